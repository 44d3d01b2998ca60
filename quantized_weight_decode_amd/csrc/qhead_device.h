// qhead_device.h -- device helpers shared by the gfx950 kernels of libqhead.
//
// Everything here is written for CDNA4 (gfx950) wave64: the FP8/FP4 -> BF16
// converts and the BF16 dot2 are gfx950 VALU instructions, and the cross-lane
// reduction uses v_permlane32_swap / v_permlane16_swap plus DPP.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace qh {

// f(integral_constant<int, 0>) ... f(integral_constant<int, N - 1>), unrolled:
// loop bodies with compile-time slot indices (register rings of loads).
template <int N, typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl<N>(f, std::make_integer_sequence<int, N>{});
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ bf16x2_t as_bf2(uint32_t u) { return __builtin_bit_cast(bf16x2_t, u); }
__device__ __forceinline__ uint32_t as_u32(bf16x2_t v) { return __builtin_bit_cast(uint32_t, v); }

// Four E4M3FN bytes -> two packed BF16 pairs (bytes 0,1 and 2,3). Every E4M3
// value is exactly representable in BF16, so the conversion is exact.
__device__ __forceinline__ void e4m3x4_to_bf16(uint32_t w, uint32_t& lo, uint32_t& hi) {
    lo = as_u32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
    hi = as_u32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
}

// Byte `sel` (0..3) of w, two E2M1 nibbles (low nibble first) -> packed BF16
// pair. Exact.
template <int SEL>
__device__ __forceinline__ uint32_t e2m1x2_to_bf16(uint32_t w) {
    return as_u32(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, SEL));
}

// acc + a.lo * b.lo + a.hi * b.hi, BF16 pairs into FP32.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(as_bf2(a), as_bf2(b), acc, false);
}

// a.lo * b.lo + a.hi * b.hi from a zero accumulator: the same instruction
// with the inline constant 0 as its addend (the compiler's own form copies a
// zero into the accumulator register first, one more VALU operation).
__device__ __forceinline__ float dot2_bf16_zero(uint32_t a, uint32_t b) {
    float r;
    asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// Round a finite FP32 value to BF16, nearest even.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Encode a finite FP32 value as E4M3FN: nearest grid point, ties to even,
// saturating at +-448, sign kept (so -0 and negative underflow give 0x80).
// Works on the binary32 bit pattern: below 2^-6 the grid is m * 2^-9, which
// a * 512 rounded to an integer gives directly; above, the 23-bit mantissa is
// rounded to 3 bits with the carry rippling into the exponent field.
__device__ __forceinline__ uint32_t f32_to_e4m3_rne_sat(float t) {
    uint32_t u = __float_as_uint(t);
    uint32_t sign = (u >> 24) & 0x80u;
    uint32_t a = u & 0x7FFFFFFFu;
    uint32_t code;
    if (a >= 0x43E00000u) {  // |t| >= 448
        code = 0x7Eu;
    } else if (a < 0x3C800000u) {  // |t| < 2^-6
        code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
    } else {
        uint32_t keep = (a >> 20) & 7u;
        uint32_t rem = a & 0xFFFFFu;
        uint32_t up = (rem > 0x80000u) | ((rem == 0x80000u) & (keep & 1u));
        uint32_t biased = (a >> 23) - 120u;  // binary32 exponent - 127 + 7
        code = ((biased << 3) | keep) + up;
    }
    return code | sign;
}

// DPP controls (gfx9 encoding).
constexpr int kDppRowRor8 = 0x128;
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kDppQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum across the 64 lanes of a wave for N values per lane (N a power of two,
// 1..64), by one fixed pairing tree whatever N is:
//   level 0: lane l with l ^ 32      (v_permlane32_swap)
//   level 1: lane l with l ^ 16      (v_permlane16_swap)
//   level 2: lane l with l ^ 8       (DPP row_ror:8)
//   level 3: lane l with l ^ 7 within each 8 lanes (DPP row_half_mirror)
//   level 4: lane l with l ^ 2       (DPP quad_perm)
//   level 5: lane l with l ^ 1       (DPP quad_perm)
// While more than one value remains, each level also halves the values a
// lane holds (reduce-scatter): lanes whose level bit is 0 keep the lower half
// of the indices. Afterwards lane l holds in v[0] the full sum of value index
// l >> (6 - log2 N); lanes sharing that index hold identical bits. Every
// value's sum is formed by the same tree, so the result of an index does not
// depend on N or on the other values.
// One DPP level of the tree over N values per lane: reduce-scatter while N > 1
// (lanes with `BIT` set keep the upper half), plain pairwise sum at N == 1.
template <int CTRL, int BIT, int N>
__device__ __forceinline__ void dpp_level(float (&v)[N], int lane) {
    if constexpr (N >= 2) {
        const bool hi = (lane & BIT) != 0;
#pragma unroll
        for (int i = 0; i < N / 2; ++i) {
            const float mine = hi ? v[i + N / 2] : v[i];
            const float send = hi ? v[i] : v[i + N / 2];
            v[i] = mine + dpp_f32<CTRL>(send);
        }
    } else {
        v[0] = v[0] + dpp_f32<CTRL>(v[0]);
    }
}

template <int N>
__device__ __forceinline__ void permlane32_level(float (&v)[N]) {
    if constexpr (N >= 2) {
#pragma unroll
        for (int i = 0; i < N / 2; ++i) {
            auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]),
                                                      __float_as_uint(v[i + N / 2]), false, false);
            v[i] = __uint_as_float(s[0]) + __uint_as_float(s[1]);
            // The upper half is dead after this level; overwriting it lets
            // the swap work in place instead of on a copy (worth it from 4
            // values on; with 2 it only perturbs the scheduling).
            if constexpr (N >= 4) v[i + N / 2] = __uint_as_float(s[1]);
        }
    } else {
        auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[0]), __float_as_uint(v[0]),
                                                  false, false);
        v[0] = __uint_as_float(s[0]) + __uint_as_float(s[1]);
    }
}

template <int N>
__device__ __forceinline__ void permlane16_level(float (&v)[N]) {
    if constexpr (N >= 2) {
#pragma unroll
        for (int i = 0; i < N / 2; ++i) {
            auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i]),
                                                      __float_as_uint(v[i + N / 2]), false, false);
            v[i] = __uint_as_float(s[0]) + __uint_as_float(s[1]);
            // The upper half is dead after this level; overwriting it lets
            // the swap work in place instead of on a copy (worth it from 4
            // values on; with 2 it only perturbs the scheduling).
            if constexpr (N >= 4) v[i + N / 2] = __uint_as_float(s[1]);
        }
    } else {
        auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[0]), __float_as_uint(v[0]),
                                                  false, false);
        v[0] = __uint_as_float(s[0]) + __uint_as_float(s[1]);
    }
}

constexpr int half_or_one(int n) { return n >= 2 ? n / 2 : 1; }

// Views the first M entries of an array as an array of M.
template <int M, int N>
__device__ __forceinline__ float (&prefix(float (&v)[N]))[M] {
    static_assert(M <= N, "prefix longer than array");
    return *reinterpret_cast<float(*)[M]>(&v[0]);
}

// Sum across the 64 lanes of a wave for N values per lane (N a power of two,
// 1..64), by one fixed pairing tree whatever N is:
//   level 0: lane l with l ^ 32      (v_permlane32_swap)
//   level 1: lane l with l ^ 16      (v_permlane16_swap)
//   level 2: lane l with l ^ 8       (DPP row_ror:8)
//   level 3: lane l with l ^ 7 within each 8 lanes (DPP row_half_mirror)
//   level 4: lane l with l ^ 2       (DPP quad_perm)
//   level 5: lane l with l ^ 1       (DPP quad_perm)
// While more than one value remains, each level also halves the values a
// lane holds (reduce-scatter): lanes whose level bit is 0 keep the lower half
// of the indices. Afterwards lane l holds in v[0] the full sum of value index
// l >> (6 - log2 N); lanes sharing that index hold identical bits. Every
// value's sum is formed by the same tree, so the result of an index does not
// depend on N or on the other values.
template <int N>
__device__ __forceinline__ void wave_reduce_scatter(float (&v)[N], int lane) {
    static_assert(N >= 1 && N <= 64 && (N & (N - 1)) == 0, "N must be a power of two <= 64");
    constexpr int N1 = half_or_one(N);
    constexpr int N2 = half_or_one(N1);
    constexpr int N3 = half_or_one(N2);
    constexpr int N4 = half_or_one(N3);
    constexpr int N5 = half_or_one(N4);
    permlane32_level<N>(v);
    permlane16_level<N1>(prefix<N1>(v));
    dpp_level<kDppRowRor8, 8, N2>(prefix<N2>(v), lane);
    dpp_level<kDppRowHalfMirror, 4, N3>(prefix<N3>(v), lane);
    dpp_level<kDppQuadXor2, 2, N4>(prefix<N4>(v), lane);
    dpp_level<kDppQuadXor1, 1, N5>(prefix<N5>(v), lane);
}

template <int N>
struct Log2 {
    static constexpr int value = 1 + Log2<N / 2>::value;
};
template <>
struct Log2<1> {
    static constexpr int value = 0;
};

constexpr int next_pow2(int n) {
    int p = 1;
    while (p < n) p *= 2;
    return p;
}

// 16-byte streaming load of weight bytes (read once per launch: non-temporal,
// so the weight stream does not evict the activations from the caches).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// A 16-byte LDS read whose words may feed inline asm: the vector passes
// through an empty asm first, which keeps it one ds_read_b128 (the compiler
// otherwise splits such a read into 4-byte reads).
__device__ __forceinline__ uint4 lds_read16(const uint4* p) {
    u32x4_t v = *reinterpret_cast<const u32x4_t*>(p);
    asm("" : "+v"(v));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint4 load_stream16(const uint8_t* p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// BF16 MFMA 16x16x32 (A: 16 rows x 32 k, B: 32 k x 16 columns, C/D
// 16 x 16 FP32; lane l holds row/column l & 15, k 8 (l >> 4) .. + 7). It adds
// the 8 products of each 16-lane group as one step, lane groups 0..3 in
// order; a step with a single nonzero BF16 pair rounds exactly like
// v_dot2_f32_bf16 on that pair.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma_bf16(const uint4& a, const uint4& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Transpose of four dwords across the four 16-lane groups: afterwards
// register q of lane group g holds what register g of lane group q held.
__device__ __forceinline__ void xpose4(uint32_t& r0, uint32_t& r1, uint32_t& r2, uint32_t& r3) {
    auto a = __builtin_amdgcn_permlane32_swap(r0, r2, false, false);
    r0 = a[0];
    r2 = a[1];
    auto b = __builtin_amdgcn_permlane32_swap(r1, r3, false, false);
    r1 = b[0];
    r3 = b[1];
    auto d = __builtin_amdgcn_permlane16_swap(r0, r1, false, false);
    r0 = d[0];
    r1 = d[1];
    auto e = __builtin_amdgcn_permlane16_swap(r2, r3, false, false);
    r2 = e[0];
    r3 = e[1];
}

}  // namespace qh
