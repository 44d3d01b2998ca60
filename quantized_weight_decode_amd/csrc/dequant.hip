// dequant.hip -- load-time FP4 -> BF16 dequantization on gfx950.
//
//  * dequant_nvfp4_bf16: an NVFP4 weight [n][k] (E2M1 nibbles, even flat
//    index = low nibble, one E4M3 scale per 16 consecutive values of a row,
//    one F32 global multiplier) to BF16 ("fp8_lut.rs", dequant_nvfp4_to_bf16,
//    whose kernel the page launches as one block of 256 threads per row):
//      out = bf16( fl32( (e2m1 * e4m3(scale)) * g ) ).
//    The E2M1 x E4M3 product is exact in binary32; g is applied with one
//    binary32 rounding; the BF16 rounding is to nearest even.
//  * dequant_fp4_e8m0_bf16: E2M1 with one E8M0 scale per group of `block`
//    consecutive values of a flat tensor, no global ("fp8_lut.rs",
//    dequant_nvfp4_e8m0_to_bf16 and FP8_E8M0_LUT: 2^(e-127), e = 0 and
//    e = 255 give 0): out = bf16( fl32(e2m1 * scale) ).
//
// Both are HBM streams (0.5625 bytes in, 2 bytes out per value). A lane
// converts one group of 8 consecutive values at a time: a 4-byte packed load
// and a 1-byte scale load, exact v_cvt_scalef32_pk_f32_fp4 conversions, the
// scale products in binary32, v_cvt_pk_bf16_f32 (nearest even) and one
// 16-byte streaming store. Consecutive lanes take consecutive groups, so
// every load and store instruction of a wave covers one contiguous span; a
// workgroup handles kUnroll * 256 groups per iteration with all loads issued
// before the first conversion.
#include "qhead_device.h"
#include "qhead_internal.h"

namespace qh {

constexpr int kDqThreads = 256;
constexpr int kUnroll = 4;

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4s_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Values 2Q and 2Q+1 of a group (byte Q of w, low nibble first) times s,
// then times g if kGlobal, packed to BF16.
template <int Q, bool kGlobal>
__device__ __forceinline__ uint32_t convert2(uint32_t w, float s, float g) {
    const auto p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, Q);
    float a = p[0] * s, b = p[1] * s;
    if (kGlobal) {
        a = a * g;
        b = b * g;
    }
    return pack_bf16x2(a, b);
}

template <bool kGlobal>
__device__ __forceinline__ u32x4s_t convert8(uint32_t w, float s, float g) {
    u32x4s_t o;
    o[0] = convert2<0, kGlobal>(w, s, g);
    o[1] = convert2<1, kGlobal>(w, s, g);
    o[2] = convert2<2, kGlobal>(w, s, g);
    o[3] = convert2<3, kGlobal>(w, s, g);
    return o;
}

// groups = total / 8; the scale of group i is scale_f32(sc[i / per_scale]).
template <bool kE8M0>
__global__ void __launch_bounds__(kDqThreads)
dequant_fp4_kernel(const uint32_t* __restrict__ wp, const uint8_t* __restrict__ sc, float g,
                   int64_t groups, int64_t per_scale, uint16_t* __restrict__ out) {
    const int64_t tile = (int64_t)kUnroll * kDqThreads;
    for (int64_t base = (int64_t)blockIdx.x * tile; base < groups;
         base += (int64_t)gridDim.x * tile) {
        uint32_t w[kUnroll];
        uint32_t e[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            int64_t i = base + u * kDqThreads + threadIdx.x;
            i = i < groups ? i : groups - 1;  // clamped: the store below is guarded
            w[u] = wp[i];
            // NVFP4: two groups of 8 per 16-value block scale (a shift, not
            // a 64-bit division per value)
            e[u] = sc[kE8M0 ? i / per_scale : i >> 1];
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t i = base + u * kDqThreads + threadIdx.x;
            float s;
            if (kE8M0)
                s = (e[u] == 0u || e[u] == 255u) ? 0.0f : __uint_as_float(e[u] << 23);
            else
                s = __builtin_amdgcn_cvt_f32_fp8(e[u], 0);
            const u32x4s_t o = convert8<!kE8M0>(w[u], s, g);
            if (i < groups)
                __builtin_nontemporal_store(o, reinterpret_cast<u32x4s_t*>(out + 8 * i));
        }
    }
}

static unsigned grid_for(int64_t groups, const DeviceInfo& dev) {
    const int64_t tile = (int64_t)kUnroll * kDqThreads;
    int64_t blocks = (groups + tile - 1) / tile;
    const int64_t cap = (int64_t)dev.num_cus * 8;
    if (blocks > cap) blocks = cap;
    return (unsigned)(blocks > 0 ? blocks : 1);
}

hipError_t run_dequant_nvfp4_bf16(const uint8_t* wp, const uint8_t* bs, float g, int64_t n, int k,
                                  uint16_t* out, const DeviceInfo& dev, hipStream_t stream) {
    const int64_t groups = n * (int64_t)k / 8;  // k % 32 == 0: a group never spans rows
    hipLaunchKernelGGL(dequant_fp4_kernel<false>, dim3(grid_for(groups, dev)), dim3(kDqThreads),
                       0, stream, reinterpret_cast<const uint32_t*>(wp), bs, g, groups,
                       (int64_t)2, out);
    return hipGetLastError();
}

hipError_t run_dequant_fp4_e8m0_bf16(const uint8_t* wp, const uint8_t* scales, int64_t total,
                                     int64_t block, uint16_t* out, const DeviceInfo& dev,
                                     hipStream_t stream) {
    const int64_t groups = total / 8;  // block % 16 == 0: a group never spans scale groups
    hipLaunchKernelGGL(dequant_fp4_kernel<true>, dim3(grid_for(groups, dev)), dim3(kDqThreads),
                       0, stream, reinterpret_cast<const uint32_t*>(wp), scales, 0.0f, groups,
                       block / 8, out);
    return hipGetLastError();
}

}  // namespace qh
