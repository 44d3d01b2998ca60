// silu_quant.hip -- the SiLU FFN product and its per-row E4M3 quantization,
// the activation of the W8A8 down projection ("w8a8_layer.rs",
// W8a8Ctx::silu_proj: bf16(silu(gate) * up), quantized in the launch that
// forms it). silu and the product are defined in binary64 with one BF16
// rounding; the quantization is quant_act_e4m3's (act_quant.hip).
#include "qhead_internal.h"
#include "quant_common.h"

namespace qh {

// Binary64 -> BF16, round to nearest even, one rounding (NaN -> 0x7FC0).
__device__ __forceinline__ uint32_t f64_to_bf16_rne(double v) {
    if (__builtin_isnan(v)) return 0x7FC0u;
    const uint32_t sign = __builtin_signbit(v) ? 0x8000u : 0u;
    const double a = __builtin_fabs(v);
    if (a == 0.0) return sign;
    if (__builtin_isinf(a)) return sign | 0x7F80u;
    int e;
    (void)__builtin_frexp(a, &e);  // a = f * 2^e, f in [0.5, 1)
    e -= 1;                        // a in [2^e, 2^(e+1))
    uint32_t bits;
    if (e < -126) {
        // subnormal BF16: units of 2^-133; a carry to 128 is the smallest normal
        bits = (uint32_t)__builtin_rint(__builtin_ldexp(a, 133));
    } else {
        double q = __builtin_rint(__builtin_ldexp(a, 7 - e));  // 128 .. 256
        if (q == 256.0) {
            q = 128.0;
            ++e;
        }
        bits = (e + 127 >= 255) ? 0x7F80u : (((uint32_t)(e + 127) << 7) | ((uint32_t)q - 128u));
    }
    return sign | bits;
}

// bf16(silu(g) * u) from BF16 bit patterns: silu(g) = g / (1 + exp(-g)) and
// the product in binary64, one BF16 rounding.
__device__ __forceinline__ uint32_t silu_mul_bf16_f64(uint32_t g16, uint32_t u16) {
    const double g = (double)__uint_as_float(g16 << 16);
    const double u = (double)__uint_as_float(u16 << 16);
    const double sg = g / (1.0 + exp(-g));
    return f64_to_bf16_rne(sg * u);
}

// The same value, computed in binary32 when that decides the BF16 rounding.
// expf (within 1 unit in the last place), the add, the division and the
// product leave the binary32 result within 7 units in its last place of the
// exact value, as long as no step leaves the normal range; when that result
// is at least 32 units away from the nearest BF16 rounding boundary (its low
// 16 bits differ from 0x8000 by 32 or more), the exact value, and so the
// binary64 evaluation, round to the same BF16. Otherwise (about one value in
// a thousand), and whenever silu(g) or the product lies outside
// 2^-100 <= |.| < 2^100 (zeros included), the binary64 path decides.
__device__ __forceinline__ uint32_t silu_mul_bf16(uint32_t g16, uint32_t u16) {
    const float g = __uint_as_float(g16 << 16);
    const float u = __uint_as_float(u16 << 16);
    const float sg = g / (1.0f + expf(-g));
    const float p = sg * u;
    const uint32_t bits = __float_as_uint(p);
    const uint32_t mag = bits & 0x7FFFFFFFu;
    const uint32_t smag = __float_as_uint(sg) & 0x7FFFFFFFu;
    const int low = (int)(bits & 0xFFFFu) - 0x8000;
    constexpr uint32_t kLo = 0x0D800000u, kHi = 0x71800000u;  // 2^-100, 2^100
    const bool safe = mag >= kLo && mag < kHi && smag >= kLo && smag < kHi &&
                      (low >= 32 || low <= -32);
    if (__builtin_expect(safe, 1)) return (bits + 0x7FFFu + ((bits >> 16) & 1u)) >> 16;
    return silu_mul_bf16_f64(g16, u16);
}

// out[i] = bf16(silu(gate[i]) * up[i]) over a flat range (the SiLU product on
// its own, the value the down projection quantizes).
__global__ void __launch_bounds__(kQuantThreads)
silu_mul_kernel(const uint16_t* __restrict__ gate, const uint16_t* __restrict__ up, int64_t n,
                uint16_t* __restrict__ out) {
    const int64_t stride = (int64_t)gridDim.x * kQuantThreads;
    for (int64_t i = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x; i < n; i += stride)
        out[i] = (uint16_t)silu_mul_bf16(gate[i], up[i]);
}

// Screen of |p| = |silu(g) * u| for the row maximum below:
//   0    p is a zero (g or u is zero, both finite);
//   -2   |p| <= |g u| < 2^-100 (silu(g) is at most |g| in magnitude);
//   -1   no bound established: a NaN or infinite operand, or |silu(g)| or |p|
//        outside [2^-100, 2^100);
//   else |p| within a relative 2^-16.
// The exponential and the reciprocal are the hardware approximations
// (v_exp_f32, v_rcp_f32); where silu(g) is in range, |g| log2(e) < 93, so the
// rounded argument of the exponential is off by less than 2^-16.5 and its
// value by less than 2^-17 relative; the remaining roundings add less than
// 2^-20.
__device__ __forceinline__ float silu_mul_screen(uint32_t g16, uint32_t u16) {
    const float g = __uint_as_float(g16 << 16);
    const float u = __uint_as_float(u16 << 16);
    constexpr float kLo = 0x1p-100f, kHi = 0x1p100f;
    const float e = __builtin_amdgcn_exp2f(-g * 1.44269504f);
    const float sg = g * __builtin_amdgcn_rcpf(1.0f + e);
    const float p = __builtin_fabsf(sg * u);
    const float asg = __builtin_fabsf(sg);
    // selects, not branches: every case is computed, the first that holds wins
    float r = (p >= kLo && p < kHi && asg >= kLo && asg < kHi) ? p : -1.0f;
    r = __builtin_fabsf(g) * __builtin_fabsf(u) < kLo ? -2.0f : r;
    r = ((g16 & 0x7FFFu) == 0 || (u16 & 0x7FFFu) == 0) ? 0.0f : r;
    r = ((g16 & 0x7F80u) == 0x7F80u || (u16 & 0x7F80u) == 0x7F80u) ? -1.0f : r;
    return r;
}

// Maximum over the 64 lanes of a wave (DPP within rows of 16 lanes, then the
// row swaps).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    auto mx = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
    v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppQuadXor1, 0xF, 0xF, false));
    v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppQuadXor2, 0xF, 0xF, false));
    v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowHalfMirror, 0xF, 0xF, false));
    v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowMirror, 0xF, 0xF, false));
    auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = mx(a[0], a[1]);
    auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return mx(b[0], b[1]);
}

// E consecutive BF16 values (E = 2, 4 or 8) as E / 2 words, one load.
template <int E>
__device__ __forceinline__ void load_words(const uint16_t* p, uint32_t (&w)[E / 2]) {
    if constexpr (E == 8) {
        const uint4 v = *reinterpret_cast<const uint4*>(p);
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    } else if constexpr (E == 4) {
        const uint2 v = *reinterpret_cast<const uint2*>(p);
        w[0] = v.x; w[1] = v.y;
    } else {
        w[0] = *reinterpret_cast<const uint32_t*>(p);
    }
}

__device__ __forceinline__ uint32_t half_of(const uint32_t* w, int i) {
    return (i & 1) ? w[i >> 1] >> 16 : w[i >> 1] & 0xFFFFu;
}

// Exact maximum of |p| (BF16 magnitude bits) over columns [k0, k1) of a row
// (multiples of E), for a workgroup of NT threads taking E columns each per
// step, BATCH steps at a time; every thread returns it.
// Each value is first screened (silu_mul_screen), and only unscreened values
// and those within 2^-5 of the largest screened value seen so far in the wave
// are evaluated exactly. The value attaining the maximum is among them: with
// screening error d <= 2^-16 and BF16 rounding of at most 2^-8 relative, its
// screened value is at least (1 - 2^-8)(1 - d) / ((1 + 2^-8)(1 + d)) > 1 - 2^-6
// times any other screened value, and the running wave maximum never exceeds
// the final one. Values known to be below 2^-100 are evaluated only when the
// maximum found is below 2^-100 too. So the result equals the maximum of the
// exact products.
template <int NT, int BATCH, int E>
__device__ __forceinline__ uint32_t range_max_bits(const uint16_t* grow, const uint16_t* urow,
                                                   int k0, int k1, uint32_t* red) {
    constexpr float kNear = 1.0f - 0x1p-5f;
    const int c_begin = k0 / E, c_end = k1 / E;
    uint32_t m = 0;
    float run = 0.0f;  // largest screened |p| of this wave so far
    for (int c0 = c_begin; c0 < c_end; c0 += BATCH * NT) {
        uint32_t g[BATCH][E / 2], u[BATCH][E / 2];
#pragma unroll
        for (int b = 0; b < BATCH; ++b) {
            const int cidx = c0 + b * NT + (int)threadIdx.x;
#pragma unroll
            for (int i = 0; i < E / 2; ++i) g[b][i] = u[b][i] = 0;
            if (cidx < c_end) {
                load_words<E>(grow + (size_t)cidx * E, g[b]);
                load_words<E>(urow + (size_t)cidx * E, u[b]);
            }
        }
        float a[BATCH][E];
        float tmax = 0.0f;
#pragma unroll
        for (int b = 0; b < BATCH; ++b)
#pragma unroll
            for (int i = 0; i < E; ++i) {
                a[b][i] = silu_mul_screen(half_of(g[b], i), half_of(u[b], i));
                tmax = __builtin_fmaxf(tmax, a[b][i]);
            }
        // non-negative floats order as their bit patterns
        run = __builtin_fmaxf(run, __uint_as_float(wave_max_u32(__float_as_uint(tmax))));
        const float thr = run * kNear;
#pragma unroll
        for (int b = 0; b < BATCH; ++b)
#pragma unroll
            for (int i = 0; i < E; ++i) {
                const float ai = a[b][i];
                if (ai == -1.0f || (ai > 0.0f && ai >= thr)) {
                    const uint32_t mag = bf16_mag(silu_mul_bf16(half_of(g[b], i), half_of(u[b], i)));
                    m = mag > m ? mag : m;
                }
            }
    }
    m = block_max_u32<NT>(m, red);
    if (m < 0x0D80u) {
        // the maximum may be one of the values below 2^-100 (0x0D80 is the
        // BF16 magnitude of 2^-100): evaluate those exactly too
        for (int cidx = c_begin + (int)threadIdx.x; cidx < c_end; cidx += NT) {
            uint32_t g[E / 2], u[E / 2];
            load_words<E>(grow + (size_t)cidx * E, g);
            load_words<E>(urow + (size_t)cidx * E, u);
#pragma unroll
            for (int i = 0; i < E; ++i) {
                if (silu_mul_screen(half_of(g, i), half_of(u, i)) == -2.0f) {
                    const uint32_t mag = bf16_mag(silu_mul_bf16(half_of(g, i), half_of(u, i)));
                    m = mag > m ? mag : m;
                }
            }
        }
        __syncthreads();  // every wave has read red
        m = block_max_u32<NT>(m, red);
    }
    return m;
}

// The same maximum for ranges a workgroup holds at once (at most NB steps of
// E columns per thread): every value is screened first, then the workgroup's
// largest screened value sets one threshold for all, and the candidates are
// gathered into an LDS list (cap entries; beyond it a thread evaluates its own
// candidates) so that their exact evaluations run on consecutive lanes
// instead of idling the other lanes of each wave. Ranges longer than NT * E *
// NB columns take range_max_bits.
template <int NT, int E, int NB>
__device__ __forceinline__ uint32_t range_max_bits_held(const uint16_t* grow, const uint16_t* urow,
                                                        int k0, int k1, uint32_t* red,
                                                        uint32_t* list, int cap,
                                                        uint32_t* count) {
    if (k1 - k0 > NT * E * NB) return range_max_bits<NT, 1, E>(grow, urow, k0, k1, red);
    constexpr float kNear = 1.0f - 0x1p-5f;
    const int c_begin = k0 / E, c_end = k1 / E;
    if (threadIdx.x == 0) *count = 0;
    uint32_t g[NB][E / 2], u[NB][E / 2];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const int cidx = c_begin + b * NT + (int)threadIdx.x;
#pragma unroll
        for (int i = 0; i < E / 2; ++i) g[b][i] = u[b][i] = 0;
        if (cidx < c_end) {
            load_words<E>(grow + (size_t)cidx * E, g[b]);
            load_words<E>(urow + (size_t)cidx * E, u[b]);
        }
    }
    float a[NB][E];
    float tmax = 0.0f;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < E; ++i) {
            a[b][i] = silu_mul_screen(half_of(g[b], i), half_of(u[b], i));
            tmax = __builtin_fmaxf(tmax, a[b][i]);
        }
    // non-negative floats order as their bit patterns
    const float thr = __uint_as_float(block_max_u32<NT>(__float_as_uint(tmax), red)) * kNear;
    uint32_t m = 0;
    bool tiny = false;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < E; ++i) {
            const float ai = a[b][i];
            tiny = tiny || ai == -2.0f;
            if (ai == -1.0f || (ai > 0.0f && ai >= thr)) {
                const uint32_t gi = half_of(g[b], i), ui = half_of(u[b], i);
                const uint32_t slot = atomicAdd(count, 1u);
                if ((int)slot < cap) {
                    list[slot] = gi | (ui << 16);
                } else {
                    const uint32_t mag = bf16_mag(silu_mul_bf16(gi, ui));
                    m = mag > m ? mag : m;
                }
            }
        }
    __syncthreads();
    const int n = min((int)*count, cap);
    for (int j = threadIdx.x; j < n; j += NT) {
        const uint32_t e = list[j];
        const uint32_t mag = bf16_mag(silu_mul_bf16(e & 0xFFFFu, e >> 16));
        m = mag > m ? mag : m;
    }
    m = block_max_u32<NT>(m, red + NT / 64);
    if (m < 0x0D80u) {
        // the maximum may be one of the values below 2^-100 (0x0D80 is the
        // BF16 magnitude of 2^-100): evaluate those exactly too
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int i = 0; i < E; ++i) {
                if (a[b][i] == -2.0f) {
                    const uint32_t mag = bf16_mag(silu_mul_bf16(half_of(g[b], i), half_of(u[b], i)));
                    m = mag > m ? mag : m;
                }
            }
        m = block_max_u32<NT>(m, red + 2 * (NT / 64));
    }
    return m;
}

// Codes of columns [kf, k1) of a row for the row maximum bits m (amax =
// BF16 value of m, scale = amax / 448), E per thread per step starting at
// column kf; the first step's operands come preloaded (gf, uf).
template <int NT, int E>
__device__ __forceinline__ void encode_range(const uint16_t* grow, const uint16_t* urow,
                                             uint8_t* qrow, int kf, int k1, uint32_t m,
                                             const uint32_t (&gf)[E / 2],
                                             const uint32_t (&uf)[E / 2]) {
    const float amax = __uint_as_float(m << 16);
    const float scale = amax / 448.0f;
    for (int k = kf; k < k1; k += NT * E) {
        uint32_t packed[(E + 3) / 4] = {};
        if (amax != 0.0f) {
            uint32_t g[E / 2], u[E / 2];
            if (k == kf) {
#pragma unroll
                for (int i = 0; i < E / 2; ++i) {
                    g[i] = gf[i];
                    u[i] = uf[i];
                }
            } else {
                load_words<E>(grow + k, g);
                load_words<E>(urow + k, u);
            }
#pragma unroll
            for (int i = 0; i < E; ++i) {
                const uint32_t pv = silu_mul_bf16(half_of(g, i), half_of(u, i));
                const uint32_t code = f32_to_e4m3_rne_sat(__uint_as_float(pv << 16) / scale);
                packed[i >> 2] |= code << (8 * (i & 3));
            }
        }
        if constexpr (E == 8)
            *reinterpret_cast<uint2*>(qrow + k) = make_uint2(packed[0], packed[1]);
        else if constexpr (E == 4)
            *reinterpret_cast<uint32_t*>(qrow + k) = packed[0];
        else
            *reinterpret_cast<uint16_t*>(qrow + k) = (uint16_t)packed[0];
    }
}

// The scale of a row from its maximum bits: amax / 448 (0 for amax = 0).
__device__ __forceinline__ float row_scale_of(uint32_t m) {
    const float amax = __uint_as_float(m << 16);
    return amax == 0.0f ? 0.0f : amax / 448.0f;
}

// Per-row E4M3 quantization of p = bf16(silu(gate) * up) ("w8a8_layer.rs",
// W8a8Ctx::silu_proj quantizes the SiLU product in the launch that forms
// it), in one launch: grid (S, rows), every workgroup finds the whole row's
// amax = max_k |p[k]| itself (range_max_bits), then encodes its slice of
// `slice` columns (slice 0 also writes the scale). The codes equal those of
// the plain definition: max of the exact products, then each product divided
// by amax / 448 and encoded.
constexpr int kSiluFusedThreads = 1024;
constexpr int kSiluListCap = 1024;
__global__ void __launch_bounds__(kSiluFusedThreads)
silu_quant_kernel(const uint16_t* __restrict__ gate, const uint16_t* __restrict__ up, int ld, int H,
                  int slice, uint8_t* __restrict__ xq, float* __restrict__ sa) {
    __shared__ uint32_t red[3 * (kSiluFusedThreads / 64)];
    __shared__ uint32_t list[kSiluListCap];
    __shared__ uint32_t count;
    const int s = blockIdx.x, r = blockIdx.y;
    const uint16_t* grow = gate + (size_t)r * ld;
    const uint16_t* urow = up + (size_t)r * ld;
    // this thread's first chunk of the slice, loaded now so that its latency
    // passes during the row maximum
    const int k1 = min(H, (s + 1) * slice);
    const int kf = s * slice + (int)threadIdx.x * 2;
    uint32_t gf[1] = {0}, uf[1] = {0};
    if (kf < k1) {
        load_words<2>(grow + kf, gf);
        load_words<2>(urow + kf, uf);
    }
    const uint32_t m = range_max_bits_held<kSiluFusedThreads, 8, 3>(grow, urow, 0, H, red, list,
                                                                    kSiluListCap, &count);
    if (s == 0 && threadIdx.x == 0) sa[r] = row_scale_of(m);
    encode_range<kSiluFusedThreads, 2>(grow, urow, xq + (size_t)r * H, kf, k1, m, gf, uf);
}

// The same quantization in two launches over K-slices (grid S x rows), for
// the few-row calls where one launch would repeat the row's screening in every
// workgroup: the first writes each slice's maximum bits to maxbuf[r * S + s],
// the second takes the row's maximum over its S words and encodes its slice.
// A thread takes 2 columns, so that the exact evaluations of a slice are
// spread over all its lanes. The maximum does not depend on the order, so the
// bytes equal silu_quant_kernel's.
constexpr int kSiluSliceCols = 2 * kQuantThreads;
__global__ void __launch_bounds__(kQuantThreads)
silu_slice_max_kernel(const uint16_t* __restrict__ gate, const uint16_t* __restrict__ up, int ld,
                      int H, uint32_t* __restrict__ maxbuf) {
    __shared__ uint32_t red[3 * (kQuantThreads / 64)];
    __shared__ uint32_t list[kSiluSliceCols];
    __shared__ uint32_t count;
    const int s = blockIdx.x, r = blockIdx.y;
    const uint32_t m = range_max_bits_held<kQuantThreads, 2, 1>(
        gate + (size_t)r * ld, up + (size_t)r * ld, s * kSiluSliceCols,
        min(H, (s + 1) * kSiluSliceCols), red, list, kSiluSliceCols, &count);
    if (threadIdx.x == 0) maxbuf[(size_t)r * gridDim.x + s] = m;
}

__global__ void __launch_bounds__(kQuantThreads)
silu_slice_quant_kernel(const uint16_t* __restrict__ gate, const uint16_t* __restrict__ up, int ld,
                        int H, const uint32_t* __restrict__ maxbuf, uint8_t* __restrict__ xq,
                        float* __restrict__ sa) {
    __shared__ uint32_t red[kQuantThreads / 64];
    const int s = blockIdx.x, r = blockIdx.y, S = gridDim.x;
    const uint16_t* grow = gate + (size_t)r * ld;
    const uint16_t* urow = up + (size_t)r * ld;
    const int k1 = min(H, (s + 1) * kSiluSliceCols);
    const int kf = s * kSiluSliceCols + (int)threadIdx.x * 2;
    uint32_t gf[1] = {0}, uf[1] = {0};
    if (kf < k1) {
        load_words<2>(grow + kf, gf);
        load_words<2>(urow + kf, uf);
    }
    uint32_t m = 0;
    for (int j = threadIdx.x; j < S; j += kQuantThreads) {
        const uint32_t v = maxbuf[(size_t)r * S + j];
        m = v > m ? v : m;
    }
    m = block_max_u32(m, red);
    if (s == 0 && threadIdx.x == 0) sa[r] = row_scale_of(m);
    encode_range<kQuantThreads, 2>(grow, urow, xq + (size_t)r * H, kf, k1, m, gf, uf);
}

hipError_t run_quant_act_silu_e4m3(const uint16_t* gate, const uint16_t* up, int ld, int rows,
                                   int H, uint8_t* xq, float* sa, hipStream_t stream) {
    // About 512 workgroups over the rows, slices of >= 1024 columns (a
    // multiple of 8): every workgroup repeats the row's screening pass, so
    // many rows take few slices each.
    int S = (512 + rows - 1) / rows;
    const int smax = (H + 1023) / 1024;
    S = S < 1 ? 1 : (S > smax ? smax : S);
    int slice = (H + S - 1) / S;
    slice = (slice + 7) / 8 * 8;
    S = (H + slice - 1) / slice;
    hipLaunchKernelGGL(silu_quant_kernel, dim3(S, rows), dim3(kSiluFusedThreads), 0, stream, gate,
                       up, ld, H, slice, xq, sa);
    return hipGetLastError();
}

hipError_t run_quant_act_silu_e4m3_split(const uint16_t* gate, const uint16_t* up, int ld,
                                         int rows, int H, uint8_t* xq, float* sa,
                                         uint32_t* maxbuf, hipStream_t stream) {
    const int S = (H + kSiluSliceCols - 1) / kSiluSliceCols;
    // rows longer than kSiluMaxSlices slices: the one-launch form
    if (S > kSiluMaxSlices) return run_quant_act_silu_e4m3(gate, up, ld, rows, H, xq, sa, stream);
    hipLaunchKernelGGL(silu_slice_max_kernel, dim3(S, rows), dim3(kQuantThreads), 0, stream, gate,
                       up, ld, H, maxbuf);
    hipLaunchKernelGGL(silu_slice_quant_kernel, dim3(S, rows), dim3(kQuantThreads), 0, stream,
                       gate, up, ld, H, maxbuf, xq, sa);
    return hipGetLastError();
}

hipError_t run_silu_mul(const uint16_t* gate, const uint16_t* up, int64_t n, uint16_t* out,
                        const DeviceInfo& dev, hipStream_t stream) {
    int64_t blocks = (n + kQuantThreads - 1) / kQuantThreads;
    if (blocks > (int64_t)dev.num_cus * 16) blocks = (int64_t)dev.num_cus * 16;
    hipLaunchKernelGGL(silu_mul_kernel, dim3((unsigned)blocks), dim3(kQuantThreads), 0, stream,
                       gate, up, n, out);
    return hipGetLastError();
}

}  // namespace qh
