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

// Per-row E4M3 quantization of p = bf16(silu(gate) * up) ("w8a8_layer.rs",
// W8a8Ctx::silu_proj quantizes the SiLU product in the launch that forms it).
// One workgroup per row; p is formed twice (once for the row maximum, once
// for the codes) instead of being stored.
__global__ void __launch_bounds__(kQuantThreads)
quant_act_silu_e4m3_kernel(const uint16_t* __restrict__ gate, const uint16_t* __restrict__ up,
                           int ld, int H, uint8_t* __restrict__ xq, float* __restrict__ sa) {
    __shared__ uint32_t red[kQuantThreads / 64];
    const int r = blockIdx.x;
    const uint16_t* grow = gate + (size_t)r * ld;
    const uint16_t* urow = up + (size_t)r * ld;
    uint8_t* qrow = xq + (size_t)r * H;

    auto products = [&](int k, uint32_t (&p)[8]) {
        const uint4 gv = *reinterpret_cast<const uint4*>(grow + k);
        const uint4 uv = *reinterpret_cast<const uint4*>(urow + k);
        const uint32_t g[4] = {gv.x, gv.y, gv.z, gv.w};
        const uint32_t u[4] = {uv.x, uv.y, uv.z, uv.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p[2 * i] = silu_mul_bf16(g[i] & 0xFFFFu, u[i] & 0xFFFFu);
            p[2 * i + 1] = silu_mul_bf16(g[i] >> 16, u[i] >> 16);
        }
    };

    uint32_t m = 0;
    for (int k = threadIdx.x * 8; k < H; k += kQuantThreads * 8) {
        uint32_t p[8];
        products(k, p);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t a = bf16_mag(p[i]);
            m = a > m ? a : m;
        }
    }
    m = block_max_u32(m, red);
    const float amax = __uint_as_float(m << 16);

    if (amax == 0.0f) {
        if (threadIdx.x == 0) sa[r] = 0.0f;
        for (int k = threadIdx.x * 8; k < H; k += kQuantThreads * 8)
            *reinterpret_cast<uint2*>(qrow + k) = make_uint2(0, 0);
        return;
    }
    const float scale = amax / 448.0f;
    if (threadIdx.x == 0) sa[r] = scale;
    for (int k = threadIdx.x * 8; k < H; k += kQuantThreads * 8) {
        uint32_t p[8];
        products(k, p);
        uint32_t packed[2] = {0, 0};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t c = f32_to_e4m3_rne_sat(__uint_as_float(p[i] << 16) / scale);
            packed[i >> 2] |= c << (8 * (i & 3));
        }
        *reinterpret_cast<uint2*>(qrow + k) = make_uint2(packed[0], packed[1]);
    }
}

// The same quantization split over K-slices, for few rows: a slice of
// `slice` columns per workgroup (grid S x rows). Pass 1 writes each slice's
// largest |p| (BF16 magnitude bits) to maxbuf[r * S + s]; pass 2 takes the
// row maximum over the S slices, recomputes p and writes the codes (slice 0
// also writes the scale). The maximum does not depend on the order, so the
// bytes equal quant_act_silu_e4m3_kernel's.
__global__ void __launch_bounds__(kQuantThreads)
silu_slice_max_kernel(const uint16_t* __restrict__ gate, const uint16_t* __restrict__ up, int ld,
                      int H, int slice, uint32_t* __restrict__ maxbuf) {
    __shared__ uint32_t red[kQuantThreads / 64];
    const int s = blockIdx.x, r = blockIdx.y;
    const uint16_t* grow = gate + (size_t)r * ld;
    const uint16_t* urow = up + (size_t)r * ld;
    const int k1 = min(H, (s + 1) * slice);
    uint32_t m = 0;
    for (int k = s * slice + threadIdx.x * 8; k < k1; k += kQuantThreads * 8) {
        const uint4 gv = *reinterpret_cast<const uint4*>(grow + k);
        const uint4 uv = *reinterpret_cast<const uint4*>(urow + k);
        const uint32_t g[4] = {gv.x, gv.y, gv.z, gv.w};
        const uint32_t u[4] = {uv.x, uv.y, uv.z, uv.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t a = bf16_mag(silu_mul_bf16(g[i] & 0xFFFFu, u[i] & 0xFFFFu));
            const uint32_t b = bf16_mag(silu_mul_bf16(g[i] >> 16, u[i] >> 16));
            m = a > m ? a : m;
            m = b > m ? b : m;
        }
    }
    m = block_max_u32(m, red);
    if (threadIdx.x == 0) maxbuf[(size_t)r * gridDim.x + s] = m;
}

__global__ void __launch_bounds__(kQuantThreads)
silu_slice_quant_kernel(const uint16_t* __restrict__ gate, const uint16_t* __restrict__ up, int ld,
                        int H, int slice, const uint32_t* __restrict__ maxbuf,
                        uint8_t* __restrict__ xq, float* __restrict__ sa) {
    __shared__ uint32_t red[kQuantThreads / 64];
    const int s = blockIdx.x, r = blockIdx.y, S = gridDim.x;
    uint32_t m = 0;
    for (int j = threadIdx.x; j < S; j += kQuantThreads) {
        const uint32_t v = maxbuf[(size_t)r * S + j];
        m = v > m ? v : m;
    }
    m = block_max_u32(m, red);
    const float amax = __uint_as_float(m << 16);
    const float scale = amax / 448.0f;
    if (s == 0 && threadIdx.x == 0) sa[r] = amax == 0.0f ? 0.0f : scale;
    const uint16_t* grow = gate + (size_t)r * ld;
    const uint16_t* urow = up + (size_t)r * ld;
    uint8_t* qrow = xq + (size_t)r * H;
    const int k1 = min(H, (s + 1) * slice);
    for (int k = s * slice + threadIdx.x * 8; k < k1; k += kQuantThreads * 8) {
        uint32_t packed[2] = {0, 0};
        if (amax != 0.0f) {
            const uint4 gv = *reinterpret_cast<const uint4*>(grow + k);
            const uint4 uv = *reinterpret_cast<const uint4*>(urow + k);
            const uint32_t g[4] = {gv.x, gv.y, gv.z, gv.w};
            const uint32_t u[4] = {uv.x, uv.y, uv.z, uv.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t lo = silu_mul_bf16(g[i] & 0xFFFFu, u[i] & 0xFFFFu);
                const uint32_t hi = silu_mul_bf16(g[i] >> 16, u[i] >> 16);
                const uint32_t pair = f32_to_e4m3_rne_sat(__uint_as_float(lo << 16) / scale) |
                                      (f32_to_e4m3_rne_sat(__uint_as_float(hi << 16) / scale) << 8);
                packed[i >> 1] |= pair << (16 * (i & 1));
            }
        }
        *reinterpret_cast<uint2*>(qrow + k) = make_uint2(packed[0], packed[1]);
    }
}

hipError_t run_quant_act_silu_e4m3(const uint16_t* gate, const uint16_t* up, int ld, int rows,
                                   int H, uint8_t* xq, float* sa, hipStream_t stream) {
    hipLaunchKernelGGL(quant_act_silu_e4m3_kernel, dim3(rows), dim3(kQuantThreads), 0, stream,
                       gate, up, ld, H, xq, sa);
    return hipGetLastError();
}

hipError_t run_quant_act_silu_e4m3_split(const uint16_t* gate, const uint16_t* up, int ld,
                                         int rows, int H, uint8_t* xq, float* sa,
                                         uint32_t* maxbuf, hipStream_t stream) {
    // slices of >= 1024 columns (a multiple of 8), at most kSiluMaxSlices per row
    int slice = (H + kSiluMaxSlices - 1) / kSiluMaxSlices;
    slice = slice < 1024 ? 1024 : slice;
    slice = (slice + 7) / 8 * 8;
    const int S = (H + slice - 1) / slice;
    hipLaunchKernelGGL(silu_slice_max_kernel, dim3(S, rows), dim3(kQuantThreads), 0, stream, gate,
                       up, ld, H, slice, maxbuf);
    hipLaunchKernelGGL(silu_slice_quant_kernel, dim3(S, rows), dim3(kQuantThreads), 0, stream,
                       gate, up, ld, H, slice, maxbuf, xq, sa);
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
