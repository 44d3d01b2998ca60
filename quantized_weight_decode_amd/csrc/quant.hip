// quant.hip -- activation quantizers and load-time weight quantization.
//
//  * quant_act_e4m3: per-row dynamic E4M3 activations for the W8A8 head
//    ("w8a8_layer.rs": W8a8Ctx::proj quantizes BF16 x into the shared scratch;
//    "lm_head_fp8_rows.rs" lm_head_fp8_run: quantization is per row). One
//    workgroup per row: exact |x| maximum on BF16 bit patterns, one binary32
//    division for the scale amax/448, one binary32 division per element, then
//    round-to-nearest-even saturating E4M3 encode.
//  * quant_act_silu_e4m3: the same quantization of bf16(silu(gate) * up), the
//    down-projection activation of a SiLU FFN ("w8a8_layer.rs",
//    W8a8Ctx::silu_proj), with silu and the product in binary64.
//  * quant_q8_1: block_q8_1 activations for the Q6_K head ("lm_head_q6k.rs":
//    kquant_q8_1_rows_bf16). One thread per 32-value block.
//  * quantize_fp8_rows / quantize_nvfp4_rows / quantize_q6k_rows: load-time
//    weight preparation in the three head formats (the FP8 head's storage,
//    "lm_head_fp8_rows.rs" Fp8Weight with Fp8PerRow scales; NVFP4 blocks of
//    16 with an F32 global, "fp8_lut.rs"; Q6_K super-blocks, "lm_head_q6k.rs").
//    The pages print no quantizer; the recipes are this library's and match
//    the CPU oracle's data-preparation functions byte for byte.
//
// Divisions are IEEE binary32 (hipcc's default correctly rounded division);
// the quantizers' bytes must equal the CPU oracle's exactly.
#include "qhead_device.h"
#include "qhead_internal.h"

namespace qh {

constexpr int kQuantThreads = 256;

__device__ __forceinline__ uint32_t bf16_mag(uint32_t two) { return two & 0x7FFFu; }

// Maximum of a per-thread value over the workgroup (kQuantThreads threads).
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* red) {
    for (int off = 32; off >= 1; off >>= 1) {
        uint32_t o = __shfl_xor(v, off, 64);
        v = v > o ? v : o;
    }
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    uint32_t m = red[0];
    for (int w = 1; w < kQuantThreads / 64; ++w) m = m > red[w] ? m : red[w];
    return m;
}

__global__ void __launch_bounds__(kQuantThreads)
quant_act_e4m3_kernel(const uint16_t* __restrict__ x, int H, uint8_t* __restrict__ xq,
                      float* __restrict__ sa) {
    __shared__ uint32_t red[kQuantThreads / 64];
    const int r = blockIdx.x;
    const uint16_t* row = x + (size_t)r * H;
    uint8_t* qrow = xq + (size_t)r * H;

    uint32_t m = 0;
    for (int k = threadIdx.x * 8; k < H; k += kQuantThreads * 8) {
        const uint4 v = *reinterpret_cast<const uint4*>(row + k);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t a = bf16_mag(w[i]), b = bf16_mag(w[i] >> 16);
            m = a > m ? a : m;
            m = b > m ? b : m;
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
        const uint4 v = *reinterpret_cast<const uint4*>(row + k);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        uint32_t packed[2] = {0, 0};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float lo = __uint_as_float(w[i] << 16) / scale;
            const float hi = __uint_as_float(w[i] & 0xFFFF0000u) / scale;
            const uint32_t pair = f32_to_e4m3_rne_sat(lo) | (f32_to_e4m3_rne_sat(hi) << 8);
            packed[i >> 1] |= pair << (16 * (i & 1));
        }
        *reinterpret_cast<uint2*>(qrow + k) = make_uint2(packed[0], packed[1]);
    }
}

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

__global__ void __launch_bounds__(kQuantThreads)
quant_q8_1_kernel(const uint16_t* __restrict__ x, int rows, int H, uint8_t* __restrict__ q8) {
    const int nb = H / 32;
    const int64_t idx = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x;
    if (idx >= (int64_t)rows * nb) return;
    const int r = (int)(idx / nb);
    const int j = (int)(idx - (int64_t)r * nb);
    const uint16_t* src = x + (size_t)r * H + (size_t)j * 32;

    uint32_t w[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint4 v = *reinterpret_cast<const uint4*>(src + 8 * i);
        w[4 * i + 0] = v.x;
        w[4 * i + 1] = v.y;
        w[4 * i + 2] = v.z;
        w[4 * i + 3] = v.w;
    }
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t a = bf16_mag(w[i]), b = bf16_mag(w[i] >> 16);
        m = a > m ? a : m;
        m = b > m ? b : m;
    }
    const float amax = __uint_as_float(m << 16);
    const float d = amax / 127.0f;
    uint32_t qw[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    int sumq = 0;
    if (amax != 0.0f) {
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const uint32_t bits = (i & 1) ? (w[i >> 1] & 0xFFFF0000u) : (w[i >> 1] << 16);
            float q = __builtin_rintf(__uint_as_float(bits) / d);
            q = fminf(fmaxf(q, -127.0f), 127.0f);
            const int qi = (int)q;
            sumq += qi;
            qw[i >> 2] |= ((uint32_t)qi & 0xFFu) << (8 * (i & 3));
        }
    }
    const uint16_t d16 = __builtin_bit_cast(uint16_t, (_Float16)d);
    const uint16_t s16 = __builtin_bit_cast(uint16_t, (_Float16)(d * (float)sumq));
    uint32_t* dst = reinterpret_cast<uint32_t*>(q8 + (size_t)idx * kQ8BlockBytes);
    dst[0] = (uint32_t)d16 | ((uint32_t)s16 << 16);
#pragma unroll
    for (int i = 0; i < 8; ++i) dst[1 + i] = qw[i];
}

__global__ void __launch_bounds__(kQuantThreads)
quantize_fp8_rows_kernel(const float* __restrict__ w, int H, uint8_t* __restrict__ codes,
                         float* __restrict__ scales) {
    __shared__ uint32_t red[kQuantThreads / 64];
    const int v = blockIdx.x;
    const float* row = w + (size_t)v * H;
    uint8_t* crow = codes + (size_t)v * H;
    uint32_t m = 0;
    for (int k = threadIdx.x * 4; k < H; k += kQuantThreads * 4) {
        const uint4 q = *reinterpret_cast<const uint4*>(row + k);
        const uint32_t a[4] = {q.x & 0x7FFFFFFFu, q.y & 0x7FFFFFFFu, q.z & 0x7FFFFFFFu,
                               q.w & 0x7FFFFFFFu};
#pragma unroll
        for (int i = 0; i < 4; ++i) m = a[i] > m ? a[i] : m;
    }
    m = block_max_u32(m, red);
    const float amax = __uint_as_float(m);
    if (amax == 0.0f) {
        if (threadIdx.x == 0) scales[v] = 0.0f;
        for (int k = threadIdx.x * 4; k < H; k += kQuantThreads * 4)
            *reinterpret_cast<uint32_t*>(crow + k) = 0u;
        return;
    }
    const float s = amax / 448.0f;
    if (threadIdx.x == 0) scales[v] = s;
    for (int k = threadIdx.x * 4; k < H; k += kQuantThreads * 4) {
        const float4 q = *reinterpret_cast<const float4*>(row + k);
        const uint32_t c = f32_to_e4m3_rne_sat(q.x / s) | (f32_to_e4m3_rne_sat(q.y / s) << 8) |
                           (f32_to_e4m3_rne_sat(q.z / s) << 16) |
                           (f32_to_e4m3_rne_sat(q.w / s) << 24);
        *reinterpret_cast<uint32_t*>(crow + k) = c;
    }
}

// Round a finite FP32 value to E2M1 (0, .5, 1, 1.5, 2, 3, 4, 6): nearest, ties
// to the even code, saturating at 6, sign kept (so -0 gives nibble 8). The
// thresholds are the midpoints between neighbours; `<=` at a midpoint keeps
// the even code below it, `<` sends the tie up to the even code above.
__device__ __forceinline__ uint32_t f32_to_e2m1_rne_sat(float t) {
    const uint32_t sign = (__float_as_uint(t) >> 28) & 8u;
    const float a = fabsf(t);
    const uint32_t c = a <= 0.25f ? 0u
                     : a < 0.75f  ? 1u
                     : a <= 1.25f ? 2u
                     : a < 1.75f  ? 3u
                     : a <= 2.5f  ? 4u
                     : a < 3.5f   ? 5u
                     : a <= 5.0f  ? 6u
                                  : 7u;
    return c | sign;
}

// Load-time NVFP4 weights with global multiplier g: per block of 16 values
// of a row, scale code = e4m3(fl32(amax / fl32(6 g))), step =
// fl32(e4m3(code) * g), nibble = e2m1(fl32(w / step)) (0 where step is 0).
// One thread per block.
__global__ void __launch_bounds__(kQuantThreads)
quantize_nvfp4_rows_kernel(const float* __restrict__ w, int64_t V, int H, float g,
                           uint8_t* __restrict__ packed, uint8_t* __restrict__ bs) {
    const int nb = H / 16;
    const int64_t idx = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x;
    if (idx >= V * nb) return;
    const int64_t v = idx / nb;
    const int b = (int)(idx - v * nb);
    const float* src = w + v * H + 16 * (int64_t)b;
    float x[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float4 q = *reinterpret_cast<const float4*>(src + 4 * i);
        x[4 * i] = q.x; x[4 * i + 1] = q.y; x[4 * i + 2] = q.z; x[4 * i + 3] = q.w;
    }
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t a = __float_as_uint(x[i]) & 0x7FFFFFFFu;
        m = a > m ? a : m;
    }
    const float six_g = 6.0f * g;
    const uint32_t code = six_g == 0.0f ? 0u : f32_to_e4m3_rne_sat(__uint_as_float(m) / six_g);
    const float step = __builtin_amdgcn_cvt_f32_fp8(code, 0) * g;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t nib = step == 0.0f ? 0u : f32_to_e2m1_rne_sat(x[i] / step);
        if (i < 8) lo |= nib << (4 * i);
        else hi |= nib << (4 * (i - 8));
    }
    *reinterpret_cast<uint2*>(packed + v * (H / 2) + 8 * (int64_t)b) = make_uint2(lo, hi);
    bs[v * nb + b] = (uint8_t)code;
}

// Load-time Q6_K super-blocks (210 bytes per 256 values; the byte placement
// of q6k_gemv.hip): per 16 values s_t = fl32(amax_t / 31); d = fp16(fl32(
// max_t s_t / 127)); sc_t = clamp(rne(fl32(s_t / d)), 0, 127) (0 where d is
// 0); q = clamp(rne(fl32(w / fl32(d * sc_t))), -32, 31) + 32 (32 where the
// step is 0). One thread per super-block.
__global__ void __launch_bounds__(kQuantThreads)
quantize_q6k_rows_kernel(const float* __restrict__ w, int64_t V, int H,
                         uint8_t* __restrict__ blocks) {
    const int nsb = H / 256;
    const int64_t idx = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x;
    if (idx >= V * nsb) return;
    const float* src = w + idx * 256;  // super-block idx of row idx / nsb
    float st[16];
    float smax = 0.0f;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 q = *reinterpret_cast<const float4*>(src + 16 * t + 4 * i);
            const uint32_t a[4] = {__float_as_uint(q.x) & 0x7FFFFFFFu,
                                   __float_as_uint(q.y) & 0x7FFFFFFFu,
                                   __float_as_uint(q.z) & 0x7FFFFFFFu,
                                   __float_as_uint(q.w) & 0x7FFFFFFFu};
#pragma unroll
            for (int j = 0; j < 4; ++j) m = a[j] > m ? a[j] : m;
        }
        st[t] = __uint_as_float(m) / 31.0f;
        smax = st[t] > smax ? st[t] : smax;
    }
    const _Float16 d16 = (_Float16)(smax / 127.0f);
    const float d = (float)d16;
    uint32_t ql[32], qh[16], scw[4];
#pragma unroll
    for (int i = 0; i < 32; ++i) ql[i] = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) qh[i] = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) scw[i] = 0;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
        int sc = 0;
        if (d > 0.0f) sc = (int)fminf(fmaxf(__builtin_rintf(st[t] / d), 0.0f), 127.0f);
        scw[t >> 2] |= (uint32_t)(sc & 0xFF) << (8 * (t & 3));
        const float step = d * (float)sc;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int e = 16 * t + i;  // element within the super-block
            int q = 32;
            if (step != 0.0f)
                q = (int)fminf(fmaxf(__builtin_rintf(src[e] / step), -32.0f), 31.0f) + 32;
            const int n = e >> 7, c = (e >> 5) & 3, l = e & 31;
            const int lb = 64 * n + l + 32 * (c & 1);      // ql byte
            const int hb = 32 * n + l;                      // qh byte
            ql[lb >> 2] |= (uint32_t)((c < 2) ? (q & 15) : ((q & 15) << 4)) << (8 * (lb & 3));
            qh[hb >> 2] |= (uint32_t)(((q >> 4) & 3) << (2 * c)) << (8 * (hb & 3));
        }
    }
    // 210 bytes at a 2-byte-aligned address: 105 halfword stores.
    uint16_t* dst = reinterpret_cast<uint16_t*>(blocks + idx * kQ6KBlockBytes);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        dst[2 * i] = (uint16_t)(ql[i] & 0xFFFFu);
        dst[2 * i + 1] = (uint16_t)(ql[i] >> 16);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        dst[64 + 2 * i] = (uint16_t)(qh[i] & 0xFFFFu);
        dst[64 + 2 * i + 1] = (uint16_t)(qh[i] >> 16);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        dst[96 + 2 * i] = (uint16_t)(scw[i] & 0xFFFFu);
        dst[96 + 2 * i + 1] = (uint16_t)(scw[i] >> 16);
    }
    dst[104] = __builtin_bit_cast(uint16_t, d16);
}

hipError_t run_quant_act_e4m3(const uint16_t* x, int rows, int H, uint8_t* xq, float* sa,
                              hipStream_t stream) {
    hipLaunchKernelGGL(quant_act_e4m3_kernel, dim3(rows), dim3(kQuantThreads), 0, stream, x, H, xq,
                       sa);
    return hipGetLastError();
}

hipError_t run_quant_act_silu_e4m3(const uint16_t* gate, const uint16_t* up, int ld, int rows,
                                   int H, uint8_t* xq, float* sa, hipStream_t stream) {
    hipLaunchKernelGGL(quant_act_silu_e4m3_kernel, dim3(rows), dim3(kQuantThreads), 0, stream,
                       gate, up, ld, H, xq, sa);
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

hipError_t run_quant_q8_1(const uint16_t* x, int rows, int H, uint8_t* q8, hipStream_t stream) {
    const int64_t blocks = ((int64_t)rows * (H / 32) + kQuantThreads - 1) / kQuantThreads;
    hipLaunchKernelGGL(quant_q8_1_kernel, dim3((unsigned)blocks), dim3(kQuantThreads), 0, stream, x,
                       rows, H, q8);
    return hipGetLastError();
}

hipError_t run_quantize_nvfp4_rows(const float* w, int64_t V, int H, float g, uint8_t* packed,
                                   uint8_t* bs, hipStream_t stream) {
    const int64_t n = V * (H / 16);
    hipLaunchKernelGGL(quantize_nvfp4_rows_kernel, dim3((unsigned)((n + kQuantThreads - 1) / kQuantThreads)),
                       dim3(kQuantThreads), 0, stream, w, V, H, g, packed, bs);
    return hipGetLastError();
}

hipError_t run_quantize_q6k_rows(const float* w, int64_t V, int H, uint8_t* blocks,
                                 hipStream_t stream) {
    const int64_t n = V * (H / 256);
    hipLaunchKernelGGL(quantize_q6k_rows_kernel, dim3((unsigned)((n + kQuantThreads - 1) / kQuantThreads)),
                       dim3(kQuantThreads), 0, stream, w, V, H, blocks);
    return hipGetLastError();
}

hipError_t run_quantize_fp8_rows(const float* w, int V, int H, uint8_t* codes, float* scales,
                                 hipStream_t stream) {
    hipLaunchKernelGGL(quantize_fp8_rows_kernel, dim3(V), dim3(kQuantThreads), 0, stream, w, H,
                       codes, scales);
    return hipGetLastError();
}

}  // namespace qh
