// weight_prep.hip -- load-time weight quantization in the three head formats
// (the FP8 head's storage, "lm_head_fp8_rows.rs" Fp8Weight with Fp8PerRow
// scales; NVFP4 blocks of 16 with an F32 global, "fp8_lut.rs"; Q6_K
// super-blocks, "lm_head_q6k.rs"). The pages print no quantizer; the recipes
// are this library's and match the CPU oracle's data-preparation functions
// byte for byte (binary32 divisions are correctly rounded).
#include "qhead_internal.h"
#include "quant_common.h"

namespace qh {

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
