// act_quant.hip -- activation quantizers of the W8A8 and Q6_K heads.
//
//  * quant_act_e4m3: per-row dynamic E4M3 activations for the W8A8 head
//    ("w8a8_layer.rs": W8a8Ctx::proj quantizes BF16 x into the shared scratch;
//    "lm_head_fp8_rows.rs" lm_head_fp8_run: quantization is per row). One
//    workgroup per row: exact |x| maximum on BF16 bit patterns, one binary32
//    division for the scale amax/448, one binary32 division per element, then
//    round-to-nearest-even saturating E4M3 encode.
//  * quant_q8_1: block_q8_1 activations for the Q6_K head ("lm_head_q6k.rs":
//    kquant_q8_1_rows_bf16). One thread per 32-value block.
//
// Divisions are IEEE binary32 (hipcc's default correctly rounded division);
// the bytes must equal the CPU oracle's exactly.
#include "qhead_internal.h"
#include "quant_common.h"

namespace qh {

// 1024 threads per row: one 8-value vector per thread for hidden sizes up
// to 8192, so a call of few rows is a single short pass.
constexpr int kActThreads = 1024;

__global__ void __launch_bounds__(kActThreads)
quant_act_e4m3_kernel(const uint16_t* __restrict__ x, int H, uint8_t* __restrict__ xq,
                      float* __restrict__ sa) {
    __shared__ uint32_t red[kActThreads / 64];
    const int r = blockIdx.x;
    const uint16_t* row = x + (size_t)r * H;
    uint8_t* qrow = xq + (size_t)r * H;

    uint32_t m = 0;
    for (int k = threadIdx.x * 8; k < H; k += kActThreads * 8) {
        const uint4 v = *reinterpret_cast<const uint4*>(row + k);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t a = bf16_mag(w[i]), b = bf16_mag(w[i] >> 16);
            m = a > m ? a : m;
            m = b > m ? b : m;
        }
    }
    m = block_max_u32<kActThreads>(m, red);
    const float amax = __uint_as_float(m << 16);

    if (amax == 0.0f) {
        if (threadIdx.x == 0) sa[r] = 0.0f;
        for (int k = threadIdx.x * 8; k < H; k += kActThreads * 8)
            *reinterpret_cast<uint2*>(qrow + k) = make_uint2(0, 0);
        return;
    }
    const float scale = amax / 448.0f;
    if (threadIdx.x == 0) sa[r] = scale;
    for (int k = threadIdx.x * 8; k < H; k += kActThreads * 8) {
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

hipError_t run_quant_act_e4m3(const uint16_t* x, int rows, int H, uint8_t* xq, float* sa,
                              hipStream_t stream) {
    hipLaunchKernelGGL(quant_act_e4m3_kernel, dim3(rows), dim3(kActThreads), 0, stream, x, H, xq,
                       sa);
    return hipGetLastError();
}

hipError_t run_quant_q8_1(const uint16_t* x, int rows, int H, uint8_t* q8, hipStream_t stream) {
    const int64_t blocks = ((int64_t)rows * (H / 32) + kQuantThreads - 1) / kQuantThreads;
    hipLaunchKernelGGL(quant_q8_1_kernel, dim3((unsigned)blocks), dim3(kQuantThreads), 0, stream, x,
                       rows, H, q8);
    return hipGetLastError();
}

}  // namespace qh
