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
// Both are HBM streams (0.5625 bytes in, 2 bytes out per value). Each thread
// converts 32 (NVFP4) or 16 (E8M0) consecutive values: one coalesced packed
// load, exact v_cvt_scalef32_pk_f32_fp4 conversions, and 16-byte streaming
// stores of the BF16 results.
#include "qhead_device.h"
#include "qhead_internal.h"

namespace qh {

constexpr int kDqThreads = 256;

// Four F32 pairs from the four bytes of w (each byte: low nibble first).
__device__ __forceinline__ void e2m1x8_to_f32(uint32_t w, float (&f)[8]) {
    const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
    f[0] = p0[0]; f[1] = p0[1]; f[2] = p1[0]; f[3] = p1[1];
    f[4] = p2[0]; f[5] = p2[1]; f[6] = p3[0]; f[7] = p3[1];
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f32_to_bf16_rne(lo) | ((uint32_t)f32_to_bf16_rne(hi) << 16);
}

typedef uint32_t u32x4s_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void store_stream16(uint16_t* p, uint32_t a, uint32_t b, uint32_t c,
                                               uint32_t d) {
    u32x4s_t v = {a, b, c, d};
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4s_t*>(p));
}

__global__ void __launch_bounds__(kDqThreads)
dequant_nvfp4_bf16_kernel(const uint8_t* __restrict__ wp, const uint8_t* __restrict__ bs, float g,
                          int64_t n, int k, uint16_t* __restrict__ out) {
    const int64_t per_row = k / 32;
    const int64_t chunks = n * per_row;
    const int64_t stride = (int64_t)gridDim.x * kDqThreads;
    for (int64_t c = (int64_t)blockIdx.x * kDqThreads + threadIdx.x; c < chunks; c += stride) {
        const int64_t v = c / per_row;
        const int j = (int)(c - v * per_row);
        const int64_t flat0 = v * k + 32 * (int64_t)j;
        const uint4 p = load_stream16(wp + flat0 / 2);
        const uint32_t sc2 = *reinterpret_cast<const uint16_t*>(bs + v * (k / 16) + 2 * j);
        const float s[2] = {__builtin_amdgcn_cvt_f32_fp8(sc2, 0),
                            __builtin_amdgcn_cvt_f32_fp8(sc2, 1)};
        const uint32_t d[4] = {p.x, p.y, p.z, p.w};
        uint32_t o[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float f[8];
            e2m1x8_to_f32(d[q], f);
            const float sq = s[q >> 1];  // dwords 0,1 hold block 0; 2,3 block 1
#pragma unroll
            for (int i = 0; i < 4; ++i)
                o[4 * q + i] = pack_bf16x2((f[2 * i] * sq) * g, (f[2 * i + 1] * sq) * g);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
            store_stream16(out + flat0 + 8 * q, o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
    }
}

__global__ void __launch_bounds__(kDqThreads)
dequant_fp4_e8m0_bf16_kernel(const uint8_t* __restrict__ wp, const uint8_t* __restrict__ scales,
                             int64_t total, int64_t block, uint16_t* __restrict__ out) {
    const int64_t chunks = total / 16;
    const int64_t stride = (int64_t)gridDim.x * kDqThreads;
    for (int64_t c = (int64_t)blockIdx.x * kDqThreads + threadIdx.x; c < chunks; c += stride) {
        const int64_t flat0 = 16 * c;
        const uint2 p = *reinterpret_cast<const uint2*>(wp + flat0 / 2);
        const uint32_t e = scales[flat0 / block];
        const float sc = (e == 0u || e == 255u) ? 0.0f : __uint_as_float(e << 23);
        uint32_t o[8];
        float f[8];
        e2m1x8_to_f32(p.x, f);
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(f[2 * i] * sc, f[2 * i + 1] * sc);
        e2m1x8_to_f32(p.y, f);
#pragma unroll
        for (int i = 0; i < 4; ++i) o[4 + i] = pack_bf16x2(f[2 * i] * sc, f[2 * i + 1] * sc);
        store_stream16(out + flat0, o[0], o[1], o[2], o[3]);
        store_stream16(out + flat0 + 8, o[4], o[5], o[6], o[7]);
    }
}

static unsigned grid_for(int64_t chunks, const DeviceInfo& dev) {
    int64_t blocks = (chunks + kDqThreads - 1) / kDqThreads;
    const int64_t cap = (int64_t)dev.num_cus * 8;
    if (blocks > cap) blocks = cap;
    return (unsigned)(blocks > 0 ? blocks : 1);
}

hipError_t run_dequant_nvfp4_bf16(const uint8_t* wp, const uint8_t* bs, float g, int64_t n, int k,
                                  uint16_t* out, const DeviceInfo& dev, hipStream_t stream) {
    hipLaunchKernelGGL(dequant_nvfp4_bf16_kernel, dim3(grid_for(n * (k / 32), dev)),
                       dim3(kDqThreads), 0, stream, wp, bs, g, n, k, out);
    return hipGetLastError();
}

hipError_t run_dequant_fp4_e8m0_bf16(const uint8_t* wp, const uint8_t* scales, int64_t total,
                                     int64_t block, uint16_t* out, const DeviceInfo& dev,
                                     hipStream_t stream) {
    hipLaunchKernelGGL(dequant_fp4_e8m0_bf16_kernel, dim3(grid_for(total / 16, dev)),
                       dim3(kDqThreads), 0, stream, wp, scales, total, block, out);
    return hipGetLastError();
}

}  // namespace qh
