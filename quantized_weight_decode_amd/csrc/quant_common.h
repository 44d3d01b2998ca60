// quant_common.h -- helpers shared by the quantizer kernels.
#pragma once

#include "qhead_device.h"

namespace qh {

constexpr int kQuantThreads = 256;

__device__ __forceinline__ uint32_t bf16_mag(uint32_t two) { return two & 0x7FFFu; }

// Maximum of a per-thread value over the workgroup (NTHREADS threads; red
// holds NTHREADS / 64 words).
template <int NTHREADS = kQuantThreads>
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* red) {
    for (int off = 32; off >= 1; off >>= 1) {
        uint32_t o = __shfl_xor(v, off, 64);
        v = v > o ? v : o;
    }
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    uint32_t m = red[0];
    for (int w = 1; w < NTHREADS / 64; ++w) m = m > red[w] ? m : red[w];
    return m;
}

}  // namespace qh
