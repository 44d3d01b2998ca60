// stream_read.hip -- a plain streaming read of a device buffer: the yardstick
// the GEMV launches are measured against. Every byte is read once with
// coalesced 16-byte non-temporal loads in the GEMV's per-wave pattern (lane l
// takes bytes [16 l, 16 l + 16) of a 1 KiB piece), with no arithmetic beyond
// an XOR that keeps the loads alive.
#include "qhead.h"
#include "qhead_device.h"
#include "qhead_internal.h"

namespace qh {

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 4;       // 1 KiB pieces per wave and iteration
constexpr int kReadBlocksPerCu = 8;  // 32 waves per CU, as the 1-row FP8 GEMV

__global__ void __launch_bounds__(kReadThreads)
stream_read_kernel(const uint8_t* __restrict__ p, int64_t nvec, uint32_t* __restrict__ xor_out) {
    constexpr int kWaves = kReadThreads / kWave;
    constexpr int64_t kChunk = (int64_t)kWave * kReadUnroll;  // vectors per wave and stage
    const int lane = threadIdx.x & 63;
    // wave-uniform: the stage loop runs on scalar branches
    const int64_t wave = (int64_t)blockIdx.x * kWaves +
                         __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t step = (int64_t)gridDim.x * kWaves * kChunk;
    const int64_t first = wave * kChunk;
    const int64_t nstage = first < nvec ? (nvec - first + step - 1) / step : 0;
    // Loads past the end re-read the last vector (in bounds) and are masked
    // out of the XOR by a select, so no branch drains the loads in flight.
    auto load = [&](int64_t s, uint4 (&v)[kReadUnroll]) {
        const int64_t base = first + s * step;
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u)
            v[u] = load_stream16(p + 16 * min(base + u * kWave + lane, nvec - 1));
        // the fold that follows stays below these loads
        __builtin_amdgcn_sched_barrier(0);
    };
    uint32_t x = 0;
    auto fold = [&](int64_t s, const uint4 (&v)[kReadUnroll]) {
        const int64_t base = first + s * step;
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) {
            const uint32_t w = v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
            x ^= (base + u * kWave + lane < nvec) ? w : 0u;
        }
    };
    // Two stages in flight: a stage's loads are issued before the previous
    // stage is folded.
    uint4 a[kReadUnroll], b[kReadUnroll];
    if (nstage > 0) load(0, a);
    int64_t s = 0;
    for (; s + 1 < nstage; s += 2) {
        load(s + 1, b);
        fold(s, a);
        load(s + 2, a);  // past the last stage: clamped re-reads, never folded
        fold(s + 1, b);
    }
    if (s < nstage) fold(s, a);
    // One word per workgroup, written with a plain store: one atomic per
    // wave on a single word would serialize at the L2 and take longer than
    // the read itself.
    __shared__ uint32_t red[kWaves];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x ^= __shfl_xor(x, m);
    if (lane == 0) red[threadIdx.x >> 6] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t y = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) y ^= red[w];
        xor_out[blockIdx.x] = y;
    }
}

hipError_t run_stream_read(const uint8_t* p, int64_t bytes, uint32_t* xor_out,
                           const DeviceInfo& dev, hipStream_t stream) {
    const int64_t nvec = bytes / 16;
    const int64_t per_block = (int64_t)kReadThreads / kWave * kWave * kReadUnroll;
    int64_t blocks = (nvec + per_block - 1) / per_block;
    const int64_t cap = (int64_t)dev.num_cus * kReadBlocksPerCu;
    if (blocks > cap) blocks = cap;
    if (blocks > QHEAD_STREAM_READ_WORDS) blocks = QHEAD_STREAM_READ_WORDS;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(kReadThreads), 0, stream, p,
                       nvec, xor_out);
    return hipGetLastError();
}

}  // namespace qh
