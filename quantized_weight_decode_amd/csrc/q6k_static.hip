// q6k_static.hip -- the Q6_K head with its q8_1 activations kept in a
// file-scope device array instead of a caller workspace, for callers that
// cannot allocate device memory (code under graph capture, serving loops that
// forbid allocation).
//
// The array `scratch` holds the q8_1 blocks of one <= 8-row chunk for hidden
// up to kQ6KStaticMaxHidden. In host code its name is only a host-side
// stand-in: the device address is looked up once per device with
// hipGetSymbolAddress (each GPU holds its own copy at its own address) and
// only that address is passed to the kernels. Nothing in a call allocates,
// frees or clears memory: the q8_1 quantizer writes every block of a chunk
// before the GEMV reads it.
#include <mutex>

#include "../../include/qhead.h"
#include "qhead_internal.h"

namespace qh {
namespace {

constexpr int kMaxDevices = 64;
constexpr size_t kScratchBytes =
    (size_t)8 * (QHEAD_Q6K_STATIC_MAX_HIDDEN / 32) * kQ8BlockBytes;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mutex;
uint8_t* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on device `dev`, looked up on the first call
// with that device current.
hipError_t scratch_address(int dev, uint8_t** out) {
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = static_cast<uint8_t*>(p);
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

bool aligned2(const void* p, uintptr_t a) {
    return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

}  // namespace
}  // namespace qh

using namespace qh;

extern "C" int qhead_q6k_static_scratch(const uint8_t* blocks, const void* scales,
                                        const uint16_t* x_bf16, int32_t rows, int32_t hidden,
                                        int32_t vocab, uint16_t* out_bf16, void* stream) {
    if (scales != nullptr) return QHEAD_ERR_ARG;
    if (rows < 0 || hidden <= 0 || vocab <= 0 || hidden % 256) return QHEAD_ERR_SHAPE;
    if (rows == 0) return QHEAD_OK;
    if (!blocks || !x_bf16 || !out_bf16) return QHEAD_ERR_NULL;
    if (!aligned2(blocks, 2) || !aligned2(x_bf16, 16) || !aligned2(out_bf16, 2))
        return QHEAD_ERR_ALIGN;
    if (hidden > QHEAD_Q6K_STATIC_MAX_HIDDEN) return QHEAD_ERR_SCRATCH;
    DeviceInfo dev;
    if (current_device(&dev) != hipSuccess) return QHEAD_ERR_HIP;
    if (!dev.is_gfx950 || dev.num_cus <= 0) return QHEAD_ERR_DEVICE;
    uint8_t* q8 = nullptr;
    if (scratch_address(dev.device, &q8) != hipSuccess) return QHEAD_ERR_HIP;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int32_t chunk = qhead_max_rows_per_launch(QHEAD_FMT_Q6K);
    for (int32_t done = 0; done < rows;) {
        const int32_t m = (rows - done) < chunk ? (rows - done) : chunk;
        hipError_t e = run_quant_q8_1(x_bf16 + (size_t)done * hidden, m, hidden, q8, s);
        if (e != hipSuccess) return QHEAD_ERR_HIP;
        e = run_q6k(blocks, q8, m, hidden, vocab, out_bf16 + (size_t)done * vocab, dev, s);
        if (e != hipSuccess) return QHEAD_ERR_HIP;
        done += m;
    }
    return QHEAD_OK;
}
