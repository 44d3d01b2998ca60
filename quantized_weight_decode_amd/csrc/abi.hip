// abi.hip -- the extern "C" entry points of libqhead.so (declared in
// include/qhead.h): argument validation, the row-chunk planner, the device
// check and the per-format chunk loops.
//
// Validation happens before any HIP call, so a rejected call touches no
// device state. The chunk loops advance x by done*hidden and out by
// done*vocab elements per chunk, as the chunk loops of lm_head_fp8_run
// ("lm_head_fp8_rows.rs") and lm_head_q6k_run ("lm_head_q6k.rs") do.
#include <mutex>
#include <string.h>

#include "../../include/qhead.h"
#include "qhead_internal.h"

namespace qh {

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_dev_mutex;
DeviceInfo g_dev[kMaxDevices];

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int max_rows(int32_t format) {
    switch (format) {
        case QHEAD_FMT_FP8:
            return 16;
        case QHEAD_FMT_W8A8:
            return 128;
        case QHEAD_FMT_NVFP4:
            return 16;
        case QHEAD_FMT_Q6K:
            return 8;
        default:
            return -1;
    }
}

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

int hip_status(hipError_t e) { return e == hipSuccess ? QHEAD_OK : QHEAD_ERR_HIP; }

int device_or_error(DeviceInfo* dev) {
    if (current_device(dev) != hipSuccess) return QHEAD_ERR_HIP;
    if (!dev->is_gfx950 || dev->num_cus <= 0) return QHEAD_ERR_DEVICE;
    return QHEAD_OK;
}

}  // namespace

hipError_t current_device(DeviceInfo* out) {
    int id = 0;
    hipError_t e = hipGetDevice(&id);
    if (e != hipSuccess) return e;
    if (id < 0 || id >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_dev_mutex);
    if (g_dev[id].device != id) {
        DeviceInfo info;
        info.device = id;
        e = hipDeviceGetAttribute(&info.num_cus, hipDeviceAttributeMultiprocessorCount, id);
        if (e != hipSuccess) return e;
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, id);
        if (e != hipSuccess) return e;
        info.is_gfx950 = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        g_dev[id] = info;
    }
    *out = g_dev[id];
    return hipSuccess;
}

}  // namespace qh

using namespace qh;

extern "C" {

const char* qhead_status_string(int status) {
    switch (status) {
        case QHEAD_OK:
            return "ok";
        case QHEAD_ERR_NULL:
            return "null pointer argument";
        case QHEAD_ERR_SHAPE:
            return "invalid shape (rows < 0, hidden/vocab <= 0, or hidden not a multiple of the "
                   "format's granule)";
        case QHEAD_ERR_ALIGN:
            return "pointer not aligned as required";
        case QHEAD_ERR_WORKSPACE:
            return "workspace missing or too small";
        case QHEAD_ERR_ARG:
            return "invalid argument";
        case QHEAD_ERR_DEVICE:
            return "current device is not gfx950 (MI355X)";
        case QHEAD_ERR_HIP:
            return "HIP call or kernel launch failed";
        case QHEAD_ERR_SCRATCH:
            return "size exceeds the library's fixed device scratch";
        default:
            return "unknown status";
    }
}

int qhead_max_rows_per_launch(int32_t format) {
    int m = max_rows(format);
    return m > 0 ? m : QHEAD_ERR_ARG;
}

int qhead_plan_chunks(int32_t format, int32_t rows, int32_t* chunk_rows, int32_t max_chunks) {
    const int m = max_rows(format);
    if (m <= 0) return QHEAD_ERR_ARG;
    if (rows < 0) return QHEAD_ERR_SHAPE;
    if (max_chunks < 0 || (max_chunks > 0 && chunk_rows == nullptr)) return QHEAD_ERR_NULL;
    int n = 0;
    for (int32_t done = 0; done < rows; ++n) {
        const int32_t c = (rows - done) < m ? (rows - done) : m;
        if (n < max_chunks) chunk_rows[n] = c;
        done += c;
    }
    return n;
}

int qhead_fp8_rowscale(const uint8_t* w_e4m3, const float* row_scale, const uint16_t* x_bf16,
                       int32_t rows, int32_t hidden, int32_t vocab, uint16_t* out_bf16,
                       void* stream) {
    if (rows < 0 || hidden <= 0 || vocab <= 0 || hidden % 16) return QHEAD_ERR_SHAPE;
    if (rows == 0) return QHEAD_OK;
    if (!w_e4m3 || !row_scale || !x_bf16 || !out_bf16) return QHEAD_ERR_NULL;
    if (!aligned(w_e4m3, 16) || !aligned(x_bf16, 16) || !aligned(row_scale, 4) ||
        !aligned(out_bf16, 2))
        return QHEAD_ERR_ALIGN;
    DeviceInfo dev;
    if (int st = device_or_error(&dev)) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int32_t chunk = max_rows(QHEAD_FMT_FP8);
    for (int32_t done = 0; done < rows;) {
        const int32_t m = (rows - done) < chunk ? (rows - done) : chunk;
        hipError_t e = run_fp8_w8a16(w_e4m3, row_scale, x_bf16 + (size_t)done * hidden, m, hidden,
                                     vocab, out_bf16 + (size_t)done * vocab, dev, s);
        if (e != hipSuccess) return QHEAD_ERR_HIP;
        done += m;
    }
    return QHEAD_OK;
}

int qhead_quant_act_e4m3(const uint16_t* x_bf16, int32_t rows, int32_t hidden, uint8_t* xq,
                         float* xscale, void* stream) {
    if (rows < 0 || hidden <= 0 || hidden % 16) return QHEAD_ERR_SHAPE;
    if (rows == 0) return QHEAD_OK;
    if (!x_bf16 || !xq || !xscale) return QHEAD_ERR_NULL;
    if (!aligned(x_bf16, 16) || !aligned(xq, 8) || !aligned(xscale, 4)) return QHEAD_ERR_ALIGN;
    DeviceInfo dev;
    if (int st = device_or_error(&dev)) return st;
    return hip_status(run_quant_act_e4m3(x_bf16, rows, hidden, xq, xscale,
                                         static_cast<hipStream_t>(stream)));
}

size_t qhead_w8a8_workspace_bytes(int32_t hidden) {
    if (hidden <= 0) return 0;
    return align256((size_t)128 * hidden) + align256(128 * sizeof(float)) +
           align256((size_t)128 * kSiluMaxSlices * sizeof(uint32_t)) +
           align256(w8a8_image_bytes(hidden));
}

// The W8A8 workspace: quantized activations, their scales, the SiLU per-slice
// maxima, then the staged-activation image of the GEMV.
namespace {
struct W8a8Workspace {
    uint8_t* xq;
    float* sa;
    uint32_t* maxbuf;
    void* image;
};
W8a8Workspace w8a8_workspace_parts(void* workspace, int32_t hidden) {
    W8a8Workspace w;
    uint8_t* p = static_cast<uint8_t*>(workspace);
    w.xq = p;
    p += align256((size_t)128 * hidden);
    w.sa = reinterpret_cast<float*>(p);
    p += align256(128 * sizeof(float));
    w.maxbuf = reinterpret_cast<uint32_t*>(p);
    p += align256((size_t)128 * kSiluMaxSlices * sizeof(uint32_t));
    w.image = p;
    return w;
}
}  // namespace

int qhead_w8a8_gemv(const uint8_t* w_e4m3, const float* row_scale, const uint8_t* xq,
                    const float* xscale, int32_t rows, int32_t hidden, int32_t vocab,
                    uint16_t* out_bf16, void* stream) {
    if (rows < 0 || hidden <= 0 || vocab <= 0 || hidden % 16) return QHEAD_ERR_SHAPE;
    if (rows == 0) return QHEAD_OK;
    if (!w_e4m3 || !row_scale || !xq || !xscale || !out_bf16) return QHEAD_ERR_NULL;
    if (!aligned(w_e4m3, 16) || !aligned(xq, 16) || !aligned(row_scale, 4) ||
        !aligned(xscale, 4) || !aligned(out_bf16, 2))
        return QHEAD_ERR_ALIGN;
    DeviceInfo dev;
    if (int st = device_or_error(&dev)) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int32_t chunk = max_rows(QHEAD_FMT_W8A8);
    for (int32_t done = 0; done < rows;) {
        const int32_t m = (rows - done) < chunk ? (rows - done) : chunk;
        hipError_t e = run_w8a8_gemv(w_e4m3, row_scale, xq + (size_t)done * hidden, xscale + done,
                                     m, hidden, vocab, out_bf16 + (size_t)done * vocab, dev, s,
                                     nullptr);
        if (e != hipSuccess) return QHEAD_ERR_HIP;
        done += m;
    }
    return QHEAD_OK;
}

int qhead_w8a8(const uint8_t* w_e4m3, const float* row_scale, const uint16_t* x_bf16,
               int32_t rows, int32_t hidden, int32_t vocab, uint16_t* out_bf16, void* workspace,
               size_t workspace_bytes, void* stream) {
    if (rows < 0 || hidden <= 0 || vocab <= 0 || hidden % 16) return QHEAD_ERR_SHAPE;
    if (rows == 0) return QHEAD_OK;
    if (!w_e4m3 || !row_scale || !x_bf16 || !out_bf16) return QHEAD_ERR_NULL;
    if (!aligned(w_e4m3, 16) || !aligned(x_bf16, 16) || !aligned(row_scale, 4) ||
        !aligned(out_bf16, 2))
        return QHEAD_ERR_ALIGN;
    if (!workspace || workspace_bytes < qhead_w8a8_workspace_bytes(hidden))
        return QHEAD_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return QHEAD_ERR_ALIGN;
    DeviceInfo dev;
    if (int st = device_or_error(&dev)) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const W8a8Workspace w = w8a8_workspace_parts(workspace, hidden);
    for (int32_t done = 0; done < rows;) {
        const int32_t m = (rows - done) < max_rows(QHEAD_FMT_W8A8) ? (rows - done)
                                                                  : max_rows(QHEAD_FMT_W8A8);
        hipError_t e = run_quant_act_e4m3(x_bf16 + (size_t)done * hidden, m, hidden, w.xq, w.sa, s);
        if (e != hipSuccess) return QHEAD_ERR_HIP;
        e = run_w8a8_gemv(w_e4m3, row_scale, w.xq, w.sa, m, hidden, vocab,
                          out_bf16 + (size_t)done * vocab, dev, s, w.image);
        if (e != hipSuccess) return QHEAD_ERR_HIP;
        done += m;
    }
    return QHEAD_OK;
}

int qhead_silu_mul_bf16(const uint16_t* gate, const uint16_t* up, int64_t n, uint16_t* out_bf16,
                        void* stream) {
    if (n < 0) return QHEAD_ERR_SHAPE;
    if (n == 0) return QHEAD_OK;
    if (!gate || !up || !out_bf16) return QHEAD_ERR_NULL;
    if (!aligned(gate, 2) || !aligned(up, 2) || !aligned(out_bf16, 2)) return QHEAD_ERR_ALIGN;
    DeviceInfo dev;
    if (int st = device_or_error(&dev)) return st;
    return hip_status(run_silu_mul(gate, up, n, out_bf16, dev, static_cast<hipStream_t>(stream)));
}

int qhead_quant_act_silu_e4m3(const uint16_t* gate, const uint16_t* up, int32_t ld,
                              int32_t rows, int32_t hidden, uint8_t* xq, float* xscale,
                              void* stream) {
    if (rows < 0 || hidden <= 0 || hidden % 16 || ld < hidden || ld % 8) return QHEAD_ERR_SHAPE;
    if (rows == 0) return QHEAD_OK;
    if (!gate || !up || !xq || !xscale) return QHEAD_ERR_NULL;
    if (!aligned(gate, 16) || !aligned(up, 16) || !aligned(xq, 8) || !aligned(xscale, 4))
        return QHEAD_ERR_ALIGN;
    DeviceInfo dev;
    if (int st = device_or_error(&dev)) return st;
    return hip_status(run_quant_act_silu_e4m3(gate, up, ld, rows, hidden, xq, xscale,
                                              static_cast<hipStream_t>(stream)));
}

int qhead_w8a8_silu(const uint8_t* w_e4m3, const float* row_scale, const uint16_t* gate,
                    const uint16_t* up, int32_t ld, int32_t rows, int32_t hidden, int32_t vocab,
                    uint16_t* out_bf16, void* workspace, size_t workspace_bytes, void* stream) {
    if (rows < 0 || hidden <= 0 || vocab <= 0 || hidden % 16 || ld < hidden || ld % 8)
        return QHEAD_ERR_SHAPE;
    if (rows == 0) return QHEAD_OK;
    if (!w_e4m3 || !row_scale || !gate || !up || !out_bf16) return QHEAD_ERR_NULL;
    if (!aligned(w_e4m3, 16) || !aligned(gate, 16) || !aligned(up, 16) ||
        !aligned(row_scale, 4) || !aligned(out_bf16, 2))
        return QHEAD_ERR_ALIGN;
    if (!workspace || workspace_bytes < qhead_w8a8_workspace_bytes(hidden))
        return QHEAD_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return QHEAD_ERR_ALIGN;
    DeviceInfo dev;
    if (int st = device_or_error(&dev)) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const W8a8Workspace w = w8a8_workspace_parts(workspace, hidden);
    for (int32_t done = 0; done < rows;) {
        const int32_t m = (rows - done) < max_rows(QHEAD_FMT_W8A8) ? (rows - done)
                                                                  : max_rows(QHEAD_FMT_W8A8);
        const size_t off = (size_t)done * ld;
        hipError_t e = run_quant_act_silu_e4m3_split(gate + off, up + off, ld, m, hidden, w.xq,
                                                     w.sa, w.maxbuf, s);
        if (e != hipSuccess) return QHEAD_ERR_HIP;
        e = run_w8a8_gemv(w_e4m3, row_scale, w.xq, w.sa, m, hidden, vocab,
                          out_bf16 + (size_t)done * vocab, dev, s, w.image);
        if (e != hipSuccess) return QHEAD_ERR_HIP;
        done += m;
    }
    return QHEAD_OK;
}

int qhead_nvfp4(const uint8_t* w_packed, const uint8_t* block_scale, const uint16_t* x_bf16,
                int32_t rows, int32_t hidden, int32_t vocab, uint16_t* out_bf16,
                float global_scale, void* stream) {
    if (rows < 0 || hidden <= 0 || vocab <= 0 || hidden % 32) return QHEAD_ERR_SHAPE;
    if (rows == 0) return QHEAD_OK;
    if (!w_packed || !block_scale || !x_bf16 || !out_bf16) return QHEAD_ERR_NULL;
    if (!aligned(w_packed, 16) || !aligned(block_scale, 2) || !aligned(x_bf16, 16) ||
        !aligned(out_bf16, 2))
        return QHEAD_ERR_ALIGN;
    DeviceInfo dev;
    if (int st = device_or_error(&dev)) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int32_t chunk = max_rows(QHEAD_FMT_NVFP4);
    for (int32_t done = 0; done < rows;) {
        const int32_t m = (rows - done) < chunk ? (rows - done) : chunk;
        hipError_t e = run_nvfp4(w_packed, block_scale, x_bf16 + (size_t)done * hidden,
                                 global_scale, m, hidden, vocab,
                                 out_bf16 + (size_t)done * vocab, dev, s);
        if (e != hipSuccess) return QHEAD_ERR_HIP;
        done += m;
    }
    return QHEAD_OK;
}

int qhead_quant_q8_1(const uint16_t* x_bf16, int32_t rows, int32_t hidden, void* q8_out,
                     void* stream) {
    if (rows < 0 || hidden <= 0 || hidden % 32) return QHEAD_ERR_SHAPE;
    if (rows == 0) return QHEAD_OK;
    if (!x_bf16 || !q8_out) return QHEAD_ERR_NULL;
    if (!aligned(x_bf16, 16) || !aligned(q8_out, 4)) return QHEAD_ERR_ALIGN;
    DeviceInfo dev;
    if (int st = device_or_error(&dev)) return st;
    return hip_status(run_quant_q8_1(x_bf16, rows, hidden, static_cast<uint8_t*>(q8_out),
                                     static_cast<hipStream_t>(stream)));
}

size_t qhead_q6k_workspace_bytes(int32_t hidden) {
    if (hidden <= 0) return 0;
    return align256((size_t)8 * (hidden / 32) * kQ8BlockBytes);
}

int qhead_q6k_gemv(const uint8_t* blocks, const void* q8, int32_t rows, int32_t hidden,
                   int32_t vocab, uint16_t* out_bf16, void* stream) {
    if (rows < 0 || hidden <= 0 || vocab <= 0 || hidden % 256) return QHEAD_ERR_SHAPE;
    if (rows == 0) return QHEAD_OK;
    if (!blocks || !q8 || !out_bf16) return QHEAD_ERR_NULL;
    if (!aligned(blocks, 2) || !aligned(q8, 4) || !aligned(out_bf16, 2)) return QHEAD_ERR_ALIGN;
    DeviceInfo dev;
    if (int st = device_or_error(&dev)) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const size_t q8_row = (size_t)(hidden / 32) * kQ8BlockBytes;
    const int32_t chunk = max_rows(QHEAD_FMT_Q6K);
    for (int32_t done = 0; done < rows;) {
        const int32_t m = (rows - done) < chunk ? (rows - done) : chunk;
        hipError_t e = run_q6k(blocks, static_cast<const uint8_t*>(q8) + (size_t)done * q8_row, m,
                               hidden, vocab, out_bf16 + (size_t)done * vocab, dev, s);
        if (e != hipSuccess) return QHEAD_ERR_HIP;
        done += m;
    }
    return QHEAD_OK;
}

int qhead_q6k(const uint8_t* blocks, const void* scales, const uint16_t* x_bf16, int32_t rows,
              int32_t hidden, int32_t vocab, uint16_t* out_bf16, void* workspace,
              size_t workspace_bytes, void* stream) {
    if (scales != nullptr) return QHEAD_ERR_ARG;
    if (rows < 0 || hidden <= 0 || vocab <= 0 || hidden % 256) return QHEAD_ERR_SHAPE;
    if (rows == 0) return QHEAD_OK;
    if (!blocks || !x_bf16 || !out_bf16) return QHEAD_ERR_NULL;
    if (!aligned(blocks, 2) || !aligned(x_bf16, 16) || !aligned(out_bf16, 2))
        return QHEAD_ERR_ALIGN;
    if (!workspace || workspace_bytes < qhead_q6k_workspace_bytes(hidden))
        return QHEAD_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return QHEAD_ERR_ALIGN;
    DeviceInfo dev;
    if (int st = device_or_error(&dev)) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t* q8 = static_cast<uint8_t*>(workspace);
    const int32_t chunk = max_rows(QHEAD_FMT_Q6K);
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

int qhead_quantize_nvfp4_rows(const float* w_f32, int32_t vocab, int32_t hidden,
                              float global_scale, uint8_t* w_packed, uint8_t* block_scale,
                              void* stream) {
    if (hidden <= 0 || vocab < 0 || hidden % 16) return QHEAD_ERR_SHAPE;
    if (vocab == 0) return QHEAD_OK;
    if (!w_f32 || !w_packed || !block_scale) return QHEAD_ERR_NULL;
    if (!aligned(w_f32, 16) || !aligned(w_packed, 8)) return QHEAD_ERR_ALIGN;
    DeviceInfo dev;
    if (int st = device_or_error(&dev)) return st;
    return hip_status(run_quantize_nvfp4_rows(w_f32, vocab, hidden, global_scale, w_packed,
                                              block_scale, static_cast<hipStream_t>(stream)));
}

int qhead_quantize_q6k_rows(const float* w_f32, int32_t vocab, int32_t hidden, uint8_t* blocks,
                            void* stream) {
    if (hidden <= 0 || vocab < 0 || hidden % 256) return QHEAD_ERR_SHAPE;
    if (vocab == 0) return QHEAD_OK;
    if (!w_f32 || !blocks) return QHEAD_ERR_NULL;
    if (!aligned(w_f32, 16) || !aligned(blocks, 2)) return QHEAD_ERR_ALIGN;
    DeviceInfo dev;
    if (int st = device_or_error(&dev)) return st;
    return hip_status(
        run_quantize_q6k_rows(w_f32, vocab, hidden, blocks, static_cast<hipStream_t>(stream)));
}

int qhead_dequant_nvfp4_bf16(const uint8_t* w_packed, const uint8_t* block_scale, int32_t rows,
                             int32_t cols, float global_scale, uint16_t* out_bf16, void* stream) {
    if (rows < 0 || cols <= 0 || cols % 32) return QHEAD_ERR_SHAPE;
    if (rows == 0) return QHEAD_OK;
    if (!w_packed || !block_scale || !out_bf16) return QHEAD_ERR_NULL;
    if (!aligned(w_packed, 16) || !aligned(block_scale, 2) || !aligned(out_bf16, 16))
        return QHEAD_ERR_ALIGN;
    DeviceInfo dev;
    if (int st = device_or_error(&dev)) return st;
    return hip_status(run_dequant_nvfp4_bf16(w_packed, block_scale, global_scale, rows, cols,
                                             out_bf16, dev, static_cast<hipStream_t>(stream)));
}

int qhead_dequant_fp4_e8m0_bf16(const uint8_t* w_packed, const uint8_t* scale_e8m0, int64_t total,
                                int64_t num_groups, uint16_t* out_bf16, void* stream) {
    if (total < 0 || num_groups <= 0) return QHEAD_ERR_SHAPE;
    if (total % num_groups) return QHEAD_ERR_SHAPE;
    if ((total / num_groups) % 16) return QHEAD_ERR_SHAPE;
    if (total == 0) return QHEAD_OK;
    if (!w_packed || !scale_e8m0 || !out_bf16) return QHEAD_ERR_NULL;
    if (!aligned(w_packed, 8) || !aligned(out_bf16, 16)) return QHEAD_ERR_ALIGN;
    DeviceInfo dev;
    if (int st = device_or_error(&dev)) return st;
    return hip_status(run_dequant_fp4_e8m0_bf16(w_packed, scale_e8m0, total, total / num_groups,
                                                out_bf16, dev, static_cast<hipStream_t>(stream)));
}

int qhead_quantize_fp8_rows(const float* w_f32, int32_t vocab, int32_t hidden, uint8_t* w_e4m3,
                            float* row_scale, void* stream) {
    if (hidden <= 0 || vocab < 0 || hidden % 16) return QHEAD_ERR_SHAPE;
    if (vocab == 0) return QHEAD_OK;
    if (!w_f32 || !w_e4m3 || !row_scale) return QHEAD_ERR_NULL;
    if (!aligned(w_f32, 16) || !aligned(w_e4m3, 4) || !aligned(row_scale, 4))
        return QHEAD_ERR_ALIGN;
    DeviceInfo dev;
    if (int st = device_or_error(&dev)) return st;
    return hip_status(run_quantize_fp8_rows(w_f32, vocab, hidden, w_e4m3, row_scale,
                                            static_cast<hipStream_t>(stream)));
}

int qhead_stream_read(const void* p, int64_t bytes, uint32_t* xor_out, void* stream) {
    if (bytes < 0 || bytes % 16) return QHEAD_ERR_SHAPE;
    if (bytes == 0) return QHEAD_OK;
    if (!p || !xor_out) return QHEAD_ERR_NULL;
    if (!aligned(p, 16) || !aligned(xor_out, 4)) return QHEAD_ERR_ALIGN;
    DeviceInfo dev;
    if (int st = device_or_error(&dev)) return st;
    return hip_status(run_stream_read(static_cast<const uint8_t*>(p), bytes, xor_out, dev,
                                      static_cast<hipStream_t>(stream)));
}

}  // extern "C"
