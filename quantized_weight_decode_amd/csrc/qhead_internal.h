// qhead_internal.h -- host-side declarations shared by the libqhead sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qh {

struct DeviceInfo {
    int device = -1;
    int num_cus = 0;
    bool is_gfx950 = false;
};

// Attributes of the current device (cached per device id).
hipError_t current_device(DeviceInfo* out);

// FP8 W8A16 (1 <= R <= 16 rows per launch).
hipError_t run_fp8_w8a16(const uint8_t* W, const float* s, const uint16_t* x, int R, int H, int V,
                         uint16_t* out, const DeviceInfo& dev, hipStream_t stream);
// W8A8 GEMV over quantized activations (1 <= R <= 128 rows per launch).
hipError_t run_w8a8_gemv(const uint8_t* W, const float* sw, const uint8_t* xq, const float* sa,
                         int R, int H, int V, uint16_t* out, const DeviceInfo& dev,
                         hipStream_t stream, void* image);
// Bytes of the staged-activation image run_w8a8_gemv may use for `H`.
size_t w8a8_image_bytes(int H);

// Activation quantizers and weight preparation.
hipError_t run_quant_act_e4m3(const uint16_t* x, int rows, int H, uint8_t* xq, float* sa,
                              hipStream_t stream);
hipError_t run_quant_act_silu_e4m3(const uint16_t* gate, const uint16_t* up, int ld, int rows,
                                   int H, uint8_t* xq, float* sa, hipStream_t stream);
// Split over K-slices; maxbuf holds rows * kSiluMaxSlices words.
hipError_t run_quant_act_silu_e4m3_split(const uint16_t* gate, const uint16_t* up, int ld,
                                         int rows, int H, uint8_t* xq, float* sa,
                                         uint32_t* maxbuf, hipStream_t stream);
hipError_t run_silu_mul(const uint16_t* gate, const uint16_t* up, int64_t n, uint16_t* out,
                        const DeviceInfo& dev, hipStream_t stream);
hipError_t run_quant_q8_1(const uint16_t* x, int rows, int H, uint8_t* q8, hipStream_t stream);
hipError_t run_quantize_fp8_rows(const float* w, int V, int H, uint8_t* codes, float* scales,
                                 hipStream_t stream);
hipError_t run_quantize_nvfp4_rows(const float* w, int64_t V, int H, float g, uint8_t* packed,
                                   uint8_t* bs, hipStream_t stream);
hipError_t run_quantize_q6k_rows(const float* w, int64_t V, int H, uint8_t* blocks,
                                 hipStream_t stream);

// Load-time FP4 -> BF16 dequantization.
hipError_t run_dequant_nvfp4_bf16(const uint8_t* wp, const uint8_t* bs, float g, int64_t n, int k,
                                  uint16_t* out, const DeviceInfo& dev, hipStream_t stream);
hipError_t run_dequant_fp4_e8m0_bf16(const uint8_t* wp, const uint8_t* scales, int64_t total,
                                     int64_t block, uint16_t* out, const DeviceInfo& dev,
                                     hipStream_t stream);

// NVFP4 (1 <= R <= 8) and Q6_K (1 <= R <= 8).
hipError_t run_nvfp4(const uint8_t* Wp, const uint8_t* bs, const uint16_t* x, float g, int R,
                     int H, int V, uint16_t* out, const DeviceInfo& dev, hipStream_t stream);
hipError_t run_q6k(const uint8_t* blocks, const uint8_t* q8, int R, int H, int V, uint16_t* out,
                   const DeviceInfo& dev, hipStream_t stream);

// Streaming read of a whole buffer (measurement yardstick).
hipError_t run_stream_read(const uint8_t* p, int64_t bytes, uint32_t* xor_out,
                           const DeviceInfo& dev, hipStream_t stream);

constexpr int kQ8BlockBytes = 36;
constexpr int kSiluMaxSlices = 64;
constexpr int kQ6KBlockBytes = 210;

}  // namespace qh
