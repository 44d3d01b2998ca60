/*
 * qhead.h -- C ABI of libqhead.so: few-row quantized-weight GEMV for an LM
 * output head on AMD Instinct MI355X (gfx950).
 *
 * The head turns `rows` BF16 hidden vectors into BF16 logits[rows][vocab]
 * against a resident low-precision weight, reading the weight once per
 * launch. Four weight formats are served:
 *
 *   qhead_fp8_rowscale  FP8 E4M3 weights, one F32 scale per weight row
 *                       (W8A16), one weight pass per <= 16 rows.
 *   qhead_w8a8          the same E4M3 bytes and scales, activations first
 *                       quantized per row to E4M3 (qhead_quant_act_e4m3),
 *                       then an FP8 x FP8 dot, in <= 128-row calls.
 *   qhead_nvfp4         NVFP4: E2M1 nibbles, E4M3 scale per 16 weights,
 *                       F32 global multiplier (W4A16), <= 16 rows per pass.
 *   qhead_q6k           Q6_K 210-byte super-blocks with activations first
 *                       quantized to q8_1 blocks (qhead_quant_q8_1), <= 8
 *                       rows per pass.
 *
 * Next to the head: qhead_w8a8_silu, the W8A8 down projection of a SiLU FFN
 * (bf16(silu(gate) * up) quantized per row, then the W8A8 GEMV); the
 * load-time conversions qhead_dequant_nvfp4_bf16 and
 * qhead_dequant_fp4_e8m0_bf16; and device-side weight preparation
 * (qhead_quantize_fp8_rows / _nvfp4_rows / _q6k_rows).
 *
 * Conventions (all entry points):
 *  - Pointers are device memory owned by the caller, unless stated. The
 *    library allocates nothing and keeps no state between calls apart from a
 *    per-device cache of device attributes.
 *  - Matrices are row-major and contiguous: x is [rows][hidden] BF16 (raw
 *    uint16 bits), out is [rows][vocab] BF16, weights are [vocab][...].
 *  - `stream` is a hipStream_t (0 = the null stream). Calls only enqueue work
 *    on it and never synchronize; a fault in a kernel surfaces at the
 *    caller's next synchronization.
 *  - Any row count >= 0 is accepted and split into launches inside the call
 *    (qhead_plan_chunks gives the split); rows == 0 returns QHEAD_OK once the
 *    shape arguments are valid, without examining the pointers (an empty
 *    tensor's NULL data pointer is fine), and enqueues nothing. Row r's
 *    logits are bit-identical whatever the number of rows in the call and
 *    however the call is split.
 *  - On a validation error nothing is enqueued and a negative status is
 *    returned (qhead_status_string names it).
 *  - Offsets are computed in 64 bits; vocab * hidden may exceed 2^31.
 *  - Concurrent calls are safe except that calls sharing one workspace must
 *    be ordered on one stream.
 *
 * Numerical contract (checked against a binary64 CPU oracle): with ref the
 * exact dot product of the dequantized operands times the scales,
 *   |out - ref| <= 2^-7 |ref| + 1e-4 sum_k |x_k w_k|
 * (plus 2^-134, half of BF16's subnormal spacing, for logits BF16 can only
 * hold as subnormals), and the quantizers' and converters' bytes are
 * exactly those of the oracle.
 *
 * Passages cited below are items of the pages "lm_head_fp8_rows.rs",
 * "w8a8_layer.rs", "fp8_lut.rs", "lm_head_q6k.rs" and "w4a16_gemv_tiers.rs".
 */
#ifndef QHEAD_H
#define QHEAD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define QHEAD_OK 0
#define QHEAD_ERR_NULL (-1)      /* a required pointer is NULL */
#define QHEAD_ERR_SHAPE (-2)     /* rows < 0, hidden/vocab <= 0, or hidden not a
                                    multiple of the format's granule */
#define QHEAD_ERR_ALIGN (-3)     /* a pointer lacks the alignment stated below */
#define QHEAD_ERR_WORKSPACE (-4) /* workspace missing or smaller than required */
#define QHEAD_ERR_ARG (-5)       /* other invalid argument (e.g. non-NULL scales
                                    for Q6_K, unknown format) */
#define QHEAD_ERR_DEVICE (-6)    /* current device is not gfx950 */
#define QHEAD_ERR_HIP (-7)       /* a HIP call or kernel launch failed */
#define QHEAD_ERR_SCRATCH (-8)   /* the call needs more than the library's fixed
                                    device scratch (qhead_q6k_static_scratch) */

/* Formats for qhead_plan_chunks / qhead_max_rows_per_launch. */
#define QHEAD_FMT_FP8 0
#define QHEAD_FMT_W8A8 1
#define QHEAD_FMT_NVFP4 2
#define QHEAD_FMT_Q6K 3

/* Human-readable name of a status code (static string). */
const char* qhead_status_string(int status);

/* Rows one weight pass serves for `format`: 16 (FP8 W8A16, the multi-row
 * kernels of "lm_head_fp8_rows.rs" module doc), 128 (W8A8, W8A8_MAX_ROWS of
 * the same doc), 16 (NVFP4: the narrow tiers W4A16_BATCHM_WIDTHS and the
 * 9..16-row batch16 tier of "w4a16_gemv_tiers.rs"), 8 (Q6_K, MAX_M of
 * "lm_head_q6k.rs"). Negative
 * status for an unknown format. */
int qhead_max_rows_per_launch(int32_t format);

/* The split of a `rows`-row call into launches: min(left, max_rows) each, in
 * order, as the chunk loops of lm_head_fp8_run ("lm_head_fp8_rows.rs") and
 * lm_head_q6k_run ("lm_head_q6k.rs") advance x by done*hidden and out by
 * done*vocab. Writes up to `max_chunks` chunk sizes to `chunk_rows` (host
 * memory; may be NULL when max_chunks is 0) and returns the number of chunks
 * (0 for rows == 0), or a negative status. Pure host function. */
int qhead_plan_chunks(int32_t format, int32_t rows, int32_t* chunk_rows, int32_t max_chunks);

/* FP8 W8A16 head ("lm_head_fp8_rows.rs": module doc, LmHeadRows,
 * lm_head_fp8_run):
 *   out[r][v] = bf16( fl32( acc[r][v] * row_scale[v] ) ),
 *   acc[r][v] = sum_k x[r][k] * e4m3(w[v][k]) accumulated in FP32.
 *  w_e4m3    [vocab][hidden] OCP E4M3FN bytes, 16-byte aligned.
 *  row_scale [vocab] F32.
 *  x_bf16    [rows][hidden] BF16, 16-byte aligned.
 *  out_bf16  [rows][vocab] BF16, 2-byte aligned.
 *  hidden must be a multiple of 16. */
int qhead_fp8_rowscale(const uint8_t* w_e4m3, const float* row_scale, const uint16_t* x_bf16,
                       int32_t rows, int32_t hidden, int32_t vocab, uint16_t* out_bf16,
                       void* stream);

/* Per-row dynamic E4M3 quantization of BF16 activations, the first step of
 * W8A8 ("w8a8_layer.rs": W8a8Ctx::proj quantizes into the shared scratch; per
 * row, "lm_head_fp8_rows.rs" lm_head_fp8_run):
 *   xscale[r] = fl32(amax_r / 448), xq[r][k] = e4m3_rne_sat(fl32(x[r][k] / xscale[r]))
 * with ties to even, saturation at +-448, the sign kept (-0 -> 0x80), and an
 * all-zero row giving xscale 0 and codes 0x00. Bit-exact contract.
 *  x_bf16 [rows][hidden], 16-byte aligned; xq [rows][hidden] bytes, 8-byte
 *  aligned; xscale [rows] F32. hidden must be a multiple of 16. */
int qhead_quant_act_e4m3(const uint16_t* x_bf16, int32_t rows, int32_t hidden, uint8_t* xq,
                         float* xscale, void* stream);

/* Bytes of workspace qhead_w8a8 and qhead_w8a8_silu need for `hidden`: the
 * quantized activations and scales of one 128-row chunk (W8a8Scratch of
 * "w8a8_layer.rs", sized by max_k and W8A8_MAX_ROWS), 32 KiB of per-slice
 * maxima for the SiLU path and the chunk's activations staged as BF16 for
 * the GEMV (64 KiB per 256 of hidden), 256-byte aligned parts. 0 for
 * hidden <= 0. */
size_t qhead_w8a8_workspace_bytes(int32_t hidden);

/* FP8 GEMV over already-quantized activations (the second step of W8A8,
 * "w8a8_layer.rs" W8a8Ctx::proj / silu_proj):
 *   out[r][v] = bf16( fl32( fl32(acc * xscale[r]) * row_scale[v] ) ),
 *   acc = sum_k e4m3(xq[r][k]) * e4m3(w[v][k]) in FP32.
 *  xq [rows][hidden] E4M3 codes, 16-byte aligned; xscale [rows] F32; other
 *  arguments as qhead_fp8_rowscale. */
int qhead_w8a8_gemv(const uint8_t* w_e4m3, const float* row_scale, const uint8_t* xq,
                    const float* xscale, int32_t rows, int32_t hidden, int32_t vocab,
                    uint16_t* out_bf16, void* stream);

/* W8A8 head: the same E4M3 weight bytes and row scales as qhead_fp8_rowscale
 * read in place ("lm_head_fp8_rows.rs" set_lm_head_w8a8), activations
 * quantized per row (qhead_quant_act_e4m3) into `workspace`, then
 * qhead_w8a8_gemv, in chunks of <= 128 rows. workspace: device memory of at
 * least qhead_w8a8_workspace_bytes(hidden) bytes, 256-byte aligned, used
 * across the chunks of this call; calls sharing it must be ordered on one
 * stream. */
int qhead_w8a8(const uint8_t* w_e4m3, const float* row_scale, const uint16_t* x_bf16,
               int32_t rows, int32_t hidden, int32_t vocab, uint16_t* out_bf16, void* workspace,
               size_t workspace_bytes, void* stream);

/* The SiLU FFN product on its own ("w8a8_layer.rs", W8a8Ctx::silu_proj:
 * bf16(silu(gate) * up)): out[i] = bf16( (g / (1 + exp(-g))) * u ) with
 * g = gate[i], u = up[i], silu and product in binary64, one BF16 rounding
 * (nearest even) -- the value qhead_quant_act_silu_e4m3 quantizes. gate, up,
 * out: n BF16 values, 2-byte aligned. Finite inputs are assumed. */
int qhead_silu_mul_bf16(const uint16_t* gate, const uint16_t* up, int64_t n, uint16_t* out_bf16,
                        void* stream);

/* Per-row E4M3 quantization of the SiLU FFN product, the down projection's
 * activation ("w8a8_layer.rs", W8a8Ctx::silu_proj: bf16(silu(gate) * up)
 * quantized in the launch that forms it):
 *   p[r][k] = bf16( (g / (1 + exp(-g))) * u ), g = gate[r*ld + k],
 *             u = up[r*ld + k], silu and product in binary64, one BF16
 *             rounding (nearest even);
 *   then xscale[r] and xq[r][k] from p exactly as qhead_quant_act_e4m3.
 *  gate, up: [rows][ld] BF16, 16-byte aligned, ld >= hidden, ld % 8 == 0;
 *  columns k >= hidden are not read. xq [rows][hidden], 8-byte aligned;
 *  xscale [rows]. hidden must be a multiple of 16. Finite products are
 *  assumed (an infinite p gives an unspecified row). */
int qhead_quant_act_silu_e4m3(const uint16_t* gate, const uint16_t* up, int32_t ld,
                              int32_t rows, int32_t hidden, uint8_t* xq, float* xscale,
                              void* stream);

/* W8A8 down projection of a SiLU FFN ("w8a8_layer.rs", W8a8Ctx::silu_proj):
 * qhead_quant_act_silu_e4m3 into `workspace`, then qhead_w8a8_gemv, in
 * chunks of <= 128 rows. The weight is [vocab][hidden] here with vocab = the
 * projection's output width and hidden = the FFN width; other arguments as
 * qhead_w8a8 and qhead_quant_act_silu_e4m3. */
int qhead_w8a8_silu(const uint8_t* w_e4m3, const float* row_scale, const uint16_t* gate,
                    const uint16_t* up, int32_t ld, int32_t rows, int32_t hidden, int32_t vocab,
                    uint16_t* out_bf16, void* workspace, size_t workspace_bytes, void* stream);

/* NVFP4 W4A16 head ("fp8_lut.rs" dequant_nvfp4_to_bf16 for the value
 * formula; "w4a16_gemv_tiers.rs" for the row tiers, here one weight pass per
 * <= 16 rows):
 *   out[r][v] = bf16( fl32( global_scale * sum_b fl32(e4m3(bs[v][b]) * p_b) ) ),
 *   p_b = sum_{k in block b} x[r][k] * e2m1(nib(v,k)) in FP32,
 * blocks b of 16 consecutive k; nib(v,k) is the low nibble of
 * w_packed[v][k/2] for even k, the high nibble for odd k.
 *  w_packed [vocab][hidden/2], 16-byte aligned; block_scale [vocab][hidden/16]
 *  E4M3 bytes, 2-byte aligned; global_scale is the direct multiplier (a
 *  caller holding the reciprocal convention passes 1/g, or 0 when g == 0).
 *  hidden must be a multiple of 32. */
int qhead_nvfp4(const uint8_t* w_packed, const uint8_t* block_scale, const uint16_t* x_bf16,
                int32_t rows, int32_t hidden, int32_t vocab, uint16_t* out_bf16,
                float global_scale, void* stream);

/* block_q8_1 quantization of BF16 rows ("lm_head_q6k.rs":
 * kquant_q8_1_rows_bf16 quantises hidden rows to block_q8_1). Per 32 values:
 * d = fl32(amax/127), q = clamp(rne(fl32(x/d)), -127, 127); the 36-byte block
 * holds fp16(d) (bytes 0-1), fp16(fl32(d * sum q)) (bytes 2-3) and q (4-35).
 * All-zero blocks give d = 0, q = 0. Bit-exact contract.
 *  q8_out [rows][hidden/32] blocks of 36 bytes, 4-byte aligned; hidden must
 *  be a multiple of 32. */
int qhead_quant_q8_1(const uint16_t* x_bf16, int32_t rows, int32_t hidden, void* q8_out,
                     void* stream);

/* Bytes of workspace qhead_q6k needs: q8_1 blocks for 8 rows (q8_scratch of
 * LmHeadQ6k, "lm_head_q6k.rs"). 0 for hidden <= 0. */
size_t qhead_q6k_workspace_bytes(int32_t hidden);

/* Q6_K x q8_1 GEMV over already-quantized activations:
 *   out[r][v] = bf16( sum_b fp16(d[v][b]) * sum_j fp16(d8[r][j]) *
 *                     sum_{t in j} sc[v][b][t] * sum_{i in t} (q6 - 32) * q8 )
 * with exact integer inner sums and FP32 outer sums.
 *  blocks [vocab][hidden/256] Q6_K super-blocks of 210 bytes (ql[128],
 *  qh[64], int8 scales[16], fp16 d), 2-byte aligned; q8 as written by
 *  qhead_quant_q8_1, 4-byte aligned. hidden must be a multiple of 256. */
int qhead_q6k_gemv(const uint8_t* blocks, const void* q8, int32_t rows, int32_t hidden,
                   int32_t vocab, uint16_t* out_bf16, void* stream);

/* Q6_K head ("lm_head_q6k.rs": set_lm_head_q6k requires hidden % 256 == 0;
 * lm_head_q6k_run quantises each <= 8-row group to q8_1, then runs the
 * GEMV). `scales` must be NULL (Q6_K blocks carry their own scales).
 * workspace: at least qhead_q6k_workspace_bytes(hidden) bytes, 256-byte
 * aligned, shared by the chunks of this call. */
int qhead_q6k(const uint8_t* blocks, const void* scales, const uint16_t* x_bf16, int32_t rows,
              int32_t hidden, int32_t vocab, uint16_t* out_bf16, void* workspace,
              size_t workspace_bytes, void* stream);

/* qhead_q6k without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops or harnesses
 * that forbid hipMalloc). The q8_1 activations of each <= 8-row chunk go to a
 * fixed device array inside the library, 8 * (QHEAD_Q6K_STATIC_MAX_HIDDEN/32)
 * blocks of 36 bytes (576 KiB), one copy per GPU, held until the process
 * ends. The call allocates, frees and clears nothing; its first call on a
 * device looks up that device's copy of the array. Every call on one GPU
 * uses the same array, so calls that may overlap on one GPU (different
 * streams, or host threads) race and must be ordered by the caller. Returns
 * QHEAD_ERR_SCRATCH, enqueuing nothing, for hidden >
 * QHEAD_Q6K_STATIC_MAX_HIDDEN; otherwise arguments, results and errors are
 * those of qhead_q6k, with bit-identical logits. */
#define QHEAD_Q6K_STATIC_MAX_HIDDEN 65536
int qhead_q6k_static_scratch(const uint8_t* blocks, const void* scales, const uint16_t* x_bf16,
                             int32_t rows, int32_t hidden, int32_t vocab, uint16_t* out_bf16,
                             void* stream);

/* Weight preparation (load time, not the decode path): quantize F32 weights
 * per row to E4M3 with row scales s_v = fl32(amax_v / 448) and codes
 * e4m3_rne_sat(fl32(w / s_v)); an all-zero row gets s = 0 and codes 0.
 *  w_f32 [vocab][hidden], 16-byte aligned; w_e4m3 [vocab][hidden], 4-byte
 *  aligned; row_scale [vocab]. hidden must be a multiple of 16. */
int qhead_quantize_fp8_rows(const float* w_f32, int32_t vocab, int32_t hidden, uint8_t* w_e4m3,
                            float* row_scale, void* stream);

/* Weight preparation, NVFP4 with global multiplier g (no page prints a
 * quantizer; value formula of "fp8_lut.rs" dequant_nvfp4_to_bf16): per block
 * of 16 values of a row, scale = e4m3_rne_sat(fl32(amax / fl32(6 g))),
 * step = fl32(e4m3(scale) * g), nibble = e2m1_rne_sat(fl32(w / step)) (ties
 * to the even code, sign kept; 0 where step is 0); even k in the low nibble.
 *  w_f32 [vocab][hidden], 16-byte aligned; w_packed [vocab][hidden/2],
 *  8-byte aligned; block_scale [vocab][hidden/16]. hidden % 16 == 0. */
int qhead_quantize_nvfp4_rows(const float* w_f32, int32_t vocab, int32_t hidden,
                              float global_scale, uint8_t* w_packed, uint8_t* block_scale,
                              void* stream);

/* Weight preparation, Q6_K super-blocks (layout of qhead_q6k_gemv): per 16
 * values s_t = fl32(amax_t / 31); d = fp16(fl32(max_t s_t / 127));
 * sc_t = clamp(rne(fl32(s_t / d)), 0, 127); q = clamp(rne(fl32(w /
 * fl32(d * sc_t))), -32, 31) + 32 (32 where the step is 0).
 *  w_f32 [vocab][hidden], 16-byte aligned; blocks [vocab][hidden/256][210],
 *  2-byte aligned. hidden % 256 == 0. */
int qhead_quantize_q6k_rows(const float* w_f32, int32_t vocab, int32_t hidden, uint8_t* blocks,
                            void* stream);

/* Load-time NVFP4 -> BF16 of a [rows][cols] weight ("fp8_lut.rs",
 * dequant_nvfp4_to_bf16: value E2M1 * E4M3 block scale * global multiplier,
 * even flat index = low nibble):
 *   out = bf16_rne( fl32( (e2m1 * e4m3(scale)) * global_scale ) ).
 *  w_packed [rows][cols/2], 16-byte aligned; block_scale [rows][cols/16],
 *  2-byte aligned; out_bf16 [rows][cols], 16-byte aligned; cols % 32 == 0.
 *  A caller holding the reciprocal global passes 1/g (0 when g == 0). */
int qhead_dequant_nvfp4_bf16(const uint8_t* w_packed, const uint8_t* block_scale, int32_t rows,
                             int32_t cols, float global_scale, uint16_t* out_bf16, void* stream);

/* Load-time E2M1 with E8M0 group scales and no global -> BF16 over a flat
 * tensor of `total` values in `num_groups` groups of total/num_groups
 * consecutive values ("fp8_lut.rs", dequant_nvfp4_e8m0_to_bf16 and the
 * FP8_E8M0_LUT: scale 2^(e-127) for e = 1..254, 0 for e = 0 and e = 255):
 *   out = bf16_rne( fl32(e2m1 * scale) ).
 *  QHEAD_ERR_SHAPE unless total % num_groups == 0 (as the page requires) and
 *  the group size is a multiple of 16. w_packed [total/2] bytes, 8-byte
 *  aligned; scale_e8m0 [num_groups]; out_bf16 [total], 16-byte aligned. */
int qhead_dequant_fp4_e8m0_bf16(const uint8_t* w_packed, const uint8_t* scale_e8m0, int64_t total,
                                int64_t num_groups, uint16_t* out_bf16, void* stream);

/* Measurement support, not part of the GEMV path: reads `bytes` bytes at `p`
 * once, with coalesced 16-byte non-temporal loads spread over the whole GPU
 * in the GEMV's per-wave pattern. The time of this call is the
 * streaming-read ceiling that the GEMV launches are compared with. Each
 * workgroup stores the XOR of the 32-bit words it read into its own word of
 * xor_out (device memory, QHEAD_STREAM_READ_WORDS words, cleared by the
 * caller first); the XOR of all those words is the XOR of the buffer, which
 * shows every word was read exactly once. p 16-byte aligned; bytes >= 0 and a
 * multiple of 16 (QHEAD_ERR_SHAPE otherwise); bytes == 0 returns QHEAD_OK and
 * enqueues nothing. */
#define QHEAD_STREAM_READ_WORDS 4096
int qhead_stream_read(const void* p, int64_t bytes, uint32_t* xor_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QHEAD_H */
