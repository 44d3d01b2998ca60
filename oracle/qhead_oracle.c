/*
 * qhead_oracle.c -- CPU oracle for the quantized few-row LM-head GEMV.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the library's compute path may call,
 * link or load this file; only the tests, the smoke check and the benchmark's
 * CPU-baseline leg use it. It shares no source with the HIP kernels.
 *
 * Every function is the plain definition of what the head computes: decode
 * each operand exactly, accumulate the dot product in binary64 in sequential k
 * order, then apply the scales in binary64. The result `ref` is the value the
 * GPU's BF16 logit must match within |gpu - ref| <= 2^-7 |ref| + 1e-4 sum|x w|,
 * where x and w are the dequantized operands the dot consumes; `absdot`
 * returns that sum |x w| next to each `ref`.
 *
 * The two activation quantizers (E4M3 per row, q8_1 per 32-block) are
 * encodings whose bytes the GPU must reproduce exactly; they are written out
 * here step by step in IEEE binary32, the precision the format fixes.
 *
 * Sources (the pages this follows; no page prints kernel code):
 *  - "lm_head_fp8_rows.rs": the FP8 E4M3 head with one F32 scale per weight
 *    row, run W8A16 or, when declared, W8A8 reading the same bytes in place;
 *    module doc, LmHeadRows, set_lm_head_w8a8, lm_head_fp8_run.
 *  - "w8a8_layer.rs": W8A8 quantizes the activation rows into a scratch and
 *    runs an FP8 x FP8 GEMV; module doc, W8a8Ctx::proj.
 *  - "fp8_lut.rs": the E2M1 table, the nibble order (even flat index = low
 *    nibble) and the NVFP4 value E2M1 * E4M3 block scale * global multiplier;
 *    dequant_nvfp4_to_bf16, dequant_nvfp4_e8m0_to_bf16.
 *  - "lm_head_q6k.rs": the head held as raw 210-byte Q6_K super-blocks of 256
 *    weights, hidden rows quantised to block_q8_1 (32 values) first; module
 *    doc, LmHeadQ6k, set_lm_head_q6k, lm_head_q6k_run.
 *
 * Readings where the pages are silent (E4M3 flavour, rounding rules, the
 * q8_1 and Q6_K byte layouts, the data-preparation quantizers) are listed in
 * the repository's design notes; each is restated at the function using it.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fPIC -shared. Floating point is
 * IEEE (SSE2 on x86-64, no contraction), so `float` expressions below are
 * single correctly rounded binary32 operations.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_API __attribute__((visibility("default")))

/* Threads the OpenMP loops below use (reported next to oracle timings). */
ORC_API int orc_num_threads(void) { return omp_get_max_threads(); }

/* ------------------------------------------------------------------ */
/* Exact decoders                                                      */
/* ------------------------------------------------------------------ */

/* OCP E4M3FN ("FP8 E4M3" of "lm_head_fp8_rows.rs"; the table itself is not
 * printed there): sign, 4-bit exponent with bias 7, 3-bit mantissa. Exponent
 * field 0 is subnormal, m * 2^-9; otherwise (8 + m) * 2^(e - 10). 0x7F and
 * 0xFF are NaN; there is no infinity. */
ORC_API double orc_e4m3(uint8_t b) {
    int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
    if (e == 15 && m == 7) return NAN;
    double mag = (e == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
    return s ? -mag : mag;
}

/* E2M1 values by nibble, as "fp8_lut.rs" lists them in
 * dequant_nvfp4_e8m0_to_bf16 (nibble 8 is negative zero). */
static const double E2M1_VALUES[16] = {
    0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
    -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0,
};

ORC_API double orc_e2m1(uint8_t nibble) { return E2M1_VALUES[nibble & 15]; }

/* BF16: the upper half of an IEEE binary32. */
ORC_API double orc_bf16(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* IEEE binary16 with subnormals: exponent field 0 gives m * 2^-24,
 * otherwise (1024 + m) * 2^(e - 25). */
ORC_API double orc_fp16(uint16_t h) {
    int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double mag;
    if (e == 31) mag = m ? NAN : INFINITY;
    else if (e == 0) mag = ldexp((double)m, -24);
    else mag = ldexp((double)(1024 + m), e - 25);
    return s ? -mag : mag;
}

/* ------------------------------------------------------------------ */
/* Encoders                                                            */
/* ------------------------------------------------------------------ */

/* Round a finite binary32 value to E4M3FN: nearest grid point, ties to the
 * even mantissa, magnitudes at or above 448 saturate to 448 (0x7E), the sign
 * is kept (a negative value that rounds to zero gives 0x80).
 * Grid: m * 2^-9 below 2^-6 (code = m, m = 0..8 where 8 is 2^-6 itself);
 * (8 + m) * 2^(e-10) in binade [2^(e-7), 2^(e-6)). */
ORC_API uint8_t orc_enc_e4m3(float t) {
    uint8_t sign = signbit(t) ? 0x80 : 0x00;
    double a = fabs((double)t);
    uint8_t code;
    if (a >= 448.0) {
        code = 0x7E;
    } else if (a < ldexp(1.0, -6)) {
        code = (uint8_t)nearbyint(a * 512.0); /* 0..8, ties to even */
    } else {
        int ex;
        frexp(a, &ex);                 /* a = f * 2^ex, f in [0.5, 1) */
        int e = ex - 1;                /* a in [2^e, 2^(e+1)) */
        double n = nearbyint(ldexp(a, 3 - e)); /* significand in units of 2^(e-3): 8..16 */
        if (n == 16.0) { e += 1; n = 8.0; }
        code = (uint8_t)(((e + 7) << 3) | ((int)n - 8));
    }
    return code | sign;
}

/* Round a finite binary32 value to E2M1 (nearest of 0, .5, 1, 1.5, 2, 3, 4, 6;
 * ties to the even code, which is the even mantissa; saturating at 6; sign
 * kept). Used only to prepare NVFP4 weights. */
ORC_API uint8_t orc_enc_e2m1(float t) {
    uint8_t sign = signbit(t) ? 8 : 0;
    double a = fabs((double)t);
    int best = 0;
    double bestd = INFINITY;
    for (int c = 0; c < 8; c++) {
        double d = fabs(E2M1_VALUES[c] - a);
        if (d < bestd || (d == bestd && (c & 1) == 0)) {
            bestd = d;
            best = c;
        }
    }
    return (uint8_t)(best | sign);
}

/* Round to IEEE binary16, nearest even, overflow to infinity. */
ORC_API uint16_t orc_fp16_rne(float f) {
    if (isnan(f)) return 0x7E00;
    uint16_t sign = signbit(f) ? 0x8000 : 0;
    double a = fabs((double)f);
    if (a == 0.0) return sign;
    int ex;
    frexp(a, &ex);
    int e = ex - 1;
    uint16_t bits;
    if (e < -14) {
        double n = nearbyint(ldexp(a, 24)); /* subnormal units of 2^-24, 0..1024 */
        bits = (uint16_t)n;
    } else {
        double n = nearbyint(ldexp(a, 10 - e)); /* 1024..2048 */
        if (n == 2048.0) { e += 1; n = 1024.0; }
        if (e + 15 >= 31) bits = 0x7C00;
        else bits = (uint16_t)(((e + 15) << 10) | ((int)n - 1024));
    }
    return bits | sign;
}

/* Round a binary64 value to BF16, nearest even (diagnostic rounding of the
 * oracle's f64 logits). */
ORC_API uint16_t orc_bf16_rne(double v) {
    if (isnan(v)) return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a == 0.0) return sign;
    if (isinf(a)) return 0x7F80 | sign;
    int ex;
    frexp(a, &ex);
    int e = ex - 1;
    uint16_t bits;
    if (e < -126) {
        double n = nearbyint(ldexp(a, 133)); /* subnormal units of 2^-133 */
        bits = (uint16_t)n;
    } else {
        double n = nearbyint(ldexp(a, 7 - e)); /* 128..256 */
        if (n == 256.0) { e += 1; n = 128.0; }
        if (e + 127 >= 255) bits = 0x7F80;
        else bits = (uint16_t)(((e + 127) << 7) | ((int)n - 128));
    }
    return bits | sign;
}

/* ------------------------------------------------------------------ */
/* Activation quantizers (bit-exact contracts)                         */
/* ------------------------------------------------------------------ */

/* Per-row dynamic E4M3 quantization of BF16 activations, the step W8A8 runs
 * before its FP8 x FP8 GEMV ("w8a8_layer.rs", W8a8Ctx::proj; per row, so
 * chunking never changes a row's bits, "lm_head_fp8_rows.rs",
 * lm_head_fp8_run). Per row r:
 *   amax  = max_k |x[r,k]|                     (exact)
 *   sa[r] = fl32(amax / 448)                   (one binary32 division)
 *   xq    = enc_e4m3(fl32(x[r,k] / sa[r]))     (one binary32 division each)
 * An all-zero row gives sa = 0 and codes 0x00. */
ORC_API void orc_quant_act_e4m3(const uint16_t* x, int rows, int hidden, uint8_t* xq,
                                float* sa) {
    for (int r = 0; r < rows; r++) {
        const uint16_t* xr = x + (size_t)r * hidden;
        float amax = 0.0f;
        for (int k = 0; k < hidden; k++) {
            float v = fabsf((float)orc_bf16(xr[k]));
            if (v > amax) amax = v;
        }
        uint8_t* qr = xq + (size_t)r * hidden;
        if (amax == 0.0f) {
            sa[r] = 0.0f;
            memset(qr, 0, (size_t)hidden);
            continue;
        }
        float scale = amax / 448.0f;
        sa[r] = scale;
        for (int k = 0; k < hidden; k++) {
            float t = (float)orc_bf16(xr[k]) / scale;
            qr[k] = orc_enc_e4m3(t);
        }
    }
}

/* SiLU product of the FFN down projection ("w8a8_layer.rs", W8a8Ctx::silu_proj:
 * the activation is bf16(silu(gate) * up), quantized per row in the same launch
 * as the W8A8 activations are). The pages do not fix silu's precision; it is
 * evaluated here in binary64, silu(g) = g / (1 + exp(-g)), times u, and the
 * binary64 value is rounded once to BF16 (nearest even). */
ORC_API uint16_t orc_silu_mul_bf16(uint16_t g_bits, uint16_t u_bits) {
    double g = orc_bf16(g_bits), u = orc_bf16(u_bits);
    double s = g / (1.0 + exp(-g));
    return orc_bf16_rne(s * u);
}

/* 1 when the binary64 SiLU product lies so close to a BF16 rounding boundary
 * that a last-bit difference in exp could change its BF16 rounding (the
 * rounding of the value scaled by 1 -+ 2^-44 differs), else 0. */
ORC_API int orc_silu_mul_ambiguous(uint16_t g_bits, uint16_t u_bits) {
    double g = orc_bf16(g_bits), u = orc_bf16(u_bits);
    double p = (g / (1.0 + exp(-g))) * u;
    uint16_t b = orc_bf16_rne(p);
    double eps = ldexp(1.0, -44);
    return orc_bf16_rne(p * (1.0 - eps)) != b || orc_bf16_rne(p * (1.0 + eps)) != b;
}

/* Elementwise orc_silu_mul_bf16 with its ambiguity flag, over n values. */
ORC_API void orc_silu_mul_bf16_array(const uint16_t* g, const uint16_t* u, int64_t n,
                                     uint16_t* out, uint8_t* ambiguous) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) {
        out[i] = orc_silu_mul_bf16(g[i], u[i]);
        ambiguous[i] = (uint8_t)orc_silu_mul_ambiguous(g[i], u[i]);
    }
}

/* Per-row E4M3 quantization of the SiLU product: p[r][k] =
 * orc_silu_mul_bf16(gate[r*ld + k], up[r*ld + k]) for k < hidden, then the
 * activation quantization above on p. Returns the number of ambiguous
 * elements (see orc_silu_mul_ambiguous). */
ORC_API int64_t orc_quant_act_silu_e4m3(const uint16_t* gate, const uint16_t* up, int ld,
                                        int rows, int hidden, uint8_t* xq, float* sa) {
    uint16_t* p = (uint16_t*)malloc((size_t)hidden * sizeof(uint16_t));
    int64_t ambiguous = 0;
    for (int r = 0; r < rows; r++) {
        const uint16_t* gr = gate + (size_t)r * ld;
        const uint16_t* ur = up + (size_t)r * ld;
        for (int k = 0; k < hidden; k++) {
            p[k] = orc_silu_mul_bf16(gr[k], ur[k]);
            ambiguous += orc_silu_mul_ambiguous(gr[k], ur[k]);
        }
        orc_quant_act_e4m3(p, 1, hidden, xq + (size_t)r * hidden, sa + r);
    }
    free(p);
    return ambiguous;
}

/* block_q8_1 quantization of BF16 rows ("lm_head_q6k.rs": hidden rows are
 * quantised to block_q8_1, 32 values a block). Per block of 32 values:
 *   amax = max |x|;  d = fl32(amax / 127)
 *   q_i  = clamp(round_half_even(fl32(x_i / d)), -127, 127)
 *   stored d16 = fp16_rne(d), s16 = fp16_rne(fl32(d * sum q_i))
 * An all-zero block gives d = 0 and q = 0. The 36-byte block is
 *   bytes 0-1 d16 (little endian), 2-3 s16, 4-35 q_0..q_31 (int8).
 * The dot product uses the stored fp16 d. */
#define Q8_BLOCK_BYTES 36
ORC_API void orc_quant_q8_1(const uint16_t* x, int rows, int hidden, uint8_t* q8) {
    int nb = hidden / 32;
    for (int r = 0; r < rows; r++) {
        for (int j = 0; j < nb; j++) {
            const uint16_t* xb = x + (size_t)r * hidden + (size_t)j * 32;
            uint8_t* blk = q8 + ((size_t)r * nb + j) * Q8_BLOCK_BYTES;
            float amax = 0.0f;
            for (int i = 0; i < 32; i++) {
                float v = fabsf((float)orc_bf16(xb[i]));
                if (v > amax) amax = v;
            }
            int8_t q[32];
            int sumq = 0;
            float d = 0.0f;
            if (amax == 0.0f) {
                memset(q, 0, sizeof q);
            } else {
                d = amax / 127.0f;
                for (int i = 0; i < 32; i++) {
                    float t = (float)orc_bf16(xb[i]) / d;
                    double n = nearbyint((double)t);
                    if (n > 127.0) n = 127.0;
                    if (n < -127.0) n = -127.0;
                    q[i] = (int8_t)n;
                    sumq += q[i];
                }
            }
            uint16_t d16 = orc_fp16_rne(d);
            uint16_t s16 = orc_fp16_rne(d * (float)sumq);
            blk[0] = (uint8_t)(d16 & 0xFF);
            blk[1] = (uint8_t)(d16 >> 8);
            blk[2] = (uint8_t)(s16 & 0xFF);
            blk[3] = (uint8_t)(s16 >> 8);
            memcpy(blk + 4, q, 32);
        }
    }
}

/* ------------------------------------------------------------------ */
/* Q6_K super-block layout                                             */
/* ------------------------------------------------------------------ */

/* A Q6_K super-block ("lm_head_q6k.rs": 256 weights in 210 bytes) read with
 * the field set of the public GGUF description: ql[128] low four bits,
 * qh[64] high two bits, scales[16] int8 (one per 16 weights), d fp16.
 * Weight i = 128 n + 32 c + l (half n, quarter c, l < 32) takes
 *   low bits  : ql[64 n + l + 32 (c & 1)], low nibble for c < 2, high for c >= 2
 *   high bits : bits 2c..2c+1 of qh[32 n + l]
 * q = low | high << 4 in 0..63, and the weight is d * scales[i / 16] * (q - 32). */
#define Q6K_BLOCK_BYTES 210

static int q6k_q(const uint8_t* blk, int i) {
    int n = i / 128, c = (i % 128) / 32, l = i % 32;
    uint8_t lb = blk[64 * n + l + 32 * (c & 1)];
    int low = (c < 2) ? (lb & 15) : (lb >> 4);
    int high = (blk[128 + 32 * n + l] >> (2 * c)) & 3;
    return low | (high << 4);
}

ORC_API void orc_q6k_decode_block(const uint8_t* blk, double* out256) {
    uint16_t dbits = (uint16_t)(blk[208] | (blk[209] << 8));
    double d = orc_fp16(dbits);
    for (int i = 0; i < 256; i++) {
        int8_t sc = (int8_t)blk[192 + i / 16];
        out256[i] = d * (double)sc * (double)(q6k_q(blk, i) - 32);
    }
}

/* ------------------------------------------------------------------ */
/* Hot-path references (binary64, sequential k)                        */
/* ------------------------------------------------------------------ */
/* Each reference computes out[r * nv + j] for vocab row vidx[j] and activation
 * row r, plus absdot = sum_k |x_k w_k| of the dequantized operands. */

/* FP8 W8A16: ref[r,v] = s[v] * sum_k bf16(x[r,k]) * e4m3(W[v,k])
 * ("lm_head_fp8_rows.rs": E4M3 head with per-row F32 scales). */
ORC_API void orc_fp8_rowscale(const uint8_t* w, const float* s, const uint16_t* x, int rows,
                              int hidden, int vocab, const int64_t* vidx, int nv, double* ref,
                              double* absdot) {
    (void)vocab;
#pragma omp parallel for schedule(dynamic, 16)
    for (int j = 0; j < nv; j++) {
        const uint8_t* wr = w + (size_t)vidx[j] * hidden;
        double sv = (double)s[vidx[j]];
        for (int r = 0; r < rows; r++) {
            const uint16_t* xr = x + (size_t)r * hidden;
            double acc = 0.0, aacc = 0.0;
            for (int k = 0; k < hidden; k++) {
                double p = orc_bf16(xr[k]) * orc_e4m3(wr[k]);
                acc += p;
                aacc += fabs(p);
            }
            ref[(size_t)r * nv + j] = acc * sv;
            absdot[(size_t)r * nv + j] = aacc * fabs(sv);
        }
    }
}

/* W8A8: ref[r,v] = sa[r] * sw[v] * sum_k e4m3(xq[r,k]) * e4m3(W[v,k]).
 * The same E4M3 bytes and row scales as the W8A16 head, read in place
 * ("lm_head_fp8_rows.rs", set_lm_head_w8a8). Every E4M3 value is n * 2^-9
 * with |n| < 2^18, so each product is an integer multiple of 2^-18 below
 * 2^36 and the binary64 sum is exact for hidden below 2^17. */
ORC_API void orc_w8a8(const uint8_t* w, const float* sw, const uint8_t* xq, const float* sa,
                      int rows, int hidden, int vocab, const int64_t* vidx, int nv, double* ref,
                      double* absdot) {
    (void)vocab;
#pragma omp parallel for schedule(dynamic, 16)
    for (int j = 0; j < nv; j++) {
        const uint8_t* wr = w + (size_t)vidx[j] * hidden;
        double sv = (double)sw[vidx[j]];
        for (int r = 0; r < rows; r++) {
            const uint8_t* xr = xq + (size_t)r * hidden;
            double acc = 0.0, aacc = 0.0;
            for (int k = 0; k < hidden; k++) {
                double p = orc_e4m3(xr[k]) * orc_e4m3(wr[k]);
                acc += p;
                aacc += fabs(p);
            }
            double scale = (double)sa[r] * sv;
            ref[(size_t)r * nv + j] = acc * scale;
            absdot[(size_t)r * nv + j] = aacc * fabs(scale);
        }
    }
}

/* NVFP4 W4A16: ref[r,v] = g * sum_k bf16(x[r,k]) * e2m1(nib(v,k)) * e4m3(bs[v,k/16]).
 * nib(v,k) is the low nibble of packed byte k/2 of row v when k is even, the
 * high nibble when odd ("fp8_lut.rs": even flat index = low nibble; value =
 * E2M1 * E4M3 block scale * global multiplier, dequant_nvfp4_to_bf16).
 * Blocks are 16 consecutive k of one row; bs is [vocab][hidden/16]. */
ORC_API void orc_nvfp4(const uint8_t* wp, const uint8_t* bs, float g, const uint16_t* x,
                       int rows, int hidden, int vocab, const int64_t* vidx, int nv, double* ref,
                       double* absdot) {
    (void)vocab;
    double gd = (double)g;
#pragma omp parallel for schedule(dynamic, 16)
    for (int j = 0; j < nv; j++) {
        const uint8_t* pr = wp + (size_t)vidx[j] * (hidden / 2);
        const uint8_t* br = bs + (size_t)vidx[j] * (hidden / 16);
        for (int r = 0; r < rows; r++) {
            const uint16_t* xr = x + (size_t)r * hidden;
            double acc = 0.0, aacc = 0.0;
            for (int k = 0; k < hidden; k++) {
                uint8_t byte = pr[k / 2];
                uint8_t nib = (k % 2 == 0) ? (byte & 15) : (byte >> 4);
                double wv = orc_e2m1(nib) * orc_e4m3(br[k / 16]);
                double p = orc_bf16(xr[k]) * wv;
                acc += p;
                aacc += fabs(p);
            }
            ref[(size_t)r * nv + j] = acc * gd;
            absdot[(size_t)r * nv + j] = aacc * fabs(gd);
        }
    }
}

/* Q6_K x q8_1: ref[r,v] = sum_k w[v,k] * a[r,k] where w is the decoded Q6_K
 * weight (d * scale * (q - 32)) and a = fp16(d16 of the block) * q8
 * ("lm_head_q6k.rs": blocks [vocab][hidden/256], activations as block_q8_1). */
ORC_API void orc_q6k(const uint8_t* blocks, const uint8_t* q8, int rows, int hidden, int vocab,
                     const int64_t* vidx, int nv, double* ref, double* absdot) {
    (void)vocab;
    int nsb = hidden / 256, nq = hidden / 32;
#pragma omp parallel for schedule(dynamic, 16)
    for (int j = 0; j < nv; j++) {
        const uint8_t* row = blocks + (size_t)vidx[j] * nsb * Q6K_BLOCK_BYTES;
        double wv[256];
        for (int r = 0; r < rows; r++) {
            double acc = 0.0, aacc = 0.0;
            for (int b = 0; b < nsb; b++) {
                orc_q6k_decode_block(row + (size_t)b * Q6K_BLOCK_BYTES, wv);
                for (int i = 0; i < 256; i++) {
                    int k = b * 256 + i;
                    const uint8_t* qb = q8 + ((size_t)r * nq + k / 32) * Q8_BLOCK_BYTES;
                    double dq = orc_fp16((uint16_t)(qb[0] | (qb[1] << 8)));
                    double a = dq * (double)(int8_t)qb[4 + k % 32];
                    double p = wv[i] * a;
                    acc += p;
                    aacc += fabs(p);
                }
            }
            ref[(size_t)r * nv + j] = acc;
            absdot[(size_t)r * nv + j] = aacc;
        }
    }
}

/* ------------------------------------------------------------------ */
/* Data preparation (weights for tests; not on the hot path)           */
/* ------------------------------------------------------------------ */
/* The pages print no weight quantizer. These choose one plausible recipe per
 * format; the GPU only ever consumes the bytes they produce. */

/* FP8 rows: s_v = fl32(amax_v / 448), codes = enc_e4m3(fl32(w / s_v));
 * an all-zero row gets s = 0 and codes 0. */
ORC_API void orc_prep_fp8_rows(const float* wf, int64_t nrows, int hidden, uint8_t* codes,
                               float* scales) {
#pragma omp parallel for schedule(static)
    for (int64_t v = 0; v < nrows; v++) {
        const float* row = wf + (size_t)v * hidden;
        uint8_t* out = codes + (size_t)v * hidden;
        float amax = 0.0f;
        for (int k = 0; k < hidden; k++) {
            float a = fabsf(row[k]);
            if (a > amax) amax = a;
        }
        if (amax == 0.0f) {
            scales[v] = 0.0f;
            memset(out, 0, (size_t)hidden);
            continue;
        }
        float s = amax / 448.0f;
        scales[v] = s;
        for (int k = 0; k < hidden; k++) out[k] = orc_enc_e4m3(row[k] / s);
    }
}

/* NVFP4 global multiplier: g = fl32(amax / (448 * 6)) over the whole weight. */
ORC_API float orc_prep_nvfp4_global(float amax_all) { return amax_all / 2688.0f; }

/* NVFP4 rows with global g: per block b of 16, bs = enc_e4m3(fl32(amax_b /
 * fl32(6 g))); step = fl32(e4m3(bs) * g); nibble = enc_e2m1(fl32(w / step)),
 * or nibble 0 where step is 0. */
ORC_API void orc_prep_nvfp4_rows(const float* wf, int64_t nrows, int hidden, float g,
                                 uint8_t* packed, uint8_t* bs) {
    float six_g = 6.0f * g;
#pragma omp parallel for schedule(static)
    for (int64_t v = 0; v < nrows; v++) {
        const float* row = wf + (size_t)v * hidden;
        uint8_t* prow = packed + (size_t)v * (hidden / 2);
        uint8_t* brow = bs + (size_t)v * (hidden / 16);
        memset(prow, 0, (size_t)hidden / 2);
        for (int b = 0; b < hidden / 16; b++) {
            float amax = 0.0f;
            for (int i = 0; i < 16; i++) {
                float a = fabsf(row[b * 16 + i]);
                if (a > amax) amax = a;
            }
            uint8_t code = (six_g == 0.0f) ? 0 : orc_enc_e4m3(amax / six_g);
            brow[b] = code;
            float step = (float)orc_e4m3(code) * g;
            for (int i = 0; i < 16; i++) {
                int k = b * 16 + i;
                uint8_t nib = (step == 0.0f) ? 0 : orc_enc_e2m1(row[k] / step);
                prow[k / 2] |= (k % 2 == 0) ? nib : (uint8_t)(nib << 4);
            }
        }
    }
}

/* Q6_K rows: per super-block, s_t = fl32(amax_t / 31) per 16 weights,
 * d = fp16_rne(fl32(max_t s_t / 127)), sc_t = clamp(rne(fl32(s_t / d)), 0, 127),
 * step = fl32(d * sc_t), q = clamp(rne(fl32(w / step)), -32, 31) + 32
 * (q = 32 where step is 0). Bytes are placed by the layout of q6k_q. */
ORC_API void orc_prep_q6k_rows(const float* wf, int64_t nrows, int hidden, uint8_t* blocks) {
    int nsb = hidden / 256;
#pragma omp parallel for schedule(static)
    for (int64_t v = 0; v < nrows; v++) {
        for (int b = 0; b < nsb; b++) {
            const float* w = wf + (size_t)v * hidden + (size_t)b * 256;
            uint8_t* blk = blocks + ((size_t)v * nsb + b) * Q6K_BLOCK_BYTES;
            memset(blk, 0, Q6K_BLOCK_BYTES);
            float st[16], smax = 0.0f;
            for (int t = 0; t < 16; t++) {
                float amax = 0.0f;
                for (int i = 0; i < 16; i++) {
                    float a = fabsf(w[t * 16 + i]);
                    if (a > amax) amax = a;
                }
                st[t] = amax / 31.0f;
                if (st[t] > smax) smax = st[t];
            }
            uint16_t dbits = orc_fp16_rne(smax / 127.0f);
            float d = (float)orc_fp16(dbits);
            blk[208] = (uint8_t)(dbits & 0xFF);
            blk[209] = (uint8_t)(dbits >> 8);
            for (int t = 0; t < 16; t++) {
                int sc = 0;
                if (d > 0.0f) {
                    double n = nearbyint((double)(st[t] / d));
                    sc = (int)(n < 0 ? 0 : (n > 127 ? 127 : n));
                }
                blk[192 + t] = (uint8_t)(int8_t)sc;
                float step = d * (float)sc;
                for (int i = 0; i < 16; i++) {
                    int idx = t * 16 + i;
                    int q = 32;
                    if (step != 0.0f) {
                        double n = nearbyint((double)(w[idx] / step));
                        if (n < -32) n = -32;
                        if (n > 31) n = 31;
                        q = (int)n + 32;
                    }
                    int n2 = idx / 128, c = (idx % 128) / 32, l = idx % 32;
                    int lo = 64 * n2 + l + 32 * (c & 1);
                    blk[lo] |= (uint8_t)((c < 2) ? (q & 15) : ((q & 15) << 4));
                    blk[128 + 32 * n2 + l] |= (uint8_t)(((q >> 4) & 3) << (2 * c));
                }
            }
        }
    }
}

/* ------------------------------------------------------------------ */
/* Load-time dequantization to BF16                                    */
/* ------------------------------------------------------------------ */

/* NVFP4 -> BF16 for a [n][k] weight ("fp8_lut.rs", dequant_nvfp4_to_bf16:
 * value E2M1 * fp8 block scale * global multiplier, even flat index = low
 * nibble). Reading of the rounding: the E2M1 x E4M3 product is exact in
 * binary32, the global multiplier is applied in binary32 (one rounding) and
 * the result is rounded to BF16, nearest even:
 *   out = bf16( fl32( (e2m1 * e4m3(bs)) * g ) ). */
ORC_API void orc_dequant_nvfp4_bf16(const uint8_t* packed, const uint8_t* bs, float g, int64_t n,
                                    int k, uint16_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t v = 0; v < n; v++) {
        for (int c = 0; c < k; c++) {
            int64_t flat = v * (int64_t)k + c;
            uint8_t byte = packed[flat / 2];
            uint8_t nib = (flat % 2 == 0) ? (byte & 15) : (byte >> 4);
            float w = (float)(orc_e2m1(nib) * orc_e4m3(bs[v * (int64_t)(k / 16) + c / 16]));
            float y = w * g;
            out[flat] = orc_bf16_rne((double)y);
        }
    }
}

/* E8M0 scale byte -> value: 2^(e - 127) for e = 1..254; e = 0 and e = 255
 * (NaN) give 0 ("fp8_lut.rs", FP8_E8M0_LUT and fp8_e8m0_to_f32). */
ORC_API double orc_e8m0(uint8_t e) {
    if (e == 0 || e == 255) return 0.0;
    return ldexp(1.0, (int)e - 127);
}

/* E2M1 with E8M0 group scales and no global -> BF16 ("fp8_lut.rs",
 * dequant_nvfp4_e8m0_to_bf16, and its E8M0 table). The tensor is `total`
 * values; value j is nibble j of `packed` (the low half of byte j/2 for even
 * j, the high half for odd j), and belongs to group j / (total/groups), whose
 * scale byte is scales[group]. Its BF16 is the nearest-even rounding of the
 * binary32 value of e2m1 * 2^(e-127) (exact in binary32 unless it overflows
 * to infinity). Each packed byte is decoded once, both of its values. */
ORC_API void orc_dequant_fp4_e8m0_bf16(const uint8_t* packed, const uint8_t* scales,
                                       int64_t total, int64_t groups, uint16_t* out) {
    const int64_t per_group = total / groups;
    const int64_t nbytes = (total + 1) / 2;
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nbytes; b++) {
        const uint8_t two = packed[b];
        const uint8_t nib[2] = {(uint8_t)(two & 15), (uint8_t)(two >> 4)};
        for (int half = 0; half < 2; half++) {
            const int64_t j = 2 * b + half;
            if (j >= total) break;
            const double value = orc_e2m1(nib[half]) * orc_e8m0(scales[j / per_group]);
            out[j] = orc_bf16_rne((double)(float)value);
        }
    }
}
