// nvfp4_gemv.hip -- NVFP4 (W4A16) head GEMV for 1..16 activation rows on gfx950.
//
// out[r][v] = bf16( fl32( g * sum_b e4m3(bs[v][b]) * p_b ) ),
// p_b = sum_{k in block b} x[r][k] * e2m1(nib(v,k)) in FP32,
// with blocks of 16 consecutive k and nib(v,k) the low nibble of packed byte
// k/2 for even k ("fp8_lut.rs": dequant_nvfp4_to_bf16's value E2M1 * E4M3
// block scale * global multiplier, and the even-index-low-nibble order stated
// for the dequant_nvfp4_bf16 kernel). The pages serve 4..8 rows with narrow
// tiers and 9..16 rows with a wide one ("w4a16_gemv_tiers.rs":
// W4A16_BATCHM_WIDTHS, select_tier, the batch16 kernel); here every row count
// 1..16 is its own instantiation, so no dead rows execute.
//
// Same structure as the FP8 kernel: persistent workgroups, BF16 activations
// staged in LDS per K-tile (8192 wide up to 8 rows, 4096 above, so that the
// rows fit in LDS), bands of T vocab rows per wave, each
// lane streaming 16 packed bytes (32 weights, two scale blocks) per 2048-wide
// segment with one coalesced non-temporal load plus a 2-byte block-scale
// load. Nibbles become BF16 pairs with v_cvt_scalef32_pk_bf16_fp4 (exact),
// block partials use v_dot2_f32_bf16, and each block partial is folded into
// the row accumulator with one FMA by its decoded E4M3 block scale. Lanes
// accumulate over groups of 4096 k (two segments) whatever the tile width;
// each group's sum goes through one fixed cross-lane tree and the group sums
// are added in k order. None of that depends on the row count, so rows are
// bit-identical for every row count.
#include "qhead_device.h"
#include "qhead_internal.h"

namespace qh {

constexpr int kF4SegK = 2048;    // k per segment: 64 lanes x 32
constexpr int kF4GroupSegs = 2;  // segments per cross-lane reduction group (4096 k)

// k per LDS tile for R rows: R * KT * 2 bytes must fit in LDS.
template <int R>
constexpr int f4_tile_k() {
    return R <= 8 ? 8192 : 4096;
}

// LDS uint4 index of activations k_rel .. k_rel+7 in a tile row: segment s,
// lane l (k 32l .. 32l+31 of the segment), quarter c (8 k each).
__device__ __forceinline__ int f4_lds_vec_index(int k_rel) {
    const int s = k_rel >> 11;
    const int w = k_rel & 2047;
    return s * 256 + ((w >> 3) & 3) * 64 + (w >> 5);
}

template <int R, int NTHREADS>
__device__ __forceinline__ void f4_stage_tile(uint4* xs, const uint16_t* x, int H, int k0,
                                              int nseg) {
    constexpr int kF4VecPerTileRow = f4_tile_k<R>() / 8;
    const int vec_per_row = nseg * (kF4SegK / 8);
    const int total = R * vec_per_row;
    for (int idx = threadIdx.x; idx < total; idx += NTHREADS) {
        const int r = idx / vec_per_row;
        const int q = idx - r * vec_per_row;
        const int k = k0 + q * 8;
        uint4 val = make_uint4(0, 0, 0, 0);
        if (k < H) val = *reinterpret_cast<const uint4*>(x + (size_t)r * H + k);
        xs[r * kF4VecPerTileRow + f4_lds_vec_index(q * 8)] = val;
    }
}

template <int R, int T, int WAVES, int MAXB, int BPC>
__global__ void __launch_bounds__(WAVES * kWave, (WAVES * BPC + 3) / 4)
nvfp4_gemv_kernel(const uint8_t* __restrict__ Wp, const uint8_t* __restrict__ bs,
                  const uint16_t* __restrict__ x, float g, int H, int V,
                  uint16_t* __restrict__ out, int nsuper) {
    constexpr int N = T * R;
    constexpr int NP = next_pow2(N);
    constexpr int M = Log2<NP>::value;
    constexpr int kF4TileK = f4_tile_k<R>();
    constexpr int kF4VecPerTileRow = kF4TileK / 8;
    static_assert(NP <= 64, "T*R must be <= 64");
    static_assert(kF4TileK % (kF4GroupSegs * kF4SegK) == 0, "a tile holds whole groups");
    __shared__ uint4 xs[R * kF4VecPerTileRow];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int TW = gridDim.x * WAVES;
    const int gw = blockIdx.x * WAVES + wave;
    const int NB = (V + T - 1) / T;
    const int NT = (H + kF4TileK - 1) / kF4TileK;
    const size_t prow = (size_t)H / 2;   // packed bytes per vocab row
    const size_t brow = (size_t)H / 16;  // block scales per vocab row

    const int my_idx = lane >> (6 - M);
    const int my_r = my_idx / T;
    const int my_t = my_idx - my_r * T;
    const bool writer = ((lane & ((1 << (6 - M)) - 1)) == 0) && (my_idx < N);
    // The DS offset field reaches 64 KiB: activation rows are addressed from
    // one base per RPB rows, the bases kept opaque so the compiler does not
    // fold them back into one add per read.
    constexpr int RPB = 32768 / kF4TileK;
    int hi_rows = RPB * kF4VecPerTileRow;
    if constexpr (R > RPB) asm volatile("" : "+v"(hi_rows));
    auto xrow_at = [&](const uint4* xrow, int r) {
        return xrow + (r / RPB) * hi_rows + (r % RPB) * kF4VecPerTileRow;
    };

    struct Item {
        uint4 w[T];
        uint32_t sc[T];
    };

    for (int sj = 0; sj < nsuper; ++sj) {
        float part[MAXB];
#pragma unroll
        for (int bi = 0; bi < MAXB; ++bi) part[bi] = 0.0f;

        for (int tt = 0; tt < NT; ++tt) {
            const int k0 = tt * kF4TileK;
            const int klen = min(kF4TileK, H - k0);
            const int nseg = (klen + kF4SegK - 1) / kF4SegK;
            if (NT > 1 || sj == 0) {
                __syncthreads();
                f4_stage_tile<R, WAVES * kWave>(xs, x, H, k0, nseg);
                __syncthreads();
            }
            const int first = (sj * MAXB) * TW + gw;
            const int nbb = first < NB ? min(MAXB, (NB - 1 - first) / TW + 1) : 0;
            const int nitems = nbb * nseg;
            // Unconditional loads: a lane past the hidden tail re-reads the
            // row's last 32 weights (times zero activations), a row past the
            // vocab tail re-reads the last row (never stored).
            auto load_item = [&](int bi, int s, Item& dst) {
                const int v0 = ((sj * MAXB + bi) * TW + gw) * T;
                const int k = min(k0 + s * kF4SegK + lane * 32, H - 32);
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    const int v = min(v0 + t, V - 1);
                    dst.w[t] = load_stream16(Wp + (size_t)v * prow + (k >> 1));
                    dst.sc[t] = *reinterpret_cast<const uint16_t*>(bs + (size_t)v * brow + (k >> 4));
                }
            };
            float acc[NP];
            int bi = 0, s = 0;
            auto step = [&](int it, const Item& cur, Item& nxt) {
                {
                    const bool last = it + 1 >= nitems;
                    const int nbi = last ? bi : ((s + 1 == nseg) ? bi + 1 : bi);
                    const int ns = last ? s : ((s + 1 == nseg) ? 0 : s + 1);
                    load_item(nbi, ns, nxt);
                }
                if (s % kF4GroupSegs == 0) {
#pragma unroll
                    for (int i = 0; i < NP; ++i) acc[i] = 0.0f;
                }
                const uint4* xrow = xs + s * 256 + lane;
                if constexpr (R <= 2) {
                    // Few rows: hold every row's 32 activations, decode one
                    // vocab row's nibbles at a time (fewer live registers).
                    uint32_t xv[R][16];
#pragma unroll
                    for (int r = 0; r < R; ++r) {
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            const uint4 q = lds_read16(xrow_at(xrow, r) + 64 * c);
                            xv[r][4 * c + 0] = q.x;
                            xv[r][4 * c + 1] = q.y;
                            xv[r][4 * c + 2] = q.z;
                            xv[r][4 * c + 3] = q.w;
                        }
                    }
#pragma unroll
                    for (int t = 0; t < T; ++t) {
                        uint32_t wb[16];
                        const uint32_t d[4] = {cur.w[t].x, cur.w[t].y, cur.w[t].z, cur.w[t].w};
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            wb[4 * i + 0] = e2m1x2_to_bf16<0>(d[i]);
                            wb[4 * i + 1] = e2m1x2_to_bf16<1>(d[i]);
                            wb[4 * i + 2] = e2m1x2_to_bf16<2>(d[i]);
                            wb[4 * i + 3] = e2m1x2_to_bf16<3>(d[i]);
                        }
                        const float b0 = __builtin_amdgcn_cvt_f32_fp8(cur.sc[t], 0);
                        const float b1 = __builtin_amdgcn_cvt_f32_fp8(cur.sc[t], 1);
                        // The 2R block chains advance side by side, one
                        // dot2 each per step (a chain's next dot2 is 2R
                        // instructions away); each still sums its 8 pairs in
                        // order.
                        float p0[R], p1[R];
#pragma unroll
                        for (int r = 0; r < R; ++r) {
                            p0[r] = dot2_bf16_zero(xv[r][0], wb[0]);
                            p1[r] = dot2_bf16_zero(xv[r][8], wb[8]);
                        }
#pragma unroll
                        for (int p = 1; p < 8; ++p) {
#pragma unroll
                            for (int r = 0; r < R; ++r) {
                                p0[r] = dot2_bf16(xv[r][p], wb[p], p0[r]);
                                p1[r] = dot2_bf16(xv[r][p + 8], wb[p + 8], p1[r]);
                            }
                        }
#pragma unroll
                        for (int r = 0; r < R; ++r) {
                            float a = acc[r * T + t];
                            a = __builtin_fmaf(b0, p0[r], a);
                            a = __builtin_fmaf(b1, p1[r], a);
                            acc[r * T + t] = a;
                        }
                    }
                } else {
                uint32_t wb[T][16];
                float bsf[T][2];
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    const uint32_t d[4] = {cur.w[t].x, cur.w[t].y, cur.w[t].z, cur.w[t].w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        wb[t][4 * i + 0] = e2m1x2_to_bf16<0>(d[i]);
                        wb[t][4 * i + 1] = e2m1x2_to_bf16<1>(d[i]);
                        wb[t][4 * i + 2] = e2m1x2_to_bf16<2>(d[i]);
                        wb[t][4 * i + 3] = e2m1x2_to_bf16<3>(d[i]);
                    }
                    bsf[t][0] = __builtin_amdgcn_cvt_f32_fp8(cur.sc[t], 0);
                    bsf[t][1] = __builtin_amdgcn_cvt_f32_fp8(cur.sc[t], 1);
                }
                // Activation rows through a two-entry ring: row r + 1 is read
                // while row r is computed.
                uint4 xr[2][4];
#pragma unroll
                for (int c = 0; c < 4; ++c) xr[0][c] = lds_read16(xrow + 64 * c);
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    if (r + 1 < R) {
#pragma unroll
                        for (int c = 0; c < 4; ++c)
                            xr[(r + 1) & 1][c] = lds_read16(xrow_at(xrow, r + 1) + 64 * c);
                    }
                    uint32_t xv[16];
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        xv[4 * c + 0] = xr[r & 1][c].x;
                        xv[4 * c + 1] = xr[r & 1][c].y;
                        xv[4 * c + 2] = xr[r & 1][c].z;
                        xv[4 * c + 3] = xr[r & 1][c].w;
                    }
                    // The 2T block chains of this row advance side by
                    // side, one dot2 each per step, so a chain's next dot2
                    // is 2T instructions away (a lone chain of dependent
                    // dot2 issues well below the VALU's rate); each still
                    // sums its 8 pairs in order.
                    float p0[T], p1[T];
#pragma unroll
                    for (int t = 0; t < T; ++t) {
                        p0[t] = dot2_bf16_zero(xv[0], wb[t][0]);
                        p1[t] = dot2_bf16_zero(xv[8], wb[t][8]);
                    }
#pragma unroll
                    for (int p = 1; p < 8; ++p) {
#pragma unroll
                        for (int t = 0; t < T; ++t) {
                            p0[t] = dot2_bf16(xv[p], wb[t][p], p0[t]);
                            p1[t] = dot2_bf16(xv[p + 8], wb[t][p + 8], p1[t]);
                        }
                    }
#pragma unroll
                    for (int t = 0; t < T; ++t) {
                        float a = acc[r * T + t];
                        a = __builtin_fmaf(bsf[t][0], p0[t], a);
                        a = __builtin_fmaf(bsf[t][1], p1[t], a);
                        acc[r * T + t] = a;
                    }
                }
                }
                if (s + 1 == nseg || (s + 1) % kF4GroupSegs == 0) {
                    // end of a 4096-k group: one tree, then add in k order
                    wave_reduce_scatter<NP>(acc, lane);
                    const bool first_group = tt == 0 && s < kF4GroupSegs;
#pragma unroll
                    for (int j = 0; j < MAXB; ++j)
                        if (j == bi) part[j] = first_group ? acc[0] : part[j] + acc[0];
                }
                if (s + 1 == nseg) {
                    ++bi;
                    s = 0;
                } else {
                    ++s;
                }
            };
            Item bufA, bufB;
            if (nitems > 0) load_item(0, 0, bufA);
            int it = 0;
#pragma unroll 1
            for (; it + 1 < nitems; it += 2) {
                step(it, bufA, bufB);
                step(it + 1, bufB, bufA);
            }
            if (it < nitems) step(it, bufA, bufB);
        }

#pragma unroll
        for (int bi = 0; bi < MAXB; ++bi) {
            const int band = (sj * MAXB + bi) * TW + gw;
            const int v = band * T + my_t;
            if (writer && band < NB && v < V)
                out[(size_t)my_r * V + v] = f32_to_bf16_rne(g * part[bi]);
        }
    }
}

template <int R, int T, int WAVES, int MAXB, int BPC>
static hipError_t launch_nvfp4(const uint8_t* Wp, const uint8_t* bs, const uint16_t* x, float g,
                               int H, int V, uint16_t* out, const DeviceInfo& dev,
                               hipStream_t stream) {
    const int64_t NB = (V + T - 1) / T;
    int64_t blocks = (NB + WAVES - 1) / WAVES;
    if (blocks > (int64_t)dev.num_cus * BPC) blocks = (int64_t)dev.num_cus * BPC;
    const int64_t TW = blocks * WAVES;
    const int64_t per_wave = (NB + TW - 1) / TW;
    const int nsuper = (int)((per_wave + MAXB - 1) / MAXB);
    hipLaunchKernelGGL((nvfp4_gemv_kernel<R, T, WAVES, MAXB, BPC>), dim3((unsigned)blocks),
                       dim3(WAVES * kWave), 0, stream, Wp, bs, x, g, H, V, out, nsuper);
    return hipGetLastError();
}

hipError_t run_nvfp4(const uint8_t* Wp, const uint8_t* bs, const uint16_t* x, float g, int R,
                     int H, int V, uint16_t* out, const DeviceInfo& dev, hipStream_t stream) {
    switch (R) {
#define QH_F4_CASE(RR, TT, WV, MB, BPC) \
    case RR:                            \
        return launch_nvfp4<RR, TT, WV, MB, BPC>(Wp, bs, x, g, H, V, out, dev, stream);
        QH_F4_CASE(1, 2, 16, 20, 1)
        QH_F4_CASE(2, 4, 8, 8, 2)
        QH_F4_CASE(3, 2, 8, 12, 2)
        QH_F4_CASE(4, 4, 12, 12, 1)
        QH_F4_CASE(5, 4, 8, 12, 1)
        QH_F4_CASE(6, 4, 8, 12, 1)
        QH_F4_CASE(7, 4, 8, 12, 1)
        QH_F4_CASE(8, 4, 8, 12, 1)
        QH_F4_CASE(9, 4, 8, 20, 1)
        QH_F4_CASE(10, 4, 8, 20, 1)
        QH_F4_CASE(11, 4, 8, 20, 1)
        QH_F4_CASE(12, 4, 8, 20, 1)
        QH_F4_CASE(13, 4, 8, 20, 1)
        QH_F4_CASE(14, 4, 8, 20, 1)
        QH_F4_CASE(15, 4, 8, 20, 1)
        QH_F4_CASE(16, 4, 8, 20, 1)
#undef QH_F4_CASE
        default:
            return hipErrorInvalidValue;
    }
}

}  // namespace qh
