// fp8_gemv.hip -- FP8 E4M3 head GEMV for 1..16 activation rows on gfx950.
//
// Computes logits[r][v] = bf16(fl32(acc * scale)) with acc = sum_k x[r][k] *
// e4m3(W[v][k]) in FP32, for the FP8 head with one F32 scale per weight row
// ("lm_head_fp8_rows.rs": module doc and lm_head_fp8_run, W8A16).
//
// Design (MI355X-first; the pages' per-row-count kernels are prior art only):
//  * One persistent workgroup of WAVES wave64s per CU. The activation rows are
//    staged once per K-tile into LDS as BF16, so the weight stream is the
//    only HBM traffic that scales with vocab.
//  * Each wave owns bands of T consecutive vocab rows. A band's row is read as
//    1 KiB segments: lane l loads bytes [16 l, 16 l + 16) of the segment, a
//    coalesced 16-byte non-temporal load, so every weight byte is fetched
//    exactly once per launch.
//  * The 16 weights a lane holds are decoded to BF16 pairs in registers
//    (v_cvt_scalef32_pk_bf16_fp8) and multiplied into FP32 accumulators with
//    v_dot2_f32_bf16 against the lane's 16 activations of each row, read from
//    LDS as two conflict-free 16-byte vectors.
//  * After a K-tile, the T*R accumulators of the band are summed over the 64
//    lanes by one fixed reduce-scatter tree (permlane swaps + DPP), then the
//    tile sums are added in tile order, scaled, rounded to BF16 and stored.
//
// Row invariance: lane->k mapping, per-lane accumulation order (segments in
// order, eight dot2 in k order), the cross-lane tree and the tile order all
// depend on hidden only, never on R, T or the launch shape, so a row's logits
// are bit-identical for every row count and every chunking.
#include "qhead_device.h"
#include "qhead_internal.h"

namespace qh {

constexpr int kSegK = 1024;        // k per wave segment: 64 lanes x 16
constexpr int kTileK = 4096;       // k per LDS tile (fixed: part of the arithmetic)
constexpr int kVecPerTileRow = kTileK / 8;  // uint4 (8 BF16) per activation row per tile

// LDS position (in uint4 units) of activations k_rel .. k_rel+7 within a
// tile row: segment s, lane l, half c (k 16l..16l+7 -> c=0, 16l+8.. -> c=1),
// laid out so that lanes read consecutive 16-byte vectors.
__device__ __forceinline__ int lds_vec_index(int k_rel) {
    const int s = k_rel >> 10;
    const int w = k_rel & 1023;
    const int l = w >> 4;
    const int c = (w >> 3) & 1;
    return s * 128 + c * 64 + l;
}

template <int R, int NTHREADS>
__device__ __forceinline__ void stage_tile(uint4* xs, const uint16_t* xin, int H, int k0, int nseg) {
    const int vec_per_row = nseg * (kSegK / 8);
    const int total = R * vec_per_row;
    for (int idx = threadIdx.x; idx < total; idx += NTHREADS) {
        const int r = idx / vec_per_row;
        const int q = idx - r * vec_per_row;
        const int k = k0 + q * 8;
        uint4 val = make_uint4(0, 0, 0, 0);
        if (k < H) val = *reinterpret_cast<const uint4*>(xin + (size_t)r * H + k);
        xs[r * kVecPerTileRow + lds_vec_index(q * 8)] = val;
    }
}

template <int R, int T, int WAVES, int MAXB, int BPC>
__global__ void __launch_bounds__(WAVES * kWave, (WAVES * BPC + 3) / 4)
fp8_gemv_kernel(const uint8_t* __restrict__ W, const float* __restrict__ wscale,
                const uint16_t* __restrict__ xin, int H, int V, uint16_t* __restrict__ out,
                int nsuper) {
    constexpr int N = T * R;
    constexpr int NP = next_pow2(N);
    constexpr int M = Log2<NP>::value;
    static_assert(NP <= 64, "T*R must be <= 64");
    __shared__ uint4 xs[R * kVecPerTileRow];

    const int lane = threadIdx.x & 63;
    // wave-uniform: keeps the band loop and its prefetch on scalar branches
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int TW = gridDim.x * WAVES;
    const int gw = blockIdx.x * WAVES + wave;
    const int NB = (V + T - 1) / T;
    const int NT = (H + kTileK - 1) / kTileK;

    // The value index this lane holds after the reduction: idx = r * T + t.
    const int my_idx = lane >> (6 - M);
    const int my_r = my_idx / T;
    const int my_t = my_idx - my_r * T;
    const bool writer = ((lane & ((1 << (6 - M)) - 1)) == 0) && (my_idx < N);
    // Offset (in 16-byte vectors) of activation row 8 in the LDS tile, kept
    // opaque so the compiler does not fold it back into per-read adds.
    int hi_rows = 8 * kVecPerTileRow;
    if constexpr (R > 8) asm volatile("" : "+v"(hi_rows));

    for (int sj = 0; sj < nsuper; ++sj) {
        float part[MAXB];
#pragma unroll
        for (int bi = 0; bi < MAXB; ++bi) part[bi] = 0.0f;

        for (int tt = 0; tt < NT; ++tt) {
            const int k0 = tt * kTileK;
            const int klen = min(kTileK, H - k0);
            const int nseg = (klen + kSegK - 1) / kSegK;
            // This wave's bands in this super-iteration, walked as one flat
            // list of (band, segment) items so that the next item's weights
            // are always in flight while the current one is computed.
            const int first = (sj * MAXB) * TW + gw;
            const int nbb = first < NB ? min(MAXB, (NB - 1 - first) / TW + 1) : 0;
            const int nitems = nbb * nseg;
            // Loads are unconditional so that no branch forces the wait
            // counter to drain: a lane past the hidden tail re-reads the
            // row's last 16 bytes (finite weights times the zero activations
            // staged there add nothing), and a row past the vocab tail
            // re-reads the last row (its sums are never stored).
            auto load_item = [&](int bi, int s, uint4(&dst)[T]) {
                const int v0 = ((sj * MAXB + bi) * TW + gw) * T;
                const int k = min(k0 + s * kSegK + lane * 16, H - 16);
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    const int v = min(v0 + t, V - 1);
                    dst[t] = load_stream16(W + (size_t)v * H + k);
                }
            };
            float acc[NP];
            int bi = 0, s = 0;
            // One (band, segment) item: issue the loads of item `it + 1` into
            // `nxt` (clamped, unconditional), then compute `cur`. Two named
            // buffers alternate, so no copy waits on a load in flight.
            auto step = [&](int it, const uint4(&cur)[T], uint4(&nxt)[T]) {
                {
                    const bool last = it + 1 >= nitems;
                    const int nbi = last ? bi : ((s + 1 == nseg) ? bi + 1 : bi);
                    const int ns = last ? s : ((s + 1 == nseg) ? 0 : s + 1);
                    load_item(nbi, ns, nxt);
                }
                // Nothing of the compute below moves above those loads: a
                // decode of `cur` hoisted above them would need a wait that
                // also covers the loads just issued.
                __builtin_amdgcn_sched_barrier(0);
                if (s == 0) {
#pragma unroll
                    for (int i = 0; i < NP; ++i) acc[i] = 0.0f;
                }
                uint32_t wb[T][8];
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    e4m3x4_to_bf16(cur[t].x, wb[t][0], wb[t][1]);
                    e4m3x4_to_bf16(cur[t].y, wb[t][2], wb[t][3]);
                    e4m3x4_to_bf16(cur[t].z, wb[t][4], wb[t][5]);
                    e4m3x4_to_bf16(cur[t].w, wb[t][6], wb[t][7]);
                }
                const uint4* xrow = xs + s * 128 + lane;
                // Rows 8 and up lie 64 KiB or more past xrow, beyond the DS
                // offset field: address them from a second base (one add per
                // item instead of one per read).
                const uint4* xrow_hi = xrow + hi_rows;
                if constexpr (R >= 4) {
                    // Rows in groups of G: for each k pair p, the G * T
                    // accumulators of a group take their dot2 one after the
                    // other, so a chain's next dot2 is G * T instructions
                    // away (the VALU issues near its peak only with many
                    // independent chains). Each accumulator still sums p in
                    // order, so the arithmetic is the same for every R. The
                    // next group's activations are read while this one runs.
                    constexpr int G = T >= 4 ? 4 : 2;  // 2-row bands: fewer live registers
                    uint32_t xg[2][G][8];
                    auto read_group = [&](int rg, uint32_t (&dst)[G][8]) {
#pragma unroll
                        for (int g = 0; g < G; ++g) {
                            if (rg + g < R) {
                                const uint4* xp = (rg + g) < 8
                                    ? xrow + (rg + g) * kVecPerTileRow
                                    : xrow_hi + (rg + g - 8) * kVecPerTileRow;
                                const uint4 xa = xp[0];
                                const uint4 xb = xp[64];
                                dst[g][0] = xa.x; dst[g][1] = xa.y; dst[g][2] = xa.z;
                                dst[g][3] = xa.w; dst[g][4] = xb.x; dst[g][5] = xb.y;
                                dst[g][6] = xb.z; dst[g][7] = xb.w;
                            }
                        }
                    };
                    read_group(0, xg[0]);
#pragma unroll
                    for (int rg = 0; rg < R; rg += G) {
                        if (rg + G < R) read_group(rg + G, xg[((rg / G) + 1) & 1]);
                        const int cb = (rg / G) & 1;
#pragma unroll
                        for (int p = 0; p < 8; ++p) {
#pragma unroll
                            for (int g = 0; g < G; ++g) {
                                if (rg + g < R) {
#pragma unroll
                                    for (int t = 0; t < T; ++t)
                                        acc[(rg + g) * T + t] =
                                            dot2_bf16(xg[cb][g][p], wb[t][p], acc[(rg + g) * T + t]);
                                }
                            }
                        }
                    }
                } else {
                // Activation rows through a ring of LA + 1 buffers: the
                // reads of row r + LA are issued before row r is computed.
                constexpr int LA = R < 2 ? R : 2;
                constexpr int NBUF = LA + 1;
                uint4 xr[NBUF][2];
#pragma unroll
                for (int r = 0; r < LA; ++r) {
                    xr[r][0] = xrow[r * kVecPerTileRow];
                    xr[r][1] = xrow[r * kVecPerTileRow + 64];
                }
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    if (r + LA < R) {
                        xr[(r + LA) % NBUF][0] = xrow[(r + LA) * kVecPerTileRow];
                        xr[(r + LA) % NBUF][1] = xrow[(r + LA) * kVecPerTileRow + 64];
                    }
                    const uint4 xa = xr[r % NBUF][0], xb = xr[r % NBUF][1];
                    const uint32_t xv[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
#pragma unroll
                    for (int t = 0; t < T; ++t) {
                        float a = acc[r * T + t];
#pragma unroll
                        for (int p = 0; p < 8; ++p) a = dot2_bf16(xv[p], wb[t][p], a);
                        acc[r * T + t] = a;
                    }
                }
                }
                if (s + 1 == nseg) {
                    wave_reduce_scatter<NP>(acc, lane);
                    // part[bi] (+)= the tile sum, with bi a run-time index into
                    // a register array: select through an unrolled compare.
#pragma unroll
                    for (int j = 0; j < MAXB; ++j)
                        if (j == bi) part[j] = (tt == 0) ? acc[0] : part[j] + acc[0];
                    ++bi;
                    s = 0;
                } else {
                    ++s;
                }
            };
            uint4 bufA[T], bufB[T];
            // Up to 4 rows (HBM-bound launches) the first item's loads go out
            // before the activation tile is staged, so their latency and the
            // staging's overlap; with more rows the registers they would hold
            // through the staging are scarcer than the latency.
            constexpr bool kEarly = R <= 4;
            if (kEarly && nitems > 0) load_item(0, 0, bufA);
            if (NT > 1 || sj == 0) {
                __syncthreads();
                stage_tile<R, WAVES * kWave>(xs, xin, H, k0, nseg);
                __syncthreads();
            }
            if (!kEarly && nitems > 0) load_item(0, 0, bufA);
            int it = 0;
#pragma unroll 1
            for (; it + 1 < nitems; it += 2) {
                step(it, bufA, bufB);
                step(it + 1, bufB, bufA);
            }
            if (it < nitems) step(it, bufA, bufB);
        }

        // Scales for all bands first (independent loads, one wait), then the
        // stores.
        float scl[MAXB];
#pragma unroll
        for (int bi = 0; bi < MAXB; ++bi) {
            const int v = min(((sj * MAXB + bi) * TW + gw) * T + my_t, V - 1);
            scl[bi] = wscale[v];
        }
#pragma unroll
        for (int bi = 0; bi < MAXB; ++bi) {
            const int band = (sj * MAXB + bi) * TW + gw;
            const int v = band * T + my_t;
            if (writer && band < NB && v < V)
                out[(size_t)my_r * V + v] = f32_to_bf16_rne(part[bi] * scl[bi]);
        }
    }
}

// ---------------------------------------------------------------- launch

// A launch shape: T vocab rows per wave, WAVES waves per workgroup, MAXB
// bands per wave between activation restagings, BPC workgroups per CU.
template <int R, int T, int WAVES, int MAXB, int BPC>
static hipError_t launch_fp8(const uint8_t* W, const float* wscale, const uint16_t* x, int H,
                             int V, uint16_t* out, const DeviceInfo& dev, hipStream_t stream) {
    const int64_t NB = (V + T - 1) / T;
    int64_t blocks = (NB + WAVES - 1) / WAVES;
    if (blocks > (int64_t)dev.num_cus * BPC) blocks = (int64_t)dev.num_cus * BPC;
    if constexpr (BPC == 1) {
        // One workgroup per CU: the fewest workgroups that take the same
        // number of band rounds, so the last round is not a partial one
        // (4 rows: 204 -> 199 us on the 155136-row head, a few CUs idle);
        // with several workgroups per CU the full grid is faster.
        const int64_t rounds = (NB + blocks * WAVES - 1) / (blocks * WAVES);
        blocks = (NB + rounds * WAVES - 1) / (rounds * WAVES);
    }
    const int64_t TW = blocks * WAVES;
    const int64_t per_wave = (NB + TW - 1) / TW;
    const int nsuper = (int)((per_wave + MAXB - 1) / MAXB);
    hipLaunchKernelGGL((fp8_gemv_kernel<R, T, WAVES, MAXB, BPC>), dim3((unsigned)blocks),
                       dim3(WAVES * kWave), 0, stream, W, wscale, x, H, V, out, nsuper);
    return hipGetLastError();
}

// Launch shape per row count, chosen by timing the 155136 x 8192 head on
// MI355X. Few rows are HBM-bound: many small workgroups keep more 16-byte
// loads in flight. From 5 rows on the VALU bounds the kernel: wider bands (T)
// cut LDS activation reads per weight byte (2R/T bytes) and 8-wave groups
// leave room for T*R accumulators. The shape never changes a row's bits.
hipError_t run_fp8_w8a16(const uint8_t* W, const float* wscale, const uint16_t* x, int R, int H,
                         int V, uint16_t* out, const DeviceInfo& dev, hipStream_t stream) {
    // Heads with few vocab rows (the SiLU down projection's 7168): with
    // 4-row bands the 9..16-row shape gives a wave fewer than two bands and
    // leaves waves idle; 2-row bands in 16-wave groups keep them busy.
    // Heads of fewer than 4 two-row bands per wave of a 32-wave-per-CU grid
    // (the 32000 x 4096 head): 1 and 2 rows take the shapes that measured
    // fastest there (32000 x 4096 with 7 rotated copies: 1 row 27.7 ->
    // 24.6 us, 2 rows 29.4 -> 25.5 us; on the 155136-row head they lose 3 %).
    const bool narrow = (int64_t)(V + 1) / 2 < (int64_t)dev.num_cus * 32 * 4;
    if (narrow && R == 1) return launch_fp8<1, 2, 4, 12, 8>(W, wscale, x, H, V, out, dev, stream);
    if (narrow && R == 2) return launch_fp8<2, 4, 16, 12, 1>(W, wscale, x, H, V, out, dev, stream);
    const bool skinny = R >= 9 && (int64_t)(V + 3) / 4 < 2 * (int64_t)dev.num_cus * 8;
    if (skinny) {
        switch (R) {
#define QH_FP8_SKINNY(RR)                                                                     \
    case RR:                                                                                  \
        return launch_fp8<RR, 2, 16, 8, 1>(W, wscale, x, H, V, out, dev, stream);
            QH_FP8_SKINNY(9)
            QH_FP8_SKINNY(10)
            QH_FP8_SKINNY(11)
            QH_FP8_SKINNY(12)
            QH_FP8_SKINNY(13)
            QH_FP8_SKINNY(14)
            QH_FP8_SKINNY(15)
            QH_FP8_SKINNY(16)
#undef QH_FP8_SKINNY
            default:
                break;
        }
    }
    switch (R) {
#define QH_FP8_CASE(RR, TT, WV, MB, BPC)                                                       \
    case RR:                                                                                  \
        return launch_fp8<RR, TT, WV, MB, BPC>(W, wscale, x, H, V, out, dev, stream);
        QH_FP8_CASE(1, 2, 8, 12, 4)
        QH_FP8_CASE(2, 4, 4, 12, 4)
        QH_FP8_CASE(3, 4, 16, 12, 1)
        QH_FP8_CASE(4, 4, 16, 12, 1)
        QH_FP8_CASE(5, 8, 8, 12, 1)
        QH_FP8_CASE(6, 8, 8, 12, 1)
        QH_FP8_CASE(7, 8, 8, 12, 1)
        QH_FP8_CASE(8, 8, 8, 12, 1)
        QH_FP8_CASE(9, 4, 8, 20, 1)
        QH_FP8_CASE(10, 4, 8, 20, 1)
        QH_FP8_CASE(11, 4, 8, 20, 1)
        QH_FP8_CASE(12, 4, 8, 20, 1)
        QH_FP8_CASE(13, 4, 8, 20, 1)
        QH_FP8_CASE(14, 4, 8, 20, 1)
        QH_FP8_CASE(15, 4, 8, 20, 1)
        QH_FP8_CASE(16, 4, 8, 20, 1)
#undef QH_FP8_CASE
        default:
            return hipErrorInvalidValue;
    }
}


}  // namespace qh
