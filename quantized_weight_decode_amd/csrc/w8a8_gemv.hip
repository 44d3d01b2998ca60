// w8a8_gemv.hip -- W8A8 head GEMV on gfx950: E4M3 weights with one F32 scale
// per weight row times per-row E4M3 activations, FP32 accumulation, BF16
// logits. The head's FP8 bytes and row scales are read in place
// ("lm_head_fp8_rows.rs": set_lm_head_w8a8; module doc: one weight pass per
// 128 rows, W8A8_MAX_ROWS), over the activations quantized into the scratch
// ("w8a8_layer.rs": W8a8Ctx::proj / silu_proj), and a row's logits do not
// depend on how many rows share the call ("w8a8_layer.rs" module doc).
//
// One arithmetic for every row count, served by two kernels:
//  * 1..15 rows: VALU kernel, one v_dot2_f32_bf16 per activation-weight pair;
//  * 16..128 rows: MFMA kernel, v_mfma_f32_16x16x32_bf16, one weight pass
//    for all rows of the launch.
// An MFMA of this shape adds the 8 products of each 16-lane group as one
// step; when exactly one BF16 pair of a step is nonzero, the step rounds
// exactly like v_dot2_f32_bf16 on that pair (checked bit for bit on the
// device over adversarial pairs and over full-length dot products). The MFMA
// kernel therefore feeds each instruction a weight operand with a single
// nonzero pair per lane group (a quarter of the instruction's products are
// useful) and adds the same pairs in the same order as the VALU kernel:
//   per 4096-k tile, 8 chains per logit; chain c takes the 16-k granules at
//   tile-local k = 16c + 128i (i = 0, 1, ...), each granule's 8 pairs in k
//   order, one dot2-rounded step per pair, starting from +0;
//   tile sum = ((c0 + c1) + (c2 + c3)) + ((c4 + c5) + (c6 + c7));
//   acc = the tile sums added in tile order;
//   out = bf16( fl32( fl32(acc * xscale[r]) * wscale[v] ) ).
// Pairs at k >= hidden have zero activations and leave a chain unchanged.
// Eight chains keep the VALU kernel's weight reads in 128-byte runs per row
// (8 lanes x 16 bytes), which stream near the rate of longer runs, while the
// MFMA kernel holds 8 chains x 8 row tiles of accumulators at 128 rows.
#include "lds_dma.h"
#include "qhead_device.h"
#include "qhead_internal.h"

namespace qh {
namespace {

constexpr int kChains = 8;
constexpr int kGranK = 16;                       // k per granule: one 16-byte weight load
constexpr int kStepK = kChains * kGranK;         // 128: one granule of each chain
constexpr int kSlabK = 2 * kStepK;               // 256: two granules of each chain
constexpr int kW8TileK = 4096;                   // k per reduction tile
constexpr int kSlabsPerTile = kW8TileK / kSlabK;  // 16
constexpr int kTileVec = kW8TileK / 8;           // uint4 of BF16 per row per tile

// 16 E4M3 bytes -> 8 BF16 pairs (pair p = bytes 2p, 2p+1), exact.
__device__ __forceinline__ void e4m3x16_to_bf16(const uint4& w, uint32_t (&p)[8]) {
    e4m3x4_to_bf16(w.x, p[0], p[1]);
    e4m3x4_to_bf16(w.y, p[2], p[3]);
    e4m3x4_to_bf16(w.z, p[4], p[5]);
    e4m3x4_to_bf16(w.w, p[6], p[7]);
}

// ------------------------------------------------------------ VALU kernel

// Stage tile columns [k0, k0 + 8 * nvec) of R rows of E4M3 codes into LDS as
// BF16 (exact), row r at xs + r * kTileVec; k >= H is staged as zero.
template <int R, int NTHREADS>
__device__ __forceinline__ void stage_codes_bf16(uint4* xs, const uint8_t* xq, int H, int k0,
                                                 int nvec) {
    const int total = R * nvec;
    for (int idx = threadIdx.x; idx < total; idx += NTHREADS) {
        const int r = idx / nvec;
        const int q = idx - r * nvec;
        const int k = k0 + q * 8;
        uint4 val = make_uint4(0, 0, 0, 0);
        if (k < H) {
            const uint2 codes = *reinterpret_cast<const uint2*>(xq + (size_t)r * H + k);
            e4m3x4_to_bf16(codes.x, val.x, val.y);
            e4m3x4_to_bf16(codes.y, val.z, val.w);
        }
        xs[r * kTileVec + q] = val;
    }
}

// The dot2 steps of one 16-k granule of every chain a lane holds: for each
// row r and vocab row t, acc[r * T + t] takes the 8 pairs of wb[t] times the
// activation pairs of row r (two 16-byte LDS words at xlo + r * RS for rows
// 0..7, xhi + (r - 8) * RS above), in pair order.
template <int R, int T, int RS, int NP>
__device__ __forceinline__ void granule_dots(float (&acc)[NP], const uint32_t (&wb)[T][8],
                                             const uint4* xlo, const uint4* xhi) {
    if constexpr (R >= 4) {
        // Rows in groups of G: for each pair p the G * T chains of a group
        // take their dot2 one after the other (independent chains keep the
        // VALU issuing); each chain still adds its pairs in k order. The next
        // group's activations are read while this one is computed.
        constexpr int G = T >= 4 ? 4 : 2;
        uint32_t xg[2][G][8];
        auto read_group = [&](int rg, uint32_t(&dst)[G][8]) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                if (rg + g < R) {
                    const uint4* xp = (rg + g) < 8 ? xlo + (rg + g) * RS : xhi + (rg + g - 8) * RS;
                    const uint4 xa = xp[0];
                    const uint4 xb = xp[1];
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
        constexpr int LA = R < 2 ? R : 2;
        constexpr int NBUF = LA + 1;
        uint4 xr[NBUF][2];
#pragma unroll
        for (int r = 0; r < LA; ++r) {
            xr[r][0] = xlo[r * RS];
            xr[r][1] = xlo[r * RS + 1];
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (r + LA < R) {
                xr[(r + LA) % NBUF][0] = xlo[(r + LA) * RS];
                xr[(r + LA) % NBUF][1] = xlo[(r + LA) * RS + 1];
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
}

// Lanes: chain c = lane bits {0, 1, 3}, vocab slot o = lane bits {2, 4, 5};
// a band is 8 slots x T consecutive vocab rows. An item is (band, 128-k
// step): lane (c, o) loads the 16 weight bytes of granule c of the step for
// each of its T rows, a 128-byte run per row across the eight chains. The
// chains of a logit sit on lanes l, l^1, l^2, ..., l^11, so the tree is three
// DPP steps: quad l^1, quad l^2, row_ror:8 (l^8).
template <int R, int T, int WAVES, int MAXB, int BPC>
__global__ void __launch_bounds__(WAVES * kWave, (WAVES * BPC + 3) / 4)
w8a8_valu_kernel(const uint8_t* __restrict__ W, const float* __restrict__ wscale,
                 const uint8_t* __restrict__ xq, const float* __restrict__ xscale, int H, int V,
                 uint16_t* __restrict__ out, int nsuper) {
    constexpr int N = T * R;
    constexpr int NP = next_pow2(N);
    constexpr int NP1 = half_or_one(NP);
    constexpr int NP2 = half_or_one(NP1);
    constexpr int NQ = half_or_one(NP2);  // values a lane holds per band after the tree
    constexpr int BAND = 8 * T;
    static_assert(NP <= 64, "T*R must be <= 64");
    __shared__ uint4 xs[R * kTileVec];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = (lane & 3) | ((lane >> 1) & 4);
    const int o = ((lane >> 2) & 1) | ((lane >> 3) & 6);
    const int TW = gridDim.x * WAVES;
    const int gw = blockIdx.x * WAVES + wave;
    const int NB = (V + BAND - 1) / BAND;
    const int NT = (H + kW8TileK - 1) / kW8TileK;
    // Offset (in 16-byte vectors) of activation row 8 in the LDS tile, kept
    // opaque so that rows 8 and up are read from a second base.
    int hi_rows = 8 * kTileVec;
    if constexpr (R > 8) asm volatile("" : "+v"(hi_rows));

    // Index (r * T + t) of the first value this lane holds after the tree:
    // each of the three levels halves the values a lane holds while more
    // than one is left (lanes with the level's bit set keep the upper half);
    // a level reached with one value left sums, and only lanes with that
    // level's bit clear store.
    int idx0 = 0;
    bool writer = true;
    {
        int n = NP;
        const int bits[3] = {lane & 1, (lane >> 1) & 1, (lane >> 3) & 1};
#pragma unroll
        for (int lv = 0; lv < 3; ++lv) {
            if (n >= 2) {
                n /= 2;
                idx0 += bits[lv] * n;
            } else if (bits[lv]) {
                writer = false;
            }
        }
    }

    for (int sj = 0; sj < nsuper; ++sj) {
        float part[MAXB][NQ];
#pragma unroll
        for (int bi = 0; bi < MAXB; ++bi)
#pragma unroll
            for (int q = 0; q < NQ; ++q) part[bi][q] = 0.0f;

        for (int tt = 0; tt < NT; ++tt) {
            const int k0 = tt * kW8TileK;
            const int klen = min(kW8TileK, H - k0);
            const int nstep = (klen + kStepK - 1) / kStepK;
            if (NT > 1 || sj == 0) {
                __syncthreads();
                stage_codes_bf16<R, WAVES * kWave>(xs, xq, H, k0, nstep * (kStepK / 8));
                __syncthreads();
            }
            const int first = (sj * MAXB) * TW + gw;
            const int nbb = first < NB ? min(MAXB, (NB - 1 - first) / TW + 1) : 0;
            const int nitems = nbb * nstep;
            // Unconditional loads: a lane past the hidden tail re-reads the
            // row's last 16 bytes (times zero activations), a row past the
            // vocab tail re-reads the last row (never stored).
            auto load_item = [&](int bi, int s, uint4(&dst)[T]) {
                const int v0 = ((sj * MAXB + bi) * TW + gw) * BAND + o * T;
                const int k = min(k0 + s * kStepK + c * kGranK, H - 16);
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    const int v = min(v0 + t, V - 1);
                    dst[t] = load_stream16(W + (size_t)v * H + k);
                }
            };
            float acc[NP];
            int bi = 0, s = 0;
            auto step = [&](int it, const uint4(&cur)[T], uint4(&nxt)[T]) {
                {
                    const bool last = it + 1 >= nitems;
                    const int nbi = last ? bi : ((s + 1 == nstep) ? bi + 1 : bi);
                    const int ns = last ? s : ((s + 1 == nstep) ? 0 : s + 1);
                    load_item(nbi, ns, nxt);
                }
                __builtin_amdgcn_sched_barrier(0);
                if (s == 0) {
#pragma unroll
                    for (int i = 0; i < NP; ++i) acc[i] = 0.0f;
                }
                uint32_t wb[T][8];
#pragma unroll
                for (int t = 0; t < T; ++t) e4m3x16_to_bf16(cur[t], wb[t]);
                const uint4* xrow = xs + s * (kStepK / 8) + 2 * c;
                granule_dots<R, T, kTileVec>(acc, wb, xrow, xrow + hi_rows);
                if (s + 1 == nstep) {
                    dpp_level<kDppQuadXor1, 1, NP>(acc, lane);
                    dpp_level<kDppQuadXor2, 2, NP1>(prefix<NP1>(acc), lane);
                    dpp_level<kDppRowRor8, 8, NP2>(prefix<NP2>(acc), lane);
#pragma unroll
                    for (int j = 0; j < MAXB; ++j)
                        if (j == bi) {
#pragma unroll
                            for (int q = 0; q < NQ; ++q)
                                part[j][q] = (tt == 0) ? acc[q] : part[j][q] + acc[q];
                        }
                    ++bi;
                    s = 0;
                } else {
                    ++s;
                }
            };
            uint4 bufA[T], bufB[T];
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
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const int idx = idx0 + q;
                const int r = idx / T;
                const int t = idx - r * T;
                const int v = band * BAND + o * T + t;
                if (writer && idx < N && band < NB && v < V) {
                    const float y = (part[bi][q] * xscale[r]) * wscale[v];
                    out[(size_t)r * V + v] = f32_to_bf16_rne(y);
                }
            }
        }
    }
}

template <int R, int T, int WAVES, int MAXB, int BPC>
hipError_t launch_valu(const uint8_t* W, const float* ws, const uint8_t* xq, const float* xs,
                       int H, int V, uint16_t* out, const DeviceInfo& dev, hipStream_t stream) {
    const int64_t NB = (V + 8 * T - 1) / (8 * T);
    int64_t blocks = (NB + WAVES - 1) / WAVES;
    if (blocks > (int64_t)dev.num_cus * BPC) blocks = (int64_t)dev.num_cus * BPC;
    const int64_t TW = blocks * WAVES;
    const int64_t per_wave = (NB + TW - 1) / TW;
    const int nsuper = (int)((per_wave + MAXB - 1) / MAXB);
    hipLaunchKernelGGL((w8a8_valu_kernel<R, T, WAVES, MAXB, BPC>), dim3((unsigned)blocks),
                       dim3(WAVES * kWave), 0, stream, W, ws, xq, xs, H, V, out, nsuper);
    return hipGetLastError();
}

// ----------------------------------------------- split VALU kernel (narrow V)

// A projection with few output rows (a few thousand, as in an FFN down
// projection) gives the kernel above too few bands, and so too few waves, to
// keep the weight stream busy. Here the KS waves of a workgroup share one band
// (8 slots x T vocab rows, the same lanes as above) and split the hidden
// dimension by 4096-k tile: wave w takes tiles w, w + KS, ... Each wave walks
// its items (tile, 128-k step) through a ring of PF loads in flight; an item
// holds the T weight granules of the lane and the step's activation codes (a
// lane of row a = lane / 8 (+ 8) and chain lane % 8 loads that granule), which
// the wave converts into a private LDS window before its lanes read the pairs
// of their chain. There is no barrier until the band ends: every wave leaves
// its tile sums (after the same tree as above) in LDS, and wave 0 adds them in
// tile order. Chains, pair order, tree and tile order equal the kernel above,
// so the logits carry the same bits.
template <int R, int T, int PF>
__global__ void __launch_bounds__(8 * kWave)
w8a8_valu_split_kernel(const uint8_t* __restrict__ W, const float* __restrict__ wscale,
                       const uint8_t* __restrict__ xq, const float* __restrict__ xscale, int H,
                       int V, uint16_t* __restrict__ out, int nbw) {
    constexpr int N = T * R;
    constexpr int NP = next_pow2(N);
    constexpr int NP1 = half_or_one(NP);
    constexpr int NP2 = half_or_one(NP1);
    constexpr int NQ = half_or_one(NP2);
    constexpr int BAND = 8 * T;
    constexpr int NA = (R + 7) / 8;               // activation loads per lane per item
    constexpr int WIN = R * kChains * 2;          // uint4 per wave window (one step)
    constexpr int kStepsPerTile = kW8TileK / kStepK;
    static_assert(NP <= 64, "T*R must be <= 64");
    static_assert(PF >= 2, "ring of at least two items");
    extern __shared__ uint4 lds_dyn[];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int KS = blockDim.x >> 6;
    const int c = (lane & 3) | ((lane >> 1) & 4);
    const int o = ((lane >> 2) & 1) | ((lane >> 3) & 6);
    const int NB = (V + BAND - 1) / BAND;
    const int NT = (H + kW8TileK - 1) / kW8TileK;
    const int last_steps = (H - (NT - 1) * kW8TileK + kStepK - 1) / kStepK;
    // this wave's tiles: wave, wave + KS, ... (the launch keeps KS <= NT)
    const int nq = (NT - wave + KS - 1) / KS;
    const bool owns_last = (NT - 1 - wave) % KS == 0;
    const int ipb = nq * kStepsPerTile - (owns_last ? kStepsPerTile - last_steps : 0);
    const int total = nbw * ipb;

    uint4* win = lds_dyn + wave * WIN;
    float* tsum = reinterpret_cast<float*>(lds_dyn + KS * WIN);

    int idx0 = 0;
    bool writer = true;
    {
        int n = NP;
        const int bits[3] = {lane & 1, (lane >> 1) & 1, (lane >> 3) & 1};
#pragma unroll
        for (int lv = 0; lv < 3; ++lv) {
            if (n >= 2) {
                n /= 2;
                idx0 += bits[lv] * n;
            } else if (bits[lv]) {
                writer = false;
            }
        }
    }

    // Item positions: band j of this workgroup, tile q of this wave, step s.
    struct Pos {
        int j, q, s;
    };
    auto steps_of = [&](int q) { return (q == nq - 1 && owns_last) ? last_steps : kStepsPerTile; };
    auto advance = [&](Pos& p) {
        if (++p.s == steps_of(p.q)) {
            p.s = 0;
            if (++p.q == nq) {
                p.q = 0;
                ++p.j;
            }
        }
    };
    // Unconditional loads: past the hidden tail a lane re-reads the row's
    // last 16 bytes (its activations are zero), past the vocab tail the last
    // row (never stored), past the last band of the grid the last row.
    auto load_item = [&](const Pos& p, uint4(&wd)[T], uint4(&ad)[NA]) __attribute__((always_inline)) {
        const int band = blockIdx.x + p.j * gridDim.x;
        const int kb = (wave + KS * p.q) * kW8TileK + p.s * kStepK;
        const int k = min(kb + c * kGranK, H - 16);
        const int v0 = band * BAND + o * T;
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int v = min(v0 + t, V - 1);
            wd[t] = load_stream16(W + (size_t)v * H + k);
        }
        const int ka = min(kb + (lane & 7) * kGranK, H - 16);
#pragma unroll
        for (int a = 0; a < NA; ++a) {
            const int r = min((lane >> 3) + 8 * a, R - 1);
            ad[a] = *reinterpret_cast<const uint4*>(xq + (size_t)r * H + ka);
        }
    };

    uint4 wring[PF][T];
    uint4 aring[PF][NA];
    float acc[NP];
    float part[NQ];
    Pos cur{0, 0, 0};
    Pos pf{0, 0, 0};
    int pf_it = 0;
#pragma unroll
    for (int i = 0; i + 1 < PF; ++i) {
        load_item(pf, wring[i], aring[i]);
        if (pf_it + 1 < total) {
            advance(pf);
            ++pf_it;
        }
    }

    auto item = [&](auto sl_tag) __attribute__((always_inline)) {
        constexpr int SL = decltype(sl_tag)::value;
        load_item(pf, wring[(SL + PF - 1) % PF], aring[(SL + PF - 1) % PF]);
        if (pf_it + 1 < total) {
            advance(pf);
            ++pf_it;
        }
        __builtin_amdgcn_sched_barrier(0);
        if (cur.s == 0) {
#pragma unroll
            for (int i = 0; i < NP; ++i) acc[i] = 0.0f;
        }
        const int tt = wave + KS * cur.q;
        const int kb = tt * kW8TileK + cur.s * kStepK;
        // this step's activations into the window: [row][chain] x 2 uint4
        {
            const bool kin = kb + (lane & 7) * kGranK < H;
#pragma unroll
            for (int a = 0; a < NA; ++a) {
                const int r = (lane >> 3) + 8 * a;
                if (r < R) {
                    uint32_t pr[8];
                    e4m3x16_to_bf16(aring[SL][a], pr);
                    uint4* dst = win + (r * kChains + (lane & 7)) * 2;
                    dst[0] = kin ? make_uint4(pr[0], pr[1], pr[2], pr[3]) : make_uint4(0, 0, 0, 0);
                    dst[1] = kin ? make_uint4(pr[4], pr[5], pr[6], pr[7]) : make_uint4(0, 0, 0, 0);
                }
            }
        }
        uint32_t wb[T][8];
#pragma unroll
        for (int t = 0; t < T; ++t) e4m3x16_to_bf16(wring[SL][t], wb[t]);
        // the window's writes come before its reads (a wave's LDS accesses
        // run in order; this keeps the compiler from moving the reads up)
        asm volatile("" ::: "memory");
        const uint4* xrow = win + 2 * c;
        granule_dots<R, T, kChains * 2>(acc, wb, xrow, xrow + 8 * kChains * 2);
        asm volatile("" ::: "memory");
        if (cur.s + 1 == steps_of(cur.q)) {
            dpp_level<kDppQuadXor1, 1, NP>(acc, lane);
            dpp_level<kDppQuadXor2, 2, NP1>(prefix<NP1>(acc), lane);
            dpp_level<kDppRowRor8, 8, NP2>(prefix<NP2>(acc), lane);
#pragma unroll
            for (int q = 0; q < NQ; ++q) tsum[(tt * NQ + q) * kWave + lane] = acc[q];
            if (cur.q == nq - 1) {
                // end of the band: its tile sums in tile order, by wave 0
                __syncthreads();
                const int band = blockIdx.x + cur.j * gridDim.x;
                if (wave == 0) {
#pragma unroll
                    for (int q = 0; q < NQ; ++q) part[q] = tsum[q * kWave + lane];
                    for (int t2 = 1; t2 < NT; ++t2)
#pragma unroll
                        for (int q = 0; q < NQ; ++q)
                            part[q] = part[q] + tsum[(t2 * NQ + q) * kWave + lane];
#pragma unroll
                    for (int q = 0; q < NQ; ++q) {
                        const int idx = idx0 + q;
                        const int r = idx / T;
                        const int t = idx - r * T;
                        const int v = band * BAND + o * T + t;
                        if (writer && idx < N && band < NB && v < V) {
                            const float y = (part[q] * xscale[r]) * wscale[v];
                            out[(size_t)r * V + v] = f32_to_bf16_rne(y);
                        }
                    }
                }
                __syncthreads();
            }
        }
        advance(cur);
    };

    int it = 0;
#pragma unroll 1
    for (; it + PF <= total; it += PF)
        static_for<PF>([&](auto sl) __attribute__((always_inline)) { item(sl); });
    static_for<PF>([&](auto sl) __attribute__((always_inline)) {
        if (it + decltype(sl)::value < total) item(sl);
    });
}

// LDS bytes of the split kernel: KS windows, then NT x NQ x 64 tile sums.
template <int R, int T>
constexpr size_t split_lds_bytes(int KS, int NT) {
    constexpr int NQ = half_or_one(half_or_one(half_or_one(next_pow2(T * R))));
    return (size_t)KS * R * kChains * 2 * 16 + (size_t)NT * NQ * kWave * 4;
}

template <int R, int T, int PF>
hipError_t launch_valu_split(const uint8_t* W, const float* ws, const uint8_t* xq, const float* xs,
                             int H, int V, uint16_t* out, const DeviceInfo& dev,
                             hipStream_t stream) {
    const int NT = (H + kW8TileK - 1) / kW8TileK;
    const int KS = NT < 8 ? NT : 8;
    const int64_t NB = (V + 8 * T - 1) / (8 * T);
    int64_t blocks = NB;
    const int64_t cap = (int64_t)dev.num_cus * 16;
    if (blocks > cap) blocks = cap;
    const int nbw = (int)((NB + blocks - 1) / blocks);
    const size_t lds = split_lds_bytes<R, T>(KS, NT);
    hipLaunchKernelGGL((w8a8_valu_split_kernel<R, T, PF>), dim3((unsigned)blocks),
                       dim3(KS * kWave), lds, stream, W, ws, xq, xs, H, V, out, nbw);
    return hipGetLastError();
}

// ------------------------------------------------------------ MFMA kernel

// A workgroup holds VTW vocab tiles of 16 rows (the B columns of the MFMA)
// and computes them for all 16 * RT activation rows (RT row tiles, the A
// rows; rows >= R are zero). CS waves share a vocab tile: wave h owns chains
// h * 8/CS .. (h + 1) * 8/CS - 1 of it. The workgroup walks the hidden
// dimension in 256-k slabs: per slab each chain c has two granules, A at
// k_s + 16c and B at k_s + 128 + 16c. The activations of a slab are staged
// in LDS by the whole workgroup as the dense A operands, [chain][lane group
// g][row] x 16 bytes holding the BF16 pairs (A pair g, A pair 4+g, B pair g,
// B pair 4+g) -- the pairs that step g of instructions 0..3 multiply. A
// lane takes the weights of four chains as two 16-byte pieces (lane group
// g: chain g of the group, granule A, then B), or, with two chains per
// wave, those of a chain pair as one piece (lane group g: chain g/2,
// granule g & 1); they are converted to BF16 pairs and transposed across
// lane groups so that dword q of lane group g holds the pair that
// instruction q's step g multiplies; instruction t then uses a weight
// operand holding only dword t, so its step g adds exactly that one pair.
// The pieces come straight from HBM (LW = 0: 16-byte loads at a row stride)
// or, with LW = 1, through LDS: the workgroup reads each slab's weights in
// 256-byte runs per row (piece p = chain + 8 * granule of row w per
// thread), PF - 1 slabs ahead, and stages them raw one slab ahead, piece p
// of workgroup row w at slot 16w + (p ^ (w & 7)) (8 lanes of a 16-byte
// access take 8 distinct bank groups when a row is written and when 8 rows'
// pieces are read). LW = 1 pays with one wave per tile (4 pieces per lane
// and slab, loads far apart otherwise); with more waves per tile the direct
// loads measured faster. At the end of each 4096-k tile the chains go
// through the tree (across the waves of a tile through LDS) and restart
// from zero.
// The staged activations come either from the E4M3 codes, loaded two slabs
// ahead and converted and written by the workgroup while the previous slab
// computes, or (IMG = 1, direct weight loads) from an image of every slab's
// staged bytes built once per call (w8a8_image_kernel), copied into LDS by
// 16-byte loads that bypass the registers (global_load_lds_dwordx4): the
// conversion, the LDS writes and their registers leave the slab loop. Both
// stage the same bytes, so the results are bit-identical.
template <int RT>
__global__ void __launch_bounds__(256)
w8a8_image_kernel(const uint8_t* __restrict__ xq, int R, int H, uint4* __restrict__ img, int NS) {
    // One (slab, chain X, row r) unit per thread: slab s's image holds at
    // X * 4 * RP + g * RP + ((r & ~15) | ((r + X) & 15)) the 16 bytes that
    // the kernel below stages there (rows >= R and columns >= H as zero).
    constexpr int RP = 16 * RT;
    constexpr int UNITS = kChains * RP;
    constexpr int SLAB_VEC = kChains * 4 * RP;
    const int idx = (int)(blockIdx.x * 256 + threadIdx.x);
    const int s = idx / UNITS;
    if (s >= NS) return;
    const int u = idx - s * UNITS;
    const int X = u % kChains;
    const int r = u / kChains;
    const int ka = s * kSlabK + X * kGranK;
    const int kb = ka + kStepK;
    uint4 ca = make_uint4(0, 0, 0, 0), cb = make_uint4(0, 0, 0, 0);
    if (r < R && ka < H) ca = *reinterpret_cast<const uint4*>(xq + (size_t)r * H + ka);
    if (r < R && kb < H) cb = *reinterpret_cast<const uint4*>(xq + (size_t)r * H + kb);
    uint32_t pa[8], pb[8];
    e4m3x16_to_bf16(ca, pa);
    e4m3x16_to_bf16(cb, pb);
    uint4* dst = img + (size_t)s * SLAB_VEC + X * 4 * RP + ((r & ~15) | ((r + X) & 15));
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) dst[gg * RP] = make_uint4(pa[gg], pa[4 + gg], pb[gg], pb[4 + gg]);
}

template <int RT, int VTW, int CS, int PF, int LW, int IMG>
__global__ void __launch_bounds__(VTW * CS * kWave, (VTW * CS + 3) / 4)
w8a8_mfma_kernel(const uint8_t* __restrict__ W, const float* __restrict__ wscale,
                 const uint8_t* __restrict__ xq, const uint4* __restrict__ img,
                 const float* __restrict__ xscale, int R, int H, int V,
                 uint16_t* __restrict__ out, int nrounds) {
    constexpr int WAVES = VTW * CS;
    constexpr int RP = 16 * RT;
    constexpr int NTHREADS = WAVES * kWave;
    constexpr int NCW = kChains / CS;            // chains per wave
    constexpr int LG = NCW >= 4 ? 4 : 2;         // chains per weight-load group
    constexpr int NLW = NCW / 2;                 // 16-byte weight pieces per lane per slab
    constexpr int WRS = NTHREADS / 16;           // LW: workgroup rows one staging pass covers
    static_assert(WRS % 8 == 0, "at least two waves per workgroup");
    constexpr int SLAB_VEC = kChains * 4 * RP;   // uint4 per staged slab
    constexpr int UNITS = kChains * RP;          // (chain, row) staging units per slab
    constexpr int UPT = (UNITS + NTHREADS - 1) / NTHREADS;
    static_assert(CS == 1 || CS == 2 || CS == 4, "8 chains over 1, 2 or 4 waves");
    static_assert(PF % 2 == 0, "the staging slots follow the slab parity");
    // the tree's exchange reuses a slab buffer: (CS - 1) partial sums per tile
    static_assert((CS - 1) * VTW * RT * kWave <= SLAB_VEC, "exchange fits a slab buffer");
    // IMG: 16-byte loads straight into LDS per lane and slab (each wave a
    // contiguous 1 KiB run per load); every weight piece of a slab is
    // converted before they are issued.
    constexpr int DPT = SLAB_VEC / NTHREADS;
    static_assert(!IMG || (LW == 0 && SLAB_VEC % NTHREADS == 0 && NCW <= 4),
                  "image staging: direct weight loads, whole loads per wave");
    __shared__ uint4 xs[2][SLAB_VEC];
    __shared__ uint4 wl[LW ? 2 : 1][LW ? VTW * 16 * 16 : 1];
    __shared__ float xsc[RP];
    // the tile sums so far of each vocab tile (kept by its wave h = 0)
    __shared__ f32x4_t partl[VTW][RT][kWave];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int vt = wave / CS;
    const int h = wave - vt * CS;
    const int i16 = lane & 15;
    const int g = lane >> 4;
    const int ntiles = (V + 15) / 16;
    const int NS = (H + kSlabK - 1) / kSlabK;
    const int total = nrounds * NS;
    const int nblk = gridDim.x;

    // Staging: this thread's units u = threadIdx.x + j * NTHREADS = (chain X,
    // row r), chains fastest, so that 8 consecutive lanes load one 128-byte
    // run of a row (a lane per row would touch a cache line per lane). In LDS
    // the row slots of chain X are rotated by X within each 16-row block:
    // row r of chain X sits at slot (r & ~15) | ((r + X) & 15). A 16-byte LDS
    // access is served 8 lanes at a time over 32 banks (128 bytes); the 8
    // lanes of a write (8 chains, one row) then take 8 distinct 16-byte bank
    // groups, and so do 8 consecutive rows of a tile that an operand read
    // takes. Rows >= R load row R - 1 and are staged as they come: an MFMA
    // row of A only feeds the same row of the result, and those rows are
    // never stored. Columns k >= H are staged as zero.
    const uint8_t* ssrc[UPT];
    int sldo[UPT], skx[UPT];
    bool sact[UPT];
#pragma unroll
    for (int j = 0; j < UPT; ++j) {
        const int u = (int)threadIdx.x + j * NTHREADS;
        sact[j] = UNITS % NTHREADS == 0 || u < UNITS;
        const int uu = min(u, UNITS - 1);
        const int X = uu % kChains;
        const int r = uu / kChains;
        ssrc[j] = xq + (size_t)min(r, R - 1) * H;
        sldo[j] = X * 4 * RP + ((r & ~15) | ((r + X) & 15));
        skx[j] = X * kGranK;
    }
    // Loads stay unconditional (clamped addresses): a load inside a branch
    // would make the compiler wait for every load in flight.
    auto stage_load = [&](int k_s, uint4(&st)[UPT][2]) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < UPT; ++j)
#pragma unroll
            for (int gb = 0; gb < 2; ++gb)
                st[j][gb] = *reinterpret_cast<const uint4*>(
                    ssrc[j] + min(k_s + gb * kStepK + skx[j], H - 16));
    };
    auto stage_write = [&](int k_s, const uint4(&st)[UPT][2], uint4* dst) __attribute__((always_inline)) {
        const bool full = k_s + kSlabK <= H;  // uniform: no column past the end
#pragma unroll
        for (int j = 0; j < UPT; ++j) {
            if (sact[j]) {
                uint32_t pa[8], pb[8];
                e4m3x16_to_bf16(st[j][0], pa);
                e4m3x16_to_bf16(st[j][1], pb);
                if (!full) {
                    const bool oka = k_s + skx[j] < H;
                    const bool okb = k_s + kStepK + skx[j] < H;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        pa[i] = oka ? pa[i] : 0u;
                        pb[i] = okb ? pb[i] : 0u;
                    }
                }
#pragma unroll
                for (int gg = 0; gg < 4; ++gg)
                    dst[sldo[j] + gg * RP] = make_uint4(pa[gg], pa[4 + gg], pb[gg], pb[4 + gg]);
            }
        }
    };
    // Weight loads of a slab of vocab tile `tile`. LG = 4: two loads per
    // group of four chains (lane group g: chain g of the group; granule A,
    // then B), a 64-byte run per row. LG = 2: one load per chain pair (lane
    // group g: chain g/2 of the pair, granule g & 1), two 32-byte runs per row.
    int wkoff[NLW];
#pragma unroll
    for (int j = 0; j < NLW; ++j) {
        int X, gb;
        if constexpr (LG == 4) {
            X = h * NCW + (j >> 1) * 4 + g;
            gb = j & 1;
        } else {
            X = h * NCW + 2 * j + (g >> 1);
            gb = g & 1;
        }
        wkoff[j] = gb * kStepK + X * kGranK;
    }
    auto row_of = [&](int round) {
        const int tile = (round * nblk + (int)blockIdx.x) * VTW + vt;
        return min(tile * 16 + i16, V - 1);
    };
    auto wload = [&](const uint8_t* wrow, int k_s, uint4(&dst)[NLW]) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < NLW; ++j) dst[j] = load_stream16(wrow + min(k_s + wkoff[j], H - 16));
    };
    // LW = 1: thread t stages piece t % 16 of workgroup rows t / 16 + j * WRS
    // (j < NLW; NLW * WRS = VTW * 16 rows), workgroup row w being row w % 16
    // of the workgroup's tile w / 16; WRS is a multiple of 8, so every j has
    // the same slot offset. The lane's own pieces sit at wrd[j].
    const int wr0 = (int)threadIdx.x >> 4;
    const int wpc = (int)threadIdx.x & 15;
    const int wslot = 16 * wr0 + (wpc ^ (wr0 & 7));
    int wrd[NLW];
#pragma unroll
    for (int j = 0; j < NLW; ++j) {
        const int w = vt * 16 + i16;
        wrd[j] = 16 * w + ((wkoff[j] / kGranK) ^ (w & 7));
    }
    auto wrow0_of = [&](int round) { return (round * nblk + (int)blockIdx.x) * VTW * 16 + wr0; };
    int wrow0 = wrow0_of(0);
    auto wload_rows = [&](int k_s, uint4(&dst)[NLW]) __attribute__((always_inline)) {
        const int ko = min(k_s + wpc * kGranK, H - 16);
#pragma unroll
        for (int j = 0; j < NLW; ++j)
            dst[j] = load_stream16(W + (size_t)min(wrow0 + j * WRS, V - 1) * H + ko);
    };
    auto wstage = [&](const uint4(&src)[NLW], uint4* dst) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < NLW; ++j) dst[wslot + j * NTHREADS] = src[j];
    };

    f32x4_t acc[NCW][RT];
    // Activation codes of the next two slabs (slot n % 2 holds slab n's).
    uint4 st[2][UPT][2];
    // Weights of PF slabs in flight: slot (it % PF) holds slab it's bytes.
    uint4 wb[PF][NLW];
    // Weight operands of the chain in hand: instruction t's holds only
    // dword t; the other dwords stay zero for the whole kernel.
    uint4 bq[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) bq[t] = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int X = 0; X < NCW; ++X)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) acc[X][rt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    for (int r = threadIdx.x; r < RP; r += NTHREADS) xsc[r] = r < R ? xscale[r] : 0.0f;
    // Positions (slab index within the hidden dimension, round) of the slab
    // being computed, of the weights PF - 1 slabs ahead and of the activation
    // codes two slabs ahead; the last two stop at the last slab.
    int cs = 0, cround = 0;
    int ws_ = 0, wround = 0, wit = 0;
    int ss = 0, sit = 0;
    auto adv = [&](int& sl, int& rd) {
        if (++sl == NS) {
            sl = 0;
            ++rd;
        }
    };
    // IMG: wave w loads uint4 [(w * DPT + j) * 64, + 64) of each slab's
    // image, lane l one of them, into the same place of the slab buffer
    // (wave-uniform base and LDS address, the lane's offset 16 l).
    const uint32_t xs_lds = IMG ? __builtin_amdgcn_readfirstlane(lds_byte_offset(&xs[0][0])) : 0u;
    const uint32_t img_voff = (uint32_t)lane * 16u;
    auto img_slab = [&](int sn, int buf, uint32_t after) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < DPT; ++j) {
            const int v0 = (wave * DPT + j) * kWave;  // first uint4 of this run
            lds_dma16(img + (size_t)sn * SLAB_VEC + v0, img_voff,
                      xs_lds + (uint32_t)((buf * SLAB_VEC + v0) * 16), after);
        }
    };
    if constexpr (IMG) {
        img_slab(0, 0, 0u);
    } else {
        stage_load(0, st[0]);
        stage_write(0, st[0], xs[0]);
        if (sit + 1 < total) {
            ++sit;
            ss = ss + 1 == NS ? 0 : ss + 1;
        }
        stage_load(ss * kSlabK, st[1]);
    }
    const uint8_t* wrow = W + (size_t)row_of(0) * H;
    // The weights PF - 1 slabs ahead: position advance and load.
    auto wnext = [&]() {
        if (wit + 1 < total) {
            ++wit;
            adv(ws_, wround);
            if (ws_ == 0) {
                if constexpr (LW) wrow0 = wrow0_of(wround);
                else wrow = W + (size_t)row_of(wround) * H;
            }
        }
    };
    auto wissue = [&](uint4(&dst)[NLW]) __attribute__((always_inline)) {
        if constexpr (LW) wload_rows(ws_ * kSlabK, dst);
        else wload(wrow, ws_ * kSlabK, dst);
    };
#pragma unroll
    for (int p = 0; p + 1 < PF; ++p) {
        wissue(wb[p]);
        wnext();
    }
    if constexpr (LW) wstage(wb[0], wl[0]);
    const float* swp = wscale + row_of(0);
    if constexpr (IMG) wait_vmcnt<0>();
    __syncthreads();

    // One slab: SL = it % PF (a compile-time slot, the loop is unrolled by PF).
    auto slab = [&](auto sl_tag, int it) __attribute__((always_inline)) {
        constexpr int SL = decltype(sl_tag)::value;
        const int s = cs;
        const bool more = it + 1 < total;
        uint4* xb = xs[SL & 1];
        // A operands of this slab, chain by chain: chain XL + 1's are read
        // while chain XL's MFMAs run (at most two chains' held at once), the
        // first while the weights are converted.
        uint4 a[NCW][RT];
        auto read_a = [&](int XL) __attribute__((always_inline)) {
            const int X = h * NCW + XL;
            const int base = (X * 4 + g) * RP + ((i16 + X) & 15);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) a[XL][rt] = xb[base + rt * 16];
        };
        read_a(0);
        // Activation codes two slabs ahead (their slot held this slab's
        // codes, already in LDS), then the weights PF - 1 slabs ahead.
        if constexpr (!IMG) {
            if (sit + 1 < total) {
                ++sit;
                ss = ss + 1 == NS ? 0 : ss + 1;
            }
            stage_load(ss * kSlabK, st[SL % 2]);
            wissue(wb[(SL + PF - 1) % PF]);
            wnext();
        }
        // This slab's weight pieces: from LDS (staged in the previous slab)
        // or the load ring.
        uint4 wv[NLW];
#pragma unroll
        for (int j = 0; j < NLW; ++j) {
            if constexpr (LW) wv[j] = wl[SL & 1][wrd[j]];
            else wv[j] = wb[SL][j];
        }
        // This tile's row scale, loaded every slab so that no load sits in
        // the branch that stores (a load there stalls the prefetches above).
        const float sw = *swp;
        // This slab's weight pieces as BF16 pairs (cw[j] from piece j).
        uint32_t cw[NLW][8];
        if constexpr (IMG) {
            // IMG: the pieces are converted first, so that the compiler's
            // wait for them comes before the next slab's image loads (the
            // first of which takes the last converted word as an input);
            // a wait placed after those loads would also wait for them.
            // The image loads then fill the other buffer (read by every
            // wave in the previous slab, before its barrier) while this
            // slab's MFMAs run, followed by the weights PF - 1 slabs ahead.
#pragma unroll
            for (int j = 0; j < NLW; ++j) e4m3x16_to_bf16(wv[j], cw[j]);
            if (more) img_slab(s + 1 == NS ? 0 : s + 1, (SL + 1) & 1, cw[NLW - 1][7]);
            wissue(wb[(SL + PF - 1) % PF]);
            wnext();
        } else if (more) {
            // The next slab's activations into the other buffer (read by
            // every wave in the previous slab, before its barrier); its
            // conversion overlaps this slab's MFMAs.
            stage_write((s + 1 == NS ? 0 : s + 1) * kSlabK, st[(SL + 1) % 2], xs[(SL + 1) & 1]);
            if constexpr (LW) wstage(wb[(SL + 1) % PF], wl[(SL + 1) & 1]);
        }
        auto chain_mfma = [&](int XL, uint32_t p0, uint32_t p1, uint32_t p2, uint32_t p3)
            __attribute__((always_inline)) {
            if (XL + 1 < NCW) read_a(XL + 1);
            bq[0].x = p0;
            bq[1].y = p1;
            bq[2].z = p2;
            bq[3].w = p3;
            // Instruction t of every row tile before instruction t + 1:
            // consecutive MFMAs use different accumulators.
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
                    acc[XL][rt] = mfma_bf16(a[XL][rt], bq[t], acc[XL][rt]);
        };
        if constexpr (LG == 4) {
#pragma unroll
            for (int j = 0; j < NCW / 4; ++j) {
                // Four chains: a1[Q] = pair g of granule A of chain Q's row,
                // a1[4+Q] its pair 4+g; a2[] the same for granule B.
                uint32_t(&a1)[8] = cw[2 * j];
                uint32_t(&a2)[8] = cw[2 * j + 1];
                if constexpr (!IMG) {
                    e4m3x16_to_bf16(wv[2 * j], a1);
                    e4m3x16_to_bf16(wv[2 * j + 1], a2);
                }
                xpose4(a1[0], a1[1], a1[2], a1[3]);
                xpose4(a1[4], a1[5], a1[6], a1[7]);
                xpose4(a2[0], a2[1], a2[2], a2[3]);
                xpose4(a2[4], a2[5], a2[6], a2[7]);
#pragma unroll
                for (int q = 0; q < 4; ++q) chain_mfma(4 * j + q, a1[q], a1[4 + q], a2[q], a2[4 + q]);
            }
        } else {
#pragma unroll
            for (int j = 0; j < NCW / 2; ++j) {
                // Chains 2j, 2j+1: o[Q] holds pair g of granule Q's row
                // (Q = 2c + granule), o[4 + Q] its pair 4 + g.
                uint32_t(&o)[8] = cw[j];
                if constexpr (!IMG) e4m3x16_to_bf16(wv[j], o);
                xpose4(o[0], o[1], o[2], o[3]);
                xpose4(o[4], o[5], o[6], o[7]);
#pragma unroll
                for (int c = 0; c < 2; ++c)
                    chain_mfma(2 * j + c, o[2 * c], o[4 + 2 * c], o[2 * c + 1], o[5 + 2 * c]);
            }
        }
        // End of a 4096-k tile (or of the hidden dimension): the tree
        // ((c0 + c1) + (c2 + c3)) + ((c4 + c5) + (c6 + c7)) -- each wave its
        // chains' subtree, the workgroup's waves of a tile through LDS in
        // this slab's (consumed) buffer -- then the tile sum in tile order,
        // and the chains restart from zero.
        if ((s + 1) % kSlabsPerTile == 0 || s + 1 == NS) {
            f32x4_t sub[RT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                if constexpr (NCW == 8)
                    sub[rt] = ((acc[0][rt] + acc[1][rt]) + (acc[2][rt] + acc[3][rt])) +
                              ((acc[4][rt] + acc[5][rt]) + (acc[6][rt] + acc[7][rt]));
                else if constexpr (NCW == 4)
                    sub[rt] = (acc[0][rt] + acc[1][rt]) + (acc[2][rt] + acc[3][rt]);
                else
                    sub[rt] = acc[0][rt] + acc[1][rt];
            }
            if constexpr (CS > 1) {
                f32x4_t* xch = reinterpret_cast<f32x4_t*>(xb);
                __syncthreads();  // every wave is done reading this slab's buffer
                if (h > 0) {
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt)
                        xch[(((h - 1) * VTW + vt) * RT + rt) * kWave + lane] = sub[rt];
                }
                __syncthreads();
                if (h == 0) {
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt) {
                        const f32x4_t s1 = xch[((0 * VTW + vt) * RT + rt) * kWave + lane];
                        if constexpr (CS == 2) {
                            sub[rt] = sub[rt] + s1;
                        } else {
                            const f32x4_t s2 = xch[((1 * VTW + vt) * RT + rt) * kWave + lane];
                            const f32x4_t s3 = xch[((2 * VTW + vt) * RT + rt) * kWave + lane];
                            sub[rt] = (sub[rt] + s1) + (s2 + s3);
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            }
            if (h == 0) {
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
                    partl[vt][rt][lane] = (s < kSlabsPerTile) ? sub[rt] : partl[vt][rt][lane] + sub[rt];
            }
#pragma unroll
            for (int X = 0; X < NCW; ++X)
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) acc[X][rt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        }
        if (s + 1 == NS && h == 0) {
            const int tile = (cround * nblk + (int)blockIdx.x) * VTW + vt;
            const int v = tile * 16 + i16;
            if (tile < ntiles && v < V) {
                // Row offsets computed here, once per vocab tile: an opaque
                // copy of V keeps them from being hoisted out of the slab
                // loop, where they would hold registers for the whole loop.
                int Vq = V;
                asm volatile("" : "+s"(Vq));
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    const f32x4_t pt = partl[vt][rt][lane];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = rt * 16 + g * 4 + e;
                        if (r < R) {
                            const float y = (pt[e] * xsc[r]) * sw;
                            out[(size_t)r * Vq + v] = f32_to_bf16_rne(y);
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
        adv(cs, cround);
        if (cs == 0) swp = wscale + row_of(cround);
        // IMG: the next slab's image has landed once nothing is in flight
        // (the weight loads issued after it are waited for too).
        if constexpr (IMG) wait_vmcnt<0>();
        __syncthreads();
    };

    int it = 0;
#pragma unroll 1
    for (; it + PF <= total; it += PF)
        static_for<PF>([&](auto sl) __attribute__((always_inline)) {
            slab(sl, it + decltype(sl)::value);
        });
    static_for<PF>([&](auto sl) __attribute__((always_inline)) {
        if (it + decltype(sl)::value < total) slab(sl, it + decltype(sl)::value);
    });
}

template <int RT, int VTW, int CS, int PF, int LW = 0, int IMG = 0>
hipError_t launch_mfma(const uint8_t* W, const float* ws, const uint8_t* xq, const float* xs,
                       int R, int H, int V, uint16_t* out, void* image, const DeviceInfo& dev,
                       hipStream_t stream) {
    const int64_t ntiles = (V + 15) / 16;
    int64_t blocks = (ntiles + VTW - 1) / VTW;
    if (blocks > (int64_t)dev.num_cus) blocks = (int64_t)dev.num_cus;
    const int nrounds = (int)((ntiles + blocks * VTW - 1) / (blocks * VTW));
    if constexpr (IMG) {
        const int NS = (H + kSlabK - 1) / kSlabK;
        const int n = NS * kChains * 16 * RT;
        hipLaunchKernelGGL((w8a8_image_kernel<RT>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                           stream, xq, R, H, static_cast<uint4*>(image), NS);
    }
    hipLaunchKernelGGL((w8a8_mfma_kernel<RT, VTW, CS, PF, LW, IMG>), dim3((unsigned)blocks),
                       dim3(VTW * CS * kWave), 0, stream, W, ws, xq,
                       static_cast<const uint4*>(image), xs, R, H, V, out, nrounds);
    return hipGetLastError();
}

// A shape with direct weight loads: through the image when the caller gives
// room for one.
template <int RT, int VTW, int CS, int PF>
hipError_t launch_mfma_direct(const uint8_t* W, const float* ws, const uint8_t* xq, const float* xs,
                              int R, int H, int V, uint16_t* out, void* image,
                              const DeviceInfo& dev, hipStream_t stream) {
    if (image)
        return launch_mfma<RT, VTW, CS, PF, 0, 1>(W, ws, xq, xs, R, H, V, out, image, dev, stream);
    return launch_mfma<RT, VTW, CS, PF, 0, 0>(W, ws, xq, xs, R, H, V, out, nullptr, dev, stream);
}

}  // namespace

size_t w8a8_image_bytes(int H) {
    // one 128-row slab image (8 chains x 4 lane groups x 128 rows x 16 bytes)
    // per 256-k slab
    return H <= 0 ? 0 : (size_t)((H + kSlabK - 1) / kSlabK) * kChains * 4 * 128 * 16;
}

// One W8A8 launch of 1..128 rows. `image` (nullable): device memory of
// w8a8_image_bytes(H) bytes, 16-byte aligned, that the shapes with direct
// weight loads (from 17 rows on heads of fewer than four vocab tiles per CU,
// from 33 rows otherwise) fill with the staged BF16 activations and copy
// from.
hipError_t run_w8a8_gemv(const uint8_t* W, const float* sw, const uint8_t* xq, const float* sa,
                         int R, int H, int V, uint16_t* out, const DeviceInfo& dev,
                         hipStream_t stream, void* image) {
    // Narrow projections (fewer than two bands of the kernel below per SIMD)
    // split the hidden dimension over the waves of a workgroup instead, when
    // its LDS (windows and tile sums) stays within 64 KiB.
    const int T_main = R <= 4 ? 2 : 4;
    const int64_t bands_main = (V + 8 * T_main - 1) / (8 * T_main);
    const int NT = (H + kW8TileK - 1) / kW8TileK;
    if (R >= 1 && R < 16 && bands_main < (int64_t)dev.num_cus * 8 &&
        split_lds_bytes<15, 4>(NT < 8 ? NT : 8, NT) <= 65536) {
        switch (R) {
#define QH_W8_SPLIT(RR)   \
    case RR:              \
        return launch_valu_split<RR, 4, 4>(W, sw, xq, sa, H, V, out, dev, stream);
            QH_W8_SPLIT(1)
            QH_W8_SPLIT(2)
            QH_W8_SPLIT(3)
            QH_W8_SPLIT(4)
            QH_W8_SPLIT(5)
            QH_W8_SPLIT(6)
            QH_W8_SPLIT(7)
            QH_W8_SPLIT(8)
            QH_W8_SPLIT(9)
            QH_W8_SPLIT(10)
            QH_W8_SPLIT(11)
            QH_W8_SPLIT(12)
            QH_W8_SPLIT(13)
            QH_W8_SPLIT(14)
            QH_W8_SPLIT(15)
#undef QH_W8_SPLIT
            default:
                break;
        }
    }
    switch (R) {
#define QH_W8_VALU(RR, TT, WV, MB, BPC)                                                   \
    case RR:                                                                              \
        return launch_valu<RR, TT, WV, MB, BPC>(W, sw, xq, sa, H, V, out, dev, stream);
        QH_W8_VALU(1, 2, 8, 12, 4)
        QH_W8_VALU(2, 2, 8, 12, 2)
        QH_W8_VALU(3, 2, 8, 12, 2)
        QH_W8_VALU(4, 2, 8, 12, 2)
        QH_W8_VALU(5, 4, 8, 4, 1)
        QH_W8_VALU(6, 4, 8, 4, 1)
        QH_W8_VALU(7, 4, 8, 4, 1)
        QH_W8_VALU(8, 4, 8, 4, 1)
        QH_W8_VALU(9, 4, 8, 2, 1)
        QH_W8_VALU(10, 4, 8, 2, 1)
        QH_W8_VALU(11, 4, 8, 2, 1)
        QH_W8_VALU(12, 4, 8, 2, 1)
        QH_W8_VALU(13, 4, 8, 2, 1)
        QH_W8_VALU(14, 4, 8, 2, 1)
        QH_W8_VALU(15, 4, 8, 2, 1)
#undef QH_W8_VALU
        default:
            break;
    }
    if (R < 16 || R > 128) return hipErrorInvalidValue;
    // Launch shapes <RT, vocab tiles per workgroup, waves per tile, weight
    // slabs in flight>, eight waves per workgroup (two per SIMD): up to 32
    // rows one wave per tile, up to 64 two, above four (2 chains each).
    // Narrow projections (fewer than 4 vocab tiles per CU) take two tiles of
    // four waves per workgroup at every row count, for more workgroups.
    const int64_t ntiles = (V + 15) / 16;
    if (ntiles < (int64_t)dev.num_cus * 4) {
        switch ((R + 15) / 16) {
            case 1:
                return launch_mfma<1, 2, 4, 4, 1>(W, sw, xq, sa, R, H, V, out, nullptr, dev,
                                                  stream);
            case 2:
                return launch_mfma_direct<2, 2, 4, 4>(W, sw, xq, sa, R, H, V, out, image, dev,
                                                      stream);
            case 3:
                return launch_mfma_direct<3, 2, 4, 4>(W, sw, xq, sa, R, H, V, out, image, dev,
                                                      stream);
            case 4:
                return launch_mfma_direct<4, 2, 4, 4>(W, sw, xq, sa, R, H, V, out, image, dev,
                                                      stream);
            default:
                break;
        }
    }
    switch ((R + 15) / 16) {
        case 1:
            return launch_mfma<1, 8, 1, 4, 1>(W, sw, xq, sa, R, H, V, out, nullptr, dev, stream);
        case 2:
            return launch_mfma<2, 8, 1, 4, 1>(W, sw, xq, sa, R, H, V, out, nullptr, dev, stream);
        case 3:
            return launch_mfma_direct<3, 4, 2, 4>(W, sw, xq, sa, R, H, V, out, image, dev, stream);
        case 4:
            return launch_mfma_direct<4, 4, 2, 4>(W, sw, xq, sa, R, H, V, out, image, dev, stream);
        case 5:
            return launch_mfma_direct<5, 2, 4, 4>(W, sw, xq, sa, R, H, V, out, image, dev, stream);
        case 6:
            return launch_mfma_direct<6, 2, 4, 4>(W, sw, xq, sa, R, H, V, out, image, dev, stream);
        case 7:
            return launch_mfma_direct<7, 2, 4, 4>(W, sw, xq, sa, R, H, V, out, image, dev, stream);
        default:
            return launch_mfma_direct<8, 2, 4, 4>(W, sw, xq, sa, R, H, V, out, image, dev, stream);
    }
}

}  // namespace qh
