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
//   per 4096-k tile, 4 chains per logit; chain c takes the 16-k granules at
//   tile-local k = 16c + 64i (i = 0, 1, ...), each granule's 8 pairs in k
//   order, one dot2-rounded step per pair, starting from +0;
//   tile sum = (chain0 + chain1) + (chain2 + chain3);
//   acc = the tile sums added in tile order;
//   out = bf16( fl32( fl32(acc * xscale[r]) * wscale[v] ) ).
// Pairs at k >= hidden have zero activations and leave a chain unchanged.
#include "qhead_device.h"
#include "qhead_internal.h"

namespace qh {
namespace {

constexpr int kChains = 4;
constexpr int kGranK = 16;                       // k per granule: one 16-byte weight load
constexpr int kStepK = kChains * kGranK;         // 64: one granule of each chain
constexpr int kSlabK = 2 * kStepK;               // 128: two granules of each chain
constexpr int kW8TileK = 4096;                   // k per reduction tile
constexpr int kSlabsPerTile = kW8TileK / kSlabK;  // 32
constexpr int kTileVec = kW8TileK / 8;           // uint4 of BF16 per row per tile

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma_bf16(const uint4& a, const uint4& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Transpose of four dwords across the four 16-lane groups: afterwards
// register q of lane group g holds what register g of lane group q held.
__device__ __forceinline__ void xpose4(uint32_t& r0, uint32_t& r1, uint32_t& r2, uint32_t& r3) {
    auto a = __builtin_amdgcn_permlane32_swap(r0, r2, false, false);
    r0 = a[0];
    r2 = a[1];
    auto b = __builtin_amdgcn_permlane32_swap(r1, r3, false, false);
    r1 = b[0];
    r3 = b[1];
    auto d = __builtin_amdgcn_permlane16_swap(r0, r1, false, false);
    r0 = d[0];
    r1 = d[1];
    auto e = __builtin_amdgcn_permlane16_swap(r2, r3, false, false);
    r2 = e[0];
    r3 = e[1];
}

// ------------------------------------------------------------ VALU kernel

// Stage tile rows [k0, k0 + 8 * nvec) of R rows of E4M3 codes into LDS as
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

// Lanes: c = lane & 3 is the chain, o = lane >> 2 one of 16 vocab slots; a
// band is 16 slots x T consecutive vocab rows. An item is (band, 64-k step):
// lane (c, o) loads the 16 weight bytes of granule c of the step for each of
// its T rows, one coalesced 64-byte piece per row across the four chains.
template <int R, int T, int WAVES, int MAXB, int BPC>
__global__ void __launch_bounds__(WAVES * kWave, (WAVES * BPC + 3) / 4)
w8a8_valu_kernel(const uint8_t* __restrict__ W, const float* __restrict__ wscale,
                 const uint8_t* __restrict__ xq, const float* __restrict__ xscale, int H, int V,
                 uint16_t* __restrict__ out, int nsuper) {
    constexpr int N = T * R;
    constexpr int NP = next_pow2(N);
    constexpr int NQ = NP >= 4 ? NP / 4 : 1;  // values a lane holds per band after the tree
    constexpr int BAND = 16 * T;
    static_assert(NP <= 64, "T*R must be <= 64");
    __shared__ uint4 xs[R * kTileVec];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane & 3;
    const int o = lane >> 2;
    const int TW = gridDim.x * WAVES;
    const int gw = blockIdx.x * WAVES + wave;
    const int NB = (V + BAND - 1) / BAND;
    const int NT = (H + kW8TileK - 1) / kW8TileK;
    // Offset (in 16-byte vectors) of activation row 8 in the LDS tile, kept
    // opaque so that rows 8 and up are read from a second base.
    int hi_rows = 8 * kTileVec;
    if constexpr (R > 8) asm volatile("" : "+v"(hi_rows));

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
                for (int t = 0; t < T; ++t) {
                    e4m3x4_to_bf16(cur[t].x, wb[t][0], wb[t][1]);
                    e4m3x4_to_bf16(cur[t].y, wb[t][2], wb[t][3]);
                    e4m3x4_to_bf16(cur[t].z, wb[t][4], wb[t][5]);
                    e4m3x4_to_bf16(cur[t].w, wb[t][6], wb[t][7]);
                }
                const uint4* xrow = xs + s * (kStepK / 8) + 2 * c;
                const uint4* xrow_hi = xrow + hi_rows;
                if constexpr (R >= 4) {
                    // Rows in groups of G: for each pair p the G * T chains of
                    // a group take their dot2 one after the other (independent
                    // chains keep the VALU issuing); each chain still adds its
                    // pairs in k order. The next group's activations are read
                    // while this one is computed.
                    constexpr int G = T >= 4 ? 4 : 2;
                    uint32_t xg[2][G][8];
                    auto read_group = [&](int rg, uint32_t(&dst)[G][8]) {
#pragma unroll
                        for (int g = 0; g < G; ++g) {
                            if (rg + g < R) {
                                const uint4* xp = (rg + g) < 8 ? xrow + (rg + g) * kTileVec
                                                               : xrow_hi + (rg + g - 8) * kTileVec;
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
                        xr[r][0] = xrow[r * kTileVec];
                        xr[r][1] = xrow[r * kTileVec + 1];
                    }
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        if (r + LA < R) {
                            xr[(r + LA) % NBUF][0] = xrow[(r + LA) * kTileVec];
                            xr[(r + LA) % NBUF][1] = xrow[(r + LA) * kTileVec + 1];
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
                if (s + 1 == nstep) {
                    // (chain0 + chain1) + (chain2 + chain3): the four chains of a
                    // logit are the four lanes of a quad.
                    dpp_level<kDppQuadXor1, 1, NP>(acc, lane);
                    dpp_level<kDppQuadXor2, 2, half_or_one(NP)>(prefix<half_or_one(NP)>(acc), lane);
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

        // Index (r * T + t) of the values this lane holds after the tree.
        int idx0;
        bool writer;
        if constexpr (NP >= 4) {
            idx0 = (c & 1) * (NP / 2) + ((c >> 1) & 1) * (NP / 4);
            writer = true;
        } else if constexpr (NP == 2) {
            idx0 = c & 1;
            writer = (c >> 1) == 0;
        } else {
            idx0 = 0;
            writer = c == 0;
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
    const int64_t NB = (V + 16 * T - 1) / (16 * T);
    int64_t blocks = (NB + WAVES - 1) / WAVES;
    if (blocks > (int64_t)dev.num_cus * BPC) blocks = (int64_t)dev.num_cus * BPC;
    const int64_t TW = blocks * WAVES;
    const int64_t per_wave = (NB + TW - 1) / TW;
    const int nsuper = (int)((per_wave + MAXB - 1) / MAXB);
    hipLaunchKernelGGL((w8a8_valu_kernel<R, T, WAVES, MAXB, BPC>), dim3((unsigned)blocks),
                       dim3(WAVES * kWave), 0, stream, W, ws, xq, xs, H, V, out, nsuper);
    return hipGetLastError();
}

// ------------------------------------------------------------ MFMA kernel

// Each wave owns tiles of 16 vocab rows (the B columns of the MFMA) for all
// 16 * RT activation rows (RT row tiles, the A rows; rows >= R are zero).
// The workgroup walks the hidden dimension in 128-k slabs: per slab each
// chain has two granules (A at k_s + 16c, B at k_s + 64 + 16c). The
// activations of a slab are staged in LDS by the whole workgroup as the
// dense A operands, [chain][lane group g][row] x 16 bytes holding the BF16
// pairs (A pair g, A pair 4+g, B pair g, B pair 4+g) -- the pairs that step
// g of instructions 0..3 multiply. The weights are loaded per lane (lane
// group g: 16 bytes of chain g, granule A, then granule B), converted to
// BF16 pairs and transposed across lane groups so that dword q of lane group
// g holds the same pair of the weight row; instruction t then uses a weight
// operand holding only dword t, so its step g adds exactly that one pair.
template <int RT, int WAVES, int BPC>
__global__ void __launch_bounds__(WAVES * kWave, (WAVES * BPC + 3) / 4)
w8a8_mfma_kernel(const uint8_t* __restrict__ W, const float* __restrict__ wscale,
                 const uint8_t* __restrict__ xq, const float* __restrict__ xscale, int R, int H,
                 int V, uint16_t* __restrict__ out, int nrounds) {
    constexpr int RP = 16 * RT;
    constexpr int NTHREADS = WAVES * kWave;
    constexpr int SLAB_VEC = kChains * 4 * RP;  // uint4 per staged slab
    constexpr int UNITS = kChains * RP;          // (chain, row) staging units per slab
    constexpr int UPT = (UNITS + NTHREADS - 1) / NTHREADS;
    __shared__ uint4 xs[2][SLAB_VEC];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int i16 = lane & 15;
    const int g = lane >> 4;
    const int ntiles = (V + 15) / 16;
    const int NS = (H + kSlabK - 1) / kSlabK;
    const int total = nrounds * NS;

    // Staging of slab `it % NS`: unit u = (chain, row) with rows fastest, so
    // consecutive threads write consecutive 16-byte LDS words.
    auto stage_load = [&](int it, uint4(&st)[UPT][2]) {
        const int k_s = (it % NS) * kSlabK;
#pragma unroll
        for (int j = 0; j < UPT; ++j) {
            const int u = threadIdx.x + j * NTHREADS;
            const int r = u % RP;
            const int X = u / RP;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int k = k_s + h * kStepK + X * kGranK;
                uint4 v = make_uint4(0, 0, 0, 0);
                if (u < UNITS && r < R && k < H) {
                    const uint2* p = reinterpret_cast<const uint2*>(xq + (size_t)r * H + k);
                    const uint2 lo = p[0], hi = p[1];
                    v = make_uint4(lo.x, lo.y, hi.x, hi.y);
                }
                st[j][h] = v;
            }
        }
    };
    auto stage_write = [&](const uint4(&st)[UPT][2], uint4* dst) {
#pragma unroll
        for (int j = 0; j < UPT; ++j) {
            const int u = threadIdx.x + j * NTHREADS;
            if (u < UNITS) {
                const int r = u % RP;
                const int X = u / RP;
                uint32_t pa[8], pb[8];
                e4m3x4_to_bf16(st[j][0].x, pa[0], pa[1]);
                e4m3x4_to_bf16(st[j][0].y, pa[2], pa[3]);
                e4m3x4_to_bf16(st[j][0].z, pa[4], pa[5]);
                e4m3x4_to_bf16(st[j][0].w, pa[6], pa[7]);
                e4m3x4_to_bf16(st[j][1].x, pb[0], pb[1]);
                e4m3x4_to_bf16(st[j][1].y, pb[2], pb[3]);
                e4m3x4_to_bf16(st[j][1].z, pb[4], pb[5]);
                e4m3x4_to_bf16(st[j][1].w, pb[6], pb[7]);
#pragma unroll
                for (int gg = 0; gg < 4; ++gg)
                    dst[(X * 4 + gg) * RP + r] = make_uint4(pa[gg], pa[4 + gg], pb[gg], pb[4 + gg]);
            }
        }
    };
    auto tile_of = [&](int it) { return ((it / NS) * (int)gridDim.x + (int)blockIdx.x) * WAVES + wave; };
    auto wload = [&](int it, uint4(&dst)[2]) {
        const int k_s = (it % NS) * kSlabK;
        const int v = min(tile_of(it) * 16 + i16, V - 1);
        const uint8_t* wrow = W + (size_t)v * H;
        dst[0] = load_stream16(wrow + min(k_s + g * kGranK, H - 16));
        dst[1] = load_stream16(wrow + min(k_s + kStepK + g * kGranK, H - 16));
    };

    f32x4_t acc[kChains][RT];
    f32x4_t part[RT];
    uint4 st[UPT][2];
    uint4 wcur[2], wnxt[2];
    if (total > 0) {
        stage_load(0, st);
        stage_write(st, xs[0]);
        wload(0, wcur);
    }
    __syncthreads();
#pragma unroll 1
    for (int it = 0; it < total; ++it) {
        const int s = it % NS;
        const bool more = it + 1 < total;
        if (more) {
            stage_load(it + 1, st);
            wload(it + 1, wnxt);
        }
        if (s % kSlabsPerTile == 0) {
#pragma unroll
            for (int X = 0; X < kChains; ++X)
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) acc[X][rt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        }
        // Weights: BF16 pairs of chain g's granules, then the transposes.
        uint32_t a1[8], a2[8];
        e4m3x4_to_bf16(wcur[0].x, a1[0], a1[1]);
        e4m3x4_to_bf16(wcur[0].y, a1[2], a1[3]);
        e4m3x4_to_bf16(wcur[0].z, a1[4], a1[5]);
        e4m3x4_to_bf16(wcur[0].w, a1[6], a1[7]);
        e4m3x4_to_bf16(wcur[1].x, a2[0], a2[1]);
        e4m3x4_to_bf16(wcur[1].y, a2[2], a2[3]);
        e4m3x4_to_bf16(wcur[1].z, a2[4], a2[5]);
        e4m3x4_to_bf16(wcur[1].w, a2[6], a2[7]);
        xpose4(a1[0], a1[1], a1[2], a1[3]);
        xpose4(a1[4], a1[5], a1[6], a1[7]);
        xpose4(a2[0], a2[1], a2[2], a2[3]);
        xpose4(a2[4], a2[5], a2[6], a2[7]);
        const uint4* xb = xs[it & 1];
#pragma unroll
        for (int X = 0; X < kChains; ++X) {
            const uint4 b0 = make_uint4(a1[X], 0, 0, 0);
            const uint4 b1 = make_uint4(0, a1[4 + X], 0, 0);
            const uint4 b2 = make_uint4(0, 0, a2[X], 0);
            const uint4 b3 = make_uint4(0, 0, 0, a2[4 + X]);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const uint4 a = xb[(X * 4 + g) * RP + rt * 16 + i16];
                f32x4_t d = acc[X][rt];
                d = mfma_bf16(a, b0, d);
                d = mfma_bf16(a, b1, d);
                d = mfma_bf16(a, b2, d);
                d = mfma_bf16(a, b3, d);
                acc[X][rt] = d;
            }
        }
        if (more) stage_write(st, xs[(it + 1) & 1]);
        // End of a 4096-k tile (or of the hidden dimension): the tree, then the
        // tile sum in tile order.
        if ((s + 1) % kSlabsPerTile == 0 || s + 1 == NS) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const f32x4_t sum = (acc[0][rt] + acc[1][rt]) + (acc[2][rt] + acc[3][rt]);
                part[rt] = (s < kSlabsPerTile) ? sum : part[rt] + sum;
            }
        }
        if (s + 1 == NS) {
            const int tile = tile_of(it);
            const int v = tile * 16 + i16;
            if (tile < ntiles && v < V) {
                const float sw = wscale[v];
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = rt * 16 + g * 4 + e;
                        if (r < R) {
                            const float y = (part[rt][e] * xscale[r]) * sw;
                            out[(size_t)r * V + v] = f32_to_bf16_rne(y);
                        }
                    }
                }
            }
        }
        __syncthreads();
        wcur[0] = wnxt[0];
        wcur[1] = wnxt[1];
    }
}

template <int RT, int WAVES, int BPC>
hipError_t launch_mfma(const uint8_t* W, const float* ws, const uint8_t* xq, const float* xs,
                       int R, int H, int V, uint16_t* out, const DeviceInfo& dev,
                       hipStream_t stream) {
    const int64_t ntiles = (V + 15) / 16;
    int64_t blocks = (ntiles + WAVES - 1) / WAVES;
    if (blocks > (int64_t)dev.num_cus * BPC) blocks = (int64_t)dev.num_cus * BPC;
    const int nrounds = (int)((ntiles + blocks * WAVES - 1) / (blocks * WAVES));
    hipLaunchKernelGGL((w8a8_mfma_kernel<RT, WAVES, BPC>), dim3((unsigned)blocks),
                       dim3(WAVES * kWave), 0, stream, W, ws, xq, xs, R, H, V, out, nrounds);
    return hipGetLastError();
}

}  // namespace

// One W8A8 launch of 1..128 rows.
hipError_t run_w8a8_gemv(const uint8_t* W, const float* sw, const uint8_t* xq, const float* sa,
                         int R, int H, int V, uint16_t* out, const DeviceInfo& dev,
                         hipStream_t stream) {
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
    switch ((R + 15) / 16) {
        case 1:
            return launch_mfma<1, 8, 1>(W, sw, xq, sa, R, H, V, out, dev, stream);
        case 2:
            return launch_mfma<2, 8, 1>(W, sw, xq, sa, R, H, V, out, dev, stream);
        case 3:
            return launch_mfma<3, 8, 1>(W, sw, xq, sa, R, H, V, out, dev, stream);
        case 4:
            return launch_mfma<4, 8, 1>(W, sw, xq, sa, R, H, V, out, dev, stream);
        case 5:
            return launch_mfma<5, 4, 1>(W, sw, xq, sa, R, H, V, out, dev, stream);
        case 6:
            return launch_mfma<6, 4, 1>(W, sw, xq, sa, R, H, V, out, dev, stream);
        case 7:
            return launch_mfma<7, 4, 1>(W, sw, xq, sa, R, H, V, out, dev, stream);
        default:
            return launch_mfma<8, 4, 1>(W, sw, xq, sa, R, H, V, out, dev, stream);
    }
}

}  // namespace qh
