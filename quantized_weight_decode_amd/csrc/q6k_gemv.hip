// q6k_gemv.hip -- Q6_K x q8_1 head GEMV for 1..8 activation rows on gfx950.
//
// The head is held as raw 210-byte Q6_K super-blocks of 256 weights
// ("lm_head_q6k.rs": LmHeadQ6k blocks [vocab][hidden/256], MAX_M = 8 rows
// per kquant_mmvq launch) and the activations as block_q8_1 of 32 values
// written by quant_q8_1. A weight is d * sc[t] * (q - 32) with q six bits
// (low four in ql, high two in qh), sc an int8 per 16 weights and d fp16;
// the byte placement follows the public GGUF description (ql[128] | qh[64] |
// scales[16] | d):
//   weight i = 128 n + 32 c + l:  ql[64 n + 32 (c & 1) + l], low nibble for
//   c < 2, high for c >= 2; qh[32 n + l] bits 2c..2c+1.
//
// out[r][v] = bf16( sum over sub-blocks t of fl32(sc_t * isum_t) * fl32(d * d8_j) )
// with isum_t = sum_{i in t} (q_i - 32) * q8_i an exact int32 (v_dot4_i32_i8)
// and j the q8_1 block holding sub-block t; FP32 accumulation otherwise.
//
// Mapping (MI355X-first): 16 lanes per super-block, lane t of the 16 owns
// sub-block t = the 16 consecutive weights 16t .. 16t+15, whose low bits are
// 16 consecutive ql bytes and whose high bits are 16 consecutive qh bytes. A
// wave covers four super-blocks (1024 weights, 840 bytes) of each of its T
// vocab rows per item. Those 840 bytes are the aligned 16-byte chunks that
// hold them (a chunk holding at least one byte of the item never crosses a
// page), loaded straight into one of a ring of DEPTH wave-private LDS
// buffers (two in every launch shape) by one fully coalesced
// global_load_lds_dwordx4 per row (lane l's chunk to slot l); each lane then
// reads its fields from LDS as aligned dwords and cuts four 6-bit codes at a
// time out of them with v_alignbit funnel shifts (super-blocks are only
// 2-byte aligned; the shift folds the misalignment and the field's bit
// position). While item it is computed from one buffer, items it + 1 ..
// it + DEPTH - 1 are in flight into the others; the wait before each item is
// placed by hand (lds_dma16), so that the later items' loads stay in flight
// across the computation. With no register ring, the weights cost no
// registers between issue and use. The -32 offset is folded into the
// integer dot: the staging step stores -32 * sum(q8) per sub-block next to
// the q8 values.
#include "lds_dma.h"
#include "qhead_device.h"
#include "qhead_internal.h"

namespace qh {

constexpr int kQTileK = 8192;                // k per LDS tile (32 super-blocks)
constexpr int kQSbPerTile = kQTileK / 256;

// LDS per workgroup, sized by the row count so that small R leaves room for
// several workgroups per CU.
// The q8 values of a super-block (256 k) take 256 bytes, unpadded: each
// 16-lane group of a 16-byte read takes one super-block's 256 contiguous
// bytes, and padding super-blocks by 16..64 bytes measured 7 times the bank
// conflict cycles of no padding (raw SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE
// 0.139 against 0.019 at 4 and 8 rows). Its 16 sub-block offsets take 16
// words, in slot sb ^ ((sb >> 1) & 1) for super-block sb: a 4-byte LDS read
// serves 32 lanes at a time over 32 banks, and the two half waves in it read
// super-blocks 4s + i and 4s + i + 2 (i = 0, 1), whose offsets then sit in
// the two different 16-bank halves.
constexpr int kQPadSb = 256;
constexpr int kOffPadSb = 16;
__device__ __forceinline__ int q_pos(int k) { return (k >> 8) * kQPadSb + (k & 255); }
__device__ __forceinline__ int off_pos(int k) {
    const int sb = k >> 8;
    return (sb ^ ((sb >> 1) & 1)) * kOffPadSb + ((k & 255) >> 4);
}

template <int R>
struct alignas(16) Q6Lds {
    int8_t q[R][kQSbPerTile * kQPadSb];     // q8 values [row][k]
    float d8[R][kQTileK / 32];              // fp16 d of each q8 block, as f32
    int32_t off[R][kQSbPerTile * kOffPadSb];  // -32 * sum of q8 per 16-value sub-block, padded
};

template <int R, int NTHREADS>
__device__ __forceinline__ void q6_stage_tile(Q6Lds<R>& L, const uint8_t* q8, int H, int k0,
                                              int klen) {
    const int nb = H / 32;
    const int jb0 = k0 / 32;
    const int nbt = klen / 32;  // q8 blocks in this tile
    for (int idx = threadIdx.x; idx < R * nbt; idx += NTHREADS) {
        const int r = idx / nbt;
        const int j = idx - r * nbt;
        const uint32_t* src =
            reinterpret_cast<const uint32_t*>(q8 + ((size_t)r * nb + jb0 + j) * kQ8BlockBytes);
        const uint32_t head = src[0];
        const _Float16 d16 = __builtin_bit_cast(_Float16, (uint16_t)(head & 0xFFFFu));
        L.d8[r][j] = (float)d16;
        // the block's 32 values as two 16-byte LDS writes (a 4-byte write
        // per value word would put 8 lanes on each bank)
        uint32_t w[8];
        int s0 = 0, s1 = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            w[i] = src[1 + i];
            const int sum4 = __builtin_amdgcn_sdot4((int)w[i], 0x01010101, 0, false);
            if (i < 4) s0 += sum4;
            else s1 += sum4;
        }
        u32x4_t* dst = reinterpret_cast<u32x4_t*>(&L.q[r][q_pos(j * 32)]);
        dst[0] = u32x4_t{w[0], w[1], w[2], w[3]};
        dst[1] = u32x4_t{w[4], w[5], w[6], w[7]};
        L.off[r][off_pos(j * 32)] = -32 * s0;
        L.off[r][off_pos(j * 32 + 16)] = -32 * s1;
    }
}

template <int R, int T, int WAVES, int MAXB, int BPC, int DEPTH>
__global__ void __launch_bounds__(WAVES * kWave, (WAVES * BPC + 3) / 4)
q6k_gemv_kernel(const uint8_t* __restrict__ blocks, const uint8_t* __restrict__ q8, int H, int V,
                uint16_t* __restrict__ out, int nsuper) {
    constexpr int N = T * R;
    constexpr int NP = next_pow2(N);
    constexpr int M = Log2<NP>::value;
    constexpr int kItemBytes = 4 * kQ6KBlockBytes;  // 840
    static_assert(NP <= 64 && R <= 8, "T*R must be <= 64, R <= 8");
    static_assert(kItemBytes + 15 <= 64 * 16, "an item must fit one 16-byte load per lane");
    static_assert((kItemBytes + 13) / 16 + 2 <= 61, "the shifted chunks stay in the row's buffer");
    static_assert(DEPTH >= 2 && (DEPTH - 1) * T <= 63, "vmcnt counts the loads of the items in flight");
    __shared__ Q6Lds<R> L;
    // wave-private weight staging, a ring of DEPTH buffers: [wave][item %
    // DEPTH][row t][1024 bytes]. Item it + DEPTH - 1 is loaded into one
    // buffer at the start of step it, while item it is read from another.
    __shared__ u32x4_t WB[WAVES][DEPTH][T][kWave];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int TW = gridDim.x * WAVES;
    const int gw = blockIdx.x * WAVES + wave;
    const int NB = (V + T - 1) / T;
    const int NT = (H + kQTileK - 1) / kQTileK;
    const int nsb = H / 256;
    const size_t rowbytes = (size_t)nsb * kQ6KBlockBytes;

    // lane -> (super-block within the item, sub-block t = 8n + 2c + h). A
    // 4-byte LDS read serves 32 lanes at a time over 32 banks; its two half
    // waves take super-blocks {0, 2} or {1, 3}. Super-blocks 2 and 3 are
    // staged 32 bytes later than their place in the item (see `stage`):
    // 137 dwords from super-block 0, 105 + 8 from 1, which puts the ql and
    // qh windows of the two half waves in disjoint banks at every item
    // misalignment (105 dwords alone leaves two qh banks shared).
    const int sbi = (((lane >> 4) & 1) << 1) | (lane >> 5);
    const int t16 = lane & 15;
    const int n = t16 >> 3, c = (t16 >> 1) & 3, h = t16 & 1;
    const int ql_off = 64 * n + 32 * (c & 1) + 16 * h;
    const int qh_off = 128 + 32 * n + 16 * h;
    const int lo_shift = (c >= 2) ? 4 : 0;
    const int hi_shift = 2 * c;
    // Byte offsets within a staged item of this lane's fields (before the
    // item's misalignment), and the bit added to 8 x the byte address of the
    // 32-bit window each field is funnel-shifted from: the low nibbles of ql
    // land in bits 0-3 of each byte, the 2-bit qh fields in bits 4-5. When
    // the qh field sits below bit 4 the window starts one byte earlier.
    // The offsets count from the block's first staging buffer and include
    // this wave's buffers (a multiple of 4 bytes).
    const int qh_back = hi_shift < 4 ? 1 : 0;
    const int p_sb = wave * (DEPTH * T * kWave * 16) + sbi * kQ6KBlockBytes + (sbi >= 2 ? 32 : 0);
    const int p_ql = p_sb + ql_off;
    const int p_qh = p_sb + qh_off - qh_back;
    const int b_qh = 8 * qh_back + hi_shift - 4;
    const int p_sc = p_sb + 192 + t16;
    const int p_d = p_sb + 208;
    const uint8_t* const wb = reinterpret_cast<const uint8_t*>(&WB[0][0][0]);
    const uint32_t wb_lds = __builtin_amdgcn_readfirstlane(lds_byte_offset(&WB[wave][0][0][0]));
    // An item's first byte is 2-byte aligned, and its position mod 4 in the
    // staging buffer depends only on the parity of its vocab row: items start
    // at multiples of 840 bytes within a row, rows are hidden/256 x 210 bytes
    // apart and bands start at even rows. So the 32-bit window of each field
    // and its funnel shift take one of two lane values, for even and odd rows
    // (a row re-read past the vocab tail may take the wrong one: its sums are
    // never stored).
    static_assert(T % 2 == 0, "bands must start at even rows");
    const int c_even = (int)(reinterpret_cast<uintptr_t>(blocks) & 3);
    const int c_odd = (c_even + 2 * (nsb & 1)) & 3;
    const int wl_even = (p_ql + c_even) & ~3, wl_odd = (p_ql + c_odd) & ~3;
    const int wh_even = (p_qh + c_even) & ~3, wh_odd = (p_qh + c_odd) & ~3;
    const uint32_t sl_even = 8 * ((p_ql + c_even) & 3) + lo_shift;
    const uint32_t sl_odd = 8 * ((p_ql + c_odd) & 3) + lo_shift;
    const uint32_t sh_even = 8 * ((p_qh + c_even) & 3) + b_qh;
    const uint32_t sh_odd = 8 * ((p_qh + c_odd) & 3) + b_qh;

    const int my_idx = lane >> (6 - M);
    const int my_r = my_idx / T;
    const int my_t = my_idx - my_r * T;
    const bool writer = ((lane & ((1 << (6 - M)) - 1)) == 0) && (my_idx < N);

    for (int sj = 0; sj < nsuper; ++sj) {
        float part[MAXB];
#pragma unroll
        for (int bi = 0; bi < MAXB; ++bi) part[bi] = 0.0f;

        for (int tt = 0; tt < NT; ++tt) {
            const int k0 = tt * kQTileK;
            const int klen = min(kQTileK, H - k0);
            const int nsb_tile = klen / 256;
            const int nseg = (nsb_tile + 3) / 4;
            if (NT > 1 || sj == 0) {
                __syncthreads();
                q6_stage_tile<R, WAVES * kWave>(L, q8, H, k0, klen);
                __syncthreads();
            }
            const int first = (sj * MAXB) * TW + gw;
            const int nbb = first < NB ? min(MAXB, (NB - 1 - first) / TW + 1) : 0;
            const int nitems = nbb * nseg;

            // First byte of item (bi, s) in row t (rows past the vocab tail
            // re-read the last row, never stored).
            auto item_ptr = [&](int bi, int s, int t) -> const uint8_t* {
                const int v = min(((sj * MAXB + bi) * TW + gw) * T + t, V - 1);
                const int sb0 = tt * kQSbPerTile + s * 4;
                return blocks + (size_t)v * rowbytes + (size_t)sb0 * kQ6KBlockBytes;
            };
            // One 16-byte aligned chunk per lane and row into LDS buffer
            // `buf`, lane l's chunk to slot l. Slot j holds chunk j, from slot
            // 28 on chunk j - 2: super-blocks 2 and 3 (item bytes >= 420 +
            // 0..14) land 32 bytes later, and slots 26 and 27 keep the tail
            // of super-block 1 (bytes < 434). The last chunk an item needs is
            // 53 (slot 55); the lanes past it load the item's last chunk
            // again, into slots no lane reads.
            const int lchunk = lane < 28 ? lane : lane - 2;
            auto issue = [&](int bi, int s, int buf) __attribute__((always_inline)) {
                const int sb0 = tt * kQSbPerTile + s * 4;
                const int nbytes = min(4, nsb - sb0) * kQ6KBlockBytes;
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    const uint8_t* p = item_ptr(bi, s, t);
                    const int mis = (int)(reinterpret_cast<uintptr_t>(p) & 15);
                    const uint32_t ch = (uint32_t)min(lchunk, (mis + nbytes - 1) >> 4);
                    lds_dma16(p - mis, 16u * ch, wb_lds + (uint32_t)((buf * T + t) * kWave * 16));
                }
            };

            float acc[NP];
            int bi = 0, s = 0;
            // (pbi, ps): the next item to load. Step it loads item it + DEPTH
            // - 1 into the buffer that step it - 1 read (all its reads were
            // consumed there), then waits for item it: the T loads of each
            // item after it that is already issued may stay in flight
            // (DEPTH - 1 items, fewer at the end). Nothing else in this loop
            // loads from vector memory, so the count is exact.
            int pbi = 0, ps = 0;
            auto load_next = [&](int buf) __attribute__((always_inline)) {
                issue(pbi, ps, buf);
                if (++ps == nseg) {
                    ps = 0;
                    ++pbi;
                }
            };
            auto step = [&](int it, int buf) __attribute__((always_inline)) {
                if (it + DEPTH - 1 < nitems) {
                    load_next(buf == 0 ? DEPTH - 1 : buf - 1);
                    wait_vmcnt<(DEPTH - 1) * T>();
                } else {
                    // items it + 1 .. nitems - 1 are in flight (wave-uniform)
                    const int left = nitems - 1 - it;
                    static_for<DEPTH - 1>([&](auto i) __attribute__((always_inline)) {
                        if (left == decltype(i)::value) wait_vmcnt<decltype(i)::value * T>();
                    });
                }
                if (s == 0) {
#pragma unroll
                    for (int i = 0; i < NP; ++i) acc[i] = 0.0f;
                }
                const int sbt = s * 4 + sbi;  // super-block within the tile
                const bool valid = sbt < nsb_tile;
                uint32_t qw[T][4];
                float wsc[T];
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    // item start within row t's staging buffer, and that
                    // rounded down to a word (wave-uniform)
                    const int st = (int)(reinterpret_cast<uintptr_t>(item_ptr(bi, s, t)) & 15) +
                                   (buf * T + t) * kWave * 16;
                    const int sw = st & ~3;
                    const uint32_t* wl =
                        reinterpret_cast<const uint32_t*>(wb + sw + ((t & 1) ? wl_odd : wl_even));
                    const uint32_t* wh =
                        reinterpret_cast<const uint32_t*>(wb + sw + ((t & 1) ? wh_odd : wh_even));
                    // alignbit takes its shift modulo 32
                    const uint32_t shl = (t & 1) ? sl_odd : sl_even;
                    const uint32_t shh = (t & 1) ? sh_odd : sh_even;
                    uint32_t qlw[5], qhw[5];
#pragma unroll
                    for (int i = 0; i < 5; ++i) {
                        qlw[i] = wl[i];
                        qhw[i] = wh[i];
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t lo = __builtin_amdgcn_alignbit(qlw[i + 1], qlw[i], shl);
                        const uint32_t hi = __builtin_amdgcn_alignbit(qhw[i + 1], qhw[i], shh);
                        qw[t][i] = (lo & 0x0F0F0F0Fu) | (hi & 0x30303030u);
                    }
                    int sc = reinterpret_cast<const int8_t*>(wb)[st + p_sc];
                    // keep sc a 32-bit value: a sign-extending byte load and
                    // one convert (otherwise the convert is narrowed to 16
                    // bits and costs an extra bit-field extract)
                    asm("" : "+v"(sc));
                    const uint16_t dbits = *reinterpret_cast<const uint16_t*>(wb + st + p_d);
                    // d * sc is exact in FP32 (11-bit times 8-bit significands)
                    const float d = (float)__builtin_bit_cast(_Float16, dbits);
                    wsc[t] = valid ? d * (float)sc : 0.0f;
                }
                const int kk = min(sbt, kQSbPerTile - 1) * 256 + 16 * t16;  // k within the tile
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const uint4 xq = *reinterpret_cast<const uint4*>(&L.q[r][q_pos(kk)]);
                    const int off = L.off[r][off_pos(kk)];
                    const float d8 = valid ? L.d8[r][kk >> 5] : 0.0f;
#pragma unroll
                    for (int t = 0; t < T; ++t) {
                        // The clamp (saturation) never acts: |is| < 2^18. It
                        // selects the three-operand encoding, so the chain
                        // starts from `off` without first copying it.
                        int is = __builtin_amdgcn_sdot4((int)qw[t][0], (int)xq.x, off, true);
                        is = __builtin_amdgcn_sdot4((int)qw[t][1], (int)xq.y, is, false);
                        is = __builtin_amdgcn_sdot4((int)qw[t][2], (int)xq.z, is, false);
                        is = __builtin_amdgcn_sdot4((int)qw[t][3], (int)xq.w, is, false);
                        acc[r * T + t] = __builtin_fmaf((float)is, wsc[t] * d8, acc[r * T + t]);
                    }
                }
                if (s + 1 == nseg) {
                    wave_reduce_scatter<NP>(acc, lane);
#pragma unroll
                    for (int j = 0; j < MAXB; ++j)
                        if (j == bi) part[j] = (tt == 0) ? acc[0] : part[j] + acc[0];
                    ++bi;
                    s = 0;
                } else {
                    ++s;
                }
            };
            for (int j = 0; j < DEPTH - 1 && j < nitems; ++j) load_next(j);
            int buf = 0;
#pragma unroll 1
            for (int it = 0; it < nitems; ++it) {
                step(it, buf);
                buf = buf + 1 == DEPTH ? 0 : buf + 1;
            }
        }

#pragma unroll
        for (int bi = 0; bi < MAXB; ++bi) {
            const int band = (sj * MAXB + bi) * TW + gw;
            const int v = band * T + my_t;
            if (writer && band < NB && v < V) out[(size_t)my_r * V + v] = f32_to_bf16_rne(part[bi]);
        }
    }
}

template <int R, int T, int WAVES, int MAXB, int BPC, int DEPTH>
static hipError_t launch_q6k(const uint8_t* blocks, const uint8_t* q8, int H, int V,
                             uint16_t* out, const DeviceInfo& dev, hipStream_t stream) {
    const int64_t NB = (V + T - 1) / T;
    int64_t nblk = (NB + WAVES - 1) / WAVES;
    if (nblk > (int64_t)dev.num_cus * BPC) nblk = (int64_t)dev.num_cus * BPC;
    const int64_t TW = nblk * WAVES;
    const int64_t per_wave = (NB + TW - 1) / TW;
    const int nsuper = (int)((per_wave + MAXB - 1) / MAXB);
    hipLaunchKernelGGL((q6k_gemv_kernel<R, T, WAVES, MAXB, BPC, DEPTH>), dim3((unsigned)nblk),
                       dim3(WAVES * kWave), 0, stream, blocks, q8, H, V, out, nsuper);
    return hipGetLastError();
}

hipError_t run_q6k(const uint8_t* blocks, const uint8_t* q8, int R, int H, int V, uint16_t* out,
                   const DeviceInfo& dev, hipStream_t stream) {
    switch (R) {
#define QH_Q6_CASE(RR, TT, WV, MB, BPC, DP) \
    case RR:                                \
        return launch_q6k<RR, TT, WV, MB, BPC, DP>(blocks, q8, H, V, out, dev, stream);
        QH_Q6_CASE(1, 4, 8, 12, 2, 2)
        QH_Q6_CASE(2, 2, 12, 8, 2, 2)
        QH_Q6_CASE(3, 4, 12, 12, 1, 2)
        QH_Q6_CASE(4, 4, 12, 12, 1, 2)
        QH_Q6_CASE(5, 4, 12, 12, 1, 2)
        QH_Q6_CASE(6, 4, 8, 12, 1, 2)
        QH_Q6_CASE(7, 4, 8, 12, 1, 2)
        QH_Q6_CASE(8, 4, 8, 12, 1, 2)
#undef QH_Q6_CASE
        default:
            return hipErrorInvalidValue;
    }
}

}  // namespace qh
