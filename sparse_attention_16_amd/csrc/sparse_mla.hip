// sparse_mla.hip — sparse attention over selected latent rows, MLA's MQA mode,
// on gfx950 matrix cores.
//
// For a query row t with selected positions idx[t, :] (page "Техотчёт
// DeepSeek-V3.2 (2025): разреженное внимание DSA и масштабирование RL",
// section "Отбор и основное внимание", equation u_t: attention only over the
// k top-scored latent entries, one entry shared by all query heads):
//   z[h,s]   = scale * <q[t,h,0:576], kv[s,0:576]>
//   out[t,h] = sum_s softmax_s(z[h,:]) kv[s, 0:512],  lse[t,h] = ln sum_s exp z[h,s]
//
// One workgroup serves one query row (or one split of its selected set) for
// all 128 heads, so every gathered 1152-byte latent row feeds 128 heads (the
// MQA property that keeps the gather coalesced).  8 waves, two per SIMD, so
// that the hardware overlaps one wave's stalls with the other wave's
// matrix-core work.  For QK and the softmax a wave owns 16 heads (the query
// operands of the 512 latent dims, 64 VGPRs, stay in registers for the whole
// row; those of the 64 rope dims sit in LDS).  For PV a wave owns 64 of the
// 512 value columns of all 128 heads (128 accumulator registers): the
// probabilities go through LDS, and every V operand read from LDS feeds eight
// head tiles.
//
// Per 32-key block:
//   gather  : the 32 selected rows -> LDS with direct-to-LDS 16-byte loads
//             into one of three buffers, two blocks ahead; dims 0..511 of a
//             row are one 1 KB load, the 64 rope dims of 8 rows share one
//             XOR-swizzled 1 KB slab;
//   S^T     : z^T[key, head] = K Q^T on the 16x16x32 bf16 MFMA; A = K rows
//             from LDS, B = query heads;
//   softmax : exp2 domain against a per-head reference max fixed at the
//             first block with a usable key;
//   P       : each wave writes its heads' probabilities (bf16) to LDS in the
//             B-operand layout of the PV MFMA (the S^T accumulator layout
//             already puts one head per lane), then every wave reads all 128;
//   PV      : O^T[c, head] += V^T P^T for the wave's value columns; A = V^T
//             read with the LDS transpose load.
// Between two barriers a wave runs S^T of block b+1 (with the loads of block
// b+2 spread over its k-steps, so that the 36 KB of loads of all waves do not
// queue up at once), then the PV of block b with block b+1's softmax stages
// placed between its MFMAs (the matrix cores and the VALU run side by side).
// The loop never touches O except through MFMAs (no online rescale).
// Exactness: p = 2^(z - m_ref) is bounded by 2^64 as long as no later logit
// exceeds the reference by more than 64 (log2 units).  Each lane tracks its
// largest rise above the reference; if any exceeds 64 at the end of the pass,
// the row is recomputed with the row's true maximum as the reference (tracked
// during the first pass), which cannot overflow.
// Split-KV (few query rows): each split writes a normalised partial and its
// lse; mla_merge_kernel combines them.
#include "dsa_device.h"
#include "kernels.h"

namespace dsa {

namespace {

constexpr int H = 128;
constexpr int D = 576;
constexpr int DV = 512;
constexpr int ROWB = D * 2;              // 1152 bytes per latent row
constexpr int BK = MLA_BK;               // 32 keys per block
constexpr int PA = 1056;                 // LDS pitch of the dims 0..511 part (1 KB + 32 B)
constexpr int RB = BK * PA;              // start of the rope slabs (8 rows x 128 B each)
constexpr int BUF_BYTES = RB + BK * 128; // 37888
constexpr int NWAVES = 8;                // 8 head groups of 16 heads
constexpr int NTHREADS = NWAVES * kWave;
constexpr int NHT = 1;                   // 16-head MFMA tiles per wave
constexpr int KSTEPS = D / 32;           // 18 k-steps (16 latent + 2 rope)
constexpr int MT = BK / 16;              // 16-key tiles per block
constexpr int CTILES = DV / 16;          // 32 value tiles
constexpr int CT_W = CTILES / NWAVES;    // 4 value tiles per wave in PV
constexpr int HT_ALL = H / 16;           // 8 head tiles
constexpr int PP = 80;                   // LDS pitch of one head's 32 probabilities (64 B + 16)
constexpr float LN2 = 0.69314718055994530942f;
constexpr float MAX_RISE = 64.f;         // log2 headroom above the reference max
constexpr int MAX_SEL = 2048;            // largest k (slots staged in LDS)

static_assert(BK == 32 && NWAVES * 4 == BK, "each wave loads 4 rows; waves 0..3 load the rope slabs");

typedef DSA_LDS uint8_t lds_u8;
typedef __attribute__((ext_vector_type(8))) short i16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;

// Maximum over the four 16-lane groups (lanes l, l^16, l^32, l^48) with two
// VALU lane swaps: no LDS traffic and no exec-mask change.
__device__ __forceinline__ float group4_max(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// The loads of one block, split for interleaving with the MFMAs.
// gather_slots reads the wave's four row positions (made scalar: each row is
// one 1 KB load from a scalar base, the lane adding 16 * lane) and, for waves
// 0..3, the lane's slab row; gather_issue(i) issues load i (rows 0..3, then
// the slab).  kvb is the sequence's first latent row (wave-uniform).
struct GatherSlots {
    uint64_t base[4];   // row bases (scalar registers)
    uint64_t kvb;
    uint32_t soff;      // slab: this lane's byte offset from kvb
};
__device__ __forceinline__ GatherSlots gather_slots(const DSA_LDS int32_t *sel, int blk, int l, uint64_t kvb) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    GatherSlots g;
    const i32x4 a = *reinterpret_cast<const DSA_LDS i32x4 *>(sel + blk * BK + 4 * wave);
    // (an unusable slot, -1, loads row 0; the validity masks exclude it)
#pragma unroll
    for (int i = 0; i < 4; ++i)
        g.base[i] = kvb + (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane(a[i] < 0 ? 0 : a[i]) * ROWB;
    const int sv = sel[blk * BK + 8 * (wave & 3) + (l >> 3)];
    const uint32_t sr = (uint32_t)(sv < 0 ? 0 : sv);
    g.soff = sr * ROWB + 1024 + 16 * ((l & 7) ^ (l >> 3));
    g.kvb = kvb;
    return g;
}
__device__ __forceinline__ void gather_issue(const GatherSlots &g, int i, int l, lds_u8 *buf) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (i < 4)
        dma16s(g.base[i], 16 * l, buf + (4 * wave + i) * PA);
    else if (wave < 4)
        dma16s(g.kvb, g.soff, buf + RB + wave * 1024);
}

}  // namespace

// S^T accumulators live in VGPRs: the QK MFMAs are written as inline asm with
// VGPR operands, which keeps the compiler from placing them in the accumulator
// registers the O tiles use (it then moves O registers out and back around
// every block).  The compiler does not know these are MFMAs, so
// the wait states an MFMA result needs before a VALU instruction reads it are
// inserted explicitly (qk_drain: 24, more than any 16x16 MFMA requires), and
// the first k-step takes an inline zero accumulator instead of a VALU-written
// one.  Accumulation is in place (dst == srcC), which back-to-back MFMAs of
// the same opcode support without wait states.
__device__ __forceinline__ void qk_first(f32x4 &d, const bf16x8 &a, const bf16x8 &b) {
    asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void qk_next(f32x4 &d, const bf16x8 &a, const bf16x8 &b) {
    asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void qk_drain(f32x4 (&s)[NHT][MT]) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s[0][0]), "+v"(s[0][1]));
}

// Grid: x = query row, y = split.  LDS (156 KB): three gather buffers, the
// index slice, the probabilities of two blocks, the rope query operands,
// per-head sums and restart flags.
// The index array and every output are separate restrict-qualified arguments
// (no store of the kernel can clobber idx).
__global__ __launch_bounds__(NTHREADS) void sparse_mla_kernel(
    MlaParams p, const int32_t *__restrict__ idx, uint16_t *__restrict__ out,
    float *__restrict__ lse, uint16_t *__restrict__ o_part, float *__restrict__ lse_part) {
    __shared__ __attribute__((aligned(1024))) uint8_t buf0[BUF_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t buf1[BUF_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t buf2[BUF_BYTES];
    __shared__ __attribute__((aligned(16))) int32_t sel[MAX_SEL];
    __shared__ __attribute__((aligned(16))) uint8_t plds[2][H * PP];   // by block parity
    __shared__ __attribute__((aligned(16))) uint8_t qrope[NWAVES * 2 * 1024];  // rope operands, per wave
    __shared__ float lsh[H];
    __shared__ int restart_flag[NWAVES];

    // rows in reverse order: in a causal batch the last rows see the most keys,
    // so the longest rows start first and the short ones fill the tail
    const int t = (int)gridDim.x - 1 - (int)blockIdx.x, split = blockIdx.y;
    const int wave = threadIdx.x >> 6, l = lane_id();
    const int row16 = l & 15, grp = l >> 4;
    const RowInfo ri = row_info(p.cu_q, p.cu_kv, p.pos0, p.B, p.total_kv, p.max_kv, t);

    // this split's slice of the selected set
    const int j0 = split * p.blocks_per_split * BK;
    int j1 = j0 + p.blocks_per_split * BK;
    j1 = j1 < p.k ? j1 : p.k;
    int nsel = (j1 > j0 && ri.ctx > 0) ? j1 - j0 : 0;
    if (p.dense) {   // the row's visible keys 0 .. nvis-1, in order
        const int je = ri.nvis < j1 ? ri.nvis : j1;
        nsel = je > j0 ? je - j0 : 0;
    }
    const int32_t *__restrict__ idx_row = idx + (int64_t)t * p.k + j0;
    int nblk = (nsel + BK - 1) / BK;

    // the slice's slot positions, padded to whole blocks; -1 marks an
    // unusable slot (outside the slice or outside [0, ctx)).  All of a
    // thread's index loads are issued before its first store.
    {
        static_assert(MAX_SEL % NTHREADS == 0, "slot fill");
        int v[MAX_SEL / NTHREADS];
#pragma unroll
        for (int u = 0; u < MAX_SEL / NTHREADS; ++u) {
            const int j = (int)threadIdx.x + u * NTHREADS;
            v[u] = j < nsel ? (p.dense ? j0 + j : idx_row[j]) : -1;
        }
#pragma unroll
        for (int u = 0; u < MAX_SEL / NTHREADS; ++u) {
            const int j = (int)threadIdx.x + u * NTHREADS;
            if (j < nblk * BK) sel[j] = (v[u] >= 0 && v[u] < ri.ctx) ? v[u] : -1;
        }
    }

    // query operands: lane holds head h0 + 16*ht + row16, dims 32*ks + 8*grp .. +7.
    // Issued now and waited for only once the first blocks' gathers are out,
    // so that the two latencies overlap.  (The two rope k-steps go to LDS,
    // each wave reading back its own.)
    const int h0 = wave * 16;
    bf16x8 qb[NHT][16], qr_in[NHT][2];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
        const uint16_t *qrow = p.q + ((int64_t)t * H + h0 + 16 * ht + row16) * D + 8 * grp;
#pragma unroll
        for (int ks = 0; ks < 16; ++ks)
            qb[ht][ks] = *reinterpret_cast<const bf16x8 *>(qrow + 32 * ks);
#pragma unroll
        for (int ks = 16; ks < KSTEPS; ++ks) qr_in[ht][ks - 16] = *reinterpret_cast<const bf16x8 *>(qrow + 32 * ks);
    }
    const DSA_LDS uint8_t *lqr = (const DSA_LDS uint8_t *)qrope + wave * 2048 + 16 * l;
    lds_barrier();   // the slot positions are visible (the query loads keep flying)

    // validity masks: lane b holds bit i = slot b*BK + i is a usable row; read
    // per block with readlane
    uint32_t maskv = 0;
    for (int it = 0; it * kWave < nsel; ++it) {
        const int j = it * kWave + l;
        const bool ok = j < nsel && sel[j] >= 0;
        const uint64_t m = __ballot(ok);
        maskv = l == 2 * it ? (uint32_t)m : (l == 2 * it + 1 ? (uint32_t)(m >> 32) : maskv);
    }
    // blocks after the last usable slot add nothing: stop there (a row of
    // n < k selected keys followed by -1 padding runs ceil(n / BK) blocks)
    {
        const uint64_t live = __ballot(maskv != 0u);
        const int nlive = live ? 64 - (int)__builtin_clzll(live) : 0;
        nblk = nblk < nlive ? nblk : nlive;
    }

    // per-lane LDS read offsets (buffer-relative)
    const int rr16 = row16 & 7;
    const int kA = row16 * PA + 16 * grp;                              // K rows, dims < 512
    const int kB = RB + (row16 >> 3) * 1024 + rr16 * 128;              // rope slab row
    const int kB16 = kB + 16 * (grp ^ rr16);                           // dims 512 + 8*grp
    const int kB17 = kB + 16 * ((4 + grp) ^ rr16);                     // dims 544 + 8*grp
    const int vA = (4 * grp + (row16 >> 2)) * PA + 8 * (row16 & 3);    // V^T transpose reads

    const DSA_LDS int32_t *lsel = (const DSA_LDS int32_t *)sel;
    // per-lane source bases of the gather: dims 0..511 (16 bytes per lane)
    // and the lane's rope chunk of its slab row
    uint64_t kvb = (uint64_t)(uintptr_t)p.kv + (uint64_t)ri.kv0 * ROWB;
    // (readfirstlane returns int: widen through uint32_t, or the low word is sign-extended)
    kvb = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(kvb >> 32)) << 32) |
          (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)kvb);
    lds_u8 *lb0 = (lds_u8 *)buf0;
    lds_u8 *lb1 = (lds_u8 *)buf1;
    lds_u8 *lb2 = (lds_u8 *)buf2;

    // pass 0's first two blocks go out now; then the query operands are
    // waited for (with them), and the rope operands stored
    auto issue_first_blocks = [&]() {
        const GatherSlots g0 = gather_slots(lsel, 0, l, kvb);
#pragma unroll
        for (int i = 0; i < 5; ++i) gather_issue(g0, i, l, lb0);
        if (nblk > 1) {
            const GatherSlots g1 = gather_slots(lsel, 1, l, kvb);
#pragma unroll
            for (int i = 0; i < 5; ++i) gather_issue(g1, i, l, lb1);
        }
    };
    if (nblk > 0) issue_first_blocks();
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): query operands (and the first blocks) landed
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
        for (int r = 0; r < 2; ++r)
            *reinterpret_cast<bf16x8 *>(qrope + (wave * 2 + r) * 1024 + 16 * l) = qr_in[ht][r];

    f32x4 o[HT_ALL][CT_W];   // O^T tiles: all heads x this wave's value columns
    float m_run[NHT], l_run[NHT], m_seen[NHT], rise[NHT];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) m_seen[ht] = -INFINITY;

    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) {
            m_run[ht] = pass == 0 ? -INFINITY : m_seen[ht];
            l_run[ht] = 0.f;
            rise[ht] = -INFINITY;
        }
#pragma unroll
        for (int ht = 0; ht < HT_ALL; ++ht)
#pragma unroll
            for (int c = 0; c < CT_W; ++c) o[ht][c] = f32x4{0.f, 0.f, 0.f, 0.f};

        // ---- S^T of block blk from buffer cur (lane = head row16, keys 4*grp+i)
        // (gl: the loads of another block, issued one per DMA_EVERY k-steps
        // so that they do not queue up behind each other)
        constexpr int DMA_EVERY = 3;
        auto qk_block = [&](int blk, const lds_u8 *cur, f32x4 (&sacc)[NHT][MT],
                            const GatherSlots &gl, bool gon, lds_u8 *gbuf, int glz) {
            const int z = blk >> 30;
            // K operands are loaded QK_AHEAD k-steps ahead of their MFMAs
            constexpr int QK_AHEAD = 2;
            const int kAz = kA + z, kB16z = kB16 + z, kB17z = kB17 + z;
            auto k_off = [&](int ks, int mt) {
                return ks < 16 ? kAz + 64 * ks + mt * 16 * PA
                               : (ks == 16 ? kB16z : kB17z) + mt * 2048;
            };
            bf16x8 kbuf[QK_AHEAD + 1][MT];
            bf16x8 qr[2];
#pragma unroll
            for (int ks = 0; ks < QK_AHEAD; ++ks)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    kbuf[ks][mt] = *reinterpret_cast<const DSA_LDS bf16x8 *>(cur + k_off(ks, mt));
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
                if (ks % DMA_EVERY == 0 && ks / DMA_EVERY < 5 && gon) gather_issue(gl, ks / DMA_EVERY, glz, gbuf);
                if (ks + QK_AHEAD < KSTEPS) {
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        kbuf[(ks + QK_AHEAD) % (QK_AHEAD + 1)][mt] = *reinterpret_cast<const DSA_LDS bf16x8 *>(
                            cur + k_off(ks + QK_AHEAD, mt));
                    if (ks + QK_AHEAD >= 16)
                        qr[ks + QK_AHEAD - 16] = *reinterpret_cast<const DSA_LDS bf16x8 *>(
                            lqr + 1024 * (ks + QK_AHEAD - 16) + z);
                }
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int ht = 0; ht < NHT; ++ht)
                        if (ks == 0)
                            qk_first(sacc[ht][mt], kbuf[0][mt], qb[ht][0]);
                        else
                            qk_next(sacc[ht][mt], kbuf[ks % (QK_AHEAD + 1)][mt], ks < 16 ? qb[ht][ks] : qr[ks - 16]);
                __builtin_amdgcn_sched_barrier(0);
            }
            qk_drain(sacc);
        };

        // ---- unusable slots of a block: logit -inf.  Only the last block of a
        // row and rows with fewer usable slots than k take this branch.
        auto mask_block = [&](uint32_t vmask, f32x4 (&sacc)[NHT][MT]) {
            if (__builtin_expect(vmask != 0xFFFFFFFFu, 0)) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const uint32_t nib = (vmask >> (16 * mt + 4 * grp)) & 0xFu;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int ht = 0; ht < NHT; ++ht)
                            if (!((nib >> i) & 1u)) sacc[ht][mt][i] = -INFINITY;
                }
            }
        };

        // ---- softmax of one block in stages (so that each stage can sit
        // between the MFMAs of another block's PV).  The head's reference is
        // the maximum of its first usable block (all 4 lane groups); until
        // then m_run is -inf and O, l are zero.  The running maximum and the
        // rise above the reference are tracked per lane, checked once per pass.
        float bz[NHT], neg_m[NHT], pv[NHT][8];
        bf16x8 pb[NHT];
        auto soft_stage = [&](int st, const f32x4 (&sacc)[NHT][MT], lds_u8 *pl) {
#pragma unroll
            for (int ht = 0; ht < NHT; ++ht) {
                if (st == 0) {
                    const float bmax = fmaxf(fmaxf(fmaxf(sacc[ht][0][0], sacc[ht][0][1]),
                                                   fmaxf(sacc[ht][0][2], sacc[ht][0][3])),
                                             fmaxf(fmaxf(sacc[ht][1][0], sacc[ht][1][1]),
                                                   fmaxf(sacc[ht][1][2], sacc[ht][1][3])));
                    bz[ht] = bmax * p.scale_log2;
                    m_seen[ht] = fmaxf(m_seen[ht], bz[ht]);
                    asm volatile("" : "+v"(bz[ht]));
                } else if (st == 1) {
                    const float ball = group4_max(bz[ht]);
                    m_run[ht] = m_run[ht] == -INFINITY ? ball : m_run[ht];
                    neg_m[ht] = m_run[ht] == -INFINITY ? 0.f : -m_run[ht];
                    rise[ht] = fmaxf(rise[ht], bz[ht] + neg_m[ht]);
                    asm volatile("" : "+v"(neg_m[ht]));
                } else if (st == 2 || st == 3) {
#pragma unroll
                    for (int e = 4 * (st - 2); e < 4 * (st - 1); ++e) {
                        pv[ht][e] = __builtin_amdgcn_exp2f(fmaf(sacc[ht][e >> 2][e & 3], p.scale_log2, neg_m[ht]));
                        asm volatile("" : "+v"(pv[ht][e]));
                    }
                } else if (st == 4) {
                    l_run[ht] += ((pv[ht][0] + pv[ht][1]) + (pv[ht][2] + pv[ht][3])) +
                                 ((pv[ht][4] + pv[ht][5]) + (pv[ht][6] + pv[ht][7]));
                    pb[ht] = bf16x8{(__bf16)pv[ht][0], (__bf16)pv[ht][1], (__bf16)pv[ht][2], (__bf16)pv[ht][3],
                                    (__bf16)pv[ht][4], (__bf16)pv[ht][5], (__bf16)pv[ht][6], (__bf16)pv[ht][7]};
                } else if (st == 5) {
                    // P to LDS: head h0 + 16*ht + row16, probabilities of the
                    // permuted key order 8*grp .. 8*grp+7 (keys 4*grp+i and 16+4*grp+i)
                    *reinterpret_cast<DSA_LDS bf16x8 *>(pl + (h0 + 16 * ht + row16) * PP + 16 * grp) = pb[ht];
                }
            }
        };

        // Pipeline.  Blocks 0 and 1 are loaded and block 0's probabilities
        // computed before the loop.  Step blk (between two barriers): load
        // block blk+2; S^T of block blk+1; PV of block blk with block blk+1's
        // softmax stages between its MFMAs.  The barrier at the end of the
        // step publishes block blk+1's probabilities and block blk+2's rows,
        // and frees block blk's buffer (which receives block blk+3) and its
        // probabilities (plds by block parity).  The last step runs the
        // softmax stages on an empty block (every slot masked: no effect).
        if (nblk > 0) {
            if (pass > 0) {   // (pass 0's first blocks were issued with the query loads)
                issue_first_blocks();
                if (nblk > 1) {
                    if (wave < 4)
                        __builtin_amdgcn_s_waitcnt(0x0F75);  // vmcnt(5)
                    else
                        __builtin_amdgcn_s_waitcnt(0x0F74);  // vmcnt(4)
                } else {
                    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
                }
            }
            lds_barrier();   // block 0 landed and visible to every wave
            f32x4 sacc[NHT][MT];
            {
                const GatherSlots gnone = gather_slots(lsel, 0, l, kvb);
                qk_block(0, lb0, sacc, gnone, false, lb2, l);
            }
            mask_block(__builtin_amdgcn_readlane(maskv, 0), sacc);
#pragma unroll
            for (int st = 0; st < 6; ++st) soft_stage(st, sacc, (lds_u8 *)plds[0]);
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads of block 1
            lds_barrier();
        }
        auto step = [&](int blk, lds_u8 *cur, lds_u8 *nx1, lds_u8 *nx2) {
            const int z = blk >> 30;
            const int lz = lane_id() + z;
            const bool ld2 = blk + 2 < nblk;
            const bool more = blk + 1 < nblk;
            f32x4 sacc[NHT][MT];
            // block blk+2's loads spread over block blk+1's S^T
            const GatherSlots g = gather_slots(lsel, ld2 ? blk + 2 : blk, lz, kvb);
            if (more) {
                qk_block(blk + 1, nx1, sacc, g, ld2, nx2, lz);
            } else {
#pragma unroll
                for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) sacc[ht][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
            mask_block(more ? __builtin_amdgcn_readlane(maskv, blk + 1) : 0u, sacc);
            lds_u8 *pl_next = (lds_u8 *)plds[(blk + 1) & 1];

            // ---- O^T += V^T P^T over this wave's value columns.  A = V^T via
            // transpose reads (all CT_W tiles, read once): 16-lane group grp
            // reads rows (keys) 4*grp + r and 16 + 4*grp + r; lane row16 of the
            // group addresses row row16/4, columns 16*ct + 4*(row16%4) .. +3.
            // B = P^T of head tile T, read from LDS one tile ahead; each B
            // operand feeds CT_W MFMAs.  Softmax stage T of block blk+1 runs
            // after head tile T's MFMAs.
            const lds_u8 *pl = (const lds_u8 *)plds[blk & 1];
            const int vAz = vA + z + 32 * CT_W * wave;
            bf16x8 va[CT_W];
#pragma unroll
            for (int ct = 0; ct < CT_W; ++ct) {
                const i16x4 lo = lds_read_tr16(cur + vAz + 32 * ct);
                const i16x4 hi = lds_read_tr16(cur + vAz + 16 * PA + 32 * ct);
                const i16x8 a8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                va[ct] = __builtin_bit_cast(bf16x8, a8);
            }
            auto p_op = [&](int T) {
                return *reinterpret_cast<const DSA_LDS bf16x8 *>(pl + (16 * T + row16) * PP + 16 * grp);
            };
            bf16x8 pt[2];
            pt[0] = p_op(0);
#pragma unroll
            for (int T = 0; T < HT_ALL; ++T) {
                if (T + 1 < HT_ALL) pt[(T + 1) & 1] = p_op(T + 1);
#pragma unroll
                for (int ct = 0; ct < CT_W; ++ct) o[T][ct] = mfma_bf16_16x16x32(va[ct], pt[T & 1], o[T][ct]);
                if (T < 6) soft_stage(T, sacc, pl_next);
                __builtin_amdgcn_sched_barrier(0);
            }
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads of block blk+2
            lds_barrier();
        };
        for (int blk = 0; blk < nblk; blk += 3) {
            step(blk, lb0, lb1, lb2);
            if (blk + 1 < nblk) step(blk + 1, lb1, lb2, lb0);
            if (blk + 2 < nblk) step(blk + 2, lb2, lb0, lb1);
        }

        // ---- the head's maximum over its 4 lane groups (the reference of a
        // second pass)
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) {
            m_seen[ht] = fmaxf(m_seen[ht], xor16_f(m_seen[ht]));
            m_seen[ht] = fmaxf(m_seen[ht], shfl_xor_f(m_seen[ht], 32));
        }
        // ---- did any head of any wave outgrow its reference max?
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): nothing of this pass left in flight
        bool restart = false;
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) restart |= rise[ht] > MAX_RISE;
        if (l == 0) restart_flag[wave] = __ballot(restart) != 0;
        __syncthreads();
        bool again = false;
#pragma unroll
        for (int w = 0; w < NWAVES; ++w) again |= restart_flag[w] != 0;
        __syncthreads();
        if (!again) break;
    }

    // ---- finish: the owner of each head reduces its sum and writes its lse;
    // every wave then normalises its value columns of all heads
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
        float l_tot = l_run[ht] + xor16_f(l_run[ht]);
        l_tot += shfl_xor_f(l_tot, 32);
        const int h = h0 + 16 * ht + row16;
        const bool empty = !(l_tot > 0.f);
        const float lse_v = empty ? -INFINITY : (m_run[ht] + log2f(l_tot)) * LN2;
        if (grp == 0) {
            lsh[h] = l_tot;
            if (p.splits == 1)
                lse[(int64_t)t * H + h] = lse_v;
            else
                lse_part[((int64_t)t * p.splits + split) * H + h] = lse_v;
        }
    }
    __syncthreads();
    // 16-byte stores: lanes grp and grp ^ 1 (l and l ^ 16, the same head)
    // exchange one 8-byte half, so that for each pair of value tiles
    // (2u, 2u+1) an even-grp lane holds 8 consecutive columns of tile 2u and
    // an odd-grp lane 8 of tile 2u+1; half the store instructions of one
    // 8-byte store per tile and lane
    static_assert(CT_W % 2 == 0, "value tiles in pairs");
    typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
    typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
    const bool odd = (grp & 1) != 0;
    uint16_t *obase = p.splits == 1 ? out + (int64_t)t * H * DV
                                    : o_part + ((int64_t)t * p.splits + split) * H * DV;
    const int cw = CT_W * 16 * wave + 16 * (grp & 1) + 4 * (grp & 2);
#pragma unroll
    for (int T = 0; T < HT_ALL; ++T) {
        const int h = 16 * T + row16;
        const float l_tot = lsh[h];
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        uint16_t *orow = obase + (int64_t)h * DV + cw;
#pragma unroll
        for (int u = 0; u < CT_W / 2; ++u) {
            const bf16x4 a = {(__bf16)(o[T][2 * u][0] * inv), (__bf16)(o[T][2 * u][1] * inv),
                              (__bf16)(o[T][2 * u][2] * inv), (__bf16)(o[T][2 * u][3] * inv)};
            const bf16x4 b = {(__bf16)(o[T][2 * u + 1][0] * inv), (__bf16)(o[T][2 * u + 1][1] * inv),
                              (__bf16)(o[T][2 * u + 1][2] * inv), (__bf16)(o[T][2 * u + 1][3] * inv)};
            const u32x2 ab = __builtin_bit_cast(u32x2, a), bb = __builtin_bit_cast(u32x2, b);
            // the half the partner needs: tile 2u+1 from an even lane, tile 2u from an odd one
            const u32x2 give = odd ? ab : bb;
            const u32x2 got = {(uint32_t)__builtin_amdgcn_ds_swizzle((int)give[0], 0x401F),
                               (uint32_t)__builtin_amdgcn_ds_swizzle((int)give[1], 0x401F)};
            const u32x4 v = odd ? u32x4{got[0], got[1], bb[0], bb[1]} : u32x4{ab[0], ab[1], got[0], got[1]};
            *reinterpret_cast<u32x4 *>(orow + 32 * u) = v;
        }
    }
}

// Combines split partials: lse = ln sum_s exp(lse_s), out = sum_s exp(lse_s - lse) o_s.
// The partials o_s are normalised and stored in bf16 (half the bytes of the
// round trip through memory; their rounding, 2^-9 relative, is of the order
// of the final bf16 rounding of out); the combination runs in fp32.  A split
// without usable keys (lse_s = -inf) wrote o_s = 0 and gets weight 0.
// Grid: x = query row, y = group of 4 heads; 64 threads x 8 value columns per
// head, the partials of four splits loaded together.
__global__ __launch_bounds__(256) void mla_merge_kernel(MlaParams p) {
    const int t = blockIdx.x;
    const int h = 4 * blockIdx.y + (threadIdx.x >> 6);
    const int c = 8 * (threadIdx.x & 63);
    const int S = p.splits;
    const float *lp = p.lse_part + (int64_t)t * S * H + h;
    const uint16_t *op = p.o_part + ((int64_t)t * S * H + h) * DV + c;
    // the first four splits' partials and lse values are loaded together,
    // before anything depends on them (one memory round trip instead of two)
    bf16x8 v4[4];
    float l4[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        v4[u] = u < S ? *reinterpret_cast<const bf16x8 *>(op + (int64_t)u * H * DV) : bf16x8{};
        l4[u] = u < S ? lp[(int64_t)u * H] : -INFINITY;
    }
    float mx = fmaxf(fmaxf(l4[0], l4[1]), fmaxf(l4[2], l4[3]));
    for (int s = 4; s < S; ++s) mx = fmaxf(mx, lp[(int64_t)s * H]);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float L = -INFINITY;
    if (mx != -INFINITY) {
        float den = 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) den += expf(l4[u] - mx);   // (exp(-inf) = 0 past S)
        for (int s = 4; s < S; ++s) den += expf(lp[(int64_t)s * H] - mx);
        L = mx + logf(den);
        auto weight = [&](float ls) { return ls == -INFINITY ? 0.f : expf(ls - L); };
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (u < S) {
                const float wgt = weight(l4[u]);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] += (float)v4[u][e] * wgt;
            }
        }
        int s = 4;
        for (; s + 4 <= S; s += 4) {
            bf16x8 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const bf16x8 *>(op + (int64_t)(s + u) * H * DV);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float wgt = weight(lp[(int64_t)(s + u) * H]);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] += (float)v[u][e] * wgt;
            }
        }
        for (; s < S; ++s) {
            const bf16x8 v = *reinterpret_cast<const bf16x8 *>(op + (int64_t)s * H * DV);
            const float wgt = weight(lp[(int64_t)s * H]);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += (float)v[e] * wgt;
        }
    }
    const bf16x8 v = {(__bf16)acc[0], (__bf16)acc[1], (__bf16)acc[2], (__bf16)acc[3],
                      (__bf16)acc[4], (__bf16)acc[5], (__bf16)acc[6], (__bf16)acc[7]};
    *reinterpret_cast<bf16x8 *>(p.out + ((int64_t)t * H + h) * DV + c) = v;
    if ((threadIdx.x & 63) == 0) p.lse[(int64_t)t * H + h] = L;
}

hipError_t launch_sparse_mla(const MlaParams &p, int T, hipStream_t s, LaunchMarks *m) {
    if (T <= 0) return hipSuccess;
    hipLaunchKernelGGL(sparse_mla_kernel, dim3(T, p.splits), dim3(NTHREADS), 0, s, p, p.idx, p.out,
                       p.lse, p.o_part, p.lse_part);
    hipError_t e = hipGetLastError();
    if (m) m->after("sparse_mla_kernel", s);
    if (e != hipSuccess || p.splits == 1) return e;
    hipLaunchKernelGGL(mla_merge_kernel, dim3(T, H / 4), dim3(256), 0, s, p);
    e = hipGetLastError();
    if (m) m->after("mla_merge_kernel", s);
    return e;
}

}  // namespace dsa
