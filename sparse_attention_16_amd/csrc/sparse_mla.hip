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
// that the hardware overlaps one wave's softmax, gather issue and barrier
// waits with the other wave's matrix-core work.  For QK and the softmax a wave
// owns 16 heads (its query operands, 72 VGPRs, stay in registers for the whole
// row).  For PV a wave owns 64 of the 512 value columns of all 128 heads (128
// accumulator registers): the probabilities go through LDS, and every V
// operand read from LDS feeds eight head tiles.
//
// Per 32-key block:
//   gather  : the 32 selected rows -> LDS with direct-to-LDS 16-byte loads
//             into one of three buffers, two blocks ahead; dims 0..511 of a
//             row are one 1 KB load, the 64 rope dims of 8 rows share one
//             XOR-swizzled 1 KB slab;
//   S^T     : z^T[key, head] = K Q^T on the 16x16x32 bf16 MFMA; A = K rows
//             from LDS, B = query heads (registers, loaded once);
//   softmax : exp2 domain against a per-head reference max fixed at the
//             first block with a usable key;
//   P       : each wave writes its heads' probabilities (bf16) to LDS in the
//             B-operand layout of the PV MFMA (the S^T accumulator layout
//             already puts one head per lane), then every wave reads all 128;
//   PV      : O^T[c, head] += V^T P^T for the wave's value columns; A = V^T
//             read with the LDS transpose load.
// The loop never touches O except through MFMAs (no online rescale).
// Exactness: p = 2^(z - m_ref) is bounded by 2^64 as long as no later logit
// exceeds the reference by more than 64 (log2 units); a block that does sets
// a restart flag, and the row is recomputed with the row's true maximum as the
// reference (tracked during the first pass), which cannot overflow.
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

// One 16-byte-per-lane direct-to-LDS load: LDS destination lds + 16 * lane.
// Issued from asm, so the compiler's wait insertion does not track it (it
// cannot tell which LDS buffer the load writes and would fence later LDS reads
// of unrelated buffers with a wait for it); the kernel waits for these loads
// explicitly with vmcnt at the top of each step (no other vector-memory load
// is issued inside the block loop).  M0 must be written one instruction ahead
// of the load.
__device__ __forceinline__ void dma16(const void *src, const DSA_LDS void *lds) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(m0)
                 : "m0");
}

// The direct-to-LDS loads of one block for this wave: wave w loads rows
// 4w..4w+3 (dims 0..511: one 1 KB load per row); waves 0..3 also load rope
// slab w (dims 512..575 of rows 8w..8w+7, 8 x 128 B), in which logical
// 16-byte chunk c of row rr sits at chunk position c ^ rr, so that a column of
// 8 rows read together lands on distinct banks.  Row positions come from the
// row's index slice staged in LDS, already clamped to [0, ctx) (unusable slots
// hold row 0 and are masked later): a wave-uniform LDS read is a short wait,
// where a scalar load of fresh index data would wait on L2 every block, and
// each load address is then a single multiply-add on the lane's base pointer.
__device__ __forceinline__ void gather_block(const uint8_t *lane_row, const uint8_t *lane_slab,
                                             const DSA_LDS int32_t *sel, int blk, lds_u8 *buf, int l) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const DSA_LDS int32_t *s4p = sel + blk * BK + 4 * wave;
    const i32x4 a = *reinterpret_cast<const DSA_LDS i32x4 *>(s4p);
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16(lane_row + (uint64_t)(uint32_t)a[i] * ROWB, buf + (4 * wave + i) * PA);
    if (wave < 4) {
        const uint32_t sr = (uint32_t)sel[blk * BK + 8 * wave + (l >> 3)];
        dma16(lane_slab + (uint64_t)sr * ROWB, buf + RB + wave * 1024);
    }
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

// Grid: x = query row, y = split.  LDS: three gather buffers, the index slice,
// the probabilities of one block, per-head sums and restart flags.
// The index array and every output are separate restrict-qualified arguments
// (no store of the kernel can clobber idx).
__global__ __launch_bounds__(NTHREADS) void sparse_mla_kernel(
    MlaParams p, const int32_t *__restrict__ idx, uint16_t *__restrict__ out,
    float *__restrict__ lse, float *__restrict__ o_part, float *__restrict__ lse_part) {
    __shared__ __attribute__((aligned(1024))) uint8_t buf0[BUF_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t buf1[BUF_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t buf2[BUF_BYTES];
    __shared__ __attribute__((aligned(16))) int32_t sel[MAX_SEL];
    __shared__ __attribute__((aligned(16))) uint8_t plds[2][H * PP];   // by block parity
    __shared__ float lsh[H];
    __shared__ int restart_flag[NWAVES];

    const int t = blockIdx.x, split = blockIdx.y;
    const int wave = threadIdx.x >> 6, l = lane_id();
    const int row16 = l & 15, grp = l >> 4;
    const RowInfo ri = row_info(p.cu_q, p.cu_kv, p.pos0, p.B, p.total_kv, p.max_kv, t);

    // this split's slice of the selected set
    const int j0 = split * p.blocks_per_split * BK;
    int j1 = j0 + p.blocks_per_split * BK;
    j1 = j1 < p.k ? j1 : p.k;
    const int nsel = (j1 > j0 && ri.ctx > 0) ? j1 - j0 : 0;
    const int32_t *__restrict__ idx_row = idx + (int64_t)t * p.k + j0;
    const int nblk = (nsel + BK - 1) / BK;

    // query operands: lane holds head h0 + 16*ht + row16, dims 32*ks + 8*grp .. +7
    const int h0 = wave * 16;
    bf16x8 qb[NHT][KSTEPS];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
        const uint16_t *qrow = p.q + ((int64_t)t * H + h0 + 16 * ht + row16) * D + 8 * grp;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks)
            qb[ht][ks] = *reinterpret_cast<const bf16x8 *>(qrow + 32 * ks);
    }
    // the slice's slot positions, clamped to [0, ctx) and padded to whole
    // blocks (unusable slots load row 0; the masks below exclude them)
    for (int j = threadIdx.x; j < nblk * BK; j += NTHREADS) {
        const int v = j < nsel ? idx_row[j] : -1;
        sel[j] = (v >= 0 && v < ri.ctx) ? v : 0;
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): query operands resident before the pipeline
    __syncthreads();

    // validity masks: lane b holds bit i = slot b*BK + i is a usable row
    // (inside the slice, inside [0, ctx)); read per block with readlane
    uint32_t maskv = 0;
    for (int it = 0; it * kWave < nsel; ++it) {
        const int j = it * kWave + l;
        const bool ok = j < nsel && (uint32_t)idx_row[j < nsel ? j : 0] < (uint32_t)ri.ctx;
        const uint64_t m = __ballot(ok);
        maskv = l == 2 * it ? (uint32_t)m : (l == 2 * it + 1 ? (uint32_t)(m >> 32) : maskv);
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
    const uint8_t *kvb = reinterpret_cast<const uint8_t *>(p.kv) + ri.kv0 * ROWB;
    const uint8_t *lane_row = kvb + 16 * l;
    const uint8_t *lane_slab = kvb + 1024 + 16 * ((l & 7) ^ (l >> 3));
    lds_u8 *lb0 = (lds_u8 *)buf0;
    lds_u8 *lb1 = (lds_u8 *)buf1;
    lds_u8 *lb2 = (lds_u8 *)buf2;

    f32x4 o[HT_ALL][CT_W];   // O^T tiles: all heads x this wave's value columns
    float m_run[NHT], l_run[NHT], m_seen[NHT];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) m_seen[ht] = -INFINITY;

    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) {
            m_run[ht] = pass == 0 ? -INFINITY : m_seen[ht];
            l_run[ht] = 0.f;
        }
#pragma unroll
        for (int ht = 0; ht < HT_ALL; ++ht)
#pragma unroll
            for (int c = 0; c < CT_W; ++c) o[ht][c] = f32x4{0.f, 0.f, 0.f, 0.f};
        bool restart = false;

        // Pipeline: blocks 0 and 1 are loaded here; block b+2 is loaded during
        // step b, after the step's barrier.
        if (nblk > 0) gather_block(lane_row, lane_slab, lsel, 0, lb0, l);
        if (nblk > 1) gather_block(lane_row, lane_slab, lsel, 1, lb1, l);
        if (nblk > 0) {   // block 0 landed and visible to every wave
            if (nblk > 1) {
                if (wave < 4)
                    __builtin_amdgcn_s_waitcnt(0x0F75);  // vmcnt(5)
                else
                    __builtin_amdgcn_s_waitcnt(0x0F74);  // vmcnt(4)
            } else {
                __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
            }
            lds_barrier();
        }

        // One block step: cur = buffer of block blk, nxt2 = buffer for blk+2
        // (the one block blk-1 used).  `cur` and `nxt2` are distinct LDS arrays
        // at compile time (the loop is unrolled by three), which lets the
        // compiler see that reads of `cur` do not wait for the loads landing
        // elsewhere.
        // One barrier per block, between the probability write and the PV:
        // before it each wave waits for its own loads of block blk+1 (issued
        // a step earlier), so after it block blk+1 is visible to every wave,
        // every wave's probabilities of block blk are in place and every wave
        // is done with block blk-1's buffer, which then receives block blk+2.
        // The probabilities are double-buffered by block parity: a wave may
        // write block blk+1's while another still reads block blk's.
        auto step = [&](int blk, lds_u8 *cur, lds_u8 *nxt2) {
            // Lane-derived values are rebuilt inside the step from an opaque
            // zero (blk >> 30 == 0 for every real block count): hoisted out of
            // the loop they would cost registers the operands need.
            const int z = blk >> 30;
            const int lz = lane_id() + z;
            const uint32_t vmask = __builtin_amdgcn_readlane(maskv, blk);

            // ---- S^T: MT key tiles x NHT head tiles, lane = (head row16, keys 4*grp+i)
            f32x4 sacc[NHT][MT];
            // K operands are loaded QK_AHEAD k-steps ahead of their MFMAs
            // (software pipeline; one wave per SIMD hides nothing by itself).
            constexpr int QK_AHEAD = 2;
            const int kAz = kA + z, kB16z = kB16 + z, kB17z = kB17 + z;
            auto k_off = [&](int ks, int mt) {
                return ks < 16 ? kAz + 64 * ks + mt * 16 * PA
                               : (ks == 16 ? kB16z : kB17z) + mt * 2048;
            };
            bf16x8 kbuf[QK_AHEAD + 1][MT];
#pragma unroll
            for (int ks = 0; ks < QK_AHEAD; ++ks)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    kbuf[ks][mt] = *reinterpret_cast<const DSA_LDS bf16x8 *>(cur + k_off(ks, mt));
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
                if (ks + QK_AHEAD < KSTEPS) {
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        kbuf[(ks + QK_AHEAD) % (QK_AHEAD + 1)][mt] = *reinterpret_cast<const DSA_LDS bf16x8 *>(
                            cur + k_off(ks + QK_AHEAD, mt));
                }
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int ht = 0; ht < NHT; ++ht)
                        if (ks == 0)
                            qk_first(sacc[ht][mt], kbuf[0][mt], qb[ht][0]);
                        else
                            qk_next(sacc[ht][mt], kbuf[ks % (QK_AHEAD + 1)][mt], qb[ht][ks]);
                __builtin_amdgcn_sched_barrier(0);
            }

            qk_drain(sacc);
            // ---- softmax numerators against the reference max
            if (vmask != 0xFFFFFFFFu) {
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
            bf16x8 pb[NHT];
#pragma unroll
            for (int ht = 0; ht < NHT; ++ht) {
                // this lane's 8 logits of the head; the restart test and the
                // running maximum work per lane (the head's 4 lane groups are
                // combined once per pass), only the first usable block needs
                // the head's block maximum across the groups
                float bmax = fmaxf(fmaxf(fmaxf(sacc[ht][0][0], sacc[ht][0][1]),
                                         fmaxf(sacc[ht][0][2], sacc[ht][0][3])),
                                   fmaxf(fmaxf(sacc[ht][1][0], sacc[ht][1][1]),
                                         fmaxf(sacc[ht][1][2], sacc[ht][1][3])));
                const float bz = bmax * p.scale_log2;
                m_seen[ht] = fmaxf(m_seen[ht], bz);
                if (m_run[ht] == -INFINITY) {    // first usable key: O and l are still zero
                    bmax = fmaxf(bmax, xor16_f(bmax));
                    bmax = fmaxf(bmax, shfl_xor_f(bmax, 32));
                    m_run[ht] = bmax * p.scale_log2;
                } else if (bz > m_run[ht] + MAX_RISE) {
                    restart = true;
                }
                const float neg_m = m_run[ht] == -INFINITY ? 0.f : -m_run[ht];
                float pv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    pv[e] = __builtin_amdgcn_exp2f(fmaf(sacc[ht][e >> 2][e & 3], p.scale_log2, neg_m));
                l_run[ht] += ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
                pb[ht] = bf16x8{(__bf16)pv[0], (__bf16)pv[1], (__bf16)pv[2], (__bf16)pv[3],
                                (__bf16)pv[4], (__bf16)pv[5], (__bf16)pv[6], (__bf16)pv[7]};
            }

            // ---- P to LDS: head h0 + 16*ht + row16, probabilities of the
            // permuted key order 8*grp .. 8*grp+7 (keys 4*grp+i and 16+4*grp+i)
            lds_u8 *pl = (lds_u8 *)plds[blk & 1];
#pragma unroll
            for (int ht = 0; ht < NHT; ++ht)
                *reinterpret_cast<DSA_LDS bf16x8 *>(pl + (h0 + 16 * ht + row16) * PP + 16 * grp) = pb[ht];
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads of block blk+1
            lds_barrier();
            if (blk + 2 < nblk) gather_block(lane_row, lane_slab, lsel, blk + 2, nxt2, lz);
            // ---- O^T += V^T P^T over this wave's value columns.  A = V^T via
            // transpose reads (all CT_W tiles, read once): 16-lane group grp
            // reads rows (keys) 4*grp + r and 16 + 4*grp + r; lane row16 of the
            // group addresses row row16/4, columns 16*ct + 4*(row16%4) .. +3.
            // B = P^T of head tile T, read from LDS one tile ahead; each B
            // operand feeds CT_W MFMAs.
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
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        for (int blk = 0; blk < nblk; blk += 3) {
            step(blk, lb0, lb2);
            if (blk + 1 < nblk) step(blk + 1, lb1, lb0);
            if (blk + 2 < nblk) step(blk + 2, lb2, lb1);
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
    const int c0 = CT_W * 16 * wave + 4 * grp;
#pragma unroll
    for (int T = 0; T < HT_ALL; ++T) {
        const int h = 16 * T + row16;
        const float l_tot = lsh[h];
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        if (p.splits == 1) {
            uint16_t *orow = out + ((int64_t)t * H + h) * DV + c0;
#pragma unroll
            for (int ct = 0; ct < CT_W; ++ct) {
                const bf16x4 v = {(__bf16)(o[T][ct][0] * inv), (__bf16)(o[T][ct][1] * inv),
                                  (__bf16)(o[T][ct][2] * inv), (__bf16)(o[T][ct][3] * inv)};
                *reinterpret_cast<bf16x4 *>(orow + 16 * ct) = v;
            }
        } else {
            float *orow = o_part + (((int64_t)t * p.splits + split) * H + h) * DV + c0;
#pragma unroll
            for (int ct = 0; ct < CT_W; ++ct) *reinterpret_cast<f32x4 *>(orow + 16 * ct) = o[T][ct] * inv;
        }
    }
}

// Combines split partials: lse = ln sum_s exp(lse_s), out = sum_s exp(lse_s - lse) o_s.
// Grid: x = query row, y = pair of heads; 128 threads x 4 value columns per head.
__global__ __launch_bounds__(256) void mla_merge_kernel(MlaParams p) {
    const int t = blockIdx.x;
    const int h = 2 * blockIdx.y + (threadIdx.x >> 7);
    const int c = 4 * (threadIdx.x & 127);
    const int S = p.splits;
    const float *lp = p.lse_part + (int64_t)t * S * H + h;
    float mx = -INFINITY;
    for (int s = 0; s < S; ++s) mx = fmaxf(mx, lp[(int64_t)s * H]);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float L = -INFINITY;
    if (mx != -INFINITY) {
        float den = 0.f;
        for (int s = 0; s < S; ++s) den += expf(lp[(int64_t)s * H] - mx);
        L = mx + logf(den);
        for (int s = 0; s < S; ++s) {
            const float ls = lp[(int64_t)s * H];
            if (ls == -INFINITY) continue;
            const f32x4 v = *reinterpret_cast<const f32x4 *>(
                p.o_part + (((int64_t)t * S + s) * H + h) * DV + c);
            acc += v * expf(ls - L);
        }
    }
    const bf16x4 v = {(__bf16)acc[0], (__bf16)acc[1], (__bf16)acc[2], (__bf16)acc[3]};
    *reinterpret_cast<bf16x4 *>(p.out + ((int64_t)t * H + h) * DV + c) = v;
    if ((threadIdx.x & 127) == 0) p.lse[(int64_t)t * H + h] = L;
}

hipError_t launch_sparse_mla(const MlaParams &p, int T, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    hipLaunchKernelGGL(sparse_mla_kernel, dim3(T, p.splits), dim3(NTHREADS), 0, s, p, p.idx, p.out,
                       p.lse, p.o_part, p.lse_part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1) return e;
    hipLaunchKernelGGL(mla_merge_kernel, dim3(T, H / 2), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace dsa
