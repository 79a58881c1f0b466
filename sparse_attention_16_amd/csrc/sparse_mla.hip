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
// MQA property that keeps the gather coalesced).  4 waves x 32 heads: each K
// or V operand read from LDS feeds two 16-head MFMA tiles.
//
// Per 64-key block:
//   gather  : 64 selected rows -> LDS with direct-to-LDS 16-byte loads
//             (row pitch 1168 B), double-buffered so the next block's gather
//             overlaps this block's math;
//   S^T     : z^T[key, head] = K Q^T on the 16x16x32 bf16 MFMA; A = K rows
//             from LDS, B = this wave's 16 query heads (registers, loaded once);
//   softmax : online (running max m and sum l per head), exp2 domain;
//   PV      : O^T[c, head] += V^T P^T; B = P^T straight from the S^T
//             accumulators (the C layout of S^T already puts one head per
//             lane), A = V^T read with the LDS transpose load.
// Split-KV (few query rows): each split writes a normalised partial and its
// lse; mla_merge_kernel combines them.
#include "dsa_device.h"
#include "kernels.h"

namespace dsa {

namespace {

constexpr int H = 128;
constexpr int D = 576;
constexpr int DV = 512;
constexpr int ROWB = D * 2;            // 1152 bytes per latent row
constexpr int PITCH = ROWB + 16;       // LDS row pitch
constexpr int BK = MLA_BK;             // 64 keys per block
constexpr int BUF_BYTES = BK * PITCH;  // 74752
constexpr int NWAVES = 8;
constexpr int NTHREADS = NWAVES * kWave;
constexpr int HPW = H / NWAVES;        // heads per wave
constexpr int NHT = HPW / 16;          // 16-head MFMA tiles per wave
constexpr int LOADS_PER_BUF = (BUF_BYTES + 1023) / 1024;  // 1 KB per wave-wide load
constexpr int KSTEPS = D / 32;         // 18
constexpr int MT = BK / 16;            // 16-key tiles per block
constexpr int KK = BK / 32;            // 32-key PV steps per block
constexpr int CTILES = DV / 16;        // 32
constexpr float LN2 = 0.69314718055994530942f;

typedef DSA_LDS uint8_t lds_u8;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(8))) short i16x8;

// Issues the direct-to-LDS loads of one 64-key block.  Load slot j (16 B) of
// the buffer maps to LDS byte 16*j = row*PITCH + col; columns >= 1152 are the
// pitch padding and load a harmless in-bounds 16 bytes of the same row.
__device__ __forceinline__ void gather_block(const MlaParams &p, const int32_t *sel, int nsel,
                                             int blk, int64_t kv0, int ctx, lds_u8 *buf) {
    const int wave = threadIdx.x >> 6, l = lane_id();
    for (int li = wave; li < LOADS_PER_BUF; li += NWAVES) {
        const int off = li * 1024 + l * 16;
        int row = off / PITCH;
        int col = off - row * PITCH;
        if (row >= BK) {
            row = BK - 1;
            col = 0;
        }
        if (col >= ROWB) col = 0;
        const int j = blk * BK + row;
        int s = j < nsel ? sel[j] : -1;
        if (s < 0 || s >= ctx) s = 0;   // masked later; any in-bounds row
        const uint8_t *src = reinterpret_cast<const uint8_t *>(p.kv) + (kv0 + s) * ROWB + col;
        __builtin_amdgcn_global_load_lds(src, buf + li * 1024, 16, 0, 0);
    }
}

}  // namespace

// Grid: x = query row, y = split.  LDS: two gather buffers + the row's idx.
__global__ __launch_bounds__(NTHREADS) void sparse_mla_kernel(MlaParams p) {
    __shared__ __attribute__((aligned(1024))) uint8_t buf0[LOADS_PER_BUF * 1024];
    __shared__ __attribute__((aligned(1024))) uint8_t buf1[LOADS_PER_BUF * 1024];
    __shared__ int32_t sel[2048];

    const int t = blockIdx.x, split = blockIdx.y;
    const int tid = threadIdx.x, wave = tid >> 6, l = lane_id();
    const int row16 = l & 15, grp = l >> 4;
    const RowInfo ri = row_info(p.cu_q, p.cu_kv, p.pos0, p.B, p.total_kv, p.max_kv, t);

    // this split's slice of the selected set
    const int j0 = split * p.blocks_per_split * BK;
    int j1 = j0 + p.blocks_per_split * BK;
    j1 = j1 < p.k ? j1 : p.k;
    const int nsel = (j1 > j0 && ri.ctx > 0) ? j1 - j0 : 0;
    const int32_t *idx_row = p.idx + (int64_t)t * p.k + j0;
    for (int j = tid; j < nsel; j += NTHREADS) {
        const int s = idx_row[j];
        sel[j] = (s >= 0 && s < ri.ctx) ? s : -1;
    }
    __syncthreads();
    const int nblk = (nsel + BK - 1) / BK;

    // query operands of this wave's 2 x 16 heads: lane holds head
    // h0 + 16*ht + row16, dims 32*ks + 8*grp .. +7
    const int h0 = wave * HPW;
    bf16x8 qb[NHT][KSTEPS];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
        const uint16_t *qrow = p.q + ((int64_t)t * H + h0 + 16 * ht + row16) * D + 8 * grp;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks)
            qb[ht][ks] = *reinterpret_cast<const bf16x8 *>(qrow + 32 * ks);
    }

    f32x4 o[NHT][CTILES];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
        for (int c = 0; c < CTILES; ++c) o[ht][c] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[NHT], l_run[NHT];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
        m_run[ht] = -INFINITY;
        l_run[ht] = 0.f;
    }

    lds_u8 *lb0 = (lds_u8 *)buf0;
    lds_u8 *lb1 = (lds_u8 *)buf1;
    if (nblk > 0) gather_block(p, sel, nsel, 0, ri.kv0, ri.ctx, lb0);

    // One block step; `cur` and `nxt` are distinct LDS arrays at compile time
    // (the loop is unrolled by two), so the compiler can see that reads of
    // `cur` do not depend on the direct-to-LDS loads still landing in `nxt`.
    auto step = [&](int blk, lds_u8 *cur, lds_u8 *nxt) {
        // block blk has landed in `cur` for every wave, and every wave is done
        // reading `nxt` (block blk-1)
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        __syncthreads();
        if (blk + 1 < nblk) gather_block(p, sel, nsel, blk + 1, ri.kv0, ri.ctx, nxt);

        // ---- S^T = K Q^T : MT key tiles of 16, lane = (head row16, keys 4*grp+i).
        // The next k-step's operand of key tile mt is loaded right after the
        // current one is consumed; the scheduling barrier keeps the compiler
        // from hoisting more LDS reads (query operands and accumulators fill
        // most of the register file).
        f32x4 sacc[NHT][MT];
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) sacc[ht][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        {
            const lds_u8 *kbase = cur + row16 * PITCH + 16 * grp;
            bf16x8 abuf[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                abuf[mt] = *reinterpret_cast<const DSA_LDS bf16x8 *>(kbase + 16 * mt * PITCH);
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const bf16x8 a = abuf[mt];
                    if (ks + 1 < KSTEPS)
                        abuf[mt] = *reinterpret_cast<const DSA_LDS bf16x8 *>(
                            kbase + 16 * mt * PITCH + 64 * (ks + 1));
#pragma unroll
                    for (int ht = 0; ht < NHT; ++ht)
                        sacc[ht][mt] = mfma_bf16_16x16x32(a, qb[ht][ks], sacc[ht][mt]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }

        // ---- online softmax (log2 domain), per head tile.  The running max
        // only moves when a block raises it by more than 8 (p stays <= 2^8),
        // so the O rescale is rare after the first block; the result is the
        // same softmax because l and O always share the max used for p.
        const int jv = blk * BK + (l & (BK - 1));
        const uint32_t vmask = (uint32_t)__ballot(jv < nsel && sel[jv] >= 0);
        bf16x8 pb[NHT][KK];
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) {
            float bmax = -INFINITY;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const uint32_t nib = (vmask >> (16 * mt + 4 * grp)) & 0xFu;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float z = ((nib >> i) & 1u) ? sacc[ht][mt][i] * p.scale_log2 : -INFINITY;
                    sacc[ht][mt][i] = z;
                    bmax = fmaxf(bmax, z);
                }
            }
            bmax = fmaxf(bmax, xor16_f(bmax));
            bmax = fmaxf(bmax, shfl_xor_f(bmax, 32));
            const bool raise = bmax > m_run[ht] + 8.f;
            if (__ballot(raise)) {
                const float alpha = raise ? exp2f(m_run[ht] - bmax) : 1.f;
                if (raise) m_run[ht] = bmax;
                l_run[ht] *= alpha;
#pragma unroll
                for (int c = 0; c < CTILES; ++c) o[ht][c] *= alpha;
            }
            const float m_use = m_run[ht] == -INFINITY ? 0.f : m_run[ht];
            float psum = 0.f;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                float pv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    pv[e] = exp2f(sacc[ht][2 * kk + (e >> 2)][e & 3] - m_use);
                    psum += pv[e];
                }
                u32x4 pk = {pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                            pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7])};
                pb[ht][kk] = __builtin_bit_cast(bf16x8, pk);
            }
            l_run[ht] += psum;
        }

        // ---- O^T += V^T P^T : A = V^T via transpose reads, one c-tile ahead.
        // 16-lane group grp reads rows (keys) 32*kk + 4*grp + r (+16 for the
        // second half); lane (row16) of the group addresses row row16/4,
        // columns 16*ct + 4*(row16%4) .. +3.
        const int tr_row = row16 >> 2, tr_col = 4 * (row16 & 3);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const lds_u8 *r0 = cur + (32 * kk + 4 * grp + tr_row) * PITCH + 2 * tr_col;
            const lds_u8 *r1 = r0 + 16 * PITCH;
            i16x4 vlo = lds_read_tr16(r0), vhi = lds_read_tr16(r1);
#pragma unroll
            for (int ct = 0; ct < CTILES; ++ct) {
                const i16x8 a8 = {vlo[0], vlo[1], vlo[2], vlo[3], vhi[0], vhi[1], vhi[2], vhi[3]};
                if (ct + 1 < CTILES) {
                    vlo = lds_read_tr16(r0 + 32 * (ct + 1));
                    vhi = lds_read_tr16(r1 + 32 * (ct + 1));
                }
                const bf16x8 a = __builtin_bit_cast(bf16x8, a8);
#pragma unroll
                for (int ht = 0; ht < NHT; ++ht)
                    o[ht][ct] = mfma_bf16_16x16x32(a, pb[ht][kk], o[ht][ct]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    for (int blk = 0; blk < nblk; blk += 2) {
        step(blk, lb0, lb1);
        if (blk + 1 < nblk) step(blk + 1, lb1, lb0);
    }

    // ---- finish: full sum per head, normalise, write
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
        float l_tot = l_run[ht] + xor16_f(l_run[ht]);
        l_tot += shfl_xor_f(l_tot, 32);
        const int h = h0 + 16 * ht + row16;
        const bool empty = !(l_tot > 0.f);
        const float inv = empty ? 0.f : 1.f / l_tot;
        const float lse_v = empty ? -INFINITY : (m_run[ht] + log2f(l_tot)) * LN2;
        if (p.splits == 1) {
            uint16_t *orow = p.out + ((int64_t)t * H + h) * DV + 4 * grp;
#pragma unroll
            for (int ct = 0; ct < CTILES; ++ct) {
                u32x2 v = {pack_bf16x2(o[ht][ct][0] * inv, o[ht][ct][1] * inv),
                           pack_bf16x2(o[ht][ct][2] * inv, o[ht][ct][3] * inv)};
                *reinterpret_cast<u32x2 *>(orow + 16 * ct) = v;
            }
            if (grp == 0) p.lse[(int64_t)t * H + h] = lse_v;
        } else {
            float *orow = p.o_part + (((int64_t)t * p.splits + split) * H + h) * DV + 4 * grp;
#pragma unroll
            for (int ct = 0; ct < CTILES; ++ct)
                *reinterpret_cast<f32x4 *>(orow + 16 * ct) = o[ht][ct] * inv;
            if (grp == 0) p.lse_part[((int64_t)t * p.splits + split) * H + h] = lse_v;
        }
    }
}

// Combines split partials: lse = ln sum_s exp(lse_s), out = sum_s exp(lse_s - lse) o_s.
// Grid: x = query row; 128 threads x 4 columns each per head loop.
__global__ __launch_bounds__(256) void mla_merge_kernel(MlaParams p) {
    const int t = blockIdx.x;
    const int S = p.splits;
    for (int h = threadIdx.x >> 7 ? 1 : 0; h < H; h += 2) {
        const float *lp = p.lse_part + ((int64_t)t * S) * H + h;
        float mx = -INFINITY;
        for (int s = 0; s < S; ++s) mx = fmaxf(mx, lp[(int64_t)s * H]);
        float den = 0.f;
        if (mx != -INFINITY)
            for (int s = 0; s < S; ++s) den += expf(lp[(int64_t)s * H] - mx);
        const float L = mx == -INFINITY ? -INFINITY : mx + logf(den);
        const int c = 4 * (threadIdx.x & 127);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (mx != -INFINITY) {
            for (int s = 0; s < S; ++s) {
                const float ls = lp[(int64_t)s * H];
                if (ls == -INFINITY) continue;
                const float wgt = expf(ls - L);
                const f32x4 v = *reinterpret_cast<const f32x4 *>(
                    p.o_part + (((int64_t)t * S + s) * H + h) * DV + c);
                acc += v * wgt;
            }
        }
        u32x2 v = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
        *reinterpret_cast<u32x2 *>(p.out + ((int64_t)t * H + h) * DV + c) = v;
        if ((threadIdx.x & 127) == 0) p.lse[(int64_t)t * H + h] = L;
    }
}

hipError_t launch_sparse_mla(const MlaParams &p, int T, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    hipLaunchKernelGGL(sparse_mla_kernel, dim3(T, p.splits), dim3(NTHREADS), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1) return e;
    hipLaunchKernelGGL(mla_merge_kernel, dim3(T), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace dsa
