// indexer_kl.hip — the lightning indexer's KL loss on gfx950.
//
// Page "Техотчёт DeepSeek-V3.2 (2025): разреженное внимание DSA и
// масштабирование RL", section "Как учили индексатор": the indexer is trained
// toward where the main attention looks.  For query row t and its key set
// (every visible key in the dense warm-up, the selected slots in the sparse
// stage):
//   q_s  = sum_h exp(z[h,s] - lse[h]),   z[h,s] = scale * <q[t,h,:], kv[s,:]>
//          (the attention's probabilities summed over the 128 heads; lse is
//          the attention's own log-sum-exp over the same set),
//   p_s  = q_s / sum_s q_s                                (L1 normalisation),
//   kl_t = sum_s p_s (ln p_s - ln softmax(I[t,:])_s)
//        = A/Q - ln Q - B/Q + ln sum_s exp(I_s),
//   where Q = sum q_s, A = sum q_s ln q_s, B = sum q_s I_s.
//
// The logits are the attention's QK^T on the bf16 16x16x32 MFMA.  Each
// 32-slot block of latent rows is loaded into LDS with direct-to-LDS loads
// (the 1 KB latent part of a row at a 1056-byte pitch; the 128-byte rope parts
// of eight rows in one XOR-swizzled 1 KB slab); Q stays in VGPRs.  Four waves
// each own 32 heads.  Per block a wave sums exp over its heads (in-lane over
// its two head tiles, then across the 16 lanes of a DPP row) and leaves one
// value per slot in LDS; after the block's barrier, wave 0 adds the four
// waves' values and accumulates Q, A, B and the running log-sum-exp of I.
#include "dsa_device.h"
#include "kernels.h"

namespace dsa {

namespace {

constexpr int H = 128, D = 576;
constexpr int BK = KL_BK;                 // 32 slots per block
constexpr int NW = 4;                     // waves; wave w owns heads 32w .. 32w+31
constexpr int NT = NW * kWave;            // 256 threads
constexpr int KS = D / 32;                // 18 k-steps (16 latent + 2 rope)
constexpr int ROWB = D * 2;               // 1152 bytes per latent row
constexpr int PA = 1056;                  // LDS pitch of a row's first 1024 bytes
constexpr int RB = BK * PA;               // rope slabs: 4 x (8 rows x 128 B)
constexpr int BUF = RB + BK * 128;        // 37888 bytes per block buffer
constexpr int NPART = 5;                  // Q, A, B, max I, sum exp(I - max)
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.69314718055994530942f;
constexpr float FLT_MIN_NORMAL = 1.17549435e-38f;
constexpr int AHEAD = 3;                  // k-steps of K operands read ahead

typedef DSA_LDS uint8_t lds_u8;

static_assert(BK == 8 * NW, "each wave loads 8 rows and one rope slab per block");

// Sum over the 16 lanes of a DPP row (row_ror 8, 4, 2, 1): every lane of the
// row ends with the row's total.
__device__ __forceinline__ float row_sum16(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x122, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x121, 0xF, 0xF, false));
    return v;
}

// Entry of slot (blk * BK + (l & 31)) of the split as loaded: the index
// entry, the position itself in the dense mode, or -1 past the split's range.
// slot_checked turns it into a position, or -1 for an unusable slot (a
// negative or out-of-context entry).  The two are apart so that a freshly
// issued index load is not consumed at once: that would make the wave wait
// for it, and with it for every gather load issued before it.
__device__ __forceinline__ int slot_entry(const int32_t *__restrict__ idx_row, int j0, int nsel, int blk, int l) {
    const int j = blk * BK + (l & 31);
    if (j >= nsel) return -1;
    if (!idx_row) return j0 + j;
    return idx_row[j];
}
__device__ __forceinline__ int slot_checked(int v, int ctx) { return (v >= 0 && v < ctx) ? v : -1; }

// Loads one block's rows into buf: wave w the latent parts of rows
// 8w .. 8w+7 (one 1 KB load each) and the rope slab of the same rows (lane l:
// row 8w + l/8, its 16-byte chunk (l%8) ^ (l/8)).  Unusable slots load row 0.
__device__ __forceinline__ void gather_block(int pv, int wave, int l, uint64_t kvb, lds_u8 *buf) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int pos = __builtin_amdgcn_readlane(pv, 8 * wave + i);
        const uint32_t row = pos < 0 ? 0u : (uint32_t)pos;
        const uint64_t base = kvb + (uint64_t)row * ROWB;
        dma16s(base, 16u * (uint32_t)l, buf + (8 * wave + i) * PA);
    }
    const int ps = __shfl(pv, 8 * wave + (l >> 3), kWave);
    const uint32_t row = ps < 0 ? 0u : (uint32_t)ps;
    dma16s(kvb, row * ROWB + 1024u + 16u * (uint32_t)((l & 7) ^ (l >> 3)), buf + RB + wave * 1024);
}

}  // namespace

// Grid: x = query row (last row first: in a causal batch the last rows see the
// most keys), y = split of the row's slots.  LDS: two block buffers and the
// per-wave slot sums of two blocks (76.8 KB: two workgroups per compute unit).
__global__ __launch_bounds__(NT, 2) void indexer_kl_kernel(KlParams p) {
    __shared__ __attribute__((aligned(1024))) uint8_t kb[2][BUF];
    __shared__ float red[2][NW][BK];

    const int t = (int)gridDim.x - 1 - (int)blockIdx.x, split = blockIdx.y;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = lane_id();
    const int row16 = l & 15, grp = l >> 4;
    const RowInfo ri = row_info(p.cu_q, p.cu_kv, p.pos0, p.B, p.total_kv, p.max_kv, t);
    const bool dense = p.idx == nullptr;

    // this split's slots [j0, j0 + nsel) of the row's [0, jend)
    const int jend = dense ? ri.nvis : p.k;
    const int j0 = split * p.blocks_per_split * BK;
    int j1 = j0 + p.blocks_per_split * BK;
    j1 = j1 < jend ? j1 : jend;
    const int nsel = j1 > j0 ? j1 - j0 : 0;
    const int32_t *__restrict__ idx_row = dense ? nullptr : p.idx + (int64_t)t * p.k + j0;
    if (ri.ctx == 0 && nsel > 0) {
        // a sequence without cache rows: nothing to load (its "row 0" is not
        // there); every slot is unusable
        if (p.p_out && !dense)
            for (int j = threadIdx.x; j < nsel; j += NT) p.p_out[(int64_t)t * p.k + j0 + j] = 0.f;
        if (threadIdx.x == 0) {
            if (p.splits == 1 && !p.p_out) {
                p.kl[t] = 0.f;
            } else {
                float *o = p.part + ((int64_t)t * p.splits + split) * NPART;
                o[0] = 0.f;
                o[1] = 0.f;
                o[2] = 0.f;
                o[3] = -INFINITY;
                o[4] = 0.f;
            }
        }
        return;
    }
    const int nblk = (nsel + BK - 1) / BK;

    // query operands: lane holds head 32*wave + 16*ht + row16, dims 32*ks + 8*grp .. +7
    bf16x8 qb[2][KS];
    float lse2[2];
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
        const int h = 32 * wave + 16 * ht + row16;
        const uint16_t *qrow = p.q + ((int64_t)t * H + h) * D + 8 * grp;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qb[ht][ks] = *reinterpret_cast<const bf16x8 *>(qrow + 32 * ks);
        const float ls = p.lse[(int64_t)t * H + h];
        // a head without a finite lse (nothing attended) contributes nothing
        lse2[ht] = ls > -INFINITY && ls < INFINITY ? ls * LOG2E : INFINITY;
    }
    uint64_t kvb = (uint64_t)(uintptr_t)p.kv + (uint64_t)ri.kv0 * ROWB;
    // (readfirstlane returns int: widen through uint32_t, or the low word is sign-extended)
    kvb = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(kvb >> 32)) << 32) |
          (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)kvb);

    // LDS read offsets of the K operands (buffer-relative): key row16 of the
    // 16-key tile, dims 32*ks + 8*grp (latent: row pitch PA; rope: the slab)
    const int rr = row16 & 7;
    const int kA = row16 * PA + 16 * grp;
    const int kR = RB + (row16 >> 3) * 1024 + rr * 128;
    const int kR16 = kR + 16 * (grp ^ rr);
    const int kR17 = kR + 16 * ((4 + grp) ^ rr);

    // wave 0, lanes 0..31 (slot l of each block): the row's partial sums
    float aQ = 0.f, aA = 0.f, aB = 0.f, mI = -INFINITY, sI = 0.f;
    const float *__restrict__ srow = p.scores + (int64_t)t * p.ld;

    int pcur = nblk > 0 ? slot_checked(slot_entry(idx_row, j0, nsel, 0, l), ri.ctx) : -1;
    int pnext = nblk > 1 ? slot_checked(slot_entry(idx_row, j0, nsel, 1, l), ri.ctx) : -1;
    float icur = 0.f, inext = 0.f;
    if (nblk > 0) {
        gather_block(pcur, wave, l, kvb, (lds_u8 *)kb[0]);
        if (wave == 0 && pcur >= 0) icur = srow[pcur];
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): block 0 and the query operands
    lds_barrier();

    for (int b = 0; b < nblk; ++b) {
        const int cur = b & 1;
        const lds_u8 *buf = (const lds_u8 *)kb[cur];
        // block b+1's rows and index scores, block b+2's positions
        if (b + 1 < nblk) {
            gather_block(pnext, wave, l, kvb, (lds_u8 *)kb[cur ^ 1]);
            if (wave == 0 && pnext >= 0) inext = srow[pnext];
        }
        // (block b+2's entries are checked only after the block's barrier,
        // which waits for every load of the wave anyway)
        int pn2 = b + 2 < nblk ? slot_entry(idx_row, j0, nsel, b + 2, l) : -1;

        // S^T = K Q^T: lane holds head (32*wave + 16*ht + row16), keys 16*mt + 4*grp + r
        f32x4 s[2][2];
#pragma unroll
        for (int ht = 0; ht < 2; ++ht)
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) s[ht][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        // K operands are read AHEAD k-steps before their MFMAs (a ring of
        // registers), so the LDS latency hides behind the MFMAs in between
        auto koff = [&](int ks, int mt) {
            return ks < 16 ? kA + mt * 16 * PA + 64 * ks : (ks == 16 ? kR16 : kR17) + mt * 2048;
        };
        bf16x8 kr[AHEAD + 1][2];
#pragma unroll
        for (int ks = 0; ks < AHEAD; ++ks)
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) kr[ks][mt] = *reinterpret_cast<const DSA_LDS bf16x8 *>(buf + koff(ks, mt));
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + AHEAD < KS) {
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
                    kr[(ks + AHEAD) % (AHEAD + 1)][mt] =
                        *reinterpret_cast<const DSA_LDS bf16x8 *>(buf + koff(ks + AHEAD, mt));
            }
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int ht = 0; ht < 2; ++ht)
                    s[ht][mt] = mfma_bf16_16x16x32(kr[ks % (AHEAD + 1)][mt], qb[ht][ks], s[ht][mt]);
            __builtin_amdgcn_sched_barrier(0);
        }

        // probabilities summed over the wave's 32 heads, one value per slot
        float e[2][4];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                e[mt][r] = row_sum16(__builtin_amdgcn_exp2f(fmaf(s[0][mt][r], p.scale_log2, -lse2[0])) +
                                     __builtin_amdgcn_exp2f(fmaf(s[1][mt][r], p.scale_log2, -lse2[1])));
        if (row16 < 8) {
            const int mt = row16 >> 2, r = row16 & 3;
            float v = e[0][0];
#pragma unroll
            for (int x = 1; x < 8; ++x) v = row16 == x ? e[x >> 2][x & 3] : v;
            red[cur][wave][16 * mt + 4 * grp + r] = v;
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's loads of block b+1
        lds_barrier();
        asm volatile("" : "+v"(pn2));   // (keeps the check below the wait)
        pn2 = slot_checked(pn2, ri.ctx);

        // wave 0: fold block b into the row's sums
        if (wave == 0 && l < BK && pcur >= 0) {
            const float qv = red[cur][0][l] + red[cur][1][l] + red[cur][2][l] + red[cur][3][l];
            const float iv = icur;
            aQ += qv;
            // (the raw exp2 flushes results below 2^-126 to 0: qv is 0 or normal)
            if (qv >= FLT_MIN_NORMAL) aA += qv * (__builtin_amdgcn_logf(qv) * LN2);
            aB += qv * iv;
            if (iv > mI) {
                sI = sI * __builtin_amdgcn_exp2f((mI - iv) * LOG2E) + 1.f;
                mI = iv;
            } else if (iv > -INFINITY) {
                sI += __builtin_amdgcn_exp2f((iv - mI) * LOG2E);
            }
            if (p.p_out) {
                const int64_t col = dense ? (int64_t)pcur : (int64_t)(j0 + b * BK + l);
                p.p_out[(int64_t)t * (dense ? p.ld : p.k) + col] = qv;
            }
        } else if (wave == 0 && l < BK && p.p_out && !dense && b * BK + l < nsel) {
            p.p_out[(int64_t)t * p.k + j0 + b * BK + l] = 0.f;   // unusable slot
        }
        pcur = pnext;
        pnext = pn2;
        icur = inext;
    }

    if (wave != 0) return;
    // the row's sums over wave 0's lanes
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) {
        aQ += shfl_xor_f(aQ, m);
        aA += shfl_xor_f(aA, m);
        aB += shfl_xor_f(aB, m);
        const float mo = shfl_xor_f(mI, m), so = shfl_xor_f(sI, m);
        const float mn = fmaxf(mI, mo);
        sI = (mI > -INFINITY ? sI * exp2f((mI - mn) * LOG2E) : 0.f) +
             (mo > -INFINITY ? so * exp2f((mo - mn) * LOG2E) : 0.f);
        mI = mn;
    }
    if (l != 0) return;
    if (p.splits == 1 && !p.p_out) {
        p.kl[t] = aQ > 0.f ? aA / aQ - logf(aQ) - aB / aQ + (mI + logf(sI)) : 0.f;
    } else {
        float *o = p.part + ((int64_t)t * p.splits + split) * NPART;
        o[0] = aQ;
        o[1] = aA;
        o[2] = aB;
        o[3] = mI;
        o[4] = sI;
    }
}

// Combines a row's split sums into kl[t] and, when p_out is given, divides
// the row's stored q_s by Q (the L1 normalisation).  One workgroup per row.
__global__ __launch_bounds__(256) void indexer_kl_finish_kernel(KlParams p) {
    __shared__ float sq;
    const int t = blockIdx.x;
    if (threadIdx.x == 0) {
        float Q = 0.f, A = 0.f, Bs = 0.f, M = -INFINITY, S = 0.f;
        for (int s = 0; s < p.splits; ++s) {
            const float *o = p.part + ((int64_t)t * p.splits + s) * NPART;
            Q += o[0];
            A += o[1];
            Bs += o[2];
            const float m = o[3], sm = o[4];
            if (m > -INFINITY) {
                const float mn = fmaxf(M, m);
                S = (M > -INFINITY ? S * expf(M - mn) : 0.f) + sm * expf(m - mn);
                M = mn;
            }
        }
        p.kl[t] = Q > 0.f ? A / Q - logf(Q) - Bs / Q + (M + logf(S)) : 0.f;
        sq = Q;
    }
    __syncthreads();
    if (!p.p_out) return;
    const float inv = sq > 0.f ? 1.f / sq : 0.f;
    const RowInfo ri = row_info(p.cu_q, p.cu_kv, p.pos0, p.B, p.total_kv, p.max_kv, t);
    const bool dense = p.idx == nullptr;
    const int n = dense ? ri.nvis : p.k;
    float *row = p.p_out + (int64_t)t * (dense ? p.ld : p.k);
    for (int j = threadIdx.x; j < n; j += 256) row[j] *= inv;
}

hipError_t launch_indexer_kl(const KlParams &p, int T, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    hipLaunchKernelGGL(indexer_kl_kernel, dim3(T, p.splits), dim3(NT), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || (p.splits == 1 && !p.p_out)) return e;
    hipLaunchKernelGGL(indexer_kl_finish_kernel, dim3(T), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace dsa
