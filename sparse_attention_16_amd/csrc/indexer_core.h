// indexer_core.h — building blocks of the lightning-indexer score on the
// gfx950 FP8 matrix cores, shared by the score kernels (indexer.hip) and the
// fused indexer + select (indexer_topk.hip), so that every path computes the
// same fp32 value for a (query row, key) pair:
//   I[t,s] = k_scale[s] * sum_j (w[t,j] * q_scale[t,j]) * max(0, sum_d q[t,j,d] k[s,d])
// (page "Техотчёт DeepSeek-V3.2 (2025): разреженное внимание DSA и
// масштабирование RL", section "Молниеносный индексатор", the I_{t,s}
// equation on FP8 inputs; the scales are positive, so they fold outside the
// ReLU exactly in real arithmetic).
//
// Lane layout of one 16-key block (16x16x128 FP8 MFMA): A = 16 indexer heads
// of one query row, B = 16 keys; the C tile gives each lane 4 heads of one key
// column.  The weighted ReLU sum runs over a lane's 16 heads, then the four
// 16-lane groups are summed for four blocks at once (reduce_scatter4), which
// leaves key l of the 64-key group in lane l.
#pragma once

#include "dsa_device.h"
#include "kernels.h"

namespace dsa {

namespace {

constexpr int HI = 64;
constexpr int DI = 128;
constexpr int ROW_BYTES = HI * DI;  // one query row of FP8 indexer queries

// Loads the A operands (4 head groups) and folded weights of one query row.
// Branch-free: an invalid row reads row t anyway (the caller passes a valid
// row index) and gets zero weights, so its scores are zero.
__device__ __forceinline__ void load_query(const IndexerParams &p, int64_t t, bool valid,
                                           i32x8 (&qa)[4], float (&wq)[4][4]) {
    const int l = lane_id();
    const int row = l & 15, grp = l >> 4;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const uint8_t *src = p.q + t * ROW_BYTES + (16 * m + row) * DI + 32 * grp;
        const i32x4 *s4 = reinterpret_cast<const i32x4 *>(src);
        const i32x4 lo = s4[0], hi = s4[1];
        qa[m] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int j = 16 * m + 4 * grp + i;
            wq[m][i] = (valid ? 1.0f : 0.0f) * (p.w[t * HI + j] * p.q_scale[t * HI + j]);
        }
    }
}

// The 16 head partials of one lane for one 16-key block: 4 MFMAs (one per
// group of 16 heads), kept in separate accumulators so that they can be in
// flight while the previous block's epilogue runs.
__device__ __forceinline__ void block_mfma(const i32x8 (&qa)[4], const i32x8 &kb, f32x4 (&c)[4]) {
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < 4; ++m) c[m] = mfma_f8_16x16x128(qa[m], kb, zero);
}

// ReLU + weighted sum over this lane's 16 heads (4 per MFMA tile).
__device__ __forceinline__ float block_epilogue(const f32x4 (&c)[4], const float (&wq)[4][4]) {
    float part = 0.f;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) part = fmaf(wq[m][i], fmaxf(c[m][i], 0.f), part);
    return part;
}

// Sum over the four 16-lane groups of four 16-key blocks at once: p[b] holds,
// in lane l, the partial (over the heads of group l/16) of key 16*b + l%16.
// Returns, in lane l, the total of key l of the 64-key group.  Two exchanges
// of the lane halves, then of the 16-lane rows (VALU lane swaps, no LDS).
__device__ __forceinline__ float reduce_scatter4(const float (&p)[4]) {
    const auto x02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[0]), __float_as_uint(p[2]), false, false);
    const auto x13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[1]), __float_as_uint(p[3]), false, false);
    const float a = __uint_as_float(x02[0]) + __uint_as_float(x02[1]);   // blocks 0 | 2, halves summed
    const float b = __uint_as_float(x13[0]) + __uint_as_float(x13[1]);   // blocks 1 | 3
    const auto y = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(y[0]) + __uint_as_float(y[1]);
}

// Direct-to-LDS loads (16 or 4 bytes per lane) from sbase + voff (scalar base,
// 32-bit lane offset) to LDS lds + size * lane.  Issued from asm: the
// compiler's wait insertion does not track them; the kernel waits with
// explicit vmcnt.  M0 must be written one instruction ahead of the load.
// The 16-byte load uses the non-temporal cache policy: its data (a decode
// row's keys) is read exactly once, and streamed from HBM this way it moves at
// about 6.4 TB/s where the default policy stays near 4 TB/s (measured on
// MI355X with a 640 MB stream after a cache flush).
__device__ __forceinline__ void dma_b128_nt(uint64_t sbase, uint32_t voff, const DSA_LDS void *lds) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sbase), "s"(m0)
                 : "m0");
}
__device__ __forceinline__ void dma_b32(uint64_t sbase, uint32_t voff, const DSA_LDS void *lds) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "s"(m0)
                 : "m0");
}
// A wave-uniform 64-bit pointer value in scalar registers.  (readfirstlane
// returns int: widen through uint32_t, or the low word is sign-extended.)
__device__ __forceinline__ uint64_t uniform_u64(uint64_t v) {
    return ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32)) << 32) |
           (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
}

// Candidate threshold of the fused select as a float: tau is an
// order-preserving score key (0 = no threshold, every visible key), and the
// float comparison score >= threshold_value(tau) selects exactly the keys with
// score_key(score) >= tau (-0 and +0 compare equal both ways).
__device__ __forceinline__ float threshold_value(uint32_t tau) {
    if (tau == 0u) return -INFINITY;
    return __uint_as_float((tau & 0x80000000u) ? (tau & 0x7FFFFFFFu) : ~tau);
}

// Appends this lane's score to the region at rbase when c holds: one ballot,
// the lane's rank among the wave's candidates, and a wave-uniform running
// count (slots past the region's capacity are counted but not written).  The
// score is stored as its fp32 bits; the select turns it into its key.  rbase
// is wave-uniform, so the stores take a scalar base and a 32-bit lane byte
// offset (slot < cap, and 4 * cap fits 32 bits).
__device__ __forceinline__ void emit_candidate(const IndexerParams &p, bool c, float score, int key, int64_t rbase,
                                               int &cnt) {
    const uint64_t m = __ballot(c);
    if (m != 0ull) {
        const int rank = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                        __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        const int slot = cnt + rank;
        if (c && slot < p.cap) {
            const uint32_t off = 4u * (uint32_t)slot;
            *reinterpret_cast<uint32_t *>(reinterpret_cast<char *>(p.cand_key + rbase) + off) = __float_as_uint(score);
            *reinterpret_cast<int32_t *>(reinterpret_cast<char *>(p.cand_pos + rbase) + off) = key;
        }
        cnt += __popcll(m);
    }
}

}  // namespace

}  // namespace dsa
