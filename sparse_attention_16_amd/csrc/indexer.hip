// indexer.hip — lightning-indexer scores on gfx950 matrix cores.
//
// Computes, for every visible (query row t, key s) pair,
//   I[t,s] = k_scale[s] * sum_j (w[t,j] * q_scale[t,j]) * max(0, sum_d q[t,j,d] k[s,d])
// which is the index score of the page "Техотчёт DeepSeek-V3.2 (2025):
// разреженное внимание DSA и масштабирование RL", section "Молниеносный
// индексатор" (the I_{t,s} equation), evaluated on FP8 inputs as that section
// prescribes.  Folding both dequantisation scales outside the ReLU is exact in
// real arithmetic because the scales are positive.
//
// Mapping onto the 16x16x128 FP8 MFMA: the contraction dim (128) is one
// instruction; A = 16 indexer heads of one query row (held in registers for
// the whole kernel), B = 16 keys.  The C tile holds 4 heads per lane for one
// key column, so the ReLU and the weighted head sum run in registers (16
// terms per lane per row).  The sum over the four 16-lane groups is done for
// four 16-key blocks at once with two rounds of VALU lane swaps (a reduce-
// scatter that leaves key l of the 64 in lane l).  Only the final fp32 score
// leaves the registers.
#include "indexer_core.h"

namespace dsa {


// ---------------------------------------------------------------------------
// Prefill variant: one workgroup = 16 consecutive query rows of one sequence
// (8 waves x 2 rows) x one chunk of keys.  Key tiles of 128 rows are staged
// once per workgroup in LDS (row pitch 144 B so that the 16 rows read by one
// B operand land on disjoint banks; two tiles, so that one barrier per tile
// suffices) and shared by all 16 query rows.
// Grid: x = row block, y = key chunk, z = sequence.
//
// Candidate mode (CAND): the score is not stored; a visible key whose score
// is >= the row's threshold is appended, in column order, to the row's
// candidate region of this key chunk (the region's running count is wave-
// uniform: one ballot and one mbcnt per 64 keys), and the region's count is
// written at the end.  Row blocks run longest first (causal rows grow with
// the block index), so the short blocks fill the tail.
// ---------------------------------------------------------------------------
constexpr int PF_ROWS = 16;
constexpr int PF_KT = 128;
constexpr int PF_PITCH = 144;

template <bool CAND>
__global__ __launch_bounds__(512) void indexer_prefill_kernel(IndexerParams p) {
    // two key tiles: the next one is written while this one is read
    __shared__ __attribute__((aligned(16))) uint8_t ktiles[2][PF_KT * PF_PITCH];
    __shared__ float kscales[2][PF_KT];

    const int b = blockIdx.z;
    const int q0 = p.cu_q[b];
    const int nq = p.cu_q[b + 1] - q0;
    const int tb = (CAND ? (int)(gridDim.x - 1 - blockIdx.x) : (int)blockIdx.x) * PF_ROWS;
    if (tb >= nq) return;
    int64_t kv0 = p.cu_kv[b], kv1 = p.cu_kv[b + 1];
    kv0 = kv0 < 0 ? 0 : (kv0 > p.total_kv ? p.total_kv : kv0);
    kv1 = kv1 < kv0 ? kv0 : (kv1 > p.total_kv ? p.total_kv : kv1);
    const int ctx = (int)((kv1 - kv0) > p.max_kv ? p.max_kv : (kv1 - kv0));
    const int last = (tb + PF_ROWS < nq ? tb + PF_ROWS : nq) - 1;
    int vis_max = p.pos0[b] + last + 1;
    vis_max = vis_max < 0 ? 0 : (vis_max > ctx ? ctx : vis_max);

    const int c0 = blockIdx.y * p.key_chunk;
    const int c_end = c0 + p.key_chunk;
    const int comp_end = c_end < vis_max ? c_end : vis_max;      // keys needing the MFMA
    const int fill_end = (!CAND && p.fill_masked) ? (c_end < ctx ? c_end : ctx) : comp_end;
    if (c0 >= fill_end) return;
    if (CAND && vis_max <= p.topk_k) return;   // every row of the block selects all it sees

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = lane_id();

    // two query rows per wave
    i32x8 qa[2][4];
    float wq[2][4][4];
    int pos[2];
    bool valid[2];
    float thr[2];        // candidate mode: the rows' score thresholds
    int cnt[2] = {0, 0};  // candidate mode: candidates found so far (wave-uniform)
    int64_t rbase[2];    // candidate mode: first slot of the rows' regions
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int tl = tb + 2 * wave + r;
        valid[r] = tl < nq;
        pos[r] = p.pos0[b] + tl;
        load_query(p, (int64_t)(q0 + (valid[r] ? tl : tb)), valid[r], qa[r], wq[r]);
        if constexpr (CAND) {
            const int64_t t = q0 + (valid[r] ? tl : tb);
            thr[r] = threshold_value(p.tau[t]);
            rbase[r] = (t * p.nseg + blockIdx.y) * (int64_t)p.cap;
        }
    }

    // register staging of the next key tile: 1024 16-byte chunks over 512
    // threads.  A key row past comp_end loads row c0 instead (a real key
    // row): the scores of such keys are never used (the candidate test, the
    // score store and the -inf fill all check key < comp_end), and their
    // scale is 0.  The loaded values are touched only by put: a select on
    // them right after the load would make the wave wait for the load, and
    // with it for every candidate store issued before it.
    i32x4 stage[2];
    float sstage = 0.f;
    auto fetch = [&](int kbase) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int c = tid + 512 * r;
            const int key = c >> 3, byte = (c & 7) * 16;
            const bool in = kbase + key < comp_end;
            stage[r] = *reinterpret_cast<const i32x4 *>(p.k + (kv0 + (in ? kbase + key : c0)) * DI + byte);
        }
        if (tid < PF_KT) sstage = (kbase + tid < comp_end) ? p.k_scale[kv0 + kbase + tid] : 0.f;
    };

    auto put = [&](int buf) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int c = tid + 512 * r;
            *reinterpret_cast<i32x4 *>(&ktiles[buf][(c >> 3) * PF_PITCH + (c & 7) * 16]) = stage[r];
        }
        if (tid < PF_KT) kscales[buf][tid] = sstage;
    };
    // One barrier per tile: tile i is read from buffer i&1 while tile i+1
    // goes from registers into the other buffer (whose last readers, tile
    // i-1's, all passed the previous barrier).  The write to the other buffer
    // comes before the tile's last group of candidate stores, so that the
    // wait for the tile loads (issued at the top of the tile) does not also
    // wait for stores issued just before it.
    if (c0 < comp_end) {
        fetch(c0);
        put(0);
        __syncthreads();
    }
    int cur = 0;
    for (int kbase = c0; kbase < comp_end; kbase += PF_KT, cur ^= 1) {
        // the next tile's loads, issued even after the last tile (they then
        // read row c0 and fill a buffer nobody reads): unconditional loads
        // and writes let the compiler see that no load is in flight at the
        // top of the loop, so it adds no wait there
        fetch(kbase + PF_KT);
        const uint8_t *ktile = ktiles[cur];
        const float *kscale = kscales[cur];

        // 8 blocks of 16 keys, software-pipelined: the MFMAs of block st+1
        // are issued before the epilogue of block st.  Rows past the end of
        // the sequence run with zero operands (no branches); their scores are
        // not stored.
        auto kload = [&](int st) {
            const uint8_t *src = &ktile[(16 * st + (l & 15)) * PF_PITCH + 32 * (l >> 4)];
            const i32x4 lo = *reinterpret_cast<const i32x4 *>(src);
            const i32x4 hi = *reinterpret_cast<const i32x4 *>(src + 16);
            return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        };
        // Software pipeline over the 8 blocks of 16 keys: each stage issues
        // the MFMAs of block st+1 (both rows) and then runs the epilogue of
        // block st, whose MFMAs the previous stage issued, so matrix-core and
        // VALU work overlap.  (The empty asm pins each epilogue to its stage:
        // otherwise it is sunk to where the sums are reduced, and every
        // block's MFMA results stay live until then.)
        f32x4 ca[2][2][4];   // [pipeline slot][row][head group]
        float part[2][4];
        {
            const i32x8 kb = kload(0);
            block_mfma(qa[0], kb, ca[0][0]);
            block_mfma(qa[1], kb, ca[0][1]);
        }
#pragma unroll
        for (int st = 0; st < PF_KT / 16; ++st) {
            if (st + 1 < PF_KT / 16) {
                const i32x8 kb = kload(st + 1);
                block_mfma(qa[0], kb, ca[(st + 1) & 1][0]);
                block_mfma(qa[1], kb, ca[(st + 1) & 1][1]);
            }
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                part[r][st & 3] = block_epilogue(ca[st & 1][r], wq[r]);
                asm volatile("" : "+v"(part[r][st & 3]));
            }
            if (st == PF_KT / 16 - 1) put(cur ^ 1);
            if ((st & 3) == 3) {
                // lane l: key kbase + 16*(st-3) + l
                const int key = kbase + 16 * (st - 3) + l;
                const float ks = key < comp_end ? kscale[16 * (st - 3) + l] : 0.f;
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    const float v = reduce_scatter4(part[r]);
                    if constexpr (CAND) {
                        const float sc = v * ks;
                        const bool c = valid[r] && key <= pos[r] && key < comp_end && sc >= thr[r];
                        emit_candidate(p, c, sc, key, rbase[r], cnt[r]);
                    } else if (valid[r] && key < fill_end) {
                        p.scores[(int64_t)(q0 + tb + 2 * wave + r) * p.ld + key] =
                            key <= pos[r] && key < comp_end ? v * ks : -INFINITY;
                    }
                }
            }
            // one pipeline stage per region: left free, the scheduler hoists
            // every block's MFMAs to the front and runs out of registers
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
    }

    if constexpr (CAND) {
#pragma unroll
        for (int r = 0; r < 2; ++r)
            if (valid[r] && l == 0) p.cand_cnt[(int64_t)(q0 + tb + 2 * wave + r) * p.nseg + blockIdx.y] = cnt[r];
        return;
    }

    // keys of this chunk that no row of the block can see: -inf when requested
    const int fill_start = comp_end > c0 ? comp_end : c0;
    if (fill_start < fill_end) {
        for (int r = 0; r < PF_ROWS; ++r) {
            const int tl = tb + r;
            if (tl >= nq) break;
            for (int s = fill_start + tid; s < fill_end; s += 512)
                p.scores[(int64_t)(q0 + tl) * p.ld + s] = -INFINITY;
        }
    }
}

// ---------------------------------------------------------------------------
// Decode variant: one workgroup = one query row x one chunk of keys; the 4
// waves split the chunk into 64-key groups (wave w: groups w, w+4, ...).  A
// key is used by a single query row, so nothing is shared: each wave streams
// its own groups, DC_NBUF deep, into a private LDS ring with direct-to-LDS
// loads (no registers held while they fly, no barriers; non-temporal, as
// each key is read once), then reads each
// 16-key B operand back as two 16-byte LDS reads.  Every load moves one
// contiguous KB (8 key rows) in its natural order, so each touches the fewest
// cache lines; the operand layout comes from the LDS reads.  Grid: x = query
// row, y = key chunk.
// ---------------------------------------------------------------------------
constexpr int DC_WAVES = 4;
// Groups in flight per wave.  One: a smaller LDS ring leaves room for more
// resident workgroups (four per compute unit), and more independent streams
// beat a deeper ring per wave (measured on the 64-sequence decode batch).
constexpr int DC_NBUF = 1;
constexpr int DC_GROUP = 64 * DI;           // bytes of one 64-key group
constexpr int DC_LOADS = 9;                 // loads per group: 8 x 1 KB of keys + the scales

// Candidate mode (CAND): wave w takes the contiguous 512 columns
// [c0 + 512w, c0 + 512w + 512) instead of every fourth group, so that its
// candidates (the visible keys whose score is >= the row's threshold) fill
// one region in column order; the region holds all of them (cap 512).
template <bool CAND>
__global__ __launch_bounds__(64 * DC_WAVES) __attribute__((amdgpu_waves_per_eu(4)))
void indexer_decode_kernel(IndexerParams p) {
    __shared__ __attribute__((aligned(16))) uint8_t kst[DC_WAVES][DC_NBUF][DC_GROUP];
    __shared__ __attribute__((aligned(16))) float sst[DC_WAVES][DC_NBUF][64];
    const int t = blockIdx.x;
    const RowInfo ri = row_info(p.cu_q, p.cu_kv, p.pos0, p.B, p.total_kv, p.max_kv, t);
    const int c0 = blockIdx.y * p.key_chunk;
    const int c_end = c0 + p.key_chunk;
    const int comp_end = c_end < ri.nvis ? c_end : ri.nvis;
    const int fill_end = (!CAND && p.fill_masked) ? (c_end < ri.ctx ? c_end : ri.ctx) : comp_end;
    if (c0 >= fill_end) return;
    if (CAND && ri.nvis <= p.topk_k) return;   // the row selects every key it sees

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l = lane_id();
    i32x8 qa[4];
    float wq[4][4];
    load_query(p, t, true, qa, wq);

    // this wave's groups: g0 = gstart, gstart + STRIDE, ... below gend
    const int STRIDE = CAND ? 64 : 64 * DC_WAVES;
    const int gstart = CAND ? c0 + CAND_DECODE_SEG * wave : c0 + 64 * wave;
    const int gend = CAND ? (gstart + CAND_DECODE_SEG < fill_end ? gstart + CAND_DECODE_SEG : fill_end) : fill_end;
    float thr = 0.f;
    int cnt = 0;
    int64_t rbase = 0;
    const int seg = gstart / CAND_DECODE_SEG;
    if constexpr (CAND) {
        thr = threshold_value(p.tau[t]);
        rbase = ((int64_t)t * p.nseg + seg) * p.cap;
    }
    const int row = l & 15, grp = l >> 4;
    const uint64_t kbase = uniform_u64((uint64_t)(uintptr_t)(p.k + ri.kv0 * DI));
    const uint64_t sbase = uniform_u64((uint64_t)(uintptr_t)(p.k_scale + ri.kv0));
    // Loads of group g0 into the wave's slot, in two halves: keys 0..31
    // (4 loads) and keys 32..63 with the scales (5 loads).  Keys past the
    // visible end load key c0 instead (their scores are not stored), so that
    // every half issues exactly its count of loads, which the vmcnt waits
    // below count on.  A half is refilled with the next group's keys as soon
    // as its two 16-key blocks are scored, so that a wave has loads in flight
    // while it scores.
    auto issue_half = [&](int g0, int h) {
        // this wave's LDS reads of the half (of the previous group) have completed
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int j = 4 * h; j < 4 * h + 4; ++j) {   // keys 8j .. 8j+7 of the group, lane l: key 8j + l/8, bytes 16*(l%8)
            const int key = g0 + 8 * j + (l >> 3);
            const uint32_t kk = (uint32_t)(key < comp_end ? key : c0);
            dma_b128_nt(kbase, kk * DI + 16 * (l & 7), (const DSA_LDS void *)&kst[wave][0][j * 1024]);
        }
        if (h == 1) {
            const int key = g0 + l;
            dma_b32(sbase, 4u * (uint32_t)(key < comp_end ? key : c0), (const DSA_LDS void *)&sst[wave][0][0]);
        }
    };
    auto score_half = [&](int h, float (&part)[4]) {
#pragma unroll
        for (int st = 2 * h; st < 2 * h + 2; ++st) {
            const uint8_t *kr = &kst[wave][0][(16 * st + row) * DI + 32 * grp];
            const i32x4 lo = *reinterpret_cast<const i32x4 *>(kr);
            const i32x4 hi = *reinterpret_cast<const i32x4 *>(kr + 16);
            const i32x8 kb = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            f32x4 c[4];
            block_mfma(qa, kb, c);
            part[st] = block_epilogue(c, wq);
        }
    };
    auto finish = [&](int g0, const float (&part)[4]) {
        const float v = reduce_scatter4(part);
        const float ks = sst[wave][0][l];
        const int key = g0 + l;
        if constexpr (CAND) {
            const float sc = v * ks;
            emit_candidate(p, key < comp_end && sc >= thr, sc, key, rbase, cnt);
        } else if (key < fill_end) {
            p.scores[(int64_t)t * p.ld + key] = key < comp_end ? v * ks : -INFINITY;
        }
    };
    static_assert(DC_NBUF == 1 && DC_LOADS == 9, "the waits below count 4 + 5 loads per group");
    if (gstart < gend) {
        issue_half(gstart, 0);
        issue_half(gstart, 1);
    }
    for (int g0 = gstart; g0 < gend; g0 += STRIDE) {
        const bool nxt = g0 + STRIDE < gend;
        float part[4];
        __builtin_amdgcn_s_waitcnt(0x0F70 | 5);   // vmcnt(5): this group's first half landed
        score_half(0, part);
        if (nxt) {
            issue_half(g0 + STRIDE, 0);
            __builtin_amdgcn_s_waitcnt(0x0F70 | 4);   // vmcnt(4): this group's second half landed
        } else {
            __builtin_amdgcn_s_waitcnt(0x0F70);       // vmcnt(0)
        }
        score_half(1, part);
        finish(g0, part);
        if (nxt) issue_half(g0 + STRIDE, 1);
    }
    if constexpr (CAND) {
        if (l == 0 && seg < p.nseg) p.cand_cnt[(int64_t)t * p.nseg + seg] = cnt;
    }
}

hipError_t launch_indexer(const IndexerParams &p, int T, int max_q, bool decode_variant,
                          hipStream_t s) {
    if (T <= 0 || p.max_kv <= 0) return hipSuccess;
    const int nchunk = (p.max_kv + p.key_chunk - 1) / p.key_chunk;
    if (decode_variant) {
        hipLaunchKernelGGL(indexer_decode_kernel<false>, dim3(T, nchunk), dim3(64 * DC_WAVES), 0, s, p);
    } else {
        const dim3 g((max_q + PF_ROWS - 1) / PF_ROWS, nchunk, p.B);
        hipLaunchKernelGGL(indexer_prefill_kernel<false>, g, dim3(512), 0, s, p);
    }
    return hipGetLastError();
}

hipError_t launch_indexer_cand(const IndexerParams &p, int T, int max_q, bool decode_variant, hipStream_t s) {
    if (T <= 0 || p.max_kv <= 0) return hipSuccess;
    const int nchunk = (p.max_kv + p.key_chunk - 1) / p.key_chunk;
    if (decode_variant) {
        if (p.key_chunk != DC_WAVES * CAND_DECODE_SEG || p.seg_w != CAND_DECODE_SEG || p.cap < CAND_DECODE_SEG)
            return hipErrorInvalidValue;
        hipLaunchKernelGGL(indexer_decode_kernel<true>, dim3(T, nchunk), dim3(64 * DC_WAVES), 0, s, p);
    } else {
        if (p.seg_w != p.key_chunk || p.nseg != nchunk) return hipErrorInvalidValue;
        const dim3 g((max_q + PF_ROWS - 1) / PF_ROWS, nchunk, p.B);
        hipLaunchKernelGGL(indexer_prefill_kernel<true>, g, dim3(512), 0, s, p);
    }
    return hipGetLastError();
}

}  // namespace dsa
