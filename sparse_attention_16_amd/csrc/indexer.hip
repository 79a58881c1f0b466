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

}  // namespace

// ---------------------------------------------------------------------------
// Prefill variant: one workgroup = 16 consecutive query rows of one sequence
// (8 waves x 2 rows) x one chunk of keys.  Key tiles of 128 rows are staged
// once per workgroup in LDS (row pitch 144 B so that the 16 rows read by one
// B operand land on disjoint banks) and shared by all 16 query rows.
// Grid: x = row block, y = key chunk, z = sequence.
// ---------------------------------------------------------------------------
constexpr int PF_ROWS = 16;
constexpr int PF_KT = 128;
constexpr int PF_PITCH = 144;

__global__ __launch_bounds__(512) void indexer_prefill_kernel(IndexerParams p) {
    __shared__ __attribute__((aligned(16))) uint8_t ktile[PF_KT * PF_PITCH];
    __shared__ float kscale[PF_KT];

    const int b = blockIdx.z;
    const int q0 = p.cu_q[b];
    const int nq = p.cu_q[b + 1] - q0;
    const int tb = blockIdx.x * PF_ROWS;
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
    const int fill_end = p.fill_masked ? (c_end < ctx ? c_end : ctx) : comp_end;
    if (c0 >= fill_end) return;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int l = lane_id();

    // two query rows per wave
    i32x8 qa[2][4];
    float wq[2][4][4];
    int pos[2];
    bool valid[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int tl = tb + 2 * wave + r;
        valid[r] = tl < nq;
        pos[r] = p.pos0[b] + tl;
        load_query(p, (int64_t)(q0 + (valid[r] ? tl : tb)), valid[r], qa[r], wq[r]);
    }

    // register staging of the next key tile: 1024 16-byte chunks over 512 threads
    i32x4 stage[2];
    float sstage = 0.f;
    auto fetch = [&](int kbase) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int c = tid + 512 * r;
            const int key = c >> 3, byte = (c & 7) * 16;
            const bool in = kbase + key < comp_end;
            const i32x4 v = *reinterpret_cast<const i32x4 *>(p.k + (kv0 + (in ? kbase + key : c0)) * DI + byte);
            stage[r] = in ? v : i32x4{0, 0, 0, 0};
        }
        if (tid < PF_KT) sstage = (kbase + tid < comp_end) ? p.k_scale[kv0 + kbase + tid] : 0.f;
    };

    if (c0 < comp_end) fetch(c0);
    for (int kbase = c0; kbase < comp_end; kbase += PF_KT) {
        __syncthreads();
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int c = tid + 512 * r;
            *reinterpret_cast<i32x4 *>(&ktile[(c >> 3) * PF_PITCH + (c & 7) * 16]) = stage[r];
        }
        if (tid < PF_KT) kscale[tid] = sstage;
        __syncthreads();
        if (kbase + PF_KT < comp_end) fetch(kbase + PF_KT);

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
            if ((st & 3) == 3) {
                // lane l: key kbase + 16*(st-3) + l
                const int key = kbase + 16 * (st - 3) + l;
                const float ks = key < comp_end ? kscale[16 * (st - 3) + l] : 0.f;
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    const float v = reduce_scatter4(part[r]);
                    if (valid[r] && key < fill_end)
                        p.scores[(int64_t)(q0 + tb + 2 * wave + r) * p.ld + key] =
                            key <= pos[r] && key < comp_end ? v * ks : -INFINITY;
                }
            }
            // one pipeline stage per region: left free, the scheduler hoists
            // every block's MFMAs to the front and runs out of registers
            __builtin_amdgcn_sched_barrier(0);
        }
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
// loads (no registers held while they fly, no barriers), then reads each
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

// Direct-to-LDS loads (16 or 4 bytes per lane) from sbase + voff (scalar base,
// 32-bit lane offset) to LDS lds + size * lane.  Issued from asm: the
// compiler's wait insertion does not track them; the kernel waits with
// explicit vmcnt.  M0 must be written one instruction ahead of the load.
__device__ __forceinline__ void dma_b128(uint64_t sbase, uint32_t voff, const DSA_LDS void *lds) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(m0)
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

__global__ __launch_bounds__(64 * DC_WAVES) void indexer_decode_kernel(IndexerParams p) {
    __shared__ __attribute__((aligned(16))) uint8_t kst[DC_WAVES][DC_NBUF][DC_GROUP];
    __shared__ __attribute__((aligned(16))) float sst[DC_WAVES][DC_NBUF][64];
    const int t = blockIdx.x;
    const RowInfo ri = row_info(p.cu_q, p.cu_kv, p.pos0, p.B, p.total_kv, p.max_kv, t);
    const int c0 = blockIdx.y * p.key_chunk;
    const int c_end = c0 + p.key_chunk;
    const int comp_end = c_end < ri.nvis ? c_end : ri.nvis;
    const int fill_end = p.fill_masked ? (c_end < ri.ctx ? c_end : ri.ctx) : comp_end;
    if (c0 >= fill_end) return;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l = lane_id();
    i32x8 qa[4];
    float wq[4][4];
    load_query(p, t, true, qa, wq);

    const int row = l & 15, grp = l >> 4;
    const uint64_t kbase = uniform_u64((uint64_t)(uintptr_t)(p.k + ri.kv0 * DI));
    const uint64_t sbase = uniform_u64((uint64_t)(uintptr_t)(p.k_scale + ri.kv0));
    // Loads of group g0 into ring slot b.  Keys past the visible end load key
    // c0 instead (their scores are not stored), so that every group issues
    // exactly DC_LOADS loads, which the vmcnt waits below count on.
    auto issue = [&](int g0, int b) {
        // this wave's LDS reads of slot b (an earlier group) have completed
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int j = 0; j < 8; ++j) {   // keys 8j .. 8j+7 of the group, lane l: key 8j + l/8, bytes 16*(l%8)
            const int key = g0 + 8 * j + (l >> 3);
            const uint32_t kk = (uint32_t)(key < comp_end ? key : c0);
            dma_b128(kbase, kk * DI + 16 * (l & 7), (const DSA_LDS void *)&kst[wave][b][j * 1024]);
        }
        const int key = g0 + l;
        dma_b32(sbase, 4u * (uint32_t)(key < comp_end ? key : c0), (const DSA_LDS void *)&sst[wave][b][0]);
    };
    auto compute = [&](int g0, int b) {
        float part[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const uint8_t *kr = &kst[wave][b][(16 * st + row) * DI + 32 * grp];
            const i32x4 lo = *reinterpret_cast<const i32x4 *>(kr);
            const i32x4 hi = *reinterpret_cast<const i32x4 *>(kr + 16);
            const i32x8 kb = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            f32x4 c[4];
            block_mfma(qa, kb, c);
            part[st] = block_epilogue(c, wq);
        }
        const float v = reduce_scatter4(part);
        const float ks = sst[wave][b][l];
        const int key = g0 + l;
        if (key < fill_end) p.scores[(int64_t)t * p.ld + key] = key < comp_end ? v * ks : -INFINITY;
    };
    constexpr int STRIDE = 64 * DC_WAVES;
    int g0 = c0 + 64 * wave;
#pragma unroll
    for (int j = 0; j < DC_NBUF; ++j)
        if (g0 + j * STRIDE < fill_end) issue(g0 + j * STRIDE, j);
    for (int i = 0; g0 < fill_end; g0 += STRIDE, ++i) {
        // wait for this group's loads; the later groups' loads (at most
        // DC_NBUF - 1 groups, issued after this one) may still fly
        static_assert(DC_NBUF >= 1 && DC_NBUF <= 3, "vmcnt waits written for a ring of 1 to 3 groups");
        const int ahead = (fill_end - 1 - g0) / STRIDE;   // groups after this one
        const int fly = ahead < DC_NBUF - 1 ? ahead : DC_NBUF - 1;   // of them already issued
        if (fly >= 2)
            __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * DC_LOADS - 16) | (1 << 14));   // vmcnt(2 * DC_LOADS) = 18
        else if (fly == 1)
            __builtin_amdgcn_s_waitcnt(0x0F70 | DC_LOADS);   // vmcnt(DC_LOADS)
        else
            __builtin_amdgcn_s_waitcnt(0x0F70);              // vmcnt(0)
        const int b = i % DC_NBUF;
        compute(g0, b);
        if (g0 + DC_NBUF * STRIDE < fill_end) issue(g0 + DC_NBUF * STRIDE, b);
    }
}

hipError_t launch_indexer(const IndexerParams &p, int T, int max_q, bool decode_variant,
                          hipStream_t s) {
    if (T <= 0 || p.max_kv <= 0) return hipSuccess;
    const int nchunk = (p.max_kv + p.key_chunk - 1) / p.key_chunk;
    if (decode_variant) {
        hipLaunchKernelGGL(indexer_decode_kernel, dim3(T, nchunk), dim3(64 * DC_WAVES), 0, s, p);
    } else {
        const dim3 g((max_q + PF_ROWS - 1) / PF_ROWS, nchunk, p.B);
        hipLaunchKernelGGL(indexer_prefill_kernel, g, dim3(512), 0, s, p);
    }
    return hipGetLastError();
}

}  // namespace dsa
