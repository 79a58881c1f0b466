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
// waves split the chunk and stream their keys straight from HBM into the B
// operand registers, one 64-key group ahead (a key is used by a single query
// row, so staging it in LDS would buy nothing).  Grid: x = query row, y = key
// chunk.
// ---------------------------------------------------------------------------
constexpr int DC_WAVES = 4;

__global__ __launch_bounds__(256) void indexer_decode_kernel(IndexerParams p) {
    const int t = blockIdx.x;
    const RowInfo ri = row_info(p.cu_q, p.cu_kv, p.pos0, p.B, p.total_kv, p.max_kv, t);
    const int c0 = blockIdx.y * p.key_chunk;
    const int c_end = c0 + p.key_chunk;
    const int comp_end = c_end < ri.nvis ? c_end : ri.nvis;
    const int fill_end = p.fill_masked ? (c_end < ri.ctx ? c_end : ri.ctx) : comp_end;
    if (c0 >= fill_end) return;

    const int wave = threadIdx.x >> 6;
    const int l = lane_id();
    i32x8 qa[4];
    float wq[4][4];
    load_query(p, t, true, qa, wq);

    // Wave w takes the 64-key groups w, w+4, ... of the chunk; the keys of
    // the next group are loaded (straight from HBM into B operands) before
    // the current group is computed.
    const int row = l & 15, grp = l >> 4;
    auto kload = [&](int g0, i32x8 (&kb)[4], float &ks) {
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const int key = g0 + 16 * st + row;
            const bool in = key < comp_end;
            const i32x4 *s4 = reinterpret_cast<const i32x4 *>(p.k + (ri.kv0 + (in ? key : c0)) * DI + 32 * grp);
            const i32x4 lo = s4[0], hi = s4[1];
            kb[st] = in ? i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]}
                        : i32x8{0, 0, 0, 0, 0, 0, 0, 0};
        }
        const int key = g0 + l;
        ks = key < comp_end ? p.k_scale[ri.kv0 + key] : 0.f;
    };
    auto compute = [&](int g0, const i32x8 (&kb)[4], float ks) {
        float part[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            f32x4 c[4];
            block_mfma(qa, kb[st], c);
            part[st] = block_epilogue(c, wq);
        }
        const float v = reduce_scatter4(part);
        const int key = g0 + l;
        if (key < fill_end) p.scores[(int64_t)t * p.ld + key] = key < comp_end ? v * ks : -INFINITY;
    };
    constexpr int STRIDE = 64 * DC_WAVES;
    i32x8 kA[4], kB[4];
    float sA = 0.f, sB = 0.f;
    int g0 = c0 + 64 * wave;
    if (g0 < fill_end) kload(g0, kA, sA);
    // unrolled by two so that both key buffers stay in registers
    for (; g0 < fill_end; g0 += 2 * STRIDE) {
        if (g0 + STRIDE < fill_end) kload(g0 + STRIDE, kB, sB);
        compute(g0, kA, sA);
        if (g0 + STRIDE >= fill_end) break;
        if (g0 + 2 * STRIDE < fill_end) kload(g0 + 2 * STRIDE, kA, sA);
        compute(g0 + STRIDE, kB, sB);
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
