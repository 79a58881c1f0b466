// topk.hip — exact per-row top-k selection of index scores on gfx950.
//
// Selection rule (page "Техотчёт DeepSeek-V3.2 (2025): разреженное внимание
// DSA и масштабирование RL", section "Отбор и основное внимание": keep the k
// key positions with the largest index scores of the query): the k largest
// fp32 scores among the row's visible columns, -0 == +0, ties to the lower
// column; all visible columns when there are at most k.  Output: the selected
// columns in ascending order, -1 padded.
//
// Method: scores become order-preserving uint32 keys staged in LDS; three
// histogram passes over 11, 11 and 10 key bits find the exact k-th largest
// key kappa and how many keys above it exist; one compaction pass in column
// order then emits every key > kappa and the lowest-column keys == kappa,
// using wave ballots and a block prefix sum, so the output is ascending.
// Rows longer than one 32768-column chunk: each chunk selects its exact local
// top-k candidates (key, column) into workspace; a merge workgroup runs the
// same select over the candidates.  The union of the chunk-local top-k sets
// contains the global top-k under the same total order, so the merge is exact.
#include "dsa_device.h"
#include "kernels.h"

namespace dsa {

namespace {

constexpr int TPB = 1024;           // threads per workgroup
constexpr int NWAVE = TPB / kWave;
constexpr int NBIN = 2048;

struct SelectShared {
    uint32_t hist[NBIN];
    uint32_t wsum_gt[NWAVE];
    uint32_t wsum_eq[NWAVE];
    uint32_t prefix;      // key bits fixed so far
    uint32_t rem;         // keys still needed inside the current prefix
    uint32_t count_gt;    // keys strictly above the threshold
    uint32_t base_gt;     // running compaction counters
    uint32_t base_eq;
};

// Block-wide exclusive scan of one value per thread (1024 threads).
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t *wtot, uint32_t &total) {
    const int l = lane_id(), w = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        uint32_t y = __shfl_up(x, d, 64);
        if (l >= d) x += y;
    }
    if (l == 63) wtot[w] = x;
    __syncthreads();
    uint32_t off = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NWAVE; ++i) {
        const uint32_t t = wtot[i];
        off += (i < w) ? t : 0u;
        tot += t;
    }
    total = tot;
    __syncthreads();
    return off + x - v;
}

// One radix pass: histogram of bits [shift, shift+width) of the keys whose
// bits above `shift+width` equal sh.prefix, then pick the bin holding the
// rem-th largest key.  Updates prefix / rem / count_gt in shared memory.
__device__ void radix_pass(const uint32_t *keys, int n, int shift, int width, SelectShared &sh) {
    const int tid = threadIdx.x;
    for (int i = tid; i < NBIN; i += TPB) sh.hist[i] = 0;
    __syncthreads();
    const uint32_t prefix = sh.prefix;
    const int hi_shift = shift + width;
    const uint32_t mask = (1u << width) - 1u;
    for (int i = tid; i < n; i += TPB) {
        const uint32_t key = keys[i];
        const bool match = hi_shift >= 32 || (key >> hi_shift) == prefix;
        if (match) atomicAdd(&sh.hist[(key >> shift) & mask], 1u);
    }
    __syncthreads();
    // thread i owns bins (2i+1, 2i) counted from the top: bin a = NBIN-1-2i, a-1
    const int a = NBIN - 1 - 2 * tid;
    const uint32_t ca = sh.hist[a], cb = sh.hist[a - 1];
    uint32_t total;
    const uint32_t above = block_excl_scan(ca + cb, sh.wsum_gt, total);
    const uint32_t rem = sh.rem;
    __syncthreads();
    if (above < rem && rem <= above + ca) {
        sh.prefix = (prefix << width) | (uint32_t)a;
        sh.rem = rem - above;
        sh.count_gt += above;
    } else if (above + ca < rem && rem <= above + ca + cb) {
        sh.prefix = (prefix << width) | (uint32_t)(a - 1);
        sh.rem = rem - above - ca;
        sh.count_gt += above + ca;
    }
    __syncthreads();
}

// Finds the exact k-th largest key kappa (returned) of keys[0..n), n > k,
// and leaves count_gt (# keys > kappa) and rem (# keys == kappa to take).
__device__ uint32_t select_threshold(const uint32_t *keys, int n, int k, SelectShared &sh) {
    if (threadIdx.x == 0) {
        sh.prefix = 0;
        sh.rem = (uint32_t)k;
        sh.count_gt = 0;
    }
    __syncthreads();
    radix_pass(keys, n, 21, 11, sh);
    radix_pass(keys, n, 10, 11, sh);
    radix_pass(keys, n, 0, 10, sh);
    return sh.prefix;
}

// Emits, in array order, every i with keys[i] > kappa plus the first `need_eq`
// i with keys[i] == kappa: emit(slot, i) with slot = rank among the emitted
// (slots >= limit are dropped; they cannot occur for a correct threshold).
template <class Emit>
__device__ void compact(const uint32_t *keys, int n, uint32_t kappa, uint32_t need_eq,
                        uint32_t limit, SelectShared &sh, Emit emit) {
    const int tid = threadIdx.x, l = lane_id(), w = tid >> 6;
    if (tid == 0) {
        sh.base_gt = 0;
        sh.base_eq = 0;
    }
    __syncthreads();
    const uint64_t lt_mask = (l == 0) ? 0ull : (~0ull >> (64 - l));
    for (int r0 = 0; r0 < n; r0 += TPB) {
        const int i = r0 + tid;
        const uint32_t key = i < n ? keys[i] : 0u;
        const bool gt = i < n && key > kappa;
        const bool eq = i < n && key == kappa;
        const uint64_t bg = __ballot(gt), be = __ballot(eq);
        if (l == 0) {
            sh.wsum_gt[w] = (uint32_t)__popcll(bg);
            sh.wsum_eq[w] = (uint32_t)__popcll(be);
        }
        __syncthreads();
        uint32_t og = sh.base_gt, oe = sh.base_eq, tg = 0, te = 0;
#pragma unroll
        for (int x = 0; x < NWAVE; ++x) {
            const uint32_t a = sh.wsum_gt[x], b = sh.wsum_eq[x];
            og += (x < w) ? a : 0u;
            oe += (x < w) ? b : 0u;
            tg += a;
            te += b;
        }
        const uint32_t gbefore = og + (uint32_t)__popcll(bg & lt_mask);
        const uint32_t ebefore = oe + (uint32_t)__popcll(be & lt_mask);
        if (gt || (eq && ebefore < need_eq)) {
            const uint32_t slot = gbefore + (ebefore < need_eq ? ebefore : need_eq);
            if (slot < limit) emit(slot, i);
        }
        __syncthreads();
        if (tid == 0) {
            sh.base_gt += tg;
            sh.base_eq += te;
        }
        __syncthreads();
    }
}

}  // namespace

// Grid: x = query row, y = chunk of the row.  Chunk c covers visible columns
// [c*TOPK_CHUNK, min((c+1)*TOPK_CHUNK, nvis)).
__global__ __launch_bounds__(TPB) void topk_chunk_kernel(TopkParams p) {
    __shared__ uint32_t keys[TOPK_CHUNK];
    __shared__ SelectShared sh;
    const int t = blockIdx.x, c = blockIdx.y, tid = threadIdx.x;
    const RowInfo ri = row_info(p.cu_q, p.cu_kv, p.pos0, p.B, p.total_kv, p.max_kv, t);
    const int n = ri.nvis, k = p.k;
    int32_t *out = p.idx + (int64_t)t * k;

    if (n <= k) {  // everything visible is selected
        if (c == 0)
            for (int j = tid; j < k; j += TPB) out[j] = j < n ? j : -1;
        return;
    }
    const int c0 = c * TOPK_CHUNK;
    if (c0 >= n) return;
    const int len = (n - c0) < TOPK_CHUNK ? (n - c0) : TOPK_CHUNK;
    const bool single = n <= TOPK_CHUNK;
    const float *row = p.scores + (int64_t)t * p.ld + c0;

    for (int i = tid; i < len; i += TPB) keys[i] = score_key(row[i]);
    __syncthreads();

    if (single) {
        const uint32_t kappa = select_threshold(keys, len, k, sh);
        const uint32_t need_eq = sh.rem;
        compact(keys, len, kappa, need_eq, (uint32_t)k, sh, [&](uint32_t slot, int i) { out[slot] = c0 + i; });
        return;
    }
    // multi-chunk row: local top-min(k, len) candidates of this chunk
    uint32_t *ck = p.cand_key + ((int64_t)t * p.nchunk + c) * k;
    int32_t *cp = p.cand_pos + ((int64_t)t * p.nchunk + c) * k;
    if (len <= k) {
        for (int j = tid; j < k; j += TPB) {
            ck[j] = j < len ? keys[j] : 0u;
            cp[j] = j < len ? c0 + j : -1;
        }
        return;
    }
    const uint32_t kappa = select_threshold(keys, len, k, sh);
    const uint32_t need_eq = sh.rem;
    compact(keys, len, kappa, need_eq, (uint32_t)k, sh, [&](uint32_t slot, int i) {
        ck[slot] = keys[i];
        cp[slot] = c0 + i;
    });
}

// Grid: x = query row.  Merges the chunk candidates of rows longer than one
// chunk.  Candidate blocks are in column order and padded with key 0 (below
// the key of every non-NaN score), so array order = column order.
__global__ __launch_bounds__(TPB) void topk_merge_kernel(TopkParams p) {
    __shared__ uint32_t keys[TOPK_MAX_CHUNKS * 2048];
    __shared__ SelectShared sh;
    const int t = blockIdx.x, tid = threadIdx.x;
    const RowInfo ri = row_info(p.cu_q, p.cu_kv, p.pos0, p.B, p.total_kv, p.max_kv, t);
    const int n = ri.nvis, k = p.k;
    if (n <= k || n <= TOPK_CHUNK) return;
    const int nch = (n + TOPK_CHUNK - 1) / TOPK_CHUNK;
    const int m = nch * k;
    const uint32_t *ck = p.cand_key + (int64_t)t * p.nchunk * k;
    const int32_t *cp = p.cand_pos + (int64_t)t * p.nchunk * k;
    for (int i = tid; i < m; i += TPB) keys[i] = ck[i];
    __syncthreads();
    const uint32_t kappa = select_threshold(keys, m, k, sh);
    const uint32_t need_eq = sh.rem;
    int32_t *out = p.idx + (int64_t)t * k;
    compact(keys, m, kappa, need_eq, (uint32_t)k, sh, [&](uint32_t slot, int i) { out[slot] = cp[i]; });
}

hipError_t launch_topk(const TopkParams &p, int T, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    dim3 g1(T, p.nchunk);
    hipLaunchKernelGGL(topk_chunk_kernel, g1, dim3(TPB), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.nchunk <= 1) return e;
    hipLaunchKernelGGL(topk_merge_kernel, dim3(T), dim3(TPB), 0, s, p);
    return hipGetLastError();
}

}  // namespace dsa
