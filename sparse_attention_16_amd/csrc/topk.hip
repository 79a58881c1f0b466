// topk.hip — exact per-row top-k selection of index scores on gfx950.
//
// Selection rule (page "Техотчёт DeepSeek-V3.2 (2025): разреженное внимание
// DSA и масштабирование RL", section "Отбор и основное внимание": keep the k
// key positions with the largest index scores of the query): the k largest
// fp32 scores among the row's visible columns, -0 == +0, ties to the lower
// column; all visible columns when there are at most k.  Output: the selected
// columns in ascending order, -1 padded.
//
// Method: scores become order-preserving uint32 keys staged in LDS.  While
// they are loaded (16-byte loads), a histogram of the top 11 key bits is
// built; its scan names the bin holding the k-th largest key.  One pass over
// the staged keys copies that bin's keys (a few percent of the row) into a
// candidate list, and two more histogram passes of 11 and 10 bits over the
// candidates give the exact k-th largest key kappa and the number of keys
// above it.  (A bin too large for the candidate list - e.g. a row of equal
// scores - runs those two passes over the whole row instead.)  A compaction
// pass in column order then emits every key > kappa and the lowest-column
// keys == kappa, using wave ballots and a block prefix sum, so the output is
// ascending with no sort.
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
constexpr int NBIN = 2048;          // 11-bit digits; the bin scan needs NBIN == 2 * TPB
constexpr int CAND_CAP = 4096;      // keys of the threshold bin kept for the fine passes

struct SelectShared {
    uint32_t hist[NBIN];
    uint32_t wsum_gt[NWAVE];
    uint32_t wsum_eq[NWAVE];
    uint32_t prefix;      // key bits fixed so far
    uint32_t rem;         // keys still needed inside the current prefix
    uint32_t count_gt;    // keys strictly above the threshold
    uint32_t base_gt;     // running compaction counters
    uint32_t base_eq;
    uint32_t ncand;       // keys copied to the candidate list
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

__device__ __forceinline__ void init_select(SelectShared &sh, int k) {
    for (int i = threadIdx.x; i < NBIN; i += TPB) sh.hist[i] = 0;
    if (threadIdx.x == 0) {
        sh.prefix = 0;
        sh.rem = (uint32_t)k;
        sh.count_gt = 0;
        sh.ncand = 0;
    }
}

// From the histogram in sh.hist (digit of `width` bits below sh.prefix), picks
// the bin holding the rem-th largest key; appends it to prefix and updates
// rem / count_gt.
__device__ void pick_bin(int width, SelectShared &sh) {
    const int tid = threadIdx.x;
    // thread i owns bins (2i+1, 2i) counted from the top: bin a = NBIN-1-2i, a-1
    const int a = NBIN - 1 - 2 * tid;
    const uint32_t ca = sh.hist[a], cb = sh.hist[a - 1];
    uint32_t total;
    const uint32_t above = block_excl_scan(ca + cb, sh.wsum_gt, total);
    const uint32_t rem = sh.rem, prefix = sh.prefix;
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

// One radix pass over keys[0..n): histogram of bits [shift, shift+width) of
// the keys whose bits above shift+width equal sh.prefix, then pick_bin.
__device__ void radix_pass(const uint32_t *keys, int n, int shift, int width, SelectShared &sh) {
    const int tid = threadIdx.x;
    for (int i = tid; i < NBIN; i += TPB) sh.hist[i] = 0;
    __syncthreads();
    const uint32_t prefix = sh.prefix;
    const int hi_shift = shift + width;
    const uint32_t mask = (1u << width) - 1u;
    for (int i = tid; i < n; i += TPB) {
        const uint32_t key = keys[i];
        if ((key >> hi_shift) == prefix) atomicAdd(&sh.hist[(key >> shift) & mask], 1u);
    }
    __syncthreads();
    pick_bin(width, sh);
}

// Stages score_key(row[0..n)) into keys[] and adds the top 11 bits of every
// key to sh.hist (which must be zero).  keys must be 16-byte aligned.
__device__ __forceinline__ void stage_keys(const float *row, int n, uint32_t *keys, SelectShared &sh) {
    const int tid = threadIdx.x;
    if ((reinterpret_cast<uintptr_t>(row) & 15) == 0) {
        const int n4 = n >> 2;
        const float4 *r4 = reinterpret_cast<const float4 *>(row);
        for (int b = 0; b < n4; b += 8 * TPB) {
            float4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int j = b + u * TPB + tid;
                v[u] = j < n4 ? r4[j] : float4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int j = b + u * TPB + tid;
                if (j < n4) {
                    const uint32_t k0 = score_key(v[u].x), k1 = score_key(v[u].y);
                    const uint32_t k2 = score_key(v[u].z), k3 = score_key(v[u].w);
                    *reinterpret_cast<uint4 *>(&keys[4 * j]) = uint4{k0, k1, k2, k3};
                    atomicAdd(&sh.hist[k0 >> 21], 1u);
                    atomicAdd(&sh.hist[k1 >> 21], 1u);
                    atomicAdd(&sh.hist[k2 >> 21], 1u);
                    atomicAdd(&sh.hist[k3 >> 21], 1u);
                }
            }
        }
        for (int i = 4 * n4 + tid; i < n; i += TPB) {
            const uint32_t key = score_key(row[i]);
            keys[i] = key;
            atomicAdd(&sh.hist[key >> 21], 1u);
        }
    } else {
        for (int i = tid; i < n; i += TPB) {
            const uint32_t key = score_key(row[i]);
            keys[i] = key;
            atomicAdd(&sh.hist[key >> 21], 1u);
        }
    }
}

// Given the top-11-bit histogram of keys[0..n) in sh.hist (n > k), finds the
// exact k-th largest key kappa (returned) and leaves count_gt (# keys > kappa)
// and rem (# keys == kappa to take).  cand: scratch for CAND_CAP keys.
__device__ uint32_t select_threshold(const uint32_t *keys, int n, SelectShared &sh,
                                     uint32_t *cand) {
    __syncthreads();
    pick_bin(11, sh);
    const uint32_t b1 = sh.prefix;
    const int l = lane_id();
    const uint64_t lt_mask = (l == 0) ? 0ull : (~0ull >> (64 - l));
    // copy the keys of bin b1 to the candidate list (order is irrelevant here)
    for (int i0 = 0; i0 < n; i0 += TPB) {
        const int i = i0 + threadIdx.x;
        const uint32_t key = i < n ? keys[i] : 0u;
        const bool m = i < n && (key >> 21) == b1;
        const uint64_t bm = __ballot(m);
        if (bm) {
            uint32_t base = 0;
            if (l == 0) base = atomicAdd(&sh.ncand, (uint32_t)__popcll(bm));
            base = __shfl(base, 0, kWave);
            const uint32_t pos = base + (uint32_t)__popcll(bm & lt_mask);
            if (m && pos < CAND_CAP) cand[pos] = key;
        }
    }
    __syncthreads();
    const uint32_t nc = sh.ncand;
    if (nc <= CAND_CAP) {
        radix_pass(cand, (int)nc, 10, 11, sh);
        radix_pass(cand, (int)nc, 0, 10, sh);
    } else {
        radix_pass(keys, n, 10, 11, sh);
        radix_pass(keys, n, 0, 10, sh);
    }
    return sh.prefix;
}

// Emits, in array order, every i with keys[i] > kappa plus the first `need_eq`
// i with keys[i] == kappa: emit(slot, i) with slot = rank among the emitted
// (slots >= limit are dropped; they cannot occur for a correct threshold).
// Each thread takes 4 consecutive keys per round (keys 16-byte aligned).
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
    for (int r0 = 0; r0 < n; r0 += 4 * TPB) {
        const int i0 = r0 + 4 * tid;
        const uint4 kk = i0 < n ? *reinterpret_cast<const uint4 *>(&keys[i0]) : uint4{0u, 0u, 0u, 0u};
        const uint32_t kv[4] = {kk.x, kk.y, kk.z, kk.w};
        bool gt[4], eq[4];
        uint32_t gb = 0, eb = 0, gtot = 0, etot = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            gt[u] = i0 + u < n && kv[u] > kappa;
            eq[u] = i0 + u < n && kv[u] == kappa;
            const uint64_t bg = __ballot(gt[u]), be = __ballot(eq[u]);
            gb += (uint32_t)__popcll(bg & lt_mask);
            eb += (uint32_t)__popcll(be & lt_mask);
            gtot += (uint32_t)__popcll(bg);
            etot += (uint32_t)__popcll(be);
        }
        if (l == 0) {
            sh.wsum_gt[w] = gtot;
            sh.wsum_eq[w] = etot;
        }
        __syncthreads();
        uint32_t g = sh.base_gt + gb, e = sh.base_eq + eb, tg = 0, te = 0;
#pragma unroll
        for (int x = 0; x < NWAVE; ++x) {
            const uint32_t a = sh.wsum_gt[x], b = sh.wsum_eq[x];
            g += (x < w) ? a : 0u;
            e += (x < w) ? b : 0u;
            tg += a;
            te += b;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (gt[u] || (eq[u] && e < need_eq)) {
                const uint32_t slot = g + (e < need_eq ? e : need_eq);
                if (slot < limit) emit(slot, i0 + u);
            }
            g += gt[u] ? 1u : 0u;
            e += eq[u] ? 1u : 0u;
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
    __shared__ __attribute__((aligned(16))) uint32_t keys[TOPK_CHUNK];
    __shared__ __attribute__((aligned(16))) uint32_t cand[CAND_CAP];
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

    init_select(sh, k);
    __syncthreads();
    stage_keys(row, len, keys, sh);

    if (single) {
        const uint32_t kappa = select_threshold(keys, len, sh, cand);
        const uint32_t need_eq = sh.rem;
        compact(keys, len, kappa, need_eq, (uint32_t)k, sh, [&](uint32_t slot, int i) { out[slot] = c0 + i; });
        return;
    }
    // multi-chunk row: local top-min(k, len) candidates of this chunk
    uint32_t *ck = p.cand_key + ((int64_t)t * p.nchunk + c) * k;
    int32_t *cp = p.cand_pos + ((int64_t)t * p.nchunk + c) * k;
    if (len <= k) {
        __syncthreads();
        for (int j = tid; j < k; j += TPB) {
            ck[j] = j < len ? keys[j] : 0u;
            cp[j] = j < len ? c0 + j : -1;
        }
        return;
    }
    const uint32_t kappa = select_threshold(keys, len, sh, cand);
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
    __shared__ __attribute__((aligned(16))) uint32_t keys[TOPK_MAX_CHUNKS * 2048];
    __shared__ __attribute__((aligned(16))) uint32_t cand[CAND_CAP];
    __shared__ SelectShared sh;
    const int t = blockIdx.x, tid = threadIdx.x;
    const RowInfo ri = row_info(p.cu_q, p.cu_kv, p.pos0, p.B, p.total_kv, p.max_kv, t);
    const int n = ri.nvis, k = p.k;
    if (n <= k || n <= TOPK_CHUNK) return;
    const int nch = (n + TOPK_CHUNK - 1) / TOPK_CHUNK;
    const int m = nch * k;
    const uint32_t *ck = p.cand_key + (int64_t)t * p.nchunk * k;
    const int32_t *cp = p.cand_pos + (int64_t)t * p.nchunk * k;
    init_select(sh, k);
    __syncthreads();
    for (int i = tid; i < m; i += TPB) {
        const uint32_t key = ck[i];
        keys[i] = key;
        atomicAdd(&sh.hist[key >> 21], 1u);
    }
    const uint32_t kappa = select_threshold(keys, m, sh, cand);
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
