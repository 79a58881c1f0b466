// topk.hip — exact per-row top-k selection of index scores on gfx950.
//
// Selection rule (page "Техотчёт DeepSeek-V3.2 (2025): разреженное внимание
// DSA и масштабирование RL", section "Отбор и основное внимание": keep the k
// key positions with the largest index scores of the query): the k largest
// fp32 scores among the row's visible columns, -0 == +0, ties to the lower
// column; all visible columns when there are at most k.  Output: the selected
// columns in ascending order, -1 padded.
//
// Method (one workgroup per row chunk, keys staged in LDS):
//   1. stage   : scores -> order-preserving uint32 keys in LDS (16-byte
//                loads issued one chunk ahead), building a histogram of the
//                top 11 key bits on the way; its scan names the bin b1 that
//                holds the k-th largest key.
//   2. extract : each wave walks its own contiguous column segment, counts
//                the keys above bin b1 and copies the keys of bin b1 (a few
//                percent of the row) into its own candidate region.  Wave-
//                local running offsets come from ballots: no atomics.
//   3. refine  : two histogram passes of 11 and 10 bits over the candidates
//                give the exact k-th largest key kappa and how many keys equal
//                to kappa are taken.  (If bin b1 overflows the candidate
//                regions - e.g. a row of equal scores - these passes run over
//                the whole row instead.)
//   4. emit    : per wave, the number of keys > kappa and == kappa in its
//                segment gives (through one block prefix) its first output
//                slot; the wave then walks its segment in column order and
//                writes every key > kappa and the lowest-column keys ==
//                kappa.  The output is ascending with no sort.
// Rows longer than one 32768-column chunk: each chunk selects its exact local
// top-k candidates (key, column) into workspace; a merge workgroup runs the
// same select over the candidates.  The union of the chunk-local top-k sets
// contains the global top-k under the same total order, so the merge is exact.
#include "dsa_device.h"
#include "kernels.h"

namespace dsa {

namespace {

constexpr int TPB = 512;            // threads per workgroup
constexpr int NWAVE = TPB / kWave;
constexpr int NBIN = 2048;          // 11-bit digits
constexpr int BPT = NBIN / TPB;     // histogram bins scanned per thread
constexpr int CAP_W = 512;          // candidate keys per wave
constexpr int CAND_CAP = CAP_W * NWAVE;
constexpr int SEG_ALIGN = 4 * kWave;  // a wave step covers 256 columns
static_assert(NBIN % TPB == 0, "bins per thread");

struct SelectShared {
    uint32_t hist[NBIN];
    uint32_t wtot[NWAVE];     // scan scratch
    uint32_t wnc[NWAVE];      // candidates found by each wave
    uint32_t wabove[NWAVE];   // keys above bin b1 in each wave's segment
    uint32_t wgt[NWAVE];      // keys > kappa in each wave's segment
    uint32_t weq[NWAVE];      // keys == kappa in each wave's segment
    uint32_t prefix;          // key bits fixed so far
    uint32_t rem;             // keys still needed inside the current prefix
};

__device__ __forceinline__ uint64_t lanes_below() {
    const int l = lane_id();
    return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// Block-wide exclusive scan of one value per thread.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t *wtot) {
    const int l = lane_id(), w = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        uint32_t y = __shfl_up(x, d, 64);
        if (l >= d) x += y;
    }
    if (l == 63) wtot[w] = x;
    lds_barrier();
    uint32_t off = 0;
#pragma unroll
    for (int i = 0; i < NWAVE; ++i) off += (i < w) ? wtot[i] : 0u;
    lds_barrier();
    return off + x - v;
}

__device__ __forceinline__ void init_select(SelectShared &sh, int k) {
    for (int i = threadIdx.x; i < NBIN; i += TPB) sh.hist[i] = 0;
    if (threadIdx.x == 0) {
        sh.prefix = 0;
        sh.rem = (uint32_t)k;
    }
}

// From the histogram in sh.hist (digit of `width` bits below sh.prefix), picks
// the bin holding the rem-th largest key; appends it to prefix, updates rem.
__device__ void pick_bin(int width, SelectShared &sh) {
    const int tid = threadIdx.x;
    // thread i owns the BPT bins top, top-1, ... counted from the top
    const int top = NBIN - 1 - BPT * tid;
    uint32_t c[BPT], sum = 0;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
        c[i] = sh.hist[top - i];
        sum += c[i];
    }
    const uint32_t above = block_excl_scan(sum, sh.wtot);
    const uint32_t rem = sh.rem, prefix = sh.prefix;
    lds_barrier();
    uint32_t acc = above;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
        if (acc < rem && rem <= acc + c[i]) {
            sh.prefix = (prefix << width) | (uint32_t)(top - i);
            sh.rem = rem - acc;
        }
        acc += c[i];
    }
    lds_barrier();
}

// Histogram pass over the keys accepted by `get(i, key)` for i in [0, n):
// bits [shift, shift+width) of the keys whose bits above equal sh.prefix.
template <class Get>
__device__ void radix_pass(int n, int shift, int width, SelectShared &sh, Get get) {
    const int tid = threadIdx.x;
    for (int i = tid; i < NBIN; i += TPB) sh.hist[i] = 0;
    lds_barrier();
    const uint32_t prefix = sh.prefix;
    const int hi_shift = shift + width;
    const uint32_t mask = (1u << width) - 1u;
    for (int i = tid; i < n; i += TPB) {
        uint32_t key;
        if (get(i, key) && (key >> hi_shift) == prefix)
            atomicAdd(&sh.hist[(key >> shift) & mask], 1u);
    }
    lds_barrier();
    pick_bin(width, sh);
}

// Column segment of wave w: [s0, s1), a multiple of 256 columns long.
__device__ __forceinline__ void wave_segment(int n, int w, int &s0, int &s1) {
    const int per = (n + NWAVE - 1) / NWAVE;
    const int seg = (per + SEG_ALIGN - 1) / SEG_ALIGN * SEG_ALIGN;
    s0 = w * seg < n ? w * seg : n;
    s1 = s0 + seg < n ? s0 + seg : n;
}

// Loads the 4 keys at columns i0..i0+3 (i0 a multiple of 4; zeros when i0 is
// past the segment).  Callers mask columns >= s1 themselves.
__device__ __forceinline__ uint4 load4(const uint32_t *keys, int i0, int s1) {
    return i0 < s1 ? *reinterpret_cast<const uint4 *>(&keys[i0]) : uint4{0u, 0u, 0u, 0u};
}

// Steps 2-4 for keys[0..n), n > k, whose top-11-bit histogram is in sh.hist
// (the caller's last LDS writes need not be fenced yet).  keys must be 16-byte
// aligned and readable up to the next multiple of 4 past n.  Calls
// emit(slot, i) for the k selected positions i, slot = rank in column order.
template <class Emit>
__device__ void select_emit(const uint32_t *keys, int n, int k, SelectShared &sh,
                            uint32_t *cand, Emit emit) {
    const int l = lane_id(), w = threadIdx.x >> 6;
    const uint64_t lt = lanes_below();
    lds_barrier();
    pick_bin(11, sh);
    const uint32_t b1 = sh.prefix;
    int s0, s1;
    wave_segment(n, w, s0, s1);

    // 2. extract: candidates of bin b1 into this wave's region, keys above b1 counted
    uint32_t *mine = cand + w * CAP_W;
    uint32_t run = 0, above = 0;
    for (int b = s0; b < s1; b += SEG_ALIGN) {
        const int i0 = b + 4 * l;
        const uint4 kk = load4(keys, i0, s1);
        const uint32_t kv[4] = {kk.x, kk.y, kk.z, kk.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const bool ok = i0 + u < s1;
            const uint32_t bin = kv[u] >> 21;
            const bool m = ok && bin == b1;
            const uint64_t bm = __ballot(m);
            above += (uint32_t)__popcll(__ballot(ok && bin > b1));
            const uint32_t pos = run + (uint32_t)__popcll(bm & lt);
            if (m && pos < CAP_W) mine[pos] = kv[u];
            run += (uint32_t)__popcll(bm);
        }
    }
    if (l == 0) {
        sh.wnc[w] = run;
        sh.wabove[w] = above;
    }
    lds_barrier();
    bool overflow = false;
#pragma unroll
    for (int x = 0; x < NWAVE; ++x) overflow |= sh.wnc[x] > CAP_W;

    // 3. refine: exact kappa
    uint32_t kappa, need_eq;
    if (!overflow) {
        auto get = [&](int i, uint32_t &key) {
            const int r = i / CAP_W, j = i - r * CAP_W;
            key = cand[i];
            return (uint32_t)j < sh.wnc[r];
        };
        radix_pass(CAND_CAP, 10, 11, sh, get);
        radix_pass(CAND_CAP, 0, 10, sh, get);
    } else {
        auto get = [&](int i, uint32_t &key) {
            key = keys[i];
            return true;
        };
        radix_pass(n, 10, 11, sh, get);
        radix_pass(n, 0, 10, sh, get);
    }
    kappa = sh.prefix;
    need_eq = sh.rem;

    // 4. emit: per-wave counts -> first slots -> ordered walk of the segment
    uint32_t gt = 0, eq = 0;
    if (!overflow) {
        gt = sh.wabove[w];  // every key above bin b1 is > kappa
        const uint32_t nc = sh.wnc[w];
        for (uint32_t j = l; j < ((nc + 63u) & ~63u); j += 64) {
            const uint32_t key = j < nc ? mine[j] : 0u;
            gt += (uint32_t)__popcll(__ballot(j < nc && key > kappa));
            eq += (uint32_t)__popcll(__ballot(j < nc && key == kappa));
        }
    } else {
        for (int b = s0; b < s1; b += SEG_ALIGN) {
            const int i0 = b + 4 * l;
            const uint4 kk = load4(keys, i0, s1);
            const uint32_t kv[4] = {kk.x, kk.y, kk.z, kk.w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const bool ok = i0 + u < s1;
                gt += (uint32_t)__popcll(__ballot(ok && kv[u] > kappa));
                eq += (uint32_t)__popcll(__ballot(ok && kv[u] == kappa));
            }
        }
    }
    if (l == 0) {
        sh.wgt[w] = gt;
        sh.weq[w] = eq;
    }
    lds_barrier();
    uint32_t g_run = 0, e_run = 0;
#pragma unroll
    for (int x = 0; x < NWAVE; ++x) {
        g_run += (x < w) ? sh.wgt[x] : 0u;
        e_run += (x < w) ? sh.weq[x] : 0u;
    }
    for (int b = s0; b < s1; b += SEG_ALIGN) {
        const int i0 = b + 4 * l;
        const uint4 kk = load4(keys, i0, s1);
        const uint32_t kv[4] = {kk.x, kk.y, kk.z, kk.w};
        bool fg[4], fe[4];
        uint32_t gb = 0, eb = 0, gtot = 0, etot = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const bool ok = i0 + u < s1;
            fg[u] = ok && kv[u] > kappa;
            fe[u] = ok && kv[u] == kappa;
            const uint64_t bg = __ballot(fg[u]), be = __ballot(fe[u]);
            gb += (uint32_t)__popcll(bg & lt);
            eb += (uint32_t)__popcll(be & lt);
            gtot += (uint32_t)__popcll(bg);
            etot += (uint32_t)__popcll(be);
        }
        uint32_t g = g_run + gb, e = e_run + eb;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (fg[u] || (fe[u] && e < need_eq)) {
                const uint32_t slot = g + (e < need_eq ? e : need_eq);
                if (slot < (uint32_t)k) emit(slot, i0 + u);
            }
            g += fg[u] ? 1u : 0u;
            e += fe[u] ? 1u : 0u;
        }
        g_run += gtot;
        e_run += etot;
    }
    lds_barrier();  // LDS (keys, candidates, counters) free for the next select
}

// Keys are staged through registers: a workgroup issues the 16-byte loads of
// its next chunk before it selects the current one, so HBM latency overlaps
// the LDS work.  PF float4 per thread cover one 32768-column chunk.
constexpr int PF = TOPK_CHUNK / (4 * TPB);

struct ChunkItem {
    int t, c;          // query row, chunk of the row
    int n;             // visible columns of the row
    int c0, len;       // first column and length of the chunk (len 0: nothing to stage)
    int n4;            // float4 loads (0 when the row is not 16-byte aligned)
    const float *row;  // scores of the chunk
};

__device__ __forceinline__ ChunkItem chunk_item(const TopkParams &p, int item) {
    ChunkItem it;
    it.t = item / p.nchunk;
    it.c = item - it.t * p.nchunk;
    const RowInfo ri = row_info(p.cu_q, p.cu_kv, p.pos0, p.B, p.total_kv, p.max_kv, it.t);
    it.n = ri.nvis;
    it.c0 = it.c * TOPK_CHUNK;
    it.len = (it.n > p.k && it.c0 < it.n) ? ((it.n - it.c0) < TOPK_CHUNK ? it.n - it.c0 : TOPK_CHUNK) : 0;
    it.row = p.scores + (int64_t)it.t * p.ld + it.c0;
    it.n4 = (reinterpret_cast<uintptr_t>(it.row) & 15) == 0 ? it.len >> 2 : 0;
    return it;
}

__device__ __forceinline__ void prefetch(const ChunkItem &it, float4 (&v)[PF]) {
    const float4 *r4 = reinterpret_cast<const float4 *>(it.row);
#pragma unroll
    for (int u = 0; u < PF; ++u) {
        const int j = u * TPB + threadIdx.x;
        v[u] = j < it.n4 ? r4[j] : float4{0.f, 0.f, 0.f, 0.f};
    }
}

// Writes score_key of the chunk into keys[] and adds the top 11 bits of every
// key to sh.hist (which must be zero).
__device__ __forceinline__ void stage_keys(const ChunkItem &it, const float4 (&v)[PF],
                                           uint32_t *keys, SelectShared &sh) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int u = 0; u < PF; ++u) {
        const int j = u * TPB + tid;
        if (j < it.n4) {
            const uint32_t k0 = score_key(v[u].x), k1 = score_key(v[u].y);
            const uint32_t k2 = score_key(v[u].z), k3 = score_key(v[u].w);
            *reinterpret_cast<uint4 *>(&keys[4 * j]) = uint4{k0, k1, k2, k3};
            atomicAdd(&sh.hist[k0 >> 21], 1u);
            atomicAdd(&sh.hist[k1 >> 21], 1u);
            atomicAdd(&sh.hist[k2 >> 21], 1u);
            atomicAdd(&sh.hist[k3 >> 21], 1u);
        }
    }
    for (int i = 4 * it.n4 + tid; i < it.len; i += TPB) {
        const uint32_t key = score_key(it.row[i]);
        keys[i] = key;
        atomicAdd(&sh.hist[key >> 21], 1u);
    }
}

}  // namespace

// Persistent: workgroup g takes the (row, chunk) items g, g + gridDim.x, ...
// of the T * nchunk items (item = row * nchunk + chunk).  Chunk c covers
// visible columns [c*TOPK_CHUNK, min((c+1)*TOPK_CHUNK, nvis)).  The loads of
// the next item are issued before the current one is selected.
__global__ __launch_bounds__(TPB) void topk_chunk_kernel(TopkParams p, int nitems) {
    __shared__ __attribute__((aligned(16))) uint32_t keys[TOPK_CHUNK];
    __shared__ __attribute__((aligned(16))) uint32_t cand[CAND_CAP];
    __shared__ SelectShared sh;
    const int tid = threadIdx.x, k = p.k;
    int item = blockIdx.x;
    if (item >= nitems) return;
    ChunkItem nxt = chunk_item(p, item);
    float4 v[PF];
    prefetch(nxt, v);
    for (; item < nitems; item += gridDim.x) {
        const ChunkItem it = nxt;
        int32_t *out = p.idx + (int64_t)it.t * k;
        if (it.len > 0) {
            init_select(sh, k);
            lds_barrier();
            stage_keys(it, v, keys, sh);
        }
        if (item + (int)gridDim.x < nitems) {
            nxt = chunk_item(p, item + gridDim.x);
            prefetch(nxt, v);
        }
        if (it.n <= k) {  // everything visible is selected
            if (it.c == 0)
                for (int j = tid; j < k; j += TPB) out[j] = j < it.n ? j : -1;
            continue;
        }
        if (it.len == 0) continue;  // chunk past the visible end
        const int c0 = it.c0, len = it.len;
        if (it.n <= TOPK_CHUNK) {
            select_emit(keys, len, k, sh, cand, [&](uint32_t slot, int i) { out[slot] = c0 + i; });
            continue;
        }
        // multi-chunk row: local top-min(k, len) candidates of this chunk
        uint32_t *ck = p.cand_key + ((int64_t)it.t * p.nchunk + it.c) * k;
        int32_t *cp = p.cand_pos + ((int64_t)it.t * p.nchunk + it.c) * k;
        if (len <= k) {
            lds_barrier();
            for (int j = tid; j < k; j += TPB) {
                ck[j] = j < len ? keys[j] : 0u;
                cp[j] = j < len ? c0 + j : -1;
            }
            lds_barrier();
            continue;
        }
        select_emit(keys, len, k, sh, cand, [&](uint32_t slot, int i) {
            ck[slot] = keys[i];
            cp[slot] = c0 + i;
        });
    }
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
    lds_barrier();
    for (int i = tid; i < m; i += TPB) {
        const uint32_t key = ck[i];
        keys[i] = key;
        atomicAdd(&sh.hist[key >> 21], 1u);
    }
    int32_t *out = p.idx + (int64_t)t * k;
    select_emit(keys, m, k, sh, cand, [&](uint32_t slot, int i) { out[slot] = cp[i]; });
}

hipError_t launch_topk(const TopkParams &p, int T, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    // one resident workgroup per compute unit (the keys fill most of the LDS)
    static int ncu = 0;
    if (ncu == 0) {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        ncu = n;
    }
    const int64_t items64 = (int64_t)T * p.nchunk;
    if (items64 > INT32_MAX) return hipErrorInvalidValue;
    const int nitems = (int)items64;
    const int grid = nitems < ncu ? nitems : ncu;
    hipLaunchKernelGGL(topk_chunk_kernel, dim3(grid), dim3(TPB), 0, s, p, nitems);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.nchunk <= 1) return e;
    hipLaunchKernelGGL(topk_merge_kernel, dim3(T), dim3(TPB), 0, s, p);
    return hipGetLastError();
}

}  // namespace dsa
