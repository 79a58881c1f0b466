// topk.hip — exact per-row top-k selection of index scores on gfx950.
//
// Selection rule (page "Техотчёт DeepSeek-V3.2 (2025): разреженное внимание
// DSA и масштабирование RL", section "Отбор и основное внимание": keep the k
// key positions with the largest index scores of the query): the k largest
// fp32 scores among the row's visible columns, -0 == +0, ties to the lower
// column; all visible columns when there are at most k.  Output: the selected
// columns in ascending order, -1 padded.
//
// Method (one 1024-thread workgroup per row chunk of up to 32768 columns; the
// chunk's scores stay in registers as order-preserving uint32 keys, thread t
// holding the 4G consecutive columns 4Gt .. 4Gt + 4G - 1):
//   1. range   : block minimum and maximum of the chunk's scores.
//   2. bin     : a 2048-bin histogram of the scores, binned by value over
//                [min, max] (a non-decreasing map, so bins keep the order);
//                a scan from the top names the bin b1 holding the k-th
//                largest key.
//   3. classify: two key thresholds a quarter bin outside b1, each checked
//                with the histogram's own bin arithmetic, split the keys:
//                those above the upper one are selected outright, those
//                below the lower one are not, and the few in between (b1
//                and its edges, about 20 keys on spread-out scores) are
//                collected in LDS and ranked (key descending, then column);
//                the first k - #outright of them are selected.  Each thread
//                ends with a bit mask of its selected keys.  If the scores
//                cannot be binned or too many keys fall in between (e.g.
//                many equal scores), three exact radix passes (11, 11, 10
//                key bits) give the k-th key kappa, and the masks take the
//                keys > kappa plus the first keys == kappa in column order.
//   4. emit    : one block scan of the masks' popcounts gives every thread
//                its first output slot; each thread writes only its selected
//                columns.  The output is ascending with no sort.
// Rows longer than one chunk: each chunk selects its exact local top-k
// candidates (key, column) into workspace; a merge workgroup runs the same
// select over the candidates.  The union of the chunk-local top-k sets
// contains the global top-k under the same total order, so the merge is exact.
#include "select_core.h"

namespace dsa {

namespace {

// One row chunk: row t, chunk c, visible columns n of the row; the chunk is
// columns [c0, c0 + len) of the row (len 0: nothing to stage).
struct ChunkItem {
    int t, c, n, c0, len;
    bool vec;          // 16-byte aligned chunk: float4 loads
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
    // 16-byte loads when rows are 16-byte aligned and ld is a multiple of 4:
    // then the load of a group with any column < len ends inside the row
    it.vec = (reinterpret_cast<uintptr_t>(it.row) & 15) == 0 && (p.ld & 3) == 0;
    return it;
}

// Issues the loads of a chunk into the LDS stage (stage[c] = score of chunk
// column c, c < len; group u of wave w: columns 4 * (u * TPB + 64 * w) + 0..255).
// 16-byte direct-to-LDS loads when rows allow them, else plain loads and LDS
// stores.  Columns past len are left unwritten (and dropped when the keys are
// formed); a 16-byte load may read up to 3 of them, still inside the row.
__device__ __forceinline__ void stage_chunk(const ChunkItem &it, float *stage, int tid, int u0, int u1) {
    const int w = tid >> 6, l = tid & 63;
    if (it.len <= 0) return;
    if (it.vec) {
        uint64_t base = (uint64_t)(uintptr_t)it.row;
        // (readfirstlane returns int: widen through uint32_t)
        base = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(base >> 32)) << 32) |
               (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)base);
#pragma unroll
        for (int u = 0; u < CH_V4; ++u) {
            const int c = 4 * (u * TPB + 64 * w + l);
            if (u >= u0 && u < u1 && c < it.len)
                dma16s(base, 4u * (uint32_t)c, (const DSA_LDS void *)(stage + 4 * (u * TPB + 64 * w)));
        }
    } else if (u0 == 0) {
        for (int c = tid; c < it.len; c += TPB) stage[c] = it.row[c];
    }
}

}  // namespace

// Persistent: workgroup g takes the (row, chunk) items g, g + gridDim.x, ...
// of the T * nchunk items (item = row * nchunk + chunk).  Chunk c covers
// visible columns [c*TOPK_CHUNK, min((c+1)*TOPK_CHUNK, nvis)).  The next
// item's scores stream into an LDS stage while the current item is selected
// from registers.
__global__ __launch_bounds__(TPB, 2) void topk_chunk_kernel(TopkParams p, int nitems) {
    __shared__ __attribute__((aligned(16))) float stage[TOPK_CHUNK];
    __shared__ SelectShared sh;
    const int tid = threadIdx.x, k = p.k, grid = (int)gridDim.x;
    int item = blockIdx.x;
    if (item >= nitems) return;
    ChunkItem nxt = chunk_item(p, item);
    stage_chunk(nxt, stage, tid, 0, CH_V4);
    // the next item's row bounds (scalar loads) are fetched one item ahead
    ChunkItem nn{};
    if (item + grid < nitems) nn = chunk_item(p, item + grid);
    for (; item < nitems; item += grid) {
        // the thread index rebuilt from an opaque zero (item < 2^30): per-key
        // column arithmetic then stays inside the loop instead of being held
        // in registers across it
        const int tz = tid + (item >> 30);
        const ChunkItem it = nxt;
        const bool has_next = item + grid < nitems;
        nxt = nn;
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this thread's part of the stage
        lds_barrier();
        // thread tz takes the G 4-column groups tz * G + u: consecutive
        // columns, and with G odd the 16-byte LDS reads of a wave fall in
        // distinct banks.  (Reads of groups u >= G stay inside the stage and
        // are dropped.)
        const int ngroups = (it.len + 4 * TPB - 1) / (4 * TPB);
        const int G = ngroups < CH_V4 ? (ngroups | 1) : CH_V4;
        float4 f4[CH_V4];
        if (G > CH_V4 / 2) {
#pragma unroll
            for (int u = 0; u < CH_V4; ++u) f4[u] = *reinterpret_cast<const float4 *>(stage + 4 * (tz * G + u));
        } else {
#pragma unroll
            for (int u = 0; u < CH_V4 / 2; ++u) f4[u] = *reinterpret_cast<const float4 *>(stage + 4 * (tz * G + u));
#pragma unroll
            for (int u = CH_V4 / 2; u < CH_V4; ++u) f4[u] = float4{0.f, 0.f, 0.f, 0.f};
        }
        // this thread's columns end at lim (its G groups, cut at the chunk's end)
        const int lim = 4 * G * (tz + 1) < it.len ? 4 * G * (tz + 1) : it.len;
        uint32_t kr[4 * CH_V4], lmin = 0xFFFFFFFFu, lmax = 0u;
#pragma unroll
        for (int u = 0; u < CH_V4; ++u) {
            const int c = 4 * (tz * G + u);
            const float f[4] = {f4[u].x, f4[u].y, f4[u].z, f4[u].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // (a mask, not a branch around the conversion)
                const uint32_t key = score_key(f[i]) & (0u - (uint32_t)(c + i < lim));
                kr[4 * u + i] = key;
                lmin = key != 0u && key < lmin ? key : lmin;
                lmax = key > lmax ? key : lmax;
            }
        }
        lds_barrier();   // stage read by every thread: the next item may land in it
        // the next item's scores, 1 KB loads per wave issued in seven parts
        // spread over the select (hook(part) issues the parts up to part), so
        // that the stage refills at a steady rate instead of in one burst that
        // stalls the issuing waves
        int issued = 0;
        auto hook = [&](int part) {
            constexpr int PART[8] = {0, 1, 2, 3, 4, 5, 6, CH_V4};
            if (has_next && part > issued) {
                stage_chunk(nxt, stage, tz, PART[issued], PART[part]);
                issued = part;
            }
        };
        hook(1);
        if (item + 2 * grid < nitems) nn = chunk_item(p, item + 2 * grid);
        int32_t *out = p.idx + (int64_t)it.t * k;
        const int c0 = it.c0;
        int len = it.len;
        // multi-chunk row: local top-min(k, len) candidates of this chunk
        const bool multi = it.n > TOPK_CHUNK;
        if (it.n <= k || len == 0 || (multi && len <= k)) {
            hook(7);
            if (it.n <= k) {  // everything visible is selected
                if (it.c == 0)
                    for (int j = tz; j < k; j += TPB) out[j] = j < it.n ? j : -1;
            } else if (len > 0) {   // the whole chunk, in column order, padded
                uint32_t *ck = p.cand_key + ((int64_t)it.t * p.nchunk + it.c) * k;
                int32_t *cp = p.cand_pos + ((int64_t)it.t * p.nchunk + it.c) * k;
                asm volatile("" : "+s"(len));   // fresh compares below, not the ones of the key loop
#pragma unroll
                for (int u = 0; u < CH_V4; ++u)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int c = 4 * (tz * G + u) + i;
                        if (u < G && c < len) {
                            ck[c] = kr[4 * u + i];
                            cp[c] = c0 + c;
                        }
                    }
                for (int j = len + tz; j < k; j += TPB) {
                    ck[j] = 0u;
                    cp[j] = -1;
                }
            }
            continue;
        }
        select_regs<CH_V4>(kr, G, lmin, lmax, k, sh, tz, multi, hook);
        hook(7);
        if (multi) {
            uint32_t *ck = p.cand_key + ((int64_t)it.t * p.nchunk + it.c) * k;
            int32_t *cp = p.cand_pos + ((int64_t)it.t * p.nchunk + it.c) * k;
            for (int j = tz; j < k; j += TPB) {
                ck[j] = sh.okey[j];
                cp[j] = c0 + sh.ocol[j];
            }
        } else {
            for (int j = tz; j < k; j += TPB) out[j] = c0 + sh.ocol[j];
        }
        lds_barrier();   // sh free for the next select
    }
}

// Grid: x = query row.  Merges the chunk candidates of rows longer than one
// chunk.  Candidate blocks are in column order and padded with key 0 (no
// key), so array order = column order.
__global__ __launch_bounds__(TPB, 2) void topk_merge_kernel(TopkParams p) {
    __shared__ SelectShared sh;
    const int t = blockIdx.x, tid = threadIdx.x;
    const RowInfo ri = row_info(p.cu_q, p.cu_kv, p.pos0, p.B, p.total_kv, p.max_kv, t);
    const int n = ri.nvis, k = p.k;
    if (n <= k || n <= TOPK_CHUNK) return;
    const int nch = (n + TOPK_CHUNK - 1) / TOPK_CHUNK;
    const int m = nch * k;
    const uint32_t *ck = p.cand_key + (int64_t)t * p.nchunk * k;
    const int32_t *cp = p.cand_pos + (int64_t)t * p.nchunk * k;
    // thread tid takes the candidates 4 * G * tid + j, j < 4 * G
    const int G = (m + 4 * TPB - 1) / (4 * TPB);
    uint32_t kr[4 * MG_V4], lmin = 0xFFFFFFFFu, lmax = 0u;
    if ((k & 3) == 0) {   // m and every row's block are multiples of 4 keys: 16-byte loads
#pragma unroll
        for (int u = 0; u < MG_V4; ++u) {
            const int c = 4 * (tid * G + u);
            const uint4 v = u < G && c < m ? *reinterpret_cast<const uint4 *>(ck + c) : uint4{0u, 0u, 0u, 0u};
            kr[4 * u] = v.x;
            kr[4 * u + 1] = v.y;
            kr[4 * u + 2] = v.z;
            kr[4 * u + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int u = 0; u < MG_V4; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = 4 * (tid * G + u) + i;
                kr[4 * u + i] = u < G && c < m ? ck[c] : 0u;
            }
    }
#pragma unroll
    for (int i = 0; i < 4 * MG_V4; ++i) {
        lmin = kr[i] != 0u && kr[i] < lmin ? kr[i] : lmin;
        lmax = kr[i] > lmax ? kr[i] : lmax;
    }
    int32_t *out = p.idx + (int64_t)t * k;
    select_regs<MG_V4>(kr, G, lmin, lmax, k, sh, tid, false, [](int) {});
    for (int j = tid; j < k; j += TPB) {
        const int c = sh.ocol[j];   // a candidate index below m (checked: it addresses cp)
        out[j] = (unsigned)c < (unsigned)m ? cp[c] : -1;
    }
}

// The selection of a row that sees no more than k keys: every visible key,
// ascending, then -1 (the select's own result for such a row, written without
// reading any score).  One row per workgroup, 4 slots per thread.
__global__ __launch_bounds__(256) void select_all_visible_kernel(TopkParams p) {
    const int t = blockIdx.x;
    const RowInfo ri = row_info(p.cu_q, p.cu_kv, p.pos0, p.B, p.total_kv, p.max_kv, t);
    int32_t *row = p.idx + (int64_t)t * p.k;
    for (int j = 4 * (int)threadIdx.x; j < p.k; j += 4 * 256) {
        if (j + 4 <= p.k && (p.k & 3) == 0) {
            const int4 v = {j < ri.nvis ? j : -1, j + 1 < ri.nvis ? j + 1 : -1,
                            j + 2 < ri.nvis ? j + 2 : -1, j + 3 < ri.nvis ? j + 3 : -1};
            *reinterpret_cast<int4 *>(row + j) = v;
        } else {
            for (int i = j; i < j + 4 && i < p.k; ++i) row[i] = i < ri.nvis ? i : -1;
        }
    }
}

hipError_t launch_select_all_visible(const TopkParams &p, int T, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    hipLaunchKernelGGL(select_all_visible_kernel, dim3(T), dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_topk(const TopkParams &p, int T, hipStream_t s, LaunchMarks *m) {
    if (T <= 0) return hipSuccess;
    if (p.nchunk > TOPK_MAX_CHUNKS) return hipErrorInvalidValue;
    // persistent grid: one workgroup per compute unit (the stage fills the LDS)
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
    if (m) m->after("topk_chunk_kernel", s);
    if (e != hipSuccess || p.nchunk <= 1) return e;
    hipLaunchKernelGGL(topk_merge_kernel, dim3(T), dim3(TPB), 0, s, p);
    e = hipGetLastError();
    if (m) m->after("topk_merge_kernel", s);
    return e;
}

}  // namespace dsa
