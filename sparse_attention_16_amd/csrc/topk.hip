// topk.hip — exact per-row top-k selection of index scores on gfx950.
//
// Selection rule (page "Техотчёт DeepSeek-V3.2 (2025): разреженное внимание
// DSA и масштабирование RL", section "Отбор и основное внимание": keep the k
// key positions with the largest index scores of the query): the k largest
// fp32 scores among the row's visible columns, -0 == +0, ties to the lower
// column; all visible columns when there are at most k.  Output: the selected
// columns in ascending order, -1 padded.
//
// Method (one 512-thread workgroup per row chunk of up to 32768 columns; the
// chunk's scores stay in registers, 64 per thread, as order-preserving uint32
// keys):
//   1. range   : block minimum and maximum of the chunk's scores.
//   2. bin     : a 2048-bin histogram of the scores, binned by value over
//                [min, max] (a non-decreasing map, so bins keep the order);
//                a scan from the top names the bin b1 holding the k-th
//                largest key and how many of its keys are taken.
//   3. kappa   : the keys of bin b1 (a handful on spread-out scores) are
//                collected in LDS and each is ranked against the others: the
//                k-th largest key kappa and the number of keys equal to kappa
//                to take follow directly.  If the bins cannot be formed or bin
//                b1 is too full (e.g. many equal scores), three exact radix
//                passes (11, 11, 10 key bits) over the register keys give
//                kappa instead.
//   4. emit    : each thread counts, per 4-column group, its keys > kappa and
//                == kappa; one block prefix over the groups in column order
//                gives every selected key its output slot.  The output is
//                ascending with no sort.
// Rows longer than one chunk: each chunk selects its exact local top-k
// candidates (key, column) into workspace; a merge workgroup runs the same
// select over the candidates.  The union of the chunk-local top-k sets
// contains the global top-k under the same total order, so the merge is exact.
#include "dsa_device.h"
#include "kernels.h"

namespace dsa {

namespace {

constexpr int TPB = 512;                                   // threads per workgroup
constexpr int NWAVE = TPB / kWave;                         // 8
constexpr int NBIN = 2048;                                 // histogram bins
constexpr int BPT = NBIN / TPB;                            // bins scanned per thread
constexpr int CCAP = TPB;                                  // candidates ranked directly (one per thread)
constexpr int CH_V4 = TOPK_CHUNK / (4 * TPB);              // 4-key groups per thread, chunk kernel
constexpr int MG_V4 = TOPK_MAX_CHUNKS * 2048 / (4 * TPB);  // 4-key groups per thread, merge kernel
constexpr int MAX_V4 = CH_V4 > MG_V4 ? CH_V4 : MG_V4;
static_assert(NBIN % TPB == 0 && CH_V4 * 4 * TPB == TOPK_CHUNK && MG_V4 * 4 * TPB == TOPK_MAX_CHUNKS * 2048,
              "register layout");
static_assert(NWAVE * MAX_V4 <= 2 * kWave, "one wave scans the group totals, two per lane");

struct SelectShared {
    // each array has one spare entry per lane after its end: writes that
    // must not count go there (a spare per lane, so that they do not collide)
    uint32_t hist[NBIN + kWave];
    uint32_t ckey[CCAP + kWave];
    int32_t ocol[2048 + kWave];      // selected columns by slot
    uint32_t okey[2048 + kWave];     // their keys
    uint32_t gsum[MAX_V4 * NWAVE];   // per (group, wave) packed counts, then their prefix
    uint32_t wtot[NWAVE];            // scan and reduction scratch
    uint32_t wmin[NWAVE], wmax[NWAVE];
    uint32_t ncand;
    uint32_t prefix;                 // bin b1, or radix key bits fixed so far
    uint32_t rem;                    // keys still needed inside the prefix
    uint32_t kappa, need_eq;
};

// Marks the register keys as changed (no instruction): values derived from
// them in an earlier phase (validity masks, bins) are recomputed instead of
// being kept live across the phases, which would not fit in the registers.
template <int N>
__device__ __forceinline__ void launder(uint32_t (&kr)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("" : "+v"(kr[i]));
}

// Score of a key (inverse of score_key; key != 0).
__device__ __forceinline__ float key_value(uint32_t key) {
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// Inclusive scan over the 64 lanes of a wave with DPP lane moves (VALU only,
// no LDS round trip): row shifts by 1, 2, 4, 8 scan each 16-lane row, then
// the last lane of row 0 is added to row 1 and 3 and that of rows 0-1 to
// rows 2-3.  Lanes a move has no source for take the identity `id`.
template <class Op>
__device__ __forceinline__ uint32_t wave_scan(uint32_t x, uint32_t id, Op op) {
    x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x111, 0xf, 0xf, false));  // row_shr:1
    x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x112, 0xf, 0xf, false));  // row_shr:2
    x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x114, 0xf, 0xf, false));  // row_shr:4
    x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x118, 0xf, 0xf, false));  // row_shr:8
    x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x142, 0xa, 0xf, false));  // row_bcast:15
    x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x143, 0xc, 0xf, false));  // row_bcast:31
    return x;
}
__device__ __forceinline__ uint32_t wave_scan_add(uint32_t x) {
    return wave_scan(x, 0u, [](uint32_t a, uint32_t b) { return a + b; });
}

// Block-wide exclusive scan of one value per thread (in thread order).
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t *wtot) {
    const int l = lane_id(), w = threadIdx.x >> 6;
    const uint32_t x = wave_scan_add(v);
    if (l == 63) wtot[w] = x;
    lds_barrier();
    uint32_t off = 0;
#pragma unroll
    for (int i = 0; i < NWAVE; ++i) off += (i < w) ? wtot[i] : 0u;
    lds_barrier();
    return off + x - v;
}

// From the counts in sh.hist (bin i = digit i, larger digits = larger keys),
// picks the bin holding the sh.rem-th largest key: sh.prefix = (prefix <<
// width) | bin, sh.rem = rank inside that bin.
__device__ __forceinline__ void pick_bin(int width, SelectShared &sh) {
    const int top = NBIN - 1 - BPT * (int)threadIdx.x;   // this thread's bins: top, top-1, ...
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

__device__ __forceinline__ void clear_hist(SelectShared &sh) {
#pragma unroll
    for (int i = 0; i < BPT; ++i) sh.hist[threadIdx.x + i * TPB] = 0u;
}

// Exact kappa by three radix passes over the register keys (key 0 = no key).
template <int NV4>
__device__ __forceinline__ void radix_kappa(uint32_t (&kr)[4 * NV4], int ngroups, int k, SelectShared &sh) {
    if (threadIdx.x == 0) {
        sh.prefix = 0;
        sh.rem = (uint32_t)k;
    }
    constexpr int SHIFT[3] = {21, 10, 0}, WIDTH[3] = {11, 11, 10};
#pragma unroll
    for (int ps = 0; ps < 3; ++ps) {
        clear_hist(sh);
        lds_barrier();
        const uint32_t prefix = sh.prefix;
        const int hi = SHIFT[ps] + WIDTH[ps];
        launder(kr);
#pragma unroll
        for (int i = 0; i < 4 * NV4; ++i) {
            if (i / 4 < ngroups) {
                const uint32_t key = kr[i];
                const bool match = key != 0u && (hi == 32 || (key >> (hi & 31)) == prefix);
                atomicAdd(&sh.hist[match ? (key >> SHIFT[ps]) & ((1u << WIDTH[ps]) - 1u) : NBIN + lane_id()], 1u);
            }
            if ((i & 3) == 3) __builtin_amdgcn_sched_barrier(0);   // one 4-key group at a time
        }
        lds_barrier();
        pick_bin(WIDTH[ps], sh);
    }
    if (threadIdx.x == 0) {
        sh.kappa = sh.prefix;
        sh.need_eq = sh.rem;
    }
    lds_barrier();
}

// Steps 1-4 over the register keys kr (key 0 = no key; key i of group u sits
// at column 4 * (u * TPB + tid) + i), at least k + 1 of them real, groups >=
// ngroups empty.  tz is the thread index, passed in so that a caller's loop
// can keep the per-key column arithmetic from being hoisted out of it and
// held in registers.  On return (after a barrier) sh.ocol[slot], slot < k,
// holds the columns of the k selected keys, slot = rank in column order, and
// sh.okey[slot] their keys when want_keys.
template <int NV4>
__device__ __forceinline__ void select_regs(uint32_t (&kr)[4 * NV4], int ngroups, int k, SelectShared &sh, int tz,
                                            bool want_keys) {
    const int tid = threadIdx.x, l = lane_id(), w = tid >> 6;
    launder(kr);

    // 1. range (keys order like scores: min/max over keys)
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
    for (int i = 0; i < 4 * NV4; ++i) {
        const uint32_t key = kr[i];
        kmin = key != 0u && key < kmin ? key : kmin;
        kmax = key > kmax ? key : kmax;
    }
    kmin = wave_scan(kmin, 0xFFFFFFFFu, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
    kmax = wave_scan(kmax, 0u, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
    if (l == 63) {   // the inclusive scan's last lane holds the wave's result
        sh.wmin[w] = kmin;
        sh.wmax[w] = kmax;
    }
    clear_hist(sh);
    if (tid == 0) {
        sh.ncand = 0;
        sh.prefix = 0;
        sh.rem = (uint32_t)k;
    }
    lds_barrier();
#pragma unroll
    for (int x = 0; x < NWAVE; ++x) {
        kmin = sh.wmin[x] < kmin ? sh.wmin[x] : kmin;
        kmax = sh.wmax[x] > kmax ? sh.wmax[x] : kmax;
    }
    const float vmin = key_value(kmin), vmax = key_value(kmax);
    const float range = vmax - vmin;
    const float inv = (float)NBIN / range;
    // value bins need a finite, positive range with a finite scale
    const bool binned = range > 0.f && range < INFINITY && inv < INFINITY;

    bool exact_done = false;
    if (binned) {
        // 2. value histogram, bin b1
        auto bin_of = [&](uint32_t key) {
            const float t = (key_value(key) - vmin) * inv;
            return (uint32_t)fminf(t, (float)(NBIN - 1));
        };
        launder(kr);
#pragma unroll
        for (int i = 0; i < 4 * NV4; ++i) {
            if (i / 4 < ngroups) atomicAdd(&sh.hist[kr[i] != 0u ? bin_of(kr[i]) : NBIN + l], 1u);
            if ((i & 3) == 3) __builtin_amdgcn_sched_barrier(0);   // one 4-key group at a time
        }
        lds_barrier();
        pick_bin(0, sh);   // prefix = b1, rem = rank inside b1
        const uint32_t b1 = sh.prefix, rem = sh.rem;
        // the bins are recomputed below, not kept from the histogram pass
        // (64 live bin values would not fit in the registers)
        launder(kr);
        float vmin2 = vmin, inv2 = inv;
        asm volatile("" : "+v"(vmin2), "+v"(inv2));
        auto bin2_of = [&](uint32_t key) {
            const float t = (key_value(key) - vmin2) * inv2;
            return (uint32_t)fminf(t, (float)(NBIN - 1));
        };
        // 3. candidates of bin b1, ranked
#pragma unroll
        for (int i = 0; i < 4 * NV4; ++i) {
            if (i / 4 >= ngroups) continue;
            const bool m = kr[i] != 0u && bin2_of(kr[i]) == b1;
            const uint64_t bal = __ballot(m);
            if (bal != 0ull) {   // wave-uniform; rare
                uint32_t base = 0;
                if (l == 0) base = atomicAdd(&sh.ncand, (uint32_t)__popcll(bal));
                base = __builtin_amdgcn_readlane(base, 0);
                const uint32_t pos = base + (uint32_t)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                      __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
                sh.ckey[m && pos < CCAP ? pos : CCAP + l] = kr[i];
            }
            if ((i & 3) == 3) __builtin_amdgcn_sched_barrier(0);
        }
        lds_barrier();
        const uint32_t nc = sh.ncand;
        if (nc <= CCAP) {
            if ((uint32_t)tid < nc) {
                const uint32_t key = sh.ckey[tid];
                uint32_t gt = 0, eq = 0;
                for (uint32_t j = 0; j < nc; ++j) {
                    const uint32_t o = sh.ckey[j];
                    gt += o > key ? 1u : 0u;
                    eq += o == key ? 1u : 0u;
                }
                // every thread holding kappa writes the same two values
                if (gt < rem && rem <= gt + eq) {
                    sh.kappa = key;
                    sh.need_eq = rem - gt;
                }
            }
            lds_barrier();
            exact_done = true;
        }
    }
    if (!exact_done) radix_kappa<NV4>(kr, ngroups, k, sh);
    const uint32_t kappa = sh.kappa, need_eq = sh.need_eq;

    launder(kr);
    // 4. emit: packed counts (keys > kappa in the low half, == kappa in the
    // high half; each at most 32768) per 4-key group, prefix in column order
    uint32_t incl[NV4];
#pragma unroll
    for (int u = 0; u < NV4; ++u) {
        if (u < ngroups) {
            uint32_t c = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t key = kr[4 * u + i];
                c += key > kappa ? 1u : (key == kappa ? 0x10000u : 0u);
            }
            const uint32_t x = wave_scan_add(c);
            incl[u] = x - c;   // exclusive within the wave
            if (l == 63) sh.gsum[u * NWAVE + w] = x;
        }
    }
    lds_barrier();
    if (w == 0) {   // exclusive prefix over (group, wave) in column order
        const int n2 = ngroups * NWAVE;
        const uint32_t a = 2 * l < n2 ? sh.gsum[2 * l] : 0u;
        const uint32_t b = 2 * l + 1 < n2 ? sh.gsum[2 * l + 1] : 0u;
        const uint32_t s = a + b;
        const uint32_t x = wave_scan_add(s);
        if (2 * l < n2) sh.gsum[2 * l] = x - s;
        if (2 * l + 1 < n2) sh.gsum[2 * l + 1] = x - s + a;
    }
    lds_barrier();
    launder(kr);
#pragma unroll
    for (int u = 0; u < NV4; ++u) {
        if (u < ngroups) {
            const uint32_t base = sh.gsum[u * NWAVE + w] + incl[u];
            uint32_t g = base & 0xFFFFu, e = base >> 16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t key = kr[4 * u + i];
                const bool fg = key > kappa, fe = key == kappa;
                const uint32_t slot = g + (e < need_eq ? e : need_eq);
                const bool take = (fg || (fe && e < need_eq)) && slot < (uint32_t)k;
                const uint32_t at = take ? slot : 2048u + (uint32_t)l;   // this lane's spare slot
                sh.ocol[at] = 4 * (u * TPB + tz) + i;
                if (want_keys) sh.okey[at] = key;
                g += fg ? 1u : 0u;
                e += fe ? 1u : 0u;
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    lds_barrier();   // selection in sh.ocol / sh.okey
}

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
__device__ __forceinline__ void stage_chunk(const ChunkItem &it, float *stage, int tid) {
    const int w = tid >> 6, l = tid & 63;
    if (it.vec) {
        uint64_t base = (uint64_t)(uintptr_t)it.row;
        // (readfirstlane returns int: widen through uint32_t)
        base = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(base >> 32)) << 32) |
               (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)base);
#pragma unroll
        for (int u = 0; u < CH_V4; ++u) {
            const int c = 4 * (u * TPB + 64 * w + l);
            if (c < it.len)
                dma16s(base, 4u * (uint32_t)c, (const DSA_LDS void *)(stage + 4 * (u * TPB + 64 * w)));
        }
    } else {
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
    const int tid = threadIdx.x, k = p.k;
    int item = blockIdx.x;
    if (item >= nitems) return;
    ChunkItem nxt = chunk_item(p, item);
    if (nxt.len > 0) stage_chunk(nxt, stage, tid);
    for (; item < nitems; item += gridDim.x) {
        // the thread index rebuilt from an opaque zero (item < 2^30): per-key
        // column arithmetic then stays inside the loop instead of being held
        // in registers across it
        const int tz = tid + (item >> 30);
        const ChunkItem it = nxt;
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this thread's part of the stage
        lds_barrier();
        uint32_t kr[4 * CH_V4];
#pragma unroll
        for (int u = 0; u < CH_V4; ++u) {
            const int c = 4 * (u * TPB + tz);
            const float4 f4 = c < it.len ? *reinterpret_cast<const float4 *>(stage + c) : float4{0.f, 0.f, 0.f, 0.f};
            const float f[4] = {f4.x, f4.y, f4.z, f4.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) kr[4 * u + i] = c + i < it.len ? score_key(f[i]) : 0u;
        }
        lds_barrier();   // stage read by every thread: the next item may land in it
        if (item + (int)gridDim.x < nitems) {
            nxt = chunk_item(p, item + gridDim.x);
            if (nxt.len > 0) stage_chunk(nxt, stage, tz);
        }
        int32_t *out = p.idx + (int64_t)it.t * k;
        if (it.n <= k) {  // everything visible is selected
            if (it.c == 0)
                for (int j = tz; j < k; j += TPB) out[j] = j < it.n ? j : -1;
            continue;
        }
        if (it.len == 0) continue;  // chunk past the visible end
        const int c0 = it.c0, len = it.len;
        const int ngroups = (len + 4 * TPB - 1) / (4 * TPB);
        // multi-chunk row: local top-min(k, len) candidates of this chunk
        const bool multi = it.n > TOPK_CHUNK;
        uint32_t *ck = p.cand_key + ((int64_t)it.t * p.nchunk + it.c) * k;
        int32_t *cp = p.cand_pos + ((int64_t)it.t * p.nchunk + it.c) * k;
        if (multi && len <= k) {   // the whole chunk, in column order, padded
#pragma unroll
            for (int u = 0; u < CH_V4; ++u)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int c = 4 * (u * TPB + tz) + i;
                    if (c < len) {
                        ck[c] = kr[4 * u + i];
                        cp[c] = c0 + c;
                    }
                }
            for (int j = len + tz; j < k; j += TPB) {
                ck[j] = 0u;
                cp[j] = -1;
            }
            continue;
        }
        select_regs<CH_V4>(kr, ngroups, k, sh, tz, multi);
        for (int j = tz; j < k; j += TPB) {
            const int col = c0 + sh.ocol[j];
            if (multi) {
                ck[j] = sh.okey[j];
                cp[j] = col;
            } else {
                out[j] = col;
            }
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
    uint32_t kr[4 * MG_V4];
#pragma unroll
    for (int u = 0; u < MG_V4; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = 4 * (u * TPB + tid) + i;
            kr[4 * u + i] = c < m ? ck[c] : 0u;
        }
    const int ngroups = (m + 4 * TPB - 1) / (4 * TPB);
    int32_t *out = p.idx + (int64_t)t * k;
    select_regs<MG_V4>(kr, ngroups, k, sh, tid, false);
    for (int j = tid; j < k; j += TPB) out[j] = cp[sh.ocol[j]];
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

hipError_t launch_topk(const TopkParams &p, int T, hipStream_t s) {
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
    if (e != hipSuccess || p.nchunk <= 1) return e;
    hipLaunchKernelGGL(topk_merge_kernel, dim3(T), dim3(TPB), 0, s, p);
    return hipGetLastError();
}

}  // namespace dsa
