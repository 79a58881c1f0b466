// topk.hip — exact per-row top-k selection of index scores on gfx950.
//
// Selection rule (page "Техотчёт DeepSeek-V3.2 (2025): разреженное внимание
// DSA и масштабирование RL", section "Отбор и основное внимание": keep the k
// key positions with the largest index scores of the query): the k largest
// fp32 scores among the row's visible columns, -0 == +0, ties to the lower
// column; all visible columns when there are at most k.  Output: the selected
// columns in ascending order, -1 padded.
//
// Method (one 1024-thread workgroup per row chunk of up to 32768 columns,
// two workgroups per compute unit; the chunk's scores are loaded straight into
// registers as order-preserving uint32 keys, column 2048 w + 64 i + l in
// register i of lane l of wave w, so every load instruction reads 64
// consecutive columns and (wave, register, lane) order is column order):
//   1. sample  : one key per lane (1024 per full chunk, spread over the
//                chunk; -inf scores left out); the rank-th largest sample,
//                rank = mu + 5 sqrt(mu) + 1 with mu = k * samples / columns
//                (the expected number of samples among the chunk's top k),
//                located by a value histogram of the samples, gives a
//                threshold a quarter bin below it.  About 1.6 k keys pass it.
//   2. compact : the keys at or above the threshold (counted per wave, one
//                barrier for the offsets) and their columns go to LDS in
//                column order.
//   3. select  : when more than k and at most 8192 keys passed, the exact
//                select of the k largest among them (lds_cand_select of
//                select_core.h: a value histogram, the bin of the k-th
//                largest, its few keys ranked, each wave writing its own
//                slots in column order); with many equal scores in that bin,
//                the register select of select_core.h.  Every key of the
//                exact top k is at or above the k-th largest key, which is at
//                or above the threshold whenever more than k keys pass it, so
//                the candidates hold the whole answer.
//   4. fallback: otherwise (a sample that missed, or many equal scores) the
//                k-th largest key kappa by radix passes over the register
//                keys, then the keys > kappa and the first keys == kappa in
//                column order, written in column order from the registers.
// Rows longer than one chunk: each chunk selects its exact local top-k
// candidates (key, column) into workspace; a merge workgroup runs the same
// select over the candidates.  The union of the chunk-local top-k sets
// contains the global top-k under the same total order, so the merge is exact.
#include "select_core.h"

namespace dsa {

namespace {

// One row chunk: row t, chunk c, visible columns n of the row; the chunk is
// columns [c0, c0 + len) of the row (len 0: nothing to select).
struct ChunkItem {
    int t, c, n, c0, len;
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
    return it;
}

constexpr int TK_WCOLS = TOPK_CHUNK / NWAVE;   // 2048 columns per wave
constexpr int TK_R = TK_WCOLS / kWave;         // 32 keys per lane
constexpr int TK_CAP = 8 * TPB;                // candidates the select takes (8 per thread)
constexpr float TK_SIGMAS = 5.f;               // sample rank margin, in standard deviations
constexpr uint32_t kNegInfKey = 0x007FFFFFu;   // score_key(-inf): the lowest real key
static_assert(TK_R == 4 * CH_V4 && TK_CAP <= 65536, "register layout");



// A wave's keys: score_key(wsrc[64 i + l]) in kr[i - i0] of lane l for the
// registers i in [i0, i0 + N), 0 for columns at or past wlen (wlen >= 1 - the
// wave's first column, so that column wlen - 1 lies inside the row).  All N
// loads are issued before any key is formed: registers wholly inside wlen
// load unmasked, a register that crosses it loads column min(c, wlen - 1).
// (The offset goes through an empty asm statement, so that a later call
// loads again instead of keeping an earlier call's keys live in between.)
template <int N>
__device__ __forceinline__ void load_keys(const float *wsrc, int i0, int wlen, uint32_t (&kr)[N]) {
    const int l = lane_id();
    int zero = 0;
    asm volatile("" : "+s"(zero));
    const float *src = wsrc + zero;
    float raw[N];
    if (kWave * (i0 + N) <= wlen) {
#pragma unroll
        for (int j = 0; j < N; ++j) raw[j] = src[kWave * (i0 + j) + l];
#pragma unroll
        for (int j = 0; j < N; ++j) kr[j] = score_key(raw[j]);
    } else {
#pragma unroll
        for (int j = 0; j < N; ++j) {
            const int c = kWave * (i0 + j) + l;
            raw[j] = src[c < wlen ? c : wlen - 1];
        }
#pragma unroll
        for (int j = 0; j < N; ++j) kr[j] = kWave * (i0 + j) + l < wlen ? score_key(raw[j]) : 0u;
    }
}

// The fallback of topk_chunk_kernel, for a chunk whose sampled threshold
// passed at most k or more than 8192 keys: kappa, the k-th largest of the
// chunk's keys, by three radix passes (11, 11, 10 key bits) of a histogram
// of the keys that match the digits fixed so far; then the keys > kappa and
// the first need_eq keys == kappa in column order, column c0 + c to dcol[slot]
// (and the key to dkey[slot] when dkey is given), slot = rank in column
// order.  The keys are loaded again, 8 registers at a time, in each pass
// (the kernel's register keys are dead by then: two waves per SIMD leave 64
// registers, too few to hold them across the passes).
__device__ __forceinline__ void chunk_radix_select(const float *wsrc, int wlen, int nreg, int wc0, int k, int c0,
                                                int32_t *dcol, uint32_t *dkey, SelectShared &sh, uint32_t *wcnt) {
    const int tid = threadIdx.x, l = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    constexpr int KG = 8;
    if (tid == 0) {
        sh.prefix = 0u;
        sh.rem = (uint32_t)k;
    }
    constexpr int SHIFT[3] = {21, 10, 0}, WIDTH[3] = {11, 11, 10};
    static_assert(NBIN >= (1 << 11), "the radix digits index the histogram");
#pragma unroll
    for (int ps = 0; ps < 3; ++ps) {
        clear_hist(sh);
        lds_barrier();
        const uint32_t prefix = sh.prefix;
        const int hi = SHIFT[ps] + WIDTH[ps];
#pragma unroll 1
        for (int g = 0; g < TK_R; g += KG) {
            if (g < nreg) {
                uint32_t kk[KG];
                load_keys<KG>(wsrc, g, wlen, kk);
#pragma unroll
                for (int j = 0; j < KG; ++j) {
                    const uint32_t key = kk[j];
                    const bool match = key != 0u && (hi == 32 || (key >> (hi & 31)) == prefix);
                    atomicAdd(&sh.hist[match ? (key >> SHIFT[ps]) & ((1u << WIDTH[ps]) - 1u) : NBIN + l], 1u);
                }
            }
        }
        lds_barrier();
        pick_bin(WIDTH[ps], sh);
    }
    const uint32_t kappa = sh.prefix, need_eq = sh.rem;
    uint32_t weq = 0;
#pragma unroll 1
    for (int g = 0; g < TK_R; g += KG) {
        if (g < nreg) {
            uint32_t kk[KG];
            load_keys<KG>(wsrc, g, wlen, kk);
#pragma unroll
            for (int j = 0; j < KG; ++j) weq += (uint32_t)__popcll(__ballot(kk[j] == kappa));
        }
    }
    if (l == 0) wcnt[w] = weq;
    lds_barrier();
    uint32_t eqb = 0;
#pragma unroll
    for (int x = 0; x < NWAVE; ++x) eqb += x < w ? wcnt[x] : 0u;
    uint32_t take = 0, wsel = 0;
#pragma unroll 1
    for (int g = 0; g < TK_R; g += KG) {
        if (g < nreg) {
            uint32_t kk[KG];
            load_keys<KG>(wsrc, g, wlen, kk);
#pragma unroll
            for (int j = 0; j < KG; ++j) {
                const bool e = kk[j] == kappa;
                const uint64_t me = __ballot(e);
                const bool tk = kk[j] > kappa || (e && eqb + lane_rank(me) < need_eq);
                eqb += (uint32_t)__popcll(me);
                take |= (tk ? 1u : 0u) << (g + j);
                wsel += (uint32_t)__popcll(__ballot(tk));
            }
        }
    }
    lds_barrier();   // every wave has read the equal counts
    if (l == 0) wcnt[w] = wsel;
    lds_barrier();
    uint32_t slot0 = 0;
#pragma unroll
    for (int x = 0; x < NWAVE; ++x) slot0 += x < w ? wcnt[x] : 0u;
#pragma unroll 1
    for (int g = 0; g < TK_R; g += KG) {
        if (g < nreg) {
            uint32_t kk[KG];
            load_keys<KG>(wsrc, g, wlen, kk);
#pragma unroll
            for (int j = 0; j < KG; ++j) {
                const bool tk = (take >> (g + j)) & 1u;
                const uint64_t mt = __ballot(tk);
                const uint32_t slot = slot0 + lane_rank(mt);
                if (tk && slot < (uint32_t)k) {   // (exactly k keys are selected)
                    dcol[slot] = c0 + wc0 + kWave * (g + j) + l;
                    if (dkey) dkey[slot] = kk[j];
                }
                slot0 += (uint32_t)__popcll(mt);
            }
        }
    }
}

}  // namespace

// Grid: one workgroup per (row, chunk) item, the last items first (in a
// causal batch the last rows see the most keys).  Chunk c covers visible
// columns [c*TOPK_CHUNK, min((c+1)*TOPK_CHUNK, nvis)).
__global__ __launch_bounds__(TPB) __attribute__((amdgpu_waves_per_eu(8))) void topk_chunk_kernel(TopkParams p,
                                                                                                 int nitems) {
    __shared__ SelectShared sh;
    __shared__ __attribute__((aligned(16))) uint32_t ckey[TK_CAP];   // candidate keys, column order, 0 after them
    __shared__ uint16_t ccol[TK_CAP];                                // their columns in the chunk
    __shared__ uint32_t wsmp[NWAVE], wcnt[NWAVE], gsum[NWAVE];       // per-wave sample and key counts, bin sums
    const int tid = threadIdx.x, l = lane_id(), k = p.k;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const ChunkItem it = chunk_item(p, nitems - 1 - (int)blockIdx.x);
    int32_t *out = p.idx + (int64_t)it.t * k;
    const int c0 = it.c0, len = it.len;
    // multi-chunk row: local top-min(k, len) candidates of this chunk
    const bool multi = it.n > TOPK_CHUNK;
    if (it.n <= k || len == 0 || (multi && len <= k)) {
        if (it.n <= k) {  // everything visible is selected
            if (it.c == 0)
                for (int j = tid; j < k; j += TPB) out[j] = j < it.n ? j : -1;
        } else if (len > 0) {   // the whole chunk, in column order, padded
            uint32_t *ck = p.cand_key + ((int64_t)it.t * p.nchunk + it.c) * k;
            int32_t *cp = p.cand_pos + ((int64_t)it.t * p.nchunk + it.c) * k;
            for (int j = tid; j < k; j += TPB) {
                ck[j] = j < len ? score_key(it.row[j]) : 0u;
                cp[j] = j < len ? c0 + j : -1;
            }
        }
        return;
    }

    // keys (0 past the chunk's end); nreg = registers of this wave that hold any
    const int wc0 = TK_WCOLS * w;
    const int nreg = len <= wc0 ? 0 : ((len - wc0 + kWave - 1) / kWave < TK_R ? (len - wc0 + kWave - 1) / kWave : TK_R);
    const float *wsrc = it.row + wc0;
    const int wlen = len - wc0;
    uint32_t kr[TK_R];
    if (nreg > 0) {
        load_keys<TK_R>(wsrc, 0, wlen, kr);
    } else {
#pragma unroll
        for (int i = 0; i < TK_R; ++i) kr[i] = 0u;
    }

    // 1. sample: lane l's key of register 4 (l % 8), spread over the wave's
    // columns.  A -inf score is left out of the sample: it would make the
    // sampled range infinite (no threshold) and can never pass a finite one.
    uint32_t sk = 0u;
#pragma unroll
    for (int i = 0; i < TK_R; i += 4) sk = (l & 7) == i / 4 ? kr[i] : sk;
    sk = sk == kNegInfKey ? 0u : sk;
    {
        const uint32_t mn = wave_scan(sk != 0u ? sk : 0xFFFFFFFFu, 0xFFFFFFFFu,
                                      [](uint32_t a, uint32_t b2) { return a < b2 ? a : b2; });
        const uint32_t mx = wave_scan(sk, 0u, [](uint32_t a, uint32_t b2) { return a > b2 ? a : b2; });
        const uint32_t ns = (uint32_t)__popcll(__ballot(sk != 0u));
        if (l == 63) {   // the inclusive scan's last lane holds the wave's result
            sh.wmin[w] = mn;
            sh.wmax[w] = mx;
            wsmp[w] = ns;
        }
    }
    clear_hist(sh);
    lds_barrier();
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u, ns = 0u;
#pragma unroll
    for (int x = 0; x < NWAVE; ++x) {
        kmin = sh.wmin[x] < kmin ? sh.wmin[x] : kmin;
        kmax = sh.wmax[x] > kmax ? sh.wmax[x] : kmax;
        ns += wsmp[x];
    }
    const float mu = (float)k * (float)ns / (float)len;
    const uint32_t rank = (uint32_t)(mu + TK_SIGMAS * sqrtf(mu)) + 1u;
    const float vmin = key_value(kmin), vmax = key_value(kmax);
    const float range = vmax - vmin;
    const float inv = (float)NBIN / range;
    uint32_t tkey = 1u;   // candidates: keys >= tkey (1: every key of the chunk)
    if (ns > rank && range > 0.f && range < INFINITY && inv < INFINITY) {
        if (sk != 0u) atomicAdd(&sh.hist[(uint32_t)fminf((key_value(sk) - vmin) * inv, (float)(NBIN - 1))], 1u);
        lds_barrier();
        uint32_t b, rem, above;
        block_pick_bin<NBIN>(sh.hist, gsum, rank, b, rem, above);   // the bin of the rank-th largest sample
        tkey = score_key(vmin + ((float)b - 0.25f) * (range / (float)NBIN));
    }
    // value bins of the candidates (3. below) span the sampled range from the
    // threshold (or the smallest sample) to the largest sample.  (Bins of the
    // key bits would be far too coarse wherever the range crosses zero or
    // several exponents.)
    const float cvlo = tkey > 1u ? key_value(tkey) : vmin;

    // 2. candidates: counts per wave, then keys and columns into LDS in column order
    // (registers from nreg on hold key 0, below every threshold: the loops
    // test nreg once per 8 registers)
    uint32_t wc = 0;
#pragma unroll
    for (int g = 0; g < TK_R; g += 8)
        if (g < nreg)
#pragma unroll
            for (int i = g; i < g + 8; ++i) wc += (uint32_t)__popcll(__ballot(kr[i] >= tkey));
    if (l == 0) wcnt[w] = wc;
    lds_barrier();
    uint32_t nc = 0, pos = 0;
#pragma unroll
    for (int x = 0; x < NWAVE; ++x) {
        pos += x < w ? wcnt[x] : 0u;
        nc += wcnt[x];
    }
    // (written whatever the count, so that no key is live past the branch
    // below; a slot past the capacity is dropped)
#pragma unroll
    for (int g = 0; g < TK_R; g += 8) {
        if (g < nreg) {
#pragma unroll
            for (int i = g; i < g + 8; ++i) {
                const bool cand = kr[i] >= tkey;
                const uint64_t m = __ballot(cand);
                const uint32_t slot = pos + lane_rank(m);
                if (cand && slot < (uint32_t)TK_CAP) {
                    ckey[slot] = kr[i];
                    ccol[slot] = (uint16_t)(wc0 + kWave * i + l);
                }
                pos += (uint32_t)__popcll(m);
            }
        }
    }
    if (nc > (uint32_t)k && nc <= (uint32_t)TK_CAP) {
        // 3. exact select over the candidates (lds_cand_select), written in
        // column order
        uint32_t *ck = multi ? p.cand_key + ((int64_t)it.t * p.nchunk + it.c) * k : nullptr;
        int32_t *cp = multi ? p.cand_pos + ((int64_t)it.t * p.nchunk + it.c) * k : out;
        if (lds_cand_select<TK_CAP>(ckey, (int)nc, k, cvlo, vmax, sh, gsum, wcnt, [&](uint32_t r, int j) {
                cp[r] = c0 + ccol[j];
                if (multi) ck[r] = ckey[j];
            }))
            return;
    }
    if (nc > (uint32_t)k && nc <= (uint32_t)TK_CAP) {
        // b1 crowded (many equal or near-equal scores) or the range not
        // binnable: the block select over the candidates
        const int G = nc <= (uint32_t)(4 * TPB) ? 1 : 2;
        for (int j = (int)nc + tid; j < 4 * G * TPB; j += TPB) ckey[j] = 0u;
        lds_barrier();
        // thread tid takes candidates 4 G tid + j
        uint32_t kc[8], lmin = 0xFFFFFFFFu, lmax = 0u;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const uint4 v = u < G ? *reinterpret_cast<const uint4 *>(ckey + 4 * (tid * G + u)) : uint4{0u, 0u, 0u, 0u};
            kc[4 * u] = v.x;
            kc[4 * u + 1] = v.y;
            kc[4 * u + 2] = v.z;
            kc[4 * u + 3] = v.w;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            lmin = kc[i] != 0u && kc[i] < lmin ? kc[i] : lmin;
            lmax = kc[i] > lmax ? kc[i] : lmax;
        }
        select_regs<2>(kc, G, lmin, lmax, k, sh, tid, multi, [](int) {});
        if (multi) {
            uint32_t *ck = p.cand_key + ((int64_t)it.t * p.nchunk + it.c) * k;
            int32_t *cp = p.cand_pos + ((int64_t)it.t * p.nchunk + it.c) * k;
            for (int j = tid; j < k; j += TPB) {
                ck[j] = sh.okey[j];
                cp[j] = c0 + ccol[sh.ocol[j]];
            }
        } else {
            for (int j = tid; j < k; j += TPB) out[j] = c0 + ccol[sh.ocol[j]];
        }
        return;
    }

    // 4. fallback
    int32_t *dcol = out;
    uint32_t *dkey = nullptr;
    if (multi) {
        dkey = p.cand_key + ((int64_t)it.t * p.nchunk + it.c) * k;
        dcol = p.cand_pos + ((int64_t)it.t * p.nchunk + it.c) * k;
    }
    chunk_radix_select(wsrc, wlen, nreg, wc0, k, c0, dcol, dkey, sh, wcnt);
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
    const int64_t items64 = (int64_t)T * p.nchunk;
    if (items64 > INT32_MAX) return hipErrorInvalidValue;
    const int nitems = (int)items64;
    const int grid = nitems;
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
