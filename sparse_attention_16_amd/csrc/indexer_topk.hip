// indexer_topk.hip — the fused indexer + top-k select of the DSA hot path:
// the index scores of a query row are never written to HBM.
//
// Page "Техотчёт DeepSeek-V3.2 (2025): разреженное внимание DSA и
// масштабирование RL": section "Молниеносный индексатор" defines the score
// I[t,s] (computed here by the same FP8 matrix-core code as indexer.hip, so the
// values are bit-identical), section "Отбор и основное внимание" the selection
// Top-k(I[t,:]) that feeds the attention (the k largest scores of the row,
// ties to the lower position; every visible key when there are at most k).
//
// An exact top-k of a row is only known once every score of the row is, so
// the kernels keep each row's *candidates* instead of its scores:
//   1. indexer_sample_kernel: the scores of an evenly strided sample of the
//      row's keys (512..1024 of them), and from them a threshold tau[t]: the
//      r-th largest sample score, with r = mu + 5 sqrt(mu) + 1 for the mu =
//      k * m / n sampled keys expected above the row's k-th largest score.
//      Rows that see at most 4096 keys get no threshold (every visible key).
//   2. the indexer in candidate mode (indexer.hip): every visible key with
//      score >= tau[t] goes, in column order, to the row's candidate regions
//      (score bits + position); about 1.3k .. 2.5k per row instead of n scores.
//   3. cand_select_kernel: the exact select over the candidates (the register
//      select of select_core.h).  It is exact whenever the candidates are at
//      least k and no region overflowed: then the k-th largest score of the
//      row is >= tau, so every key that can be selected is a candidate.  Rows
//      where that check fails (a threshold drawn too high, or too many equal
//      scores) are queued.
//   4. idx_fallback_kernel: each queued row is recomputed on chip: its scores,
//      32768 columns at a time, into LDS, the select of each chunk, and a merge
//      of the chunks' top-k.  Nothing of the row reaches HBM but its chunk
//      candidates.
// The sample makes the threshold a statistical guess, the check makes the
// result exact: the output is the top-k of the scores under the same total
// order as dsa_topk (score descending, position ascending, -0 == +0).
#include "indexer_core.h"
#include "select_core.h"

namespace dsa {

namespace {

constexpr int SMP_MIN = 512;        // sampled keys per row, at least ...
constexpr int SMP_MAX = 1024;       // ... and at most
constexpr int SMP_RATE = 32;        // one sampled key per this many columns, between those bounds
constexpr int NO_SAMPLE = 4096;     // rows seeing at most this many keys take every visible key
constexpr float SMP_SIGMA = 5.f;    // margin of the threshold rank, in standard deviations
constexpr int ST_ROWS = 16;         // query rows per sample workgroup (8 waves x 2)
constexpr int ST_KT = 128;          // sampled keys per LDS tile
constexpr int ST_PITCH = 144;       // LDS row pitch of a tile (16 rows of a B operand on disjoint banks)
constexpr int MAX_SEG = 512;        // candidate regions per row, at most (262144 / 512)

static_assert(MAX_SEG * CAND_DECODE_SEG >= TOPK_CHUNK * TOPK_MAX_CHUNKS, "region prefix array");
static_assert(CAND_SELECT_MAX == 4 * 4 * TPB, "select register layout");

// Offset of the strided sample of a row block (a hash of its indices; any
// value below the stride is correct).
__device__ __forceinline__ int sample_offset(int block, int seq, int stride) {
    return (int)(((uint32_t)block * 2654435761u + (uint32_t)seq * 40503u) % (uint32_t)stride);
}

// The rank-th largest of a wave's keys kr (0 = no key; 1 <= rank <= the
// number of keys): radix select on 8-bit digits from the most significant.
// Per digit, a 256-bin histogram (LDS atomics into the wave's own `hist`) of
// the keys that match the digits fixed so far, then the largest digit with at
// least `need` of them at or above it.  Equal to the largest x with
// #(keys >= x) >= rank (what a bisection on the key bits finds), in 4 rounds
// instead of 32.
template <int N>
__device__ uint32_t wave_rank_key(const uint32_t (&kr)[N], int rank, uint32_t *hist) {
    typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
    const int l = lane_id();
    uint32_t prefix = 0u, pmask = 0u;
    uint32_t need = (uint32_t)rank;
    for (int d = 3; d >= 0; --d) {
        const int sh = 8 * d;
        *reinterpret_cast<u32x4 *>(hist + 4 * l) = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const uint32_t x = kr[i];
            if (x != 0u && (x & pmask) == prefix) atomicAdd(&hist[(x >> sh) & 255u], 1u);
        }
        const u32x4 c = *reinterpret_cast<const u32x4 *>(hist + 4 * l);   // bins 4l .. 4l+3
        const uint32_t incl = wave_scan_add(c[0] + c[1] + c[2] + c[3]);
        const uint32_t above = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63) - incl;   // keys in bins > 4l+3
        const uint32_t g3 = above + c[3], g2 = g3 + c[2], g1 = g2 + c[1], g0 = g1 + c[0];
        const uint64_t m = __ballot(g0 >= need);
        if (m == 0ull) return 0u;   // (fewer keys than rank: not called so)
        const int L = 63 - (int)__builtin_clzll(m);
        const int j = g3 >= need ? 3 : (g2 >= need ? 2 : (g1 >= need ? 1 : 0));
        const uint32_t gb = j == 3 ? g3 : (j == 2 ? g2 : (j == 1 ? g1 : g0));
        const uint32_t cb = c[j];
        const int jl = __builtin_amdgcn_readlane(j, L);
        need -= (uint32_t)__builtin_amdgcn_readlane((int)gb, L) - (uint32_t)__builtin_amdgcn_readlane((int)cb, L);
        prefix |= (uint32_t)(4 * L + jl) << sh;
        pmask |= 255u << sh;
    }
    return prefix;
}

}  // namespace

// ---------------------------------------------------------------------------
// 1. Thresholds.  Grid: x = block of 16 query rows, z = sequence; 8 waves x 2
// rows as in the prefill indexer.  The block samples the keys o + i * stride,
// i < m, of its longest row (m = clamp(n / 32, 512, 1024)); each row uses the
// sampled keys it can see.  The sampled scores go to LDS as keys; each wave
// then takes the r-th largest of its rows' samples (wave_rank_key), with no
// further barrier.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(512) void indexer_sample_kernel(IdxTopkParams tp) {
    const IndexerParams &p = tp.ix;
    __shared__ __attribute__((aligned(16))) uint8_t ktile[2][ST_KT * ST_PITCH];
    __shared__ float kscale[2][ST_KT];
    __shared__ uint32_t samp[ST_ROWS][SMP_MAX];

    if (blockIdx.x == 0 && blockIdx.z == 0 && threadIdx.x == 0) {
        for (int i = 0; i < FB_LIST; ++i) tp.fb[i] = 0;   // queues empty, counts 0 (this kernel runs first)
    }
    const int b = blockIdx.z;
    const int q0 = p.cu_q[b];
    const int nq = p.cu_q[b + 1] - q0;
    const int tb = blockIdx.x * ST_ROWS;
    if (tb >= nq) return;
    int64_t kv0 = p.cu_kv[b], kv1 = p.cu_kv[b + 1];
    kv0 = kv0 < 0 ? 0 : (kv0 > p.total_kv ? p.total_kv : kv0);
    kv1 = kv1 < kv0 ? kv0 : (kv1 > p.total_kv ? p.total_kv : kv1);
    const int ctx = (int)((kv1 - kv0) > p.max_kv ? p.max_kv : (kv1 - kv0));
    const int last = (tb + ST_ROWS < nq ? tb + ST_ROWS : nq) - 1;
    int n_hi = p.pos0[b] + last + 1;
    n_hi = n_hi < 0 ? 0 : (n_hi > ctx ? ctx : n_hi);

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int l = lane_id();
    const int k = tp.k;
    bool valid[2];
    int pos[2], nvis[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int tl = tb + 2 * wave + r;
        valid[r] = tl < nq;
        pos[r] = p.pos0[b] + tl;
        const int nv = pos[r] + 1;
        nvis[r] = nv < 0 ? 0 : (nv > ctx ? ctx : nv);
    }
    if (n_hi <= NO_SAMPLE || n_hi <= k) {   // block-uniform: no row of the block needs a threshold
#pragma unroll
        for (int r = 0; r < 2; ++r)
            if (valid[r] && l == 0) tp.tau[q0 + tb + 2 * wave + r] = 0u;
        return;
    }
    int m = n_hi / SMP_RATE;
    m = m < SMP_MIN ? SMP_MIN : (m > SMP_MAX ? SMP_MAX : m);
    const int stride = n_hi / m;   // >= 4; sampled key i at o + i * stride < m * stride <= n_hi
    const int o = sample_offset(blockIdx.x, b, stride);

    i32x8 qa[2][4];
    float wq[2][4][4];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int tl = tb + 2 * wave + r;
        load_query(p, (int64_t)(q0 + (valid[r] ? tl : tb)), valid[r], qa[r], wq[r]);
    }

    // Sampled key tiles of 128 rows (1024 16-byte pieces over 512 threads),
    // double-buffered: the next tile's loads fly while this tile is scored,
    // and go from registers to the other LDS buffer after it.  A piece past
    // the m sampled keys loads the first sampled row instead: its score is
    // never stored (i < m below), and nothing touches the loaded registers
    // before their LDS write, so the wave waits for the loads only there.
    i32x4 stage[2];
    float sst = 0.f;
    auto fetch = [&](int i0) {
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
            const int c = tid + 512 * rr;
            const int key = c >> 3, byte = (c & 7) * 16;
            const int i = i0 + key;
            const int s = i < m ? o + i * stride : o;
            stage[rr] = *reinterpret_cast<const i32x4 *>(p.k + (kv0 + s) * DI + byte);
        }
        if (tid < ST_KT) sst = i0 + tid < m ? p.k_scale[kv0 + o + (i0 + tid) * stride] : 0.f;
    };
    auto put = [&](int buf) {
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
            const int c = tid + 512 * rr;
            *reinterpret_cast<i32x4 *>(&ktile[buf][(c >> 3) * ST_PITCH + (c & 7) * 16]) = stage[rr];
        }
        if (tid < ST_KT) kscale[buf][tid] = sst;
    };
    fetch(0);
    put(0);
    __syncthreads();
    int cur = 0;
    for (int i0 = 0; i0 < m; i0 += ST_KT, cur ^= 1) {
        fetch(i0 + ST_KT);   // (past the last tile: the first sampled row, into a buffer nobody reads)
        float part[2][4];
#pragma unroll
        for (int st = 0; st < ST_KT / 16; ++st) {
            const uint8_t *src = &ktile[cur][(16 * st + (l & 15)) * ST_PITCH + 32 * (l >> 4)];
            const i32x4 lo = *reinterpret_cast<const i32x4 *>(src);
            const i32x4 hi = *reinterpret_cast<const i32x4 *>(src + 16);
            const i32x8 kb = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                f32x4 c[4];
                block_mfma(qa[r], kb, c);
                part[r][st & 3] = block_epilogue(c, wq[r]);
            }
            if ((st & 3) == 3) {
                const int j = 16 * (st - 3) + l;   // lane l: sampled key i0 + j
                const int i = i0 + j;
                const int s = o + i * stride;
                const float ks = kscale[cur][j];
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    const float v = reduce_scatter4(part[r]);
                    if (i < m) samp[2 * wave + r][i] = (valid[r] && s <= pos[r]) ? score_key(v * ks) : 0u;
                }
            }
        }
        put(cur ^ 1);
        __syncthreads();
    }

#pragma unroll
    for (int r = 0; r < 2; ++r) {
        if (!valid[r]) continue;
        const int n = nvis[r];
        uint32_t kr[SMP_MAX / kWave];
        int mt = 0;   // sampled keys this row sees
#pragma unroll
        for (int j = 0; j < SMP_MAX / kWave; ++j) {
            const int i = j * kWave + l;
            kr[j] = i < m ? samp[2 * wave + r][i] : 0u;
            mt += __popcll(__ballot(kr[j] != 0u));
        }
        uint32_t tau = 0u;
        if (n > NO_SAMPLE && n > k && mt > 0) {
            const float mu = (float)k * (float)mt / (float)n;
            const int rank = (int)ceilf(mu + SMP_SIGMA * sqrtf(mu)) + 1;
            // the rank-th largest sampled key (the key tile is free now: each
            // wave's histogram takes 1 KB of it)
            if (rank <= mt) tau = wave_rank_key(kr, rank, reinterpret_cast<uint32_t *>(ktile[0]) + 256 * wave);
        }
        if (l == 0) tp.tau[q0 + tb + 2 * wave + r] = tau;
    }
}

// Threshold of one query row per workgroup (decode-shaped batches, where a
// sequence has a single query row and a 16-row block would score 15 empty
// rows).  Same sample grid as above for a block of one row (so the same
// threshold); the 8 waves each gather and score 128 sampled keys in one pass
// (B operands loaded straight into registers), wave 0 selects.  Grid: x = row.
__global__ __launch_bounds__(512) void indexer_sample_row_kernel(IdxTopkParams tp) {
    const IndexerParams &p = tp.ix;
    __shared__ uint32_t samp[SMP_MAX];
    __shared__ __attribute__((aligned(16))) uint32_t hist[256];
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        for (int i = 0; i < FB_LIST; ++i) tp.fb[i] = 0;   // queues empty, counts 0 (this kernel runs first)
    }
    const int t = blockIdx.x;
    // the row's sequence and visible keys (row_info's arithmetic, from one
    // search of cu_q: the sample offset needs the sequence as well)
    const int b = find_seq(p.cu_q, p.B, t);
    int n;
    int64_t kv0;
    {
        int64_t a = p.cu_kv[b], e = p.cu_kv[b + 1];
        a = a < 0 ? 0 : (a > p.total_kv ? p.total_kv : a);
        e = e < a ? a : (e > p.total_kv ? p.total_kv : e);
        const int64_t c = e - a;
        const int ctx = (int)(c > p.max_kv ? p.max_kv : c);
        const int nv = p.pos0[b] + (t - p.cu_q[b]) + 1;
        n = nv < 0 ? 0 : (nv > ctx ? ctx : nv);
        kv0 = a;
    }
    const int k = tp.k;
    const int tid = threadIdx.x, wave = tid >> 6, l = lane_id();
    if (n <= NO_SAMPLE || n <= k) {
        if (tid == 0) tp.tau[t] = 0u;
        return;
    }
    const int block = (t - p.cu_q[b]) / ST_ROWS;
    int m = n / SMP_RATE;
    m = m < SMP_MIN ? SMP_MIN : (m > SMP_MAX ? SMP_MAX : m);
    const int stride = n / m;
    const int o = sample_offset(block, b, stride);
    i32x8 qa[4];
    float wq[4][4];
    load_query(p, t, true, qa, wq);
    // wave w: sampled keys 128w + 16st + (l & 15), st < 8; all gathers first
    i32x8 kb[8];
#pragma unroll
    for (int st = 0; st < 8; ++st) {
        const int i = 128 * wave + 16 * st + (l & 15);
        const int s = i < m ? o + i * stride : o;
        const uint8_t *src = p.k + (kv0 + s) * DI + 32 * (l >> 4);
        const i32x4 lo = *reinterpret_cast<const i32x4 *>(src);
        const i32x4 hi = *reinterpret_cast<const i32x4 *>(src + 16);
        kb[st] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    float ks[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int i = 128 * wave + 64 * h + l;
        ks[h] = i < m ? p.k_scale[kv0 + o + i * stride] : 0.f;
    }
    float part[4];
#pragma unroll
    for (int st = 0; st < 8; ++st) {
        f32x4 c[4];
        block_mfma(qa, kb[st], c);
        part[st & 3] = block_epilogue(c, wq);
        if ((st & 3) == 3) {
            const int h = st >> 2;
            const int i = 128 * wave + 64 * h + l;
            const float v = reduce_scatter4(part);
            if (i < SMP_MAX) samp[i] = i < m ? score_key(v * ks[h]) : 0u;
        }
    }
    __syncthreads();
    if (wave != 0) return;
    uint32_t kr[SMP_MAX / kWave];
#pragma unroll
    for (int j = 0; j < SMP_MAX / kWave; ++j) kr[j] = samp[j * kWave + l];
    const float mu = (float)k * (float)m / (float)n;
    const int rank = (int)ceilf(mu + SMP_SIGMA * sqrtf(mu)) + 1;
    const uint32_t tau = rank <= m ? wave_rank_key(kr, rank, hist) : 0u;
    if (l == 0) tp.tau[t] = tau;
}

// ---------------------------------------------------------------------------
// 3. Exact select over a row's candidates.
//
// cand_select_wave_kernel: one wave per query row, no barriers.  The
// region counts give the row's candidate array (the non-empty regions in
// order, in per-wave LDS), each lane loads a run of consecutive candidates
// as keys (lane-major order = column order; at most 4096 per row), the k-th
// largest key kappa comes from a bisection on the key bits (ballot counts),
// and each lane writes its selected positions (keys > kappa, then the first
// keys == kappa in column order up to k) at its scanned offset: ascending.
// Rows with more candidates go to a queue for the workgroup select below;
// rows whose candidates cannot be complete go to the recompute queue.
// ---------------------------------------------------------------------------
constexpr int SEL_WAVES = 4;        // rows per workgroup of the wave select
constexpr int SEL_R = 64;           // candidates per lane, at most (the contiguous select)
constexpr int SEL_WAVE_MAX = SEL_R * kWave;
// The multi-region select holds RR candidates per lane, its taken-register
// mask in two words: 64 for contexts up to 32768 keys (rows keep ~3.4k
// candidates), 88 beyond (~3.9k at 64K, ~4.7k at 128K, which would overflow
// 64 and go to the workgroup select; 88 still fits two waves per SIMD).
constexpr int SEL_R_LONG = 88;
constexpr int SEL_LONG_CTX = 32768;   // longest context that takes the 64-register select
static_assert(SEL_R <= 64 && SEL_R_LONG <= 128, "taken-register masks");
constexpr int SEL_BINS = 256;      // value bins of the wave select's histogram
constexpr int SEL_BLOCK_ROWS = 4;   // batches of at most this many rows per compute unit: workgroup select

namespace {

// Exclusive prefix over the wave's lanes (DPP inclusive scan minus own).
__device__ __forceinline__ uint32_t wave_excl_add(uint32_t v) { return wave_scan_add(v) - v; }

}  // namespace

template <int SEL_R_MR>
__global__ __launch_bounds__(64 * SEL_WAVES) void cand_select_wave_kernel(IdxTopkParams tp, int T) {
    constexpr int SEL_WAVE_MAX_MR = SEL_R_MR * kWave;
    const IndexerParams &p = tp.ix;
    __shared__ int32_t npre_s[SEL_WAVES][MAX_SEG + 1];
    __shared__ int16_t nreg_s[SEL_WAVES][MAX_SEG];
    __shared__ uint32_t hist_s[SEL_WAVES][SEL_BINS];
    __shared__ uint32_t list_s[SEL_WAVES][kWave];
    const int wave = threadIdx.x >> 6, l = lane_id(), k = tp.k;
    const int t = blockIdx.x * SEL_WAVES + wave;
    if (t >= T) return;
    int32_t *npre = npre_s[wave];
    int16_t *nreg = nreg_s[wave];
    const RowInfo ri = row_info(p.cu_q, p.cu_kv, p.pos0, p.B, p.total_kv, p.max_kv, t);
    const int n = ri.nvis;
    int32_t *out = tp.idx + (int64_t)t * k;
    if (n <= k) {   // every visible key, ascending, then -1
        for (int j = l; j < k; j += kWave) out[j] = j < n ? j : -1;
        return;
    }
    // the row's non-empty regions: npre[e] = first candidate, nreg[e] = region
    const int nseg_t = (n + p.seg_w - 1) / p.seg_w;
    const int64_t rows0 = (int64_t)t * p.nseg;
    uint32_t off = 0, nr = 0;
    bool ovf = false;
    for (int base = 0; base < nseg_t; base += kWave) {
        const int r = base + l;
        int cnt = r < nseg_t ? p.cand_cnt[rows0 + r] : 0;
        if (cnt > p.cap || cnt < 0) {
            ovf = true;
            cnt = 0;
        }
        const uint32_t incl = wave_scan_add((uint32_t)cnt);
        const uint64_t nz = __ballot(cnt > 0);
        const int rank = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(nz >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)nz, 0u));
        if (cnt > 0) {
            npre[nr + rank] = (int32_t)(off + incl - (uint32_t)cnt);
            nreg[nr + rank] = (int16_t)r;
        }
        off += (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
        nr += (uint32_t)__popcll(nz);
    }
    if (l == 0) npre[nr] = (int32_t)off;
    const int c = (int)off;
    const uint32_t tau = tp.tau[t];
    if (__ballot(ovf) != 0ull || (tau != 0u && c < k) || (tau == 0u && c != n) || c > CAND_SELECT_MAX) {
        if (l == 0) {
            const int slot = atomicAdd(&tp.fb[0], 1);
            tp.fb[FB_LIST + slot] = t;
        }
        return;
    }
    if (l == 0) atomicAdd(&tp.fb[2], c);
    if (c > SEL_WAVE_MAX_MR) {   // too many for one wave's registers: the workgroup select takes it
        if (l == 0) {
            const int slot = atomicAdd(&tp.fb[3], 1);
            tp.fb[FB_LIST + T + slot] = t;
        }
        return;
    }
    // lane l: candidates l*R .. l*R + R - 1 (R = ceil(c / 64)), in column order
    const int R = (c + kWave - 1) / kWave;
    const int j0 = l * R;
    auto entry_of = [&](int j) {
        int lo = 0, hi = (int)nr - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (npre[mid] <= j) lo = mid; else hi = mid - 1;
        }
        return lo;
    };
    const int e0 = j0 < c ? entry_of(j0) : 0;
    const int64_t a_safe = (rows0 + nreg[0]) * p.cap;   // a valid slot (the first candidate)
    // Slot of each of this lane's candidates, walking the (non-empty) regions
    // forward: consecutive candidates cross at most one boundary.  The loads
    // are all issued before any of their values is used.
    uint32_t kr[SEL_R_MR];
    if (nr == 1) {   // the whole row in one region (prefill layout): consecutive slots
#pragma unroll
        for (int i = 0; i < SEL_R_MR; ++i) {
            const int j = j0 + i;
            kr[i] = p.cand_key[i < R && j < c ? a_safe + j : a_safe];
        }
    } else {
        int e = e0, bnd = npre[e0 + 1];
        int64_t dlt = (rows0 + nreg[e0]) * p.cap - npre[e0];
#pragma unroll
        for (int i = 0; i < SEL_R_MR; ++i) {
            const int j = j0 + i;
            const bool in = i < R && j < c;
            if (in && j >= bnd) {
                ++e;
                bnd = npre[e + 1];
                dlt = (rows0 + nreg[e]) * p.cap - npre[e];
            }
            kr[i] = p.cand_key[in ? dlt + j : a_safe];
        }
    }
#pragma unroll
    for (int i = 0; i < SEL_R_MR; ++i) kr[i] = (i < R && j0 + i < c) ? score_key(__uint_as_float(kr[i])) : 0u;
    // kappa, the k-th largest key.  A 256-bin histogram of the keys by value
    // over [min, max] (a non-decreasing map, so bins keep the order) names the
    // bin b1 that holds it; b1's keys (a few dozen on spread-out scores) are
    // gathered into one register per lane and bisected.  A range that cannot
    // be binned, or a crowded b1 (many equal scores), takes the bisection over
    // all keys instead.
    uint32_t kappa = 0u;
    bool found = false;
    {
        uint32_t lmn = 0xFFFFFFFFu, lmx = 0u;
#pragma unroll
        for (int i = 0; i < SEL_R_MR; ++i) {
            lmn = kr[i] != 0u && kr[i] < lmn ? kr[i] : lmn;
            lmx = kr[i] > lmx ? kr[i] : lmx;
        }
        const uint32_t kmin = (uint32_t)__builtin_amdgcn_readlane(
            (int)wave_scan(lmn, 0xFFFFFFFFu, [](uint32_t a, uint32_t b2) { return a < b2 ? a : b2; }), 63);
        const uint32_t kmax = (uint32_t)__builtin_amdgcn_readlane(
            (int)wave_scan(lmx, 0u, [](uint32_t a, uint32_t b2) { return a > b2 ? a : b2; }), 63);
        const float vmin = key_value(kmin), vmax = key_value(kmax);
        const float range = vmax - vmin;
        const float inv = (float)SEL_BINS / range;
        if (range > 0.f && range < INFINITY && inv < INFINITY) {
            uint32_t *hist = hist_s[wave];
#pragma unroll
            for (int q = 0; q < SEL_BINS / kWave; ++q) hist[q * kWave + l] = 0u;
            auto bin_of = [&](uint32_t key) {
                return (uint32_t)fminf((key_value(key) - vmin) * inv, (float)(SEL_BINS - 1));
            };
#pragma unroll
            for (int i = 0; i < SEL_R_MR; ++i)
                if (kr[i] != 0u) atomicAdd(&hist[bin_of(kr[i])], 1u);
            // lane l owns bins top - 4l - q (q < 4), scanned from the top
            uint32_t c4[SEL_BINS / kWave], sum = 0;
#pragma unroll
            for (int q = 0; q < SEL_BINS / kWave; ++q) {
                c4[q] = hist[SEL_BINS - 1 - (SEL_BINS / kWave) * l - q];
                sum += c4[q];
            }
            uint32_t above = wave_excl_add(sum);
            int my_b1 = -1;
            uint32_t my_rem = 0;
#pragma unroll
            for (int q = 0; q < SEL_BINS / kWave; ++q) {
                if (above < (uint32_t)k && (uint32_t)k <= above + c4[q]) {
                    my_b1 = SEL_BINS - 1 - (SEL_BINS / kWave) * l - q;
                    my_rem = (uint32_t)k - above;
                }
                above += c4[q];
            }
            const uint64_t own = __ballot(my_b1 >= 0);   // exactly one lane
            const int src = (int)__builtin_ctzll(own);
            const uint32_t b1 = (uint32_t)__builtin_amdgcn_readlane(my_b1, src);
            const uint32_t rem = (uint32_t)__builtin_amdgcn_readlane((int)my_rem, src);
            const uint32_t nb1 = hist[b1];
            if (nb1 <= (uint32_t)kWave) {
                uint32_t *lst = list_s[wave];
                uint32_t cnt = 0;
#pragma unroll
                for (int i = 0; i < SEL_R_MR; ++i) {
                    const bool inb = kr[i] != 0u && bin_of(kr[i]) == b1;
                    const uint64_t m = __ballot(inb);
                    if (inb) {
                        const uint32_t r2 = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                                      __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
                        lst[cnt + r2] = kr[i];
                    }
                    cnt += (uint32_t)__popcll(m);
                }
                const uint32_t xk = (uint32_t)l < nb1 ? lst[l] : 0u;
                // the rem-th largest of b1's keys
                uint32_t x = 0u;
                for (int bit = 31; bit >= 0; --bit) {
                    const uint32_t y = x | (1u << bit);
                    if ((uint32_t)__popcll(__ballot(xk >= y)) >= rem) x = y;
                }
                kappa = x;
                found = true;
            }
        }
    }
    if (!found) {
        // the largest x with #(keys >= x) >= k, i.e. the k-th largest key
        uint32_t x = 0u;
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t y = x | (1u << bit);
            int cnt = 0;
#pragma unroll
            for (int i = 0; i < SEL_R_MR; ++i) cnt += __popcll(__ballot(kr[i] >= y));
            if (cnt >= k) x = y;
        }
        kappa = x;
    }
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int i = 0; i < SEL_R_MR; ++i) {
        gt += kr[i] > kappa ? 1u : 0u;
        eq += kr[i] == kappa ? 1u : 0u;
    }
    // keys == kappa taken in column order until k are selected
    const uint32_t gt_all = (uint32_t)__builtin_amdgcn_readlane((int)wave_scan_add(gt), 63);
    const uint32_t need_eq = (uint32_t)k - gt_all;
    const uint32_t eq_before = wave_excl_add(eq);
    uint32_t eq_take = need_eq > eq_before ? need_eq - eq_before : 0u;
    eq_take = eq_take < eq ? eq_take : eq;
    uint32_t slot = wave_excl_add(gt + eq_take);
    // selected candidates as a bit mask, then their positions (loads first,
    // into the key registers), then the ascending writes
    uint64_t take[2] = {0ull, 0ull};   // bit i % 64 of word i / 64: register i taken
#pragma unroll
    for (int i = 0; i < SEL_R_MR; ++i) {
        bool tk = kr[i] > kappa;
        if (kr[i] == kappa && eq_take != 0u) {
            tk = true;
            --eq_take;
        }
        take[i / 64] |= (uint64_t)(tk ? 1u : 0u) << (i % 64);
    }
    if (nr == 1) {
#pragma unroll
        for (int i = 0; i < SEL_R_MR; ++i) kr[i] = (uint32_t)p.cand_pos[(take[i / 64] >> (i % 64)) & 1ull ? a_safe + j0 + i : a_safe];
    } else {
        int e = e0, bnd = npre[e0 + 1];
        int64_t dlt = (rows0 + nreg[e0]) * p.cap - npre[e0];
#pragma unroll
        for (int i = 0; i < SEL_R_MR; ++i) {
            const int j = j0 + i;
            const bool in = i < R && j < c;
            if (in && j >= bnd) {
                ++e;
                bnd = npre[e + 1];
                dlt = (rows0 + nreg[e]) * p.cap - npre[e];
            }
            kr[i] = (uint32_t)p.cand_pos[(take[i / 64] >> (i % 64)) & 1ull ? dlt + j : a_safe];
        }
    }
#pragma unroll
    for (int i = 0; i < SEL_R_MR; ++i)
        if ((take[i / 64] >> (i % 64)) & 1ull) out[slot++] = (int32_t)kr[i];
}

// cand_select_wave_contig_kernel: the same select with candidate j = 64 i + l
// in register i of lane l, so that each load and store instruction covers 64
// consecutive candidates ((register, lane) order is column order).  Launched
// when every row has one candidate region (a candidate's slot is then the
// region's base + j; with several regions finding a candidate's region costs
// more than the lane-run layout's forward walk, so such batches take the
// kernel above).
__global__ __launch_bounds__(64 * SEL_WAVES) void cand_select_wave_contig_kernel(IdxTopkParams tp, int T) {
    const IndexerParams &p = tp.ix;
    __shared__ int32_t npre_s[SEL_WAVES][MAX_SEG + 1];
    __shared__ int16_t nreg_s[SEL_WAVES][MAX_SEG];
    __shared__ uint32_t hist_s[SEL_WAVES][SEL_BINS];
    __shared__ uint32_t list_s[SEL_WAVES][kWave];
    const int wave = threadIdx.x >> 6, l = lane_id(), k = tp.k;
    const int t = blockIdx.x * SEL_WAVES + wave;
    if (t >= T) return;
    int32_t *npre = npre_s[wave];
    int16_t *nreg = nreg_s[wave];
    const RowInfo ri = row_info(p.cu_q, p.cu_kv, p.pos0, p.B, p.total_kv, p.max_kv, t);
    const int n = ri.nvis;
    int32_t *out = tp.idx + (int64_t)t * k;
    if (n <= k) {   // every visible key, ascending, then -1
        for (int j = l; j < k; j += kWave) out[j] = j < n ? j : -1;
        return;
    }
    // the row's non-empty regions: npre[e] = first candidate, nreg[e] = region
    const int nseg_t = (n + p.seg_w - 1) / p.seg_w;
    const int64_t rows0 = (int64_t)t * p.nseg;
    uint32_t off = 0, nr = 0;
    bool ovf = false;
    for (int base = 0; base < nseg_t; base += kWave) {
        const int r = base + l;
        int cnt = r < nseg_t ? p.cand_cnt[rows0 + r] : 0;
        if (cnt > p.cap || cnt < 0) {
            ovf = true;
            cnt = 0;
        }
        const uint32_t incl = wave_scan_add((uint32_t)cnt);
        const uint64_t nz = __ballot(cnt > 0);
        const int rank = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(nz >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)nz, 0u));
        if (cnt > 0) {
            npre[nr + rank] = (int32_t)(off + incl - (uint32_t)cnt);
            nreg[nr + rank] = (int16_t)r;
        }
        off += (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
        nr += (uint32_t)__popcll(nz);
    }
    if (l == 0) npre[nr] = (int32_t)off;
    const int c = (int)off;
    const uint32_t tau = tp.tau[t];
    if (__ballot(ovf) != 0ull || (tau != 0u && c < k) || (tau == 0u && c != n) || c > CAND_SELECT_MAX) {
        if (l == 0) {
            const int slot = atomicAdd(&tp.fb[0], 1);
            tp.fb[FB_LIST + slot] = t;
        }
        return;
    }
    if (l == 0) atomicAdd(&tp.fb[2], c);
    if (c > SEL_WAVE_MAX) {   // too many for one wave's registers: the workgroup select takes it
        if (l == 0) {
            const int slot = atomicAdd(&tp.fb[3], 1);
            tp.fb[FB_LIST + T + slot] = t;
        }
        return;
    }
    // Candidate j = 64 i + l is register i of lane l (R = ceil(c / 64)
    // registers in use): each load instruction reads 64 consecutive
    // candidates, and (register, lane) order is column order.  The row has one
    // region (the kernel is launched for one region per row), so candidate j
    // sits at the region's base + j; the candidate arrays are padded by 64
    // slots, so a register's 64 loads stay inside them even past the row's
    // last candidate (values there are discarded), and every load is a fixed
    // offset from one lane address.  (The loads are all issued before any of
    // their values is used.)
    const int R = __builtin_amdgcn_readfirstlane((c + kWave - 1) / kWave);   // (wave-uniform: scalar branches below)
    const int64_t a_safe = (rows0 + nreg[0]) * p.cap;   // the region's first slot
    const uint32_t *ckey = p.cand_key + a_safe;
    const int32_t *cpos = p.cand_pos + a_safe;
    uint32_t kr[SEL_R];
#pragma unroll
    for (int i = 0; i < SEL_R; ++i) kr[i] = i < R ? ckey[kWave * i + l] : 0u;
#pragma unroll
    for (int i = 0; i < SEL_R; ++i) kr[i] = (i < R && kWave * i + l < c) ? score_key(__uint_as_float(kr[i])) : 0u;
    // kappa, the k-th largest key.  A 256-bin histogram of the keys by value
    // over [min, max] (a non-decreasing map, so bins keep the order) names the
    // bin b1 that holds it; b1's keys (a few dozen on spread-out scores) are
    // gathered into one register per lane and bisected.  A range that cannot
    // be binned, or a crowded b1 (many equal scores), takes the bisection over
    // all keys instead.
    uint32_t kappa = 0u;
    bool found = false;
    {
        uint32_t lmn = 0xFFFFFFFFu, lmx = 0u;
#pragma unroll
        for (int i = 0; i < SEL_R; ++i) {
            lmn = kr[i] != 0u && kr[i] < lmn ? kr[i] : lmn;
            lmx = kr[i] > lmx ? kr[i] : lmx;
        }
        const uint32_t kmin = (uint32_t)__builtin_amdgcn_readlane(
            (int)wave_scan(lmn, 0xFFFFFFFFu, [](uint32_t a, uint32_t b2) { return a < b2 ? a : b2; }), 63);
        const uint32_t kmax = (uint32_t)__builtin_amdgcn_readlane(
            (int)wave_scan(lmx, 0u, [](uint32_t a, uint32_t b2) { return a > b2 ? a : b2; }), 63);
        const float vmin = key_value(kmin), vmax = key_value(kmax);
        const float range = vmax - vmin;
        const float inv = (float)SEL_BINS / range;
        if (range > 0.f && range < INFINITY && inv < INFINITY) {
            uint32_t *hist = hist_s[wave];
#pragma unroll
            for (int q = 0; q < SEL_BINS / kWave; ++q) hist[q * kWave + l] = 0u;
            auto bin_of = [&](uint32_t key) {
                return (uint32_t)fminf((key_value(key) - vmin) * inv, (float)(SEL_BINS - 1));
            };
#pragma unroll
            for (int i = 0; i < SEL_R; ++i)
                if (kr[i] != 0u) atomicAdd(&hist[bin_of(kr[i])], 1u);
            // lane l owns bins top - 4l - q (q < 4), scanned from the top
            uint32_t c4[SEL_BINS / kWave], sum = 0;
#pragma unroll
            for (int q = 0; q < SEL_BINS / kWave; ++q) {
                c4[q] = hist[SEL_BINS - 1 - (SEL_BINS / kWave) * l - q];
                sum += c4[q];
            }
            uint32_t above = wave_excl_add(sum);
            int my_b1 = -1;
            uint32_t my_rem = 0;
#pragma unroll
            for (int q = 0; q < SEL_BINS / kWave; ++q) {
                if (above < (uint32_t)k && (uint32_t)k <= above + c4[q]) {
                    my_b1 = SEL_BINS - 1 - (SEL_BINS / kWave) * l - q;
                    my_rem = (uint32_t)k - above;
                }
                above += c4[q];
            }
            const uint64_t own = __ballot(my_b1 >= 0);   // exactly one lane
            const int src = (int)__builtin_ctzll(own);
            const uint32_t b1 = (uint32_t)__builtin_amdgcn_readlane(my_b1, src);
            const uint32_t rem = (uint32_t)__builtin_amdgcn_readlane((int)my_rem, src);
            const uint32_t nb1 = hist[b1];
            if (nb1 <= (uint32_t)kWave) {
                uint32_t *lst = list_s[wave];
                uint32_t cnt = 0;
#pragma unroll
                for (int i = 0; i < SEL_R; ++i) {
                    const bool inb = kr[i] != 0u && bin_of(kr[i]) == b1;
                    const uint64_t m = __ballot(inb);
                    if (inb) {
                        const uint32_t r2 = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                                      __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
                        lst[cnt + r2] = kr[i];
                    }
                    cnt += (uint32_t)__popcll(m);
                }
                const uint32_t xk = (uint32_t)l < nb1 ? lst[l] : 0u;
                // the rem-th largest of b1's keys
                uint32_t x = 0u;
                for (int bit = 31; bit >= 0; --bit) {
                    const uint32_t y = x | (1u << bit);
                    if ((uint32_t)__popcll(__ballot(xk >= y)) >= rem) x = y;
                }
                kappa = x;
                found = true;
            }
        }
    }
    if (!found) {
        // the largest x with #(keys >= x) >= k, i.e. the k-th largest key
        uint32_t x = 0u;
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t y = x | (1u << bit);
            int cnt = 0;
#pragma unroll
            for (int i = 0; i < SEL_R; ++i) cnt += __popcll(__ballot(kr[i] >= y));
            if (cnt >= k) x = y;
        }
        kappa = x;
    }
    // keys > kappa, then keys == kappa in column order until k are selected
    uint32_t gt = 0;
#pragma unroll
    for (int i = 0; i < SEL_R; ++i) gt += kr[i] > kappa ? 1u : 0u;
    const uint32_t gt_all = (uint32_t)__builtin_amdgcn_readlane((int)wave_scan_add(gt), 63);
    uint32_t eq_left = (uint32_t)k - gt_all;
    uint64_t take = 0ull;
#pragma unroll
    for (int i = 0; i < SEL_R; ++i) {
        const bool e = kr[i] == kappa;
        const uint64_t me = __ballot(e);
        const uint32_t er = __builtin_amdgcn_mbcnt_hi((uint32_t)(me >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)me, 0u));
        const bool tk = kr[i] > kappa || (e && er < eq_left);
        const uint32_t ne = (uint32_t)__popcll(me);
        eq_left -= ne < eq_left ? ne : eq_left;
        take |= (uint64_t)(tk ? 1u : 0u) << i;
    }
    // the selected candidates' positions (loads first, into the key
    // registers), then the writes in (register, lane) order: ascending
#pragma unroll
    for (int i = 0; i < SEL_R; ++i) kr[i] = (take >> i) & 1ull ? (uint32_t)cpos[kWave * i + l] : 0u;
    uint32_t base = 0;
#pragma unroll
    for (int i = 0; i < SEL_R; ++i) {
        const bool tk = (take >> i) & 1ull;
        const uint64_t mt = __ballot(tk);
        const uint32_t r = __builtin_amdgcn_mbcnt_hi((uint32_t)(mt >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mt, 0u));
        if (tk) out[base + r] = (int32_t)kr[i];
        base += (uint32_t)__popcll(mt);
    }
}

// cand_select_kernel: the register select of select_core.h over one row's
// candidates (up to 16384) per 1024-thread workgroup.  Two modes: every row
// (grid = rows; batches of few rows, e.g. decode, where one workgroup per row
// is faster than one wave), with the completeness checks; or the rows the wave
// select queued (persistent workgroups, checks already done).  The candidates
// are loaded 4G per thread (G <= 4); positions are looked up afterwards.
__global__ __launch_bounds__(TPB, 2) void cand_select_kernel(IdxTopkParams tp, int T, int from_queue) {
    const IndexerParams &p = tp.ix;
    __shared__ SelectShared sh;
    __shared__ int32_t npre[MAX_SEG + 1];
    __shared__ int16_t nreg[MAX_SEG];
    __shared__ int next, nnz, fail;
    const int tid = threadIdx.x, k = tp.k;
    const int queued = from_queue ? *static_cast<volatile int32_t *>(&tp.fb[3]) : 1;
    if (queued == 0) return;
    for (int it = 0;; ++it) {
        int t;
        if (from_queue) {
            if (tid == 0) next = atomicAdd(&tp.fb[4], 1);
            lds_barrier();
            const int qi = next;
            lds_barrier();
            if (qi >= queued) break;
            t = tp.fb[FB_LIST + T + qi];
        } else {
            if (it > 0) break;
            t = blockIdx.x;
        }
        const RowInfo ri = row_info(p.cu_q, p.cu_kv, p.pos0, p.B, p.total_kv, p.max_kv, t);
        const int n = ri.nvis;
        int32_t *out = tp.idx + (int64_t)t * k;
        if (n <= k) {   // (every-row mode) every visible key, ascending, then -1
            for (int j = tid; j < k; j += TPB) out[j] = j < n ? j : -1;
            continue;
        }
        const int nseg_t = (n + p.seg_w - 1) / p.seg_w;
        const int64_t rows0 = (int64_t)t * p.nseg;
        int cv = tid < nseg_t ? p.cand_cnt[rows0 + tid] : 0;
        const bool ovf = cv > p.cap || cv < 0;
        cv = ovf ? 0 : cv;
        if (tid == 0) fail = 0;
        lds_barrier();
        if (ovf) fail = 1;
        const uint32_t off = block_excl_scan((uint32_t)cv, sh.wtot);
        const uint32_t nz = block_excl_scan(cv > 0 ? 1u : 0u, sh.wtot);
        if (cv > 0) {
            npre[nz] = (int32_t)off;
            nreg[nz] = (int16_t)tid;
        }
        if (tid == nseg_t - 1) {
            npre[nz + (cv > 0 ? 1 : 0)] = (int32_t)(off + cv);
            nnz = (int)nz + (cv > 0 ? 1 : 0);
        }
        lds_barrier();
        const int nr = nnz;
        const int c = npre[nr];
        if (!from_queue) {
            // exact only if every key that can be selected is a candidate
            const uint32_t tau = tp.tau[t];
            if (fail || (tau != 0u && c < k) || (tau == 0u && c != n) || c > CAND_SELECT_MAX) {
                if (tid == 0) {
                    const int slot = atomicAdd(&tp.fb[0], 1);
                    tp.fb[FB_LIST + slot] = t;
                }
                continue;
            }
            if (tid == 0) atomicAdd(&tp.fb[2], c);
        }
        auto entry_of = [&](int j) {
            int lo = 0, hi = nr - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (npre[mid] <= j) lo = mid; else hi = mid - 1;
            }
            return lo;
        };
        auto slot_of = [&](int j, int e) { return (rows0 + nreg[e]) * p.cap + (j - npre[e]); };
        // thread tid: candidates 4G*tid .. 4G*tid + 4G - 1 of the row (column order)
        const int G = (c + 4 * TPB - 1) / (4 * TPB);
        const int j0 = 4 * G * tid;
        int e = j0 < c ? entry_of(j0) : 0;
        uint32_t kr[16], lmin = 0xFFFFFFFFu, lmax = 0u;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int j = j0 + i;
            const bool in = i / 4 < G && j < c;
            e += (in && j >= npre[e + 1]) ? 1 : 0;
            kr[i] = in ? score_key(__uint_as_float(p.cand_key[slot_of(j, e)])) : 0u;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            lmin = kr[i] != 0u && kr[i] < lmin ? kr[i] : lmin;
            lmax = kr[i] > lmax ? kr[i] : lmax;
        }
        select_regs<4>(kr, G, lmin, lmax, k, sh, tid, false, [](int) {});
        // sh.ocol: the selected candidates' indices, ascending (= column order)
        for (int j = tid; j < k; j += TPB) {
            const int cj = sh.ocol[j];
            out[j] = p.cand_pos[slot_of(cj, entry_of(cj))];
        }
        lds_barrier();   // sh, npre free for the next row
    }
}

// ---------------------------------------------------------------------------
// 4. Recompute of the queued rows.  Persistent workgroups take rows from the
// queue; per row, each 32768-column chunk is scored into LDS (16 waves, 64-key
// groups, the same MFMA and epilogue as the indexer), then selected like the
// top-k chunk kernel.  A row of one chunk writes its idx directly; longer rows
// keep each chunk's top-k (key, position) in the row's own candidate area,
// and a final register select merges them (exact: the union of the chunks'
// top-k sets under one total order holds the row's top-k).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(TPB) void idx_fallback_kernel(IdxTopkParams tp) {
    const IndexerParams &p = tp.ix;
    __shared__ __attribute__((aligned(16))) float stage[TOPK_CHUNK];
    __shared__ SelectShared sh;
    __shared__ int next;
    const int tid = threadIdx.x, k = tp.k;
    const int wave = tid >> 6, l = lane_id();
    const int queued = *static_cast<volatile int32_t *>(&tp.fb[0]);
    if (queued == 0) return;   // (the usual case: every row's candidates were complete)
    for (;;) {
        if (tid == 0) next = atomicAdd(&tp.fb[1], 1);
        lds_barrier();
        const int qi = next;
        lds_barrier();
        if (qi >= queued) break;
        const int t = tp.fb[FB_LIST + qi];
        const RowInfo ri = row_info(p.cu_q, p.cu_kv, p.pos0, p.B, p.total_kv, p.max_kv, t);
        const int n = ri.nvis;   // > k: only such rows are queued
        const int nch = (n + TOPK_CHUNK - 1) / TOPK_CHUNK;
        int32_t *out = tp.idx + (int64_t)t * k;
        const int64_t cbase = (int64_t)t * p.nseg * p.cap;   // the row's candidate area (>= nch * k slots)
        uint32_t *ck = p.cand_key + cbase;
        int32_t *cp = p.cand_pos + cbase;
        for (int ch = 0; ch < nch; ++ch) {
            const int c0 = ch * TOPK_CHUNK;
            const int len = n - c0 < TOPK_CHUNK ? n - c0 : TOPK_CHUNK;
            {   // scores of columns [c0, c0 + len): wave w takes the 64-key groups w, w + 16, ...
                i32x8 qa[4];
                float wq[4][4];
                load_query(p, t, true, qa, wq);
                for (int g = wave; 64 * g < len; g += TPB / kWave) {
                    float part[4];
#pragma unroll
                    for (int bb = 0; bb < 4; ++bb) {
                        const int key = c0 + 64 * g + 16 * bb + (l & 15);
                        const int kc = key < c0 + len ? key : c0;
                        const uint8_t *src = p.k + (ri.kv0 + kc) * DI + 32 * (l >> 4);
                        const i32x4 lo = *reinterpret_cast<const i32x4 *>(src);
                        const i32x4 hi = *reinterpret_cast<const i32x4 *>(src + 16);
                        const i32x8 kb = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                        f32x4 c[4];
                        block_mfma(qa, kb, c);
                        part[bb] = block_epilogue(c, wq);
                    }
                    const float v = reduce_scatter4(part);
                    const int key = c0 + 64 * g + l;
                    if (key < c0 + len) stage[key - c0] = v * p.k_scale[ri.kv0 + key];
                }
            }
            lds_barrier();
            if (nch > 1 && len <= k) {
                // the whole (last) chunk is its own top-k: in column order, padded
                for (int j = tid; j < k; j += TPB) {
                    ck[ch * k + j] = j < len ? score_key(stage[j]) : 0u;
                    cp[ch * k + j] = j < len ? c0 + j : -1;
                }
            } else {
                // keys from the stage, thread tz holding the 4G consecutive columns
                // 4G*tz + j (G odd: the 16-byte LDS reads of a wave hit distinct banks)
                const int tz = tid;
                const int ngroups = (len + 4 * TPB - 1) / (4 * TPB);
                const int G = ngroups < CH_V4 ? (ngroups | 1) : CH_V4;
                const int lim = 4 * G * (tz + 1) < len ? 4 * G * (tz + 1) : len;
                uint32_t kr[4 * CH_V4], lmin = 0xFFFFFFFFu, lmax = 0u;
#pragma unroll
                for (int u = 0; u < CH_V4; ++u) {
                    const int cc = 4 * (tz * G + u);
                    const float4 f4 = (u < G && cc < TOPK_CHUNK) ? *reinterpret_cast<const float4 *>(stage + cc)
                                                                  : float4{0.f, 0.f, 0.f, 0.f};
                    const float f[4] = {f4.x, f4.y, f4.z, f4.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t key = score_key(f[i]) & (0u - (uint32_t)(cc + i < lim));
                        kr[4 * u + i] = key;
                        lmin = key != 0u && key < lmin ? key : lmin;
                        lmax = key > lmax ? key : lmax;
                    }
                }
                select_regs<CH_V4>(kr, G, lmin, lmax, k, sh, tz, nch > 1, [](int) {});
                if (nch == 1) {
                    for (int j = tid; j < k; j += TPB) out[j] = sh.ocol[j];
                } else {
                    for (int j = tid; j < k; j += TPB) {
                        ck[ch * k + j] = sh.okey[j];
                        cp[ch * k + j] = c0 + sh.ocol[j];
                    }
                }
            }
            lds_barrier();   // stage and sh free for the next chunk
        }
        if (nch > 1) {
            // merge the chunks' candidates (this workgroup's own global writes)
            __threadfence();
            __syncthreads();
            const int m = nch * k;
            const int G = (m + 4 * TPB - 1) / (4 * TPB);
            uint32_t kr[4 * MG_V4], lmin = 0xFFFFFFFFu, lmax = 0u;
#pragma unroll
            for (int i = 0; i < 4 * MG_V4; ++i) {
                const int j = 4 * G * tid + i;
                kr[i] = i / 4 < G && j < m ? ck[j] : 0u;
                lmin = kr[i] != 0u && kr[i] < lmin ? kr[i] : lmin;
                lmax = kr[i] > lmax ? kr[i] : lmax;
            }
            select_regs<MG_V4>(kr, G, lmin, lmax, k, sh, tid, false, [](int) {});
            for (int j = tid; j < k; j += TPB) out[j] = cp[sh.ocol[j]];
            lds_barrier();
        }
    }
}

hipError_t launch_indexer_topk(const IdxTopkParams &tp, int T, int max_q, bool decode_variant, hipStream_t s,
                               LaunchMarks *marks) {
    if (T <= 0) return hipSuccess;
    const IndexerParams &p = tp.ix;
    if (p.nseg * p.seg_w < p.max_kv || p.nseg > MAX_SEG) return hipErrorInvalidValue;
    if (decode_variant) {
        hipLaunchKernelGGL(indexer_sample_row_kernel, dim3(T), dim3(512), 0, s, tp);
    } else {
        hipLaunchKernelGGL(indexer_sample_kernel, dim3((max_q + ST_ROWS - 1) / ST_ROWS, 1, p.B), dim3(512), 0, s,
                           tp);
    }
    hipError_t e = hipGetLastError();
    if (marks) marks->after(decode_variant ? "indexer_sample_row_kernel" : "indexer_sample_kernel", s);
    if (e != hipSuccess) return e;
    if (p.max_kv > 0) {
        if ((e = launch_indexer_cand(p, T, max_q, decode_variant, s)) != hipSuccess) return e;
        if (marks) marks->after(decode_variant ? "indexer_decode_kernel<cand>" : "indexer_prefill_kernel<cand>", s);
    }
    static int ncu = 0;
    if (ncu == 0) {
        int dev = 0, nn = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&nn, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || nn <= 0)
            nn = 256;
        ncu = nn;
    }
    if (T <= SEL_BLOCK_ROWS * ncu) {
        // few rows: one workgroup per row
        hipLaunchKernelGGL(cand_select_kernel, dim3(T), dim3(TPB), 0, s, tp, T, 0);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (marks) marks->after("cand_select_kernel", s);
    } else {
        // many rows: one wave per row; rows with too many candidates for a wave queued
        if (p.nseg == 1)   // one region per row: the coalesced layout
            hipLaunchKernelGGL(cand_select_wave_contig_kernel, dim3((T + SEL_WAVES - 1) / SEL_WAVES),
                               dim3(64 * SEL_WAVES), 0, s, tp, T);
        else
            hipLaunchKernelGGL(p.max_kv > SEL_LONG_CTX ? cand_select_wave_kernel<SEL_R_LONG> : cand_select_wave_kernel<SEL_R>,
                               dim3((T + SEL_WAVES - 1) / SEL_WAVES),
                               dim3(64 * SEL_WAVES), 0, s, tp, T);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (marks) marks->after(p.nseg == 1 ? "cand_select_wave_contig_kernel" : "cand_select_wave_kernel", s);
        hipLaunchKernelGGL(cand_select_kernel, dim3(T < 2 * ncu ? T : 2 * ncu), dim3(TPB), 0, s, tp, T, 1);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (marks) marks->after("cand_select_kernel", s);
    }
    hipLaunchKernelGGL(idx_fallback_kernel, dim3(T < ncu ? T : ncu), dim3(TPB), 0, s, tp);
    e = hipGetLastError();
    if (marks) marks->after("idx_fallback_kernel", s);
    return e;
}

}  // namespace dsa
