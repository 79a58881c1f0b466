// api.hip — the extern "C" entry points declared in include/dsa.h: host-side
// validation, workspace layout and kernel dispatch.  No allocation, no state.
#include "dsa.h"
#include "kernels.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

namespace {

using namespace dsa;

constexpr int kHI = 64, kDI = 128, kH = 128, kD = 576, kDv = 512, kKMax = 2048;
constexpr int kMaxKvTopk = TOPK_CHUNK * TOPK_MAX_CHUNKS;  // 262144
constexpr size_t kAlign = 256;

inline bool al16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline size_t up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

dsa_status check_batch(const dsa_batch *b) {
    if (!b || !b->cu_q || !b->cu_kv || !b->pos0) return DSA_ERR_INVALID_ARG;
    if (b->batch < 1 || b->total_q < 0 || b->max_q < 0 || b->max_kv < 0 || b->total_kv < 0)
        return DSA_ERR_INVALID_ARG;
    if (b->max_q > b->total_q || (int64_t)b->max_kv > b->total_kv) return DSA_ERR_INVALID_ARG;
    if (b->max_kv > (1 << 24) || b->batch > 65535) return DSA_ERR_UNSUPPORTED;
    return DSA_OK;
}

int topk_chunks(int max_kv) { return max_kv <= 0 ? 1 : (max_kv + TOPK_CHUNK - 1) / TOPK_CHUNK; }

size_t topk_ws(const dsa_batch *b, int k) {
    const int nch = topk_chunks(b->max_kv);
    if (nch <= 1) return 0;
    return 2 * up((size_t)b->total_q * nch * k * 4);
}

// Compute units of the current device (256 on MI355X), queried once.
int device_cus() {
    static int ncu = 0;
    if (ncu == 0) {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        ncu = n;
    }
    return ncu;
}

// Split-KV factor for the attention: enough workgroups to give every compute
// unit one (the attention workgroup fills a compute unit's LDS, so a second
// round of workgroups would repeat the per-workgroup query load and partial
// write instead of overlapping them).
int mla_splits(int T, int k) {
    const int nblk = (k + MLA_BK - 1) / MLA_BK;
    const int ncu = device_cus();
    if (T <= 0 || T >= ncu) return 1;
    int s = (ncu + T - 1) / T;
    if (s > nblk) s = nblk;
    return s < 1 ? 1 : s;
}

size_t mla_ws(const dsa_batch *b, int k) {
    const int s = mla_splits(b->total_q, k);
    if (s <= 1) return 0;
    return up((size_t)b->total_q * s * kH * kDv * 2) + up((size_t)b->total_q * s * kH * 4);
}

// Splits of the KL loss: enough workgroups for two per compute unit (the
// kernel's LDS allows two), each split a whole number of 32-slot blocks.
int kl_splits(int T, int64_t slots) {
    const int64_t nblk = (slots + KL_BK - 1) / KL_BK;
    const int want = 2 * device_cus();
    if (T <= 0 || T >= want || nblk <= 1) return 1;
    int64_t s = (want + T - 1) / T;
    if (s > nblk) s = nblk;
    return s < 1 ? 1 : (int)s;
}

// Partial sums of the KL loss (both stages: the larger split count).
size_t kl_ws(const dsa_batch *b, int k) {
    const int s1 = kl_splits(b->total_q, k), s2 = kl_splits(b->total_q, b->max_kv);
    const int s = s1 > s2 ? s1 : s2;
    return up((size_t)b->total_q * s * 5 * 4);
}

// Backward workspace, for one chunk of at most BWD_CHUNK query rows (k
// rounded up to whole 32-slot blocks): P and scale * dZ per (row, slot, head)
// in bf16, each slot's 576 sums in bf16, the slot list by cache row, and the
// counting-sort arrays over the N cache rows.
int bwd_kpad(int k) { return (k + 31) / 32 * 32; }
struct BwdWs {
    size_t ps, dzs, g, list, cnt, cur, bsum, total;
};
BwdWs bwd_layout(const dsa_batch *b, int k) {
    const size_t tc = (size_t)(b->total_q < BWD_CHUNK ? b->total_q : BWD_CHUNK);
    const size_t slots = tc * bwd_kpad(k);
    const size_t n = (size_t)b->total_kv;
    const size_t nb = (n + 1 + 1023) / 1024;
    BwdWs w;
    w.ps = 0;
    w.dzs = w.ps + up(slots * kH * 2);
    w.g = w.dzs + up(slots * kH * 2);
    w.list = w.g + up(slots * kD * 2);
    w.cnt = w.list + up(slots * 4);
    w.cur = w.cnt + up((n + 1) * 4);
    w.bsum = w.cur + up((n + 1) * 4);
    w.total = w.bsum + up((nb + 1) * 4);
    return w;
}
size_t bwd_ws(const dsa_batch *b, int k) { return b->total_q > 0 ? bwd_layout(b, k).total : 0; }

// Slot budget of the dense attention: the longest context (at least 1).
int dense_slots(const dsa_batch *b) { return b->max_kv < 1 ? 1 : b->max_kv; }

// Candidate regions of the fused indexer + select.  Region width: the decode
// indexer's per-wave range (512 columns); for prefill, the widest power-of-two
// key range per indexer workgroup (up to the whole row) that still gives at
// least 8 workgroups per compute unit.  Slots per region: every column for
// decode; at most 8192 for prefill (a row's candidates are ~1.3k..2.5k when
// the sampled threshold is right; more overflow, and the row is recomputed
// on chip).  A row's area also holds the recompute's per-chunk candidates,
// k per 32768 columns.
struct CandLayout {
    int seg_w = 0, nseg = 0, cap = 0;
    size_t tau = 0, cnt = 0, key = 0, pos = 0, fb = 0, total = 0;
};
CandLayout cand_layout(const dsa_batch *b, int k, bool decode) {
    CandLayout c;
    if (decode) {
        c.seg_w = CAND_DECODE_SEG;
    } else {
        const int64_t rowblocks = (int64_t)((b->max_q + 15) / 16) * b->batch;
        int full = 2048;
        while (full < b->max_kv) full <<= 1;
        c.seg_w = 2048;
        for (int w = full; w > 2048; w >>= 1)
            if (rowblocks * ((b->max_kv + w - 1) / w) >= 8LL * device_cus()) {
                c.seg_w = w;
                break;
            }
    }
    c.nseg = b->max_kv <= 0 ? 1 : (b->max_kv + c.seg_w - 1) / c.seg_w;
    c.cap = decode ? CAND_DECODE_SEG : (c.seg_w < CAND_CAP ? c.seg_w : CAND_CAP);
    const int64_t need = (int64_t)k * topk_chunks(b->max_kv);
    if ((int64_t)c.nseg * c.cap < need) c.cap = (int)((need + c.nseg - 1) / c.nseg);
    const size_t T = (size_t)b->total_q, slots = T * c.nseg * c.cap;
    c.tau = 0;
    c.cnt = c.tau + up(T * 4);
    c.key = c.cnt + up(T * c.nseg * 4);
    // (64 slots of padding after each array: a select register's 64 loads may
    // run past the last row's last candidate)
    c.pos = c.key + up((slots + 64) * 4);
    c.fb = c.pos + up((slots + 64) * 4);
    c.total = c.fb + up((FB_LIST + 2 * T) * 4);
    return c;
}

size_t idxtopk_ws(const dsa_batch *b, int k, bool decode) { return b->total_q > 0 ? cand_layout(b, k, decode).total : 0; }

// Fused entries: candidates (none for short sequences, which skip the select),
// the selection when the caller does not take it, split-KV partials.
size_t fwd_cand_ws(const dsa_batch *b, int k, bool decode) { return b->max_kv <= k ? 0 : idxtopk_ws(b, k, decode); }
size_t fwd_ws(const dsa_batch *b, int k, bool decode) {
    return fwd_cand_ws(b, k, decode) + up((size_t)b->total_q * k * 4) + mla_ws(b, k);
}

// Keys per indexer workgroup.  Prefill takes the widest chunk of 8192, 4096
// or 2048 keys that still gives at least 8 workgroups per compute unit (each
// workgroup loads its 16 query rows once per chunk: 32K prefill 4.34 -> 4.10
// ms going from 2048 to 8192); decode keeps 2048.
int indexer_chunk(const dsa_batch *b, bool decode) {
    if (decode) return 2048;
    const int64_t rowblocks = (int64_t)((b->max_q + 15) / 16) * b->batch;
    for (int c = 8192; c > 2048; c >>= 1)
        if (rowblocks * ((b->max_kv + c - 1) / c) >= 8LL * device_cus()) return c;
    return 2048;
}

IndexerParams make_indexer(const dsa_batch *b, const uint8_t *q, const float *qs, const float *w,
                           const uint8_t *k, const float *ks, float *scores, int64_t ld, int chunk,
                           int fill) {
    IndexerParams p;
    p.cu_q = b->cu_q;
    p.cu_kv = b->cu_kv;
    p.pos0 = b->pos0;
    p.B = b->batch;
    p.total_kv = b->total_kv;
    p.max_kv = b->max_kv;
    p.q = q;
    p.q_scale = qs;
    p.w = w;
    p.k = k;
    p.k_scale = ks;
    p.scores = scores;
    p.ld = ld;
    p.key_chunk = chunk;
    p.fill_masked = fill;
    p.tau = nullptr;
    p.cand_key = nullptr;
    p.cand_pos = nullptr;
    p.cand_cnt = nullptr;
    p.seg_w = p.nseg = p.cap = p.topk_k = 0;
    return p;
}

// The fused indexer + select over the candidate layout at ws.
IdxTopkParams make_idxtopk(const dsa_batch *b, const uint8_t *q, const float *qs, const float *w, const uint8_t *kk,
                           const float *ks, int k, int32_t *idx, void *ws, bool decode) {
    const CandLayout c = cand_layout(b, k, decode);
    char *base = static_cast<char *>(ws);
    IdxTopkParams tp;
    tp.ix = make_indexer(b, q, qs, w, kk, ks, nullptr, 0, decode ? 4 * CAND_DECODE_SEG : c.seg_w, 0);
    tp.tau = reinterpret_cast<uint32_t *>(base + c.tau);
    tp.ix.tau = tp.tau;
    tp.ix.cand_cnt = reinterpret_cast<int32_t *>(base + c.cnt);
    tp.ix.cand_key = reinterpret_cast<uint32_t *>(base + c.key);
    tp.ix.cand_pos = reinterpret_cast<int32_t *>(base + c.pos);
    tp.ix.seg_w = c.seg_w;
    tp.ix.nseg = c.nseg;
    tp.ix.cap = c.cap;
    tp.ix.topk_k = k;
    tp.k = k;
    tp.idx = idx;
    tp.fb = reinterpret_cast<int32_t *>(base + c.fb);
    return tp;
}

TopkParams make_topk(const dsa_batch *b, const float *scores, int64_t ld, int k, int32_t *idx,
                     void *ws) {
    TopkParams p;
    p.cu_q = b->cu_q;
    p.cu_kv = b->cu_kv;
    p.pos0 = b->pos0;
    p.B = b->batch;
    p.total_kv = b->total_kv;
    p.max_kv = b->max_kv;
    p.scores = scores;
    p.ld = ld;
    p.k = k;
    p.idx = idx;
    p.nchunk = topk_chunks(b->max_kv);
    const size_t half = topk_ws(b, k) / 2;
    p.cand_key = reinterpret_cast<uint32_t *>(ws);
    p.cand_pos = ws ? reinterpret_cast<int32_t *>(static_cast<char *>(ws) + half) : nullptr;
    return p;
}

MlaParams make_mla(const dsa_batch *b, const uint16_t *q, const uint16_t *kv, const int32_t *idx,
                   int k, float scale, uint16_t *out, float *lse, void *ws, int dense = 0) {
    MlaParams p;
    p.cu_q = b->cu_q;
    p.cu_kv = b->cu_kv;
    p.pos0 = b->pos0;
    p.B = b->batch;
    p.total_kv = b->total_kv;
    p.max_kv = b->max_kv;
    p.q = q;
    p.kv = kv;
    p.idx = idx;
    p.k = k;
    p.dense = dense;
    p.scale_log2 = scale * 1.4426950408889634f;
    p.out = out;
    p.lse = lse;
    p.splits = mla_splits(b->total_q, k);
    const int nblk = (k + MLA_BK - 1) / MLA_BK;
    p.blocks_per_split = (nblk + p.splits - 1) / p.splits;
    p.o_part = nullptr;
    p.lse_part = nullptr;
    if (p.splits > 1) {
        p.o_part = reinterpret_cast<uint16_t *>(ws);
        p.lse_part = reinterpret_cast<float *>(static_cast<char *>(ws) +
                                               up((size_t)b->total_q * p.splits * kH * kDv * 2));
    }
    return p;
}

dsa_status hip_status(hipError_t e) { return e == hipSuccess ? DSA_OK : DSA_ERR_HIP; }

// Per-launch timing of the fused entries: an event is recorded on the stream
// before the first launch and after each one, so consecutive events bracket
// one kernel each (the profiling entry point passes one; null elsewhere).
struct Timeline final : LaunchMarks {
    static constexpr int kMax = 16;
    hipEvent_t ev[kMax + 1] = {};
    const char *name[kMax] = {};
    int n = 0;        // kernels recorded
    bool ok = true;   // every event recorded
    void after(const char *kernel, hipStream_t s) override {
        if (n >= kMax) return;
        name[n] = kernel;
        if (hipEventRecord(ev[n + 1], s) != hipSuccess) ok = false;
        ++n;
    }
};

// Softmax scales must be positive and finite: the attention kernels take the
// maximum of the scaled logits as the maximum of the raw ones, and a masked
// slot's -inf logit times a scale <= 0 is NaN or +inf.
bool valid_scale(float scale) { return std::isfinite(scale) && scale > 0.f; }

// Diagnostics, switched on from the environment and read at every call:
//   DSA_LOG=1           one line per entry call on stderr: the batch, k, the
//                       workspace given, the launch plan of the fused entries
//                       and the status returned;
//   DSA_DEBUG_CHECKS=1  every selection an entry produces (dsa_topk,
//                       dsa_indexer_topk, the fused entries) is validated on
//                       the device; a row that is not min(k, visible)
//                       ascending visible positions followed by -1 makes the
//                       call return DSA_ERR_CHECK.  The check drains the
//                       stream, so it has no place under graph capture.
bool env_flag(const char *name) {
    const char *v = std::getenv(name);
    return v && v[0] && !(v[0] == '0' && v[1] == 0);
}

std::mutex g_log_mu;

void log_line(const char *fmt, ...) {
    std::lock_guard<std::mutex> lock(g_log_mu);
    va_list ap;
    va_start(ap, fmt);
    std::fputs("[dsa] ", stderr);
    std::vfprintf(stderr, fmt, ap);
    std::fputc('\n', stderr);
    va_end(ap);
}

template <typename F>
dsa_status traced(const char *entry, const dsa_batch *b, int k, size_t ws_bytes, F &&body) {
    const dsa_status st = body();
    if (env_flag("DSA_LOG")) {
        if (b)
            log_line("%s B=%d total_q=%d max_q=%d max_kv=%d total_kv=%lld k=%d ws=%zu -> %s", entry, b->batch,
                     b->total_q, b->max_q, b->max_kv, (long long)b->total_kv, k, ws_bytes, dsa_status_string(st));
        else
            log_line("%s -> %s", entry, dsa_status_string(st));
    }
    return st;
}

dsa_status debug_check(const char *entry, const dsa_batch *b, const int32_t *idx, int k, hipStream_t s) {
    if (!env_flag("DSA_DEBUG_CHECKS") || b->total_q <= 0) return DSA_OK;
    int bad = 0;
    if (check_selection(b->cu_q, b->cu_kv, b->pos0, b->batch, b->total_kv, b->max_kv, b->total_q, idx, k, s,
                        &bad) != hipSuccess)
        return DSA_ERR_HIP;
    if (bad > 0) {
        log_line("%s: debug check: %d of %d rows break the selection contract", entry, bad, b->total_q);
        return DSA_ERR_CHECK;
    }
    if (env_flag("DSA_LOG")) log_line("%s: debug check: %d rows ok", entry, b->total_q);
    return DSA_OK;
}

dsa_status check_k(int k) {
    if (k < 1 || k > kKMax) return DSA_ERR_UNSUPPORTED;
    return DSA_OK;
}

dsa_status run_fwd(const dsa_fwd_args *a, uint16_t *out, float *lse, int32_t *idx_out, void *ws,
                   size_t ws_bytes, void *stream, bool decode, Timeline *tl = nullptr) {
    if (!a) return DSA_ERR_INVALID_ARG;
    dsa_status st = check_batch(&a->batch);
    if (st != DSA_OK) return st;
    if (a->HI != kHI || a->DI != kDI || a->H != kH || a->D != kD || a->Dv != kDv)
        return DSA_ERR_UNSUPPORTED;
    if ((st = check_k(a->k)) != DSA_OK) return st;
    if (a->batch.max_kv > kMaxKvTopk) return DSA_ERR_UNSUPPORTED;
    if (!valid_scale(a->scale)) return DSA_ERR_INVALID_ARG;
    const dsa_batch *b = &a->batch;
    if (b->total_q == 0) return DSA_OK;
    if (!a->q_fp8 || !a->q_scale || !a->w || !a->q || !out || !lse) return DSA_ERR_INVALID_ARG;
    if (b->total_kv > 0 && (!a->k_fp8 || !a->k_scale || !a->kv)) return DSA_ERR_INVALID_ARG;
    const void *ptrs[] = {a->q_fp8, a->q_scale, a->w, a->q, out, lse};
    for (const void *p : ptrs)
        if (!al16(p)) return DSA_ERR_INVALID_ARG;
    if (b->total_kv > 0 && (!al16(a->k_fp8) || !al16(a->k_scale) || !al16(a->kv)))
        return DSA_ERR_INVALID_ARG;
    if (idx_out && !al16(idx_out)) return DSA_ERR_INVALID_ARG;
    const size_t need = fwd_ws(b, a->k, decode);
    if (need > 0 && (!ws || ws_bytes < need || !al16(ws))) return DSA_ERR_WORKSPACE;

    hipStream_t s = static_cast<hipStream_t>(stream);
    char *w = static_cast<char *>(ws);
    void *cws = w;
    w += fwd_cand_ws(b, a->k, decode);
    int32_t *idx = reinterpret_cast<int32_t *>(w);
    w += up((size_t)b->total_q * a->k * 4);
    if (idx_out) idx = idx_out;
    void *mws = w;

    // Short sequences (every context within k): the select keeps every visible
    // key, so the result is dense causal attention.  Run it without scoring or
    // selecting ("MHA with mask"); the split layout is the one the three-step
    // path uses for this k, so both give the same bits.
    if (b->max_kv <= a->k) {
        if (env_flag("DSA_LOG"))
            log_line("%s plan: short mode (every visible key), attention splits %d", decode ? "decode" : "prefill",
                     mla_splits(b->total_q, a->k));
        if (idx_out) {
            TopkParams tp = make_topk(b, nullptr, 0, a->k, idx_out, nullptr);
            if ((st = hip_status(launch_select_all_visible(tp, b->total_q, s))) != DSA_OK) return st;
            if (tl) tl->after("select_all_visible_kernel", s);
            if ((st = debug_check("select_all_visible", b, idx_out, a->k, s)) != DSA_OK) return st;
        }
        MlaParams mp = make_mla(b, a->q, a->kv, nullptr, a->k, a->scale, out, lse, mws, 1);
        return hip_status(launch_sparse_mla(mp, b->total_q, s, tl));
    }

    // indexer -> top-k with the scores kept on chip (candidates only)
    IdxTopkParams tp = make_idxtopk(b, a->q_fp8, a->q_scale, a->w, a->k_fp8, a->k_scale, a->k, idx, cws, decode);
    if (env_flag("DSA_LOG")) {
        const CandLayout c = cand_layout(b, a->k, decode);
        log_line("%s plan: candidate regions of %d columns x %d per row (cap %d), %s select, attention splits %d",
                 decode ? "decode" : "prefill", c.seg_w, c.nseg, c.cap,
                 b->total_q <= 4 * device_cus() ? "workgroup" : "wave", mla_splits(b->total_q, a->k));
    }
    if ((st = hip_status(launch_indexer_topk(tp, b->total_q, b->max_q, decode, s, tl))) != DSA_OK) return st;
    if ((st = debug_check("indexer_topk", b, idx, a->k, s)) != DSA_OK) return st;
    MlaParams mp = make_mla(b, a->q, a->kv, idx, a->k, a->scale, out, lse, mws);
    return hip_status(launch_sparse_mla(mp, b->total_q, s, tl));
}

// Static scratch of the allocation-free decode entry: device memory that the
// library owns for the process's lifetime, one copy per GPU (each at its own
// address).  Host code never passes the array's name to a kernel (on the host
// it is a stand-in, not a device address): the address is taken once per
// device with hipGetSymbolAddress, with that device current, and kept.
constexpr size_t kScratchBytes = size_t(128) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch`, or null on a HIP error.
void *scratch_on_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

namespace dsa {
// (peaks.hip) attainable MFMA and HBM rates; waits for `s`
hipError_t measure_peaks(void *buf, size_t bytes, hipStream_t s, dsa_peaks *out);
}  // namespace dsa

extern "C" {

dsa_status dsa_quantize_queries(const float *q, int64_t T, int HI, int DI, uint8_t *q_fp8,
                                float *q_scale, void *stream) {
    return traced("dsa_quantize_queries", nullptr, 0, 0, [&]() -> dsa_status {
        if (HI != kHI || DI != kDI) return DSA_ERR_UNSUPPORTED;
        if (T < 0) return DSA_ERR_INVALID_ARG;
        if (T == 0) return DSA_OK;
        if (T > INT32_MAX) return DSA_ERR_UNSUPPORTED;
        if (!q || !q_fp8 || !q_scale || !al16(q) || !al16(q_fp8) || !al16(q_scale)) return DSA_ERR_INVALID_ARG;
        return hip_status(launch_quant_queries(q, T, q_fp8, q_scale, static_cast<hipStream_t>(stream)));
    });
}

dsa_status dsa_append_cache(const float *k_new, const uint16_t *kv_new, int64_t R, int DI, int D,
                            const int64_t *dst_rows, uint8_t *k_fp8, float *k_scale, uint16_t *kv,
                            int64_t N, void *stream) {
    return traced("dsa_append_cache", nullptr, 0, 0, [&]() -> dsa_status {
        if (DI != kDI || D != kD) return DSA_ERR_UNSUPPORTED;
        if (R < 0 || N < 0) return DSA_ERR_INVALID_ARG;
        if (R == 0) return DSA_OK;
        if (R > (int64_t)INT32_MAX * 8) return DSA_ERR_UNSUPPORTED;
        if (!k_new || !dst_rows || !k_fp8 || !k_scale) return DSA_ERR_INVALID_ARG;
        if ((kv_new == nullptr) != (kv == nullptr)) return DSA_ERR_INVALID_ARG;
        const void *ptrs[] = {k_new, dst_rows, k_fp8, k_scale};
        for (const void *p : ptrs)
            if (!al16(p)) return DSA_ERR_INVALID_ARG;
        if (kv_new && (!al16(kv_new) || !al16(kv))) return DSA_ERR_INVALID_ARG;
        return hip_status(launch_append_cache(k_new, kv_new, R, dst_rows, k_fp8, k_scale, kv, N,
                                              static_cast<hipStream_t>(stream)));
    });
}

dsa_status dsa_indexer_scores(const dsa_batch *batch, const uint8_t *q_fp8, const float *q_scale,
                              const float *w, const uint8_t *k_fp8, const float *k_scale, int HI,
                              int DI, float *scores, int64_t ld, void *stream) {
    return traced("dsa_indexer_scores", batch, 0, 0, [&]() -> dsa_status {
        dsa_status st = check_batch(batch);
        if (st != DSA_OK) return st;
        if (HI != kHI || DI != kDI) return DSA_ERR_UNSUPPORTED;
        if (batch->total_q == 0 || batch->max_kv == 0) return DSA_OK;
        if (!q_fp8 || !q_scale || !w || !k_fp8 || !k_scale || !scores) return DSA_ERR_INVALID_ARG;
        if (ld < batch->max_kv) return DSA_ERR_INVALID_ARG;
        const void *ptrs[] = {q_fp8, q_scale, w, k_fp8, k_scale, scores};
        for (const void *p : ptrs)
            if (!al16(p)) return DSA_ERR_INVALID_ARG;
        const bool decode = batch->max_q < 16;
        IndexerParams p = make_indexer(batch, q_fp8, q_scale, w, k_fp8, k_scale, scores, ld,
                                       indexer_chunk(batch, decode), 1);
        return hip_status(launch_indexer(p, batch->total_q, batch->max_q, decode,
                                         static_cast<hipStream_t>(stream)));
    });
}

dsa_status dsa_topk(const dsa_batch *batch, const float *scores, int64_t ld, int k, int32_t *idx,
                    void *ws, size_t ws_bytes, void *stream) {
    return traced("dsa_topk", batch, k, ws_bytes, [&]() -> dsa_status {
        dsa_status st = check_batch(batch);
        if (st != DSA_OK) return st;
        if ((st = check_k(k)) != DSA_OK) return st;
        if (batch->max_kv > kMaxKvTopk) return DSA_ERR_UNSUPPORTED;
        if (batch->total_q == 0) return DSA_OK;
        if (!scores || !idx) return DSA_ERR_INVALID_ARG;
        if (ld < batch->max_kv) return DSA_ERR_INVALID_ARG;
        if (!al16(scores) || !al16(idx)) return DSA_ERR_INVALID_ARG;
        const size_t need = topk_ws(batch, k);
        if (need > 0 && (!ws || ws_bytes < need || !al16(ws))) return DSA_ERR_WORKSPACE;
        TopkParams p = make_topk(batch, scores, ld, k, idx, ws);
        if ((st = hip_status(launch_topk(p, batch->total_q, static_cast<hipStream_t>(stream)))) != DSA_OK) return st;
        return debug_check("dsa_topk", batch, idx, k, static_cast<hipStream_t>(stream));
    });
}

dsa_status dsa_indexer_topk(const dsa_batch *batch, const uint8_t *q_fp8, const float *q_scale, const float *w,
                            const uint8_t *k_fp8, const float *k_scale, int HI, int DI, int k, int32_t *idx, void *ws,
                            size_t ws_bytes, void *stream) {
    return traced("dsa_indexer_topk", batch, k, ws_bytes, [&]() -> dsa_status {
        dsa_status st = check_batch(batch);
        if (st != DSA_OK) return st;
        if (HI != kHI || DI != kDI) return DSA_ERR_UNSUPPORTED;
        if ((st = check_k(k)) != DSA_OK) return st;
        if (batch->max_kv > kMaxKvTopk) return DSA_ERR_UNSUPPORTED;
        if (batch->total_q == 0) return DSA_OK;
        if (!q_fp8 || !q_scale || !w || !idx) return DSA_ERR_INVALID_ARG;
        if (batch->total_kv > 0 && (!k_fp8 || !k_scale)) return DSA_ERR_INVALID_ARG;
        const void *ptrs[] = {q_fp8, q_scale, w, idx};
        for (const void *p : ptrs)
            if (!al16(p)) return DSA_ERR_INVALID_ARG;
        if (batch->total_kv > 0 && (!al16(k_fp8) || !al16(k_scale))) return DSA_ERR_INVALID_ARG;
        const bool decode = batch->max_q < 16;
        const size_t need = idxtopk_ws(batch, k, decode);
        if (!ws || ws_bytes < need || !al16(ws)) return DSA_ERR_WORKSPACE;
        IdxTopkParams tp = make_idxtopk(batch, q_fp8, q_scale, w, k_fp8, k_scale, k, idx, ws, decode);
        if ((st = hip_status(launch_indexer_topk(tp, batch->total_q, batch->max_q, decode,
                                                 static_cast<hipStream_t>(stream)))) != DSA_OK)
            return st;
        return debug_check("dsa_indexer_topk", batch, idx, k, static_cast<hipStream_t>(stream));
    });
}

dsa_status dsa_sparse_mla_fwd(const dsa_batch *batch, const uint16_t *q, const uint16_t *kv,
                              const int32_t *idx, int k, int H, int D, int Dv, float scale,
                              uint16_t *out, float *lse, void *ws, size_t ws_bytes, void *stream) {
    return traced("dsa_sparse_mla_fwd", batch, k, ws_bytes, [&]() -> dsa_status {
        dsa_status st = check_batch(batch);
        if (st != DSA_OK) return st;
        if (H != kH || D != kD || Dv != kDv) return DSA_ERR_UNSUPPORTED;
        if ((st = check_k(k)) != DSA_OK) return st;
        if (batch->max_kv > MAX_KV_ATTN) return DSA_ERR_UNSUPPORTED;
        if (!valid_scale(scale)) return DSA_ERR_INVALID_ARG;
        if (batch->total_q == 0) return DSA_OK;
        if (!q || !idx || !out || !lse) return DSA_ERR_INVALID_ARG;
        if (batch->total_kv > 0 && !kv) return DSA_ERR_INVALID_ARG;
        if (!al16(q) || !al16(idx) || !al16(out) || !al16(lse) || (kv && !al16(kv)))
            return DSA_ERR_INVALID_ARG;
        const size_t need = mla_ws(batch, k);
        if (need > 0 && (!ws || ws_bytes < need || !al16(ws))) return DSA_ERR_WORKSPACE;
        MlaParams p = make_mla(batch, q, kv, idx, k, scale, out, lse, ws);
        return hip_status(launch_sparse_mla(p, batch->total_q, static_cast<hipStream_t>(stream)));
    });
}

dsa_status dsa_dense_mla_fwd(const dsa_batch *batch, const uint16_t *q, const uint16_t *kv, int H, int D,
                             int Dv, float scale, uint16_t *out, float *lse, void *ws, size_t ws_bytes,
                             void *stream) {
    return traced("dsa_dense_mla_fwd", batch, 0, ws_bytes, [&]() -> dsa_status {
        dsa_status st = check_batch(batch);
        if (st != DSA_OK) return st;
        if (H != kH || D != kD || Dv != kDv) return DSA_ERR_UNSUPPORTED;
        if (batch->max_kv > kKMax) return DSA_ERR_UNSUPPORTED;
        if (!valid_scale(scale)) return DSA_ERR_INVALID_ARG;
        if (batch->total_q == 0) return DSA_OK;
        if (!q || !out || !lse) return DSA_ERR_INVALID_ARG;
        if (batch->total_kv > 0 && !kv) return DSA_ERR_INVALID_ARG;
        if (!al16(q) || !al16(out) || !al16(lse) || (kv && !al16(kv))) return DSA_ERR_INVALID_ARG;
        const int kd = dense_slots(batch);
        const size_t need = mla_ws(batch, kd);
        if (need > 0 && (!ws || ws_bytes < need || !al16(ws))) return DSA_ERR_WORKSPACE;
        MlaParams p = make_mla(batch, q, kv, nullptr, kd, scale, out, lse, ws, 1);
        return hip_status(launch_sparse_mla(p, batch->total_q, static_cast<hipStream_t>(stream)));
    });
}

dsa_status dsa_indexer_kl_fwd(const dsa_batch *batch, const uint16_t *q, const uint16_t *kv, const float *lse,
                              int H, int D, float scale, const float *scores, int64_t ld, const int32_t *idx,
                              int k, float *kl, float *p_out, void *ws, size_t ws_bytes, void *stream) {
    return traced("dsa_indexer_kl_fwd", batch, k, ws_bytes, [&]() -> dsa_status {
        dsa_status st = check_batch(batch);
        if (st != DSA_OK) return st;
        if (H != kH || D != kD) return DSA_ERR_UNSUPPORTED;
        if (idx && (st = check_k(k)) != DSA_OK) return st;
        if (batch->max_kv > MAX_KV_ATTN) return DSA_ERR_UNSUPPORTED;
        if (!valid_scale(scale)) return DSA_ERR_INVALID_ARG;
        if (batch->total_q == 0) return DSA_OK;
        if (!q || !lse || !scores || !kl) return DSA_ERR_INVALID_ARG;
        if (batch->total_kv > 0 && !kv) return DSA_ERR_INVALID_ARG;
        if (ld < batch->max_kv || ld < 1) return DSA_ERR_INVALID_ARG;
        if (!al16(q) || !al16(lse) || !al16(scores) || !al16(kl) || (kv && !al16(kv)) || (idx && !al16(idx)) ||
            (p_out && !al16(p_out)))
            return DSA_ERR_INVALID_ARG;
        const size_t need = kl_ws(batch, idx ? k : 1);
        if (!ws || ws_bytes < need || !al16(ws)) return DSA_ERR_WORKSPACE;
        KlParams p;
        p.cu_q = batch->cu_q;
        p.cu_kv = batch->cu_kv;
        p.pos0 = batch->pos0;
        p.B = batch->batch;
        p.total_kv = batch->total_kv;
        p.max_kv = batch->max_kv;
        p.q = q;
        p.kv = kv;
        p.lse = lse;
        p.scale_log2 = scale * 1.4426950408889634f;
        p.scores = scores;
        p.ld = ld;
        p.idx = idx;
        p.k = idx ? k : 0;
        p.kl = kl;
        p.p_out = p_out;
        const int64_t slots = idx ? k : batch->max_kv;
        p.splits = kl_splits(batch->total_q, slots);
        const int64_t nblk = (slots + KL_BK - 1) / KL_BK;
        p.blocks_per_split = (int)((nblk + p.splits - 1) / p.splits);
        if (p.blocks_per_split < 1) p.blocks_per_split = 1;
        p.part = static_cast<float *>(ws);
        return hip_status(launch_indexer_kl(p, batch->total_q, static_cast<hipStream_t>(stream)));
    });
}

dsa_status dsa_sparse_mla_bwd(const dsa_batch *batch, const uint16_t *q, const uint16_t *kv, const int32_t *idx,
                              int k, int H, int D, int Dv, float scale, const uint16_t *out, const float *lse,
                              const uint16_t *dout, float *dq, float *dkv, void *ws, size_t ws_bytes,
                              void *stream) {
    return traced("dsa_sparse_mla_bwd", batch, k, ws_bytes, [&]() -> dsa_status {
        dsa_status st = check_batch(batch);
        if (st != DSA_OK) return st;
        if (H != kH || D != kD || Dv != kDv) return DSA_ERR_UNSUPPORTED;
        if ((st = check_k(k)) != DSA_OK) return st;
        if (batch->max_kv > MAX_KV_ATTN) return DSA_ERR_UNSUPPORTED;
        if (!valid_scale(scale)) return DSA_ERR_INVALID_ARG;
        if (batch->total_q == 0 && batch->total_kv == 0) return DSA_OK;
        if (batch->total_kv > 0 && (!kv || !dkv)) return DSA_ERR_INVALID_ARG;
        if (batch->total_q > 0 && (!q || !idx || !out || !lse || !dout || !dq)) return DSA_ERR_INVALID_ARG;
        const void *ptrs[] = {q, kv, idx, out, lse, dout, dq, dkv};
        for (const void *ptr : ptrs)
            if (ptr && !al16(ptr)) return DSA_ERR_INVALID_ARG;
        const size_t need = bwd_ws(batch, k);
        if (batch->total_q > 0 && (!ws || ws_bytes < need || !al16(ws))) return DSA_ERR_WORKSPACE;
        BwdParams p;
        p.cu_q = batch->cu_q;
        p.cu_kv = batch->cu_kv;
        p.pos0 = batch->pos0;
        p.B = batch->batch;
        p.total_kv = batch->total_kv;
        p.max_kv = batch->max_kv;
        p.q = q;
        p.kv = kv;
        p.idx = idx;
        p.k = k;
        p.kpad = bwd_kpad(k);
        p.scale = scale;
        p.scale_log2 = scale * 1.4426950408889634f;
        p.out = out;
        p.lse = lse;
        p.dout = dout;
        p.dq = dq;
        p.dkv = dkv;
        char *w = static_cast<char *>(ws);
        const BwdWs lay = bwd_layout(batch, k);
        p.t0 = 0;
        p.tc = 0;
        p.ps = w ? reinterpret_cast<uint16_t *>(w + lay.ps) : nullptr;
        p.dzs = w ? reinterpret_cast<uint16_t *>(w + lay.dzs) : nullptr;
        p.g = w ? reinterpret_cast<uint16_t *>(w + lay.g) : nullptr;
        p.list = w ? reinterpret_cast<int32_t *>(w + lay.list) : nullptr;
        p.cnt = w ? reinterpret_cast<int32_t *>(w + lay.cnt) : nullptr;
        p.cur = w ? reinterpret_cast<int32_t *>(w + lay.cur) : nullptr;
        p.bsum = w ? reinterpret_cast<int32_t *>(w + lay.bsum) : nullptr;
        return hip_status(launch_sparse_mla_bwd(p, batch->total_q, static_cast<hipStream_t>(stream)));
    });
}

dsa_status dsa_prefill_fwd(const dsa_fwd_args *args, uint16_t *out, float *lse, int32_t *idx_out,
                           void *ws, size_t ws_bytes, void *stream) {
    const dsa_batch *b = args ? &args->batch : nullptr;
    return traced("dsa_prefill_fwd", b, args ? args->k : 0, ws_bytes, [&]() -> dsa_status {
        return run_fwd(args, out, lse, idx_out, ws, ws_bytes, stream, false);
    });
}

dsa_status dsa_decode_fwd(const dsa_fwd_args *args, uint16_t *out, float *lse, int32_t *idx_out,
                          void *ws, size_t ws_bytes, void *stream) {
    const dsa_batch *b = args ? &args->batch : nullptr;
    return traced("dsa_decode_fwd", b, args ? args->k : 0, ws_bytes, [&]() -> dsa_status {
        return run_fwd(args, out, lse, idx_out, ws, ws_bytes, stream, true);
    });
}

dsa_status dsa_decode_fwd_noalloc(const dsa_fwd_args *args, uint16_t *out, float *lse, int32_t *idx_out,
                                  void *stream) {
    const dsa_batch *b = args ? &args->batch : nullptr;
    return traced("dsa_decode_fwd_noalloc", b, args ? args->k : 0, kScratchBytes, [&]() -> dsa_status {
        if (!args) return DSA_ERR_INVALID_ARG;
        dsa_status st = check_batch(&args->batch);
        if (st != DSA_OK) return st;
        if ((st = check_k(args->k)) != DSA_OK) return st;
        if (args->batch.max_kv > kMaxKvTopk) return DSA_ERR_UNSUPPORTED;
        if (args->batch.total_q == 0) return DSA_OK;
        if (fwd_ws(&args->batch, args->k, true) > kScratchBytes) return DSA_ERR_WORKSPACE;
        void *ws = scratch_on_current_device();
        if (!ws) return DSA_ERR_HIP;
        return run_fwd(args, out, lse, idx_out, ws, kScratchBytes, stream, true);
    });
}

size_t dsa_decode_fwd_noalloc_max_bytes(void) { return kScratchBytes; }

dsa_status dsa_check_selection(const dsa_batch *batch, const int32_t *idx, int k, void *stream, int *bad_rows) {
    return traced("dsa_check_selection", batch, k, 0, [&]() -> dsa_status {
        if (!bad_rows) return DSA_ERR_INVALID_ARG;
        *bad_rows = 0;
        dsa_status st = check_batch(batch);
        if (st != DSA_OK) return st;
        if ((st = check_k(k)) != DSA_OK) return st;
        if (batch->total_q == 0) return DSA_OK;
        if (!idx || !al16(idx)) return DSA_ERR_INVALID_ARG;
        return hip_status(check_selection(batch->cu_q, batch->cu_kv, batch->pos0, batch->batch, batch->total_kv,
                                          batch->max_kv, batch->total_q, idx, k, static_cast<hipStream_t>(stream),
                                          bad_rows));
    });
}

dsa_status dsa_measure_peaks(void *buf, size_t bytes, void *stream, dsa_peaks *out) {
    return traced("dsa_measure_peaks", nullptr, 0, bytes, [&]() -> dsa_status {
        if (!out || !buf || !al16(buf) || bytes < ((size_t)64 << 20)) return DSA_ERR_INVALID_ARG;
        *out = dsa_peaks{0.0, 0.0, 0.0, 0.0};
        return hip_status(measure_peaks(buf, bytes, static_cast<hipStream_t>(stream), out));
    });
}

dsa_status dsa_fwd_profile(const dsa_fwd_args *args, int decode, uint16_t *out, float *lse, int32_t *idx_out,
                           void *ws, size_t ws_bytes, void *stream, dsa_kernel_time *times, int max_times,
                           int *n_times) {
    if (!times || !n_times || max_times < 1) return DSA_ERR_INVALID_ARG;
    *n_times = 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    Timeline tl;
    int made = 0;
    dsa_status st = DSA_OK;
    for (; made <= Timeline::kMax; ++made)
        if (hipEventCreate(&tl.ev[made]) != hipSuccess) {
            st = DSA_ERR_HIP;
            break;
        }
    if (st == DSA_OK && hipEventRecord(tl.ev[0], s) != hipSuccess) st = DSA_ERR_HIP;
    if (st == DSA_OK) st = run_fwd(args, out, lse, idx_out, ws, ws_bytes, stream, decode != 0, &tl);
    if (st == DSA_OK && tl.n > 0) {
        if (!tl.ok || hipEventSynchronize(tl.ev[tl.n]) != hipSuccess) st = DSA_ERR_HIP;
        // the fused select's counts (its queue header): rows queued for the
        // recompute, -, candidates selected, rows handed to the workgroup select
        int32_t fb[4] = {-1, -1, -1, -1};
        const dsa_batch *b = &args->batch;
        if (st == DSA_OK && b->max_kv > args->k && b->total_q > 0) {
            const CandLayout c = cand_layout(b, args->k, decode != 0);
            if (hipMemcpy(fb, static_cast<char *>(ws) + c.fb, sizeof(fb), hipMemcpyDeviceToHost) != hipSuccess)
                st = DSA_ERR_HIP;
        }
        for (int i = 0; st == DSA_OK && i < tl.n && i < max_times; ++i) {
            float ms = 0.f;
            if (hipEventElapsedTime(&ms, tl.ev[i], tl.ev[i + 1]) != hipSuccess) st = DSA_ERR_HIP;
            times[i].kernel = tl.name[i];
            times[i].ms = ms;
            times[i].items = -1;
            if (std::strcmp(tl.name[i], "cand_select_wave_kernel") == 0 ||
                std::strcmp(tl.name[i], "cand_select_wave_contig_kernel") == 0)
                times[i].items = fb[2];
            if (std::strcmp(tl.name[i], "idx_fallback_kernel") == 0) times[i].items = fb[0];
            *n_times = i + 1;
        }
        // the workgroup select took every row (few rows) or the rows the wave
        // select handed on (then a wave select ran before it)
        bool wave_sel = false;
        for (int i = 0; i < *n_times; ++i)
            wave_sel |= std::strncmp(times[i].kernel, "cand_select_wave", 16) == 0;
        for (int i = 0; st == DSA_OK && i < *n_times; ++i)
            if (std::strcmp(times[i].kernel, "cand_select_kernel") == 0 && fb[3] >= 0)
                times[i].items = wave_sel ? fb[3] : args->batch.total_q;
    }
    for (int i = 0; i < made; ++i) (void)hipEventDestroy(tl.ev[i]);
    return st;
}

size_t dsa_workspace_size(dsa_ws_entry entry, const dsa_batch *batch, int k, int H, int Dv) {
    if (!batch || batch->batch < 1 || batch->total_q < 0 || batch->max_kv < 0 || k < 1 ||
        k > kKMax || H != kH || Dv != kDv)
        return 0;
    switch (entry) {
        case DSA_WS_TOPK: return topk_ws(batch, k);
        case DSA_WS_SPARSE_MLA: return mla_ws(batch, k);
        case DSA_WS_PREFILL: return fwd_ws(batch, k, false);
        case DSA_WS_DECODE: return fwd_ws(batch, k, true);
        case DSA_WS_INDEXER_TOPK:
            return batch->max_kv > kMaxKvTopk ? 0 : idxtopk_ws(batch, k, batch->max_q < 16);
        case DSA_WS_DENSE_MLA: return batch->max_kv > kKMax ? 0 : mla_ws(batch, dense_slots(batch));
        case DSA_WS_INDEXER_KL: return batch->max_kv > MAX_KV_ATTN ? 0 : kl_ws(batch, k);
        case DSA_WS_SPARSE_MLA_BWD: return batch->max_kv > MAX_KV_ATTN ? 0 : bwd_ws(batch, k);
    }
    return 0;
}

const char *dsa_status_string(dsa_status s) {
    switch (s) {
        case DSA_OK: return "ok";
        case DSA_ERR_INVALID_ARG: return "invalid argument";
        case DSA_ERR_UNSUPPORTED: return "unsupported shape";
        case DSA_ERR_WORKSPACE: return "workspace missing or too small";
        case DSA_ERR_HIP: return "HIP runtime error at launch";
        case DSA_ERR_CHECK: return "debug check failed: an output breaks its contract";
    }
    return "unknown status";
}

const char *dsa_version(void) { return "dsa-mi355x 0.1.0 (gfx950)"; }

}  // extern "C"
