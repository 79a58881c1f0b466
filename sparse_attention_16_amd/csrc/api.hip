// api.hip — the extern "C" entry points declared in include/dsa.h: host-side
// validation, workspace layout and kernel dispatch.  No allocation, no state.
#include "dsa.h"
#include "kernels.h"

#include <cmath>
#include <cstring>

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

int64_t score_ld(int max_kv) { return ((int64_t)max_kv + 63) / 64 * 64; }

// Slot budget of the dense attention: the longest context (at least 1).
int dense_slots(const dsa_batch *b) { return b->max_kv < 1 ? 1 : b->max_kv; }

size_t fwd_ws(const dsa_batch *b, int k) {
    return up((size_t)b->total_q * score_ld(b->max_kv) * 4) + up((size_t)b->total_q * k * 4) +
           topk_ws(b, k) + mla_ws(b, k);
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
    return p;
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

dsa_status check_k(int k) {
    if (k < 1 || k > kKMax) return DSA_ERR_UNSUPPORTED;
    return DSA_OK;
}

dsa_status run_fwd(const dsa_fwd_args *a, uint16_t *out, float *lse, int32_t *idx_out, void *ws,
                   size_t ws_bytes, void *stream, bool decode) {
    if (!a) return DSA_ERR_INVALID_ARG;
    dsa_status st = check_batch(&a->batch);
    if (st != DSA_OK) return st;
    if (a->HI != kHI || a->DI != kDI || a->H != kH || a->D != kD || a->Dv != kDv)
        return DSA_ERR_UNSUPPORTED;
    if ((st = check_k(a->k)) != DSA_OK) return st;
    if (a->batch.max_kv > kMaxKvTopk) return DSA_ERR_UNSUPPORTED;
    if (!std::isfinite(a->scale)) return DSA_ERR_INVALID_ARG;
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
    const size_t need = fwd_ws(b, a->k);
    if (need > 0 && (!ws || ws_bytes < need || !al16(ws))) return DSA_ERR_WORKSPACE;

    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t ld = score_ld(b->max_kv);
    char *w = static_cast<char *>(ws);
    float *scores = reinterpret_cast<float *>(w);
    w += up((size_t)b->total_q * ld * 4);
    int32_t *idx = reinterpret_cast<int32_t *>(w);
    w += up((size_t)b->total_q * a->k * 4);
    if (idx_out) idx = idx_out;
    void *tws = w;
    w += topk_ws(b, a->k);
    void *mws = w;

    // Short sequences (every context within k): the select keeps every visible
    // key, so the result is dense causal attention.  Run it without scoring or
    // selecting ("MHA with mask"); the split layout is the one the three-step
    // path uses for this k, so both give the same bits.
    if (b->max_kv <= a->k) {
        if (idx_out) {
            TopkParams tp = make_topk(b, nullptr, 0, a->k, idx_out, nullptr);
            if ((st = hip_status(launch_select_all_visible(tp, b->total_q, s))) != DSA_OK) return st;
        }
        MlaParams mp = make_mla(b, a->q, a->kv, nullptr, a->k, a->scale, out, lse, mws, 1);
        return hip_status(launch_sparse_mla(mp, b->total_q, s));
    }

    if (b->max_kv > 0) {
        IndexerParams ip = make_indexer(b, a->q_fp8, a->q_scale, a->w, a->k_fp8, a->k_scale, scores,
                                        ld, indexer_chunk(b, decode), 0);
        if ((st = hip_status(launch_indexer(ip, b->total_q, b->max_q, decode, s))) != DSA_OK)
            return st;
    }
    TopkParams tp = make_topk(b, scores, ld, a->k, idx, tws);
    if ((st = hip_status(launch_topk(tp, b->total_q, s))) != DSA_OK) return st;
    MlaParams mp = make_mla(b, a->q, a->kv, idx, a->k, a->scale, out, lse, mws);
    return hip_status(launch_sparse_mla(mp, b->total_q, s));
}

}  // namespace

extern "C" {

dsa_status dsa_quantize_queries(const float *q, int64_t T, int HI, int DI, uint8_t *q_fp8,
                                float *q_scale, void *stream) {
    if (HI != kHI || DI != kDI) return DSA_ERR_UNSUPPORTED;
    if (T < 0) return DSA_ERR_INVALID_ARG;
    if (T == 0) return DSA_OK;
    if (T > INT32_MAX) return DSA_ERR_UNSUPPORTED;
    if (!q || !q_fp8 || !q_scale || !al16(q) || !al16(q_fp8) || !al16(q_scale)) return DSA_ERR_INVALID_ARG;
    return hip_status(launch_quant_queries(q, T, q_fp8, q_scale, static_cast<hipStream_t>(stream)));
}

dsa_status dsa_append_cache(const float *k_new, const uint16_t *kv_new, int64_t R, int DI, int D,
                            const int64_t *dst_rows, uint8_t *k_fp8, float *k_scale, uint16_t *kv,
                            int64_t N, void *stream) {
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
}

dsa_status dsa_indexer_scores(const dsa_batch *batch, const uint8_t *q_fp8, const float *q_scale,
                              const float *w, const uint8_t *k_fp8, const float *k_scale, int HI,
                              int DI, float *scores, int64_t ld, void *stream) {
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
}

dsa_status dsa_topk(const dsa_batch *batch, const float *scores, int64_t ld, int k, int32_t *idx,
                    void *ws, size_t ws_bytes, void *stream) {
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
    return hip_status(launch_topk(p, batch->total_q, static_cast<hipStream_t>(stream)));
}

dsa_status dsa_sparse_mla_fwd(const dsa_batch *batch, const uint16_t *q, const uint16_t *kv,
                              const int32_t *idx, int k, int H, int D, int Dv, float scale,
                              uint16_t *out, float *lse, void *ws, size_t ws_bytes, void *stream) {
    dsa_status st = check_batch(batch);
    if (st != DSA_OK) return st;
    if (H != kH || D != kD || Dv != kDv) return DSA_ERR_UNSUPPORTED;
    if ((st = check_k(k)) != DSA_OK) return st;
    if (batch->max_kv > MAX_KV_ATTN) return DSA_ERR_UNSUPPORTED;
    if (!std::isfinite(scale)) return DSA_ERR_INVALID_ARG;
    if (batch->total_q == 0) return DSA_OK;
    if (!q || !idx || !out || !lse) return DSA_ERR_INVALID_ARG;
    if (batch->total_kv > 0 && !kv) return DSA_ERR_INVALID_ARG;
    if (!al16(q) || !al16(idx) || !al16(out) || !al16(lse) || (kv && !al16(kv)))
        return DSA_ERR_INVALID_ARG;
    const size_t need = mla_ws(batch, k);
    if (need > 0 && (!ws || ws_bytes < need || !al16(ws))) return DSA_ERR_WORKSPACE;
    MlaParams p = make_mla(batch, q, kv, idx, k, scale, out, lse, ws);
    return hip_status(launch_sparse_mla(p, batch->total_q, static_cast<hipStream_t>(stream)));
}

dsa_status dsa_dense_mla_fwd(const dsa_batch *batch, const uint16_t *q, const uint16_t *kv, int H, int D,
                             int Dv, float scale, uint16_t *out, float *lse, void *ws, size_t ws_bytes,
                             void *stream) {
    dsa_status st = check_batch(batch);
    if (st != DSA_OK) return st;
    if (H != kH || D != kD || Dv != kDv) return DSA_ERR_UNSUPPORTED;
    if (batch->max_kv > kKMax) return DSA_ERR_UNSUPPORTED;
    if (!std::isfinite(scale)) return DSA_ERR_INVALID_ARG;
    if (batch->total_q == 0) return DSA_OK;
    if (!q || !out || !lse) return DSA_ERR_INVALID_ARG;
    if (batch->total_kv > 0 && !kv) return DSA_ERR_INVALID_ARG;
    if (!al16(q) || !al16(out) || !al16(lse) || (kv && !al16(kv))) return DSA_ERR_INVALID_ARG;
    const int kd = dense_slots(batch);
    const size_t need = mla_ws(batch, kd);
    if (need > 0 && (!ws || ws_bytes < need || !al16(ws))) return DSA_ERR_WORKSPACE;
    MlaParams p = make_mla(batch, q, kv, nullptr, kd, scale, out, lse, ws, 1);
    return hip_status(launch_sparse_mla(p, batch->total_q, static_cast<hipStream_t>(stream)));
}

dsa_status dsa_indexer_kl_fwd(const dsa_batch *batch, const uint16_t *q, const uint16_t *kv, const float *lse,
                              int H, int D, float scale, const float *scores, int64_t ld, const int32_t *idx,
                              int k, float *kl, float *p_out, void *ws, size_t ws_bytes, void *stream) {
    dsa_status st = check_batch(batch);
    if (st != DSA_OK) return st;
    if (H != kH || D != kD) return DSA_ERR_UNSUPPORTED;
    if (idx && (st = check_k(k)) != DSA_OK) return st;
    if (batch->max_kv > MAX_KV_ATTN) return DSA_ERR_UNSUPPORTED;
    if (!std::isfinite(scale)) return DSA_ERR_INVALID_ARG;
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
}

dsa_status dsa_sparse_mla_bwd(const dsa_batch *batch, const uint16_t *q, const uint16_t *kv, const int32_t *idx,
                              int k, int H, int D, int Dv, float scale, const uint16_t *out, const float *lse,
                              const uint16_t *dout, float *dq, float *dkv, void *ws, size_t ws_bytes,
                              void *stream) {
    dsa_status st = check_batch(batch);
    if (st != DSA_OK) return st;
    if (H != kH || D != kD || Dv != kDv) return DSA_ERR_UNSUPPORTED;
    if ((st = check_k(k)) != DSA_OK) return st;
    if (batch->max_kv > MAX_KV_ATTN) return DSA_ERR_UNSUPPORTED;
    if (!std::isfinite(scale)) return DSA_ERR_INVALID_ARG;
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
}

dsa_status dsa_prefill_fwd(const dsa_fwd_args *args, uint16_t *out, float *lse, int32_t *idx_out,
                           void *ws, size_t ws_bytes, void *stream) {
    return run_fwd(args, out, lse, idx_out, ws, ws_bytes, stream, false);
}

dsa_status dsa_decode_fwd(const dsa_fwd_args *args, uint16_t *out, float *lse, int32_t *idx_out,
                          void *ws, size_t ws_bytes, void *stream) {
    return run_fwd(args, out, lse, idx_out, ws, ws_bytes, stream, true);
}

size_t dsa_workspace_size(dsa_ws_entry entry, const dsa_batch *batch, int k, int H, int Dv) {
    if (!batch || batch->batch < 1 || batch->total_q < 0 || batch->max_kv < 0 || k < 1 ||
        k > kKMax || H != kH || Dv != kDv)
        return 0;
    switch (entry) {
        case DSA_WS_TOPK: return topk_ws(batch, k);
        case DSA_WS_SPARSE_MLA: return mla_ws(batch, k);
        case DSA_WS_PREFILL:
        case DSA_WS_DECODE: return fwd_ws(batch, k);
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
    }
    return "unknown status";
}

const char *dsa_version(void) { return "dsa-mi355x 0.1.0 (gfx950)"; }

}  // extern "C"
