// kernels.h — launch parameters of the gfx950 kernels and their host-side
// launchers (one per kernel family).  Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

struct IndexerParams {
    const int32_t *cu_q;
    const int64_t *cu_kv;
    const int32_t *pos0;
    int B;
    int64_t total_kv;
    int max_kv;
    const uint8_t *q;       // [T, 64, 128] e4m3
    const float *q_scale;   // [T, 64]
    const float *w;         // [T, 64]
    const uint8_t *k;       // [N, 128] e4m3
    const float *k_scale;   // [N]
    float *scores;          // [T, ld]
    int64_t ld;
    int key_chunk;          // keys per workgroup
    int fill_masked;        // write -inf for s in [nvis, ctx)
    // Candidate mode (the fused indexer + select; scores are not written):
    // the visible keys of row t whose score key (score_key of the fp32 score)
    // is >= tau[t] go, in column order, to the row's candidate regions.
    // Region r of row t covers columns [r * seg_w, (r + 1) * seg_w) and holds
    // up to cap (key, position) pairs at slot (t * nseg + r) * cap; cand_cnt
    // receives the number found (more than cap: the region overflowed).
    const uint32_t *tau;    // [T]
    uint32_t *cand_key;     // [T * nseg * cap]
    int32_t *cand_pos;      // [T * nseg * cap]
    int32_t *cand_cnt;      // [T * nseg]
    int seg_w, nseg, cap;
    int topk_k;             // k of the select (row blocks that see at most k keys need no candidates)
};

// The fused indexer + select (indexer_topk.hip): a sampled threshold per row,
// the indexer in candidate mode, an exact select over the candidates, and an
// on-chip recompute for rows whose threshold failed.
struct IdxTopkParams {
    IndexerParams ix;       // inputs, candidate regions and thresholds
    uint32_t *tau;          // [T] written by the sample kernel (same array as ix.tau)
    int k;
    int32_t *idx;           // [T, k] out
    int32_t *fb;            // [FB_LIST + 2T]: recompute queue (count, next), candidates selected
                            // over (all rows), workgroup-select queue (count, next), then the
                            // recompute queue's rows [T] and the workgroup-select queue's rows [T]
};
constexpr int FB_LIST = 5;

struct TopkParams {
    const int32_t *cu_q;
    const int64_t *cu_kv;
    const int32_t *pos0;
    int B;
    int64_t total_kv;
    int max_kv;
    const float *scores;    // [T, ld]
    int64_t ld;
    int k;
    int32_t *idx;           // [T, k]
    uint32_t *cand_key;     // [T, nchunk, k] workspace (rows longer than one chunk)
    int32_t *cand_pos;      // [T, nchunk, k]
    int nchunk;             // chunks per row = ceil(max_kv / TOPK_CHUNK)
};

struct MlaParams {
    const int32_t *cu_q;
    const int64_t *cu_kv;
    const int32_t *pos0;
    int B;
    int64_t total_kv;
    int max_kv;
    const uint16_t *q;      // [T, 128, 576] bf16
    const uint16_t *kv;     // [N, 576] bf16
    const int32_t *idx;     // [T, k] (unused when dense)
    int k;                  // slots per row (dense: the slot budget, >= every row's visible count)
    int dense;              // 1: slot j of a row is position j for j < its visible count (idx unused)
    float scale_log2;       // softmax scale * log2(e)
    uint16_t *out;          // [T, 128, 512] bf16
    float *lse;             // [T, 128]
    int splits;             // workgroups per query row (split-KV)
    int blocks_per_split;   // MLA_BK-key blocks per split
    uint16_t *o_part;       // [T, splits, 128, 512] bf16 (splits > 1)
    float *lse_part;        // [T, splits, 128]
};

struct KlParams {
    const int32_t *cu_q;
    const int64_t *cu_kv;
    const int32_t *pos0;
    int B;
    int64_t total_kv;
    int max_kv;
    const uint16_t *q;      // [T, 128, 576] bf16
    const uint16_t *kv;     // [N, 576] bf16
    const float *lse;       // [T, 128] attention log-sum-exp (natural log)
    float scale_log2;       // softmax scale * log2(e)
    const float *scores;    // [T, ld] index scores
    int64_t ld;
    const int32_t *idx;     // [T, k] selected slots, or null: every visible key
    int k;
    float *kl;              // [T]
    float *p_out;           // nullable: [T, k] per slot, or [T, ld] per column
    int splits;             // workgroups per row
    int blocks_per_split;   // KL_BK-slot blocks per split
    float *part;            // [T, splits, 5] partial sums (workspace)
};

struct BwdParams {
    const int32_t *cu_q;
    const int64_t *cu_kv;
    const int32_t *pos0;
    int B;
    int64_t total_kv;
    int max_kv;
    const uint16_t *q;      // [T, 128, 576] bf16
    const uint16_t *kv;     // [N, 576] bf16
    const int32_t *idx;     // [T, k]
    int k;
    int kpad;               // k rounded up to whole 32-slot blocks
    float scale;            // softmax scale
    float scale_log2;       // scale * log2(e)
    const uint16_t *out;    // [T, 128, 512] bf16 forward output
    const float *lse;       // [T, 128] forward log-sum-exp (natural log)
    const uint16_t *dout;   // [T, 128, 512] bf16 gradient of out
    float *dq;              // [T, 128, 576] out
    float *dkv;             // [N, 576] out (zeroed, then accumulated)
    int t0, tc;             // the chunk of query rows [t0, t0 + tc) a launch works on
    // workspace of one chunk (row t at t - t0)
    uint16_t *ps;           // [tc, kpad, 128] bf16: P
    uint16_t *dzs;          // [tc, kpad, 128] bf16: scale * dZ
    uint16_t *g;            // [tc, kpad, 576] bf16: each slot's sum over heads (its dkv contribution)
    int32_t *cnt;           // [N + 1] slots per cache row, then their exclusive prefix
    int32_t *cur;           // [N] fill cursors
    int32_t *list;          // [tc * kpad] the chunk's usable slots ((t - t0) * kpad + j), by cache row
    int32_t *bsum;          // [scan blocks + 1] scan block totals
};

constexpr int BWD_CHUNK = 4096;       // query rows per pass of the backward

constexpr int TOPK_CHUNK = 32768;     // columns selected per workgroup in LDS
constexpr int TOPK_MAX_CHUNKS = 8;    // merge capacity: 8 x 2048 candidates
constexpr int MLA_BK = 32;            // keys per gathered block
constexpr int KL_BK = 32;             // slots per block of the KL loss
constexpr int MAX_KV_ATTN = 1 << 21;  // per-sequence rows the gathers address with 32-bit offsets
constexpr int CAND_DECODE_SEG = 512;  // columns per candidate region of the decode indexer (one wave's range)
constexpr int CAND_CAP = 8192;        // candidate slots per region of the prefill indexer, at most
constexpr int CAND_SELECT_MAX = 16384;  // candidates one select workgroup holds in registers

// Per-kernel timing hook: a launcher that enqueues several kernels calls
// after(kernel name) right after each launch (null: no timing).
struct LaunchMarks {
    virtual void after(const char *kernel, hipStream_t s) = 0;
    virtual ~LaunchMarks() = default;
};

hipError_t launch_indexer(const IndexerParams &p, int T, int max_q, bool decode_variant,
                          hipStream_t s);
// indexer in candidate mode (p.tau, p.cand_*): prefill or decode layout
hipError_t launch_indexer_cand(const IndexerParams &p, int T, int max_q, bool decode_variant, hipStream_t s);
// the fused indexer + select: sample -> candidate indexer -> select -> recompute of failed rows
hipError_t launch_indexer_topk(const IdxTopkParams &p, int T, int max_q, bool decode_variant, hipStream_t s,
                               LaunchMarks *m = nullptr);
hipError_t launch_topk(const TopkParams &p, int T, hipStream_t s, LaunchMarks *m = nullptr);
hipError_t launch_select_all_visible(const TopkParams &p, int T, hipStream_t s);
// Debug mode: counts (into *bad_out, after draining the stream) the rows of
// idx [T, k] that are not min(k, visible) ascending visible positions followed
// by -1.
hipError_t check_selection(const int32_t *cu_q, const int64_t *cu_kv, const int32_t *pos0, int B, int64_t total_kv,
                           int max_kv, int T, const int32_t *idx, int k, hipStream_t s, int *bad_out);
hipError_t launch_sparse_mla(const MlaParams &p, int T, hipStream_t s, LaunchMarks *m = nullptr);
hipError_t launch_sparse_mla_bwd(const BwdParams &p, int T, hipStream_t s);
hipError_t launch_indexer_kl(const KlParams &p, int T, hipStream_t s);
hipError_t launch_quant_queries(const float *q, int64_t T, uint8_t *q_fp8, float *q_scale, hipStream_t s);
hipError_t launch_append_cache(const float *k_new, const uint16_t *kv_new, int64_t R, const int64_t *dst,
                               uint8_t *k_fp8, float *k_scale, uint16_t *kv, int64_t N, hipStream_t s);

}  // namespace dsa
