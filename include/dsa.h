/*
 * dsa.h — C ABI of the MI355X (gfx950) DeepSeek Sparse Attention hot path.
 *
 * The operations follow these pages (cited by title and section):
 *   [R] "Техотчёт DeepSeek-V3.2 (2025): разреженное внимание DSA и
 *       масштабирование RL" (ai.flicky.cc):
 *         "Молниеносный индексатор" — index score
 *             I[t,s] = sum_j w[t,j] * ReLU(q[t,j] . k[s]) over a few FP8 heads,
 *             q and w from the current token, k from an earlier one;
 *         "Отбор и основное внимание" — u_t = Attn(h_t, {c_s : I[t,s] in
 *             Top-k(I[t,:])}), k = 2048, computed in MLA's MQA mode: one
 *             latent KV row is shared by every query head.
 *   [N] neurosova.ru news item on DeepSeek-V3.2, "DeepSeek Sparse Attention":
 *       a low-precision indexer over all token pairs, a selector keeping the
 *       top-k key/value positions per query, MQA + MLA on the selected set.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  * Pointers named in the argument lists are DEVICE pointers owned by the
 *    caller.  The library never allocates, frees or retains them, and keeps no
 *    state between calls besides its loaded code objects.  Calls only enqueue
 *    work on `stream` (a hipStream_t passed as void*, NULL = default stream)
 *    and return; outputs are ready once the caller synchronises the stream.
 *  * Host-side validation runs before any launch: a null pointer, a size or
 *    stride that does not fit, a misaligned pointer (16 bytes for every
 *    array except the batch arrays) or an unsupported shape returns an error
 *    status and launches nothing.  Errors reported by the HIP runtime at
 *    launch return DSA_ERR_HIP; faults inside kernels surface when the caller
 *    synchronises.  No C++ exception crosses this interface.
 *  * Supported shapes: indexer heads HI = 64 of dim DI = 128 (FP8 E4M3FN, the
 *    OCP format, max 448); query heads H = 128 over D = 576 bf16 dims
 *    (512 latent + 64 rope), value = the first Dv = 512 dims; 1 <= k <= 2048.
 *    Anything else returns DSA_ERR_UNSUPPORTED.
 *  * Diagnostics, read from the environment at every call: DSA_LOG=1 prints
 *    one line per call on stderr (batch, k, workspace given, the fused
 *    entries' launch plan, the status); DSA_DEBUG_CHECKS=1 validates every
 *    selection an entry produces (dsa_topk, dsa_indexer_topk, the fused
 *    entries) with dsa_check_selection, which drains the stream, and returns
 *    DSA_ERR_CHECK if a row breaks the contract.  Both are off by default and
 *    have no place under graph capture.
 *  * Every `scale` argument (the softmax scale of the attention) must be
 *    finite and > 0, else DSA_ERR_INVALID_ARG.
 *  * Positions: score columns and idx entries are positions local to their
 *    sequence (0 = the sequence's first cache row).  Query row cu_q[b]+i sits
 *    at absolute position pos0[b]+i and sees the keys 0..min(pos, ctx_b-1)
 *    (the key of its own position included), where ctx_b = cu_kv[b+1]-cu_kv[b].
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DSA_OK = 0,
    DSA_ERR_INVALID_ARG = 1,   /* null pointer, bad size, stride or alignment */
    DSA_ERR_UNSUPPORTED = 2,   /* shape outside the supported set above */
    DSA_ERR_WORKSPACE = 3,     /* workspace null or smaller than required */
    DSA_ERR_HIP = 4,           /* the HIP runtime rejected a launch */
    DSA_ERR_CHECK = 5          /* debug mode (DSA_DEBUG_CHECKS) found an output that
                                  breaks its contract */
} dsa_status;

/* Ragged batch of B sequences.  The scalars are host values (used for
 * validation and grid sizing); the three arrays are device arrays that must
 * agree with them.  Kernels clamp every cache access to [0, total_kv), so a
 * descriptor whose arrays disagree with its scalars yields wrong values but
 * no out-of-bounds access. */
typedef struct {
    int32_t batch;           /* B >= 1 */
    int32_t total_q;         /* T = cu_q[B] >= 0 */
    int32_t max_q;           /* max over b of cu_q[b+1]-cu_q[b] */
    int32_t max_kv;          /* max over b of ctx_b, <= 2^24 */
    int64_t total_kv;        /* N = cu_kv[B] */
    const int32_t *cu_q;     /* [B+1] device, non-decreasing, cu_q[0] = 0 */
    const int64_t *cu_kv;    /* [B+1] device, non-decreasing, cu_kv[0] = 0 */
    const int32_t *pos0;     /* [B]   device, position of each sequence's first query */
} dsa_batch;

/* Index scores, [R] "Молниеносный индексатор":
 *   I[t,s] = k_scale[s] * sum_j (w[t,j] * q_scale[t,j]) * max(0, sum_d q[t,j,d] * k[s,d])
 * which equals eq. I on the dequantised inputs q[t,j,:]*q_scale[t,j] and
 * k[s,:]*k_scale[s] (the scales are positive and ReLU is positively
 * homogeneous).  FP8 products accumulate in fp32 on the matrix cores.
 *   q_fp8   [T, HI, DI] uint8 E4M3FN codes      q_scale [T, HI] fp32 (> 0)
 *   w       [T, HI]     fp32 head weights
 *   k_fp8   [N, DI]     uint8 E4M3FN codes      k_scale [N] fp32 (> 0)
 *   scores  [T, ld]     fp32 out: columns s < ctx_b of row t are written,
 *                       -inf where s > pos (causally masked); columns >= ctx_b
 *                       are left untouched.  ld >= max_kv.                    */
dsa_status dsa_indexer_scores(const dsa_batch *batch,
                              const uint8_t *q_fp8, const float *q_scale, const float *w,
                              const uint8_t *k_fp8, const float *k_scale,
                              int HI, int DI, float *scores, int64_t ld, void *stream);

/* Top-k selection, [R] "Отбор и основное внимание" (Top-k(I[t,:])):
 * for every query row, the k largest scores among its visible columns
 * s <= min(pos, ctx_b-1), compared as fp32 values (-0 == +0), ties to the
 * lower s; every visible column when there are at most k.  Output idx [T, k]
 * int32: the selected positions in ascending order, padded with -1.
 * Scores must be NaN-free.  Rows longer than 32768 columns are selected in
 * 32768-column chunks whose exact local top-k candidates are merged; this
 * needs workspace (dsa_workspace_size(DSA_WS_TOPK, ...)); ws may be NULL
 * when that size is 0. */
dsa_status dsa_topk(const dsa_batch *batch, const float *scores, int64_t ld, int k,
                    int32_t *idx, void *ws, size_t ws_bytes, void *stream);

/* Index scores and top-k selection in one call, with the scores kept on chip
 * ([R] "Молниеносный индексатор" for I[t,s], "Отбор и основное внимание"
 * for Top-k(I[t,:]) and its data flow: the cheap selection feeds the
 * attention; the T x N score matrix is never written).  The result equals
 * dsa_indexer_scores followed by dsa_topk on the same inputs, bit for bit:
 * the same fp32 scores (same arithmetic), the same exact selection (k largest
 * visible scores, -0 == +0, ties to the lower position, ascending, -1 padded).
 * How: a strided sample of each row's keys sets a score threshold; the
 * indexer keeps only the keys at or above it (with their positions) as
 * candidates, and an exact select over them is checked to be complete (at
 * least k candidates, no region overflow).  Rows that fail the check (rare:
 * a threshold drawn too high, many equal scores) are recomputed on chip,
 * 32768 columns at a time, still without writing scores.
 *   inputs as dsa_indexer_scores; idx [T, k] int32 out.
 * Workspace (required): dsa_workspace_size(DSA_WS_INDEXER_TOPK, ...): the
 * candidate lists, about 8 bytes x min(8192, columns) per query row for
 * prefill-shaped batches (max_q >= 16), 8 bytes per cached column for
 * decode-shaped ones.  Supported: max_kv <= 262144, 1 <= k <= 2048. */
dsa_status dsa_indexer_topk(const dsa_batch *batch,
                            const uint8_t *q_fp8, const float *q_scale, const float *w,
                            const uint8_t *k_fp8, const float *k_scale, int HI, int DI,
                            int k, int32_t *idx, void *ws, size_t ws_bytes, void *stream);

/* Sparse attention in MLA's MQA mode, [R] "Отбор и основное внимание", eq. u,
 * and [N]: for each query row t and head h,
 *   z_s = scale * sum_{d<D} q[t,h,d] * kv[s,d]   over s in idx[t,:]
 *   out[t,h,c] = sum_s softmax(z)_s * kv[s,c]     for c < Dv
 *   lse[t,h]   = ln sum_s exp(z_s)
 * Every head uses the same selected rows.  Entries of idx that are -1 or
 * outside [0, ctx_b) are skipped; a row with no valid entry gives out = 0 and
 * lse = -inf.  Accumulation in fp32 (online softmax), output rounded to bf16.
 *   q   [T, H, D] bf16      kv [N, D] bf16 (latent rows; value = first Dv)
 *   idx [T, k] int32        out [T, H, Dv] bf16        lse [T, H] fp32
 * Workspace (dsa_workspace_size(DSA_WS_SPARSE_MLA, ...)) holds split-KV
 * partial results when the batch has few query rows; it may be 0 bytes.
 * Supported contexts: max_kv <= 2^21. */
dsa_status dsa_sparse_mla_fwd(const dsa_batch *batch, const uint16_t *q, const uint16_t *kv,
                              const int32_t *idx, int k, int H, int D, int Dv, float scale,
                              uint16_t *out, float *lse, void *ws, size_t ws_bytes,
                              void *stream);

/* "MHA with mask", the short-sequence mode of [R] "Стоимость": for short
 * sequences the pages run a separate masked dense mode that reproduces DSA's
 * result.  Each query row attends to every key it can see (positions
 * 0..min(pos, ctx_b-1)), with the same arithmetic, layouts and outputs as
 * dsa_sparse_mla_fwd:
 *   z_s = scale * sum_{d<D} q[t,h,d] * kv[s,d]     for s = 0 .. nvis_t - 1
 *   out[t,h,c] = sum_s softmax(z)_s * kv[s,c]  (c < Dv),  lse[t,h] = ln sum_s exp(z_s)
 * Where every row sees at most k keys, DSA's top-k keeps all of them, so
 * this equals the indexer -> top-k -> dsa_sparse_mla_fwd path (the fused
 * entries below switch to it on their own).  No scores, no idx.  The
 * attention stays in MLA's latent (MQA) form over the 576-dim cache rows; a
 * per-head decompressed form would need the up-projections, which are not
 * inputs of this library.
 *   q [T, H, D] bf16, kv [N, D] bf16, out [T, H, Dv] bf16, lse [T, H] fp32
 * Supported: max_kv <= 2048 (else DSA_ERR_UNSUPPORTED).  A row that sees no
 * key gives out = 0, lse = -inf.  Workspace:
 * dsa_workspace_size(DSA_WS_DENSE_MLA, ...) (split-KV partials; may be 0). */
dsa_status dsa_dense_mla_fwd(const dsa_batch *batch, const uint16_t *q, const uint16_t *kv, int H, int D,
                             int Dv, float scale, uint16_t *out, float *lse, void *ws, size_t ws_bytes,
                             void *stream);

/* Indexer KL loss, [R] "Как учили индексатор": the indexer learns where the
 * main attention looks.  For query row t over its key set (idx == NULL: every
 * visible key, the dense warm-up; else the valid slots of idx[t,:], the sparse
 * stage; a position listed twice is two slots):
 *   q_s   = sum_h exp(scale * <q[t,h,:], kv[s,:]> - lse[t,h])
 *           (the attention's probabilities summed over the heads),
 *   p_s   = q_s / sum_s q_s                        (L1 normalisation),
 *   kl[t] = sum_s p_s * (ln p_s - ln softmax_s(scores[t, s]))   (natural log).
 * lse must be the attention's log-sum-exp over the same set (what
 * dsa_sparse_mla_fwd / dsa_dense_mla_fwd return for it); a head with a
 * non-finite lse contributes nothing.  A row with no usable slot gives 0.
 *   q [T, H, D] bf16, kv [N, D] bf16, lse [T, H] fp32, scores [T, ld] fp32
 *   (the index scores, e.g. from dsa_indexer_scores), idx [T, k] int32 or NULL
 *   kl [T] fp32 out; p_out (nullable) fp32 out: the target p, [T, k] per slot
 *   (0 for unusable slots) in the sparse stage, [T, ld] per column (columns
 *   0..nvis-1 written) in the dense one.
 * Supported: H = 128, D = 576, 1 <= k <= 2048, max_kv <= 2^21, ld >= max_kv.
 * Workspace (required): dsa_workspace_size(DSA_WS_INDEXER_KL, batch, k, ...)
 * with the same k (any 1..2048 for the dense stage). */
dsa_status dsa_indexer_kl_fwd(const dsa_batch *batch, const uint16_t *q, const uint16_t *kv, const float *lse,
                              int H, int D, float scale, const float *scores, int64_t ld, const int32_t *idx,
                              int k, float *kl, float *p_out, void *ws, size_t ws_bytes, void *stream);

/* Backward of dsa_sparse_mla_fwd over the same selection, for the sparse
 * training stage of [R] "Как учили индексатор" (all parameters learn).  With
 * P[h,j] = exp(scale <q[t,h,:], kv[s_j,:]> - lse[t,h]) over the valid slots j
 * of idx[t,:] (positions s_j), dP[h,j] = <dout[t,h,:], kv[s_j,:Dv]> and
 * delta[h] = <dout[t,h,:], out[t,h,:]>:
 *   dZ[h,j]      = P[h,j] (dP[h,j] - delta[h])
 *   dq[t,h,:]    = scale * sum_j dZ[h,j] kv[s_j,:]
 *   dkv[s_j,:]  += scale * sum_h dZ[h,j] q[t,h,:]      (all D dims: the key)
 *   dkv[s_j,:Dv] += sum_h P[h,j] dout[t,h,:]           (the value)
 * summed over every row and slot that selects a cache row (a position listed
 * twice counts twice).  out and lse are the forward's outputs for the same
 * inputs.  P and dZ are rounded to bf16 before the products that consume them
 * (the usual precision of attention backward passes), and so is each slot's
 * dkv contribution before it is summed per cache row; accumulation in fp32.
 *   q [T,H,D] bf16, kv [N,D] bf16, idx [T,k] int32, out [T,H,Dv] bf16,
 *   lse [T,H] fp32, dout [T,H,Dv] bf16
 *   dq [T,H,D] fp32 out (overwritten); dkv [N,D] fp32 out (overwritten; the
 *   order in which a cache row's contributions are added varies from call to
 *   call, and so do its low bits).
 * Supported: H = 128, D = 576, Dv = 512, 1 <= k <= 2048, max_kv <= 2^21.
 * Workspace (required when T > 0): dsa_workspace_size(DSA_WS_SPARSE_MLA_BWD,
 * ...): the rows are processed in chunks of 4096, and the workspace holds one
 * chunk (about 1.7 KB per (row, slot) plus 8 bytes per cache row). */
dsa_status dsa_sparse_mla_bwd(const dsa_batch *batch, const uint16_t *q, const uint16_t *kv, const int32_t *idx,
                              int k, int H, int D, int Dv, float scale, const uint16_t *out, const float *lse,
                              const uint16_t *dout, float *dq, float *dkv, void *ws, size_t ws_bytes,
                              void *stream);

/* All inputs of one DSA forward (indexer + top-k + sparse MQA attention). */
typedef struct {
    dsa_batch batch;
    const uint8_t *q_fp8;    /* [T, HI, DI] */
    const float *q_scale;    /* [T, HI] */
    const float *w;          /* [T, HI] */
    const uint8_t *k_fp8;    /* [N, DI] indexer key cache */
    const float *k_scale;    /* [N] */
    const uint16_t *q;       /* [T, H, D] bf16 */
    const uint16_t *kv;      /* [N, D] bf16 latent cache */
    int32_t HI, DI, H, D, Dv, k;
    float scale;             /* softmax scale, finite and > 0, e.g. 1/sqrt(D) */
} dsa_fwd_args;

/* The whole hot path in one call, following the data flow of [R]
 * "Отбор и основное внимание" (cheap selection first, then attention over the
 * k selected rows): index scores -> top-k -> sparse MQA attention, the first
 * two as dsa_indexer_topk (no score matrix in memory).  Results equal
 * dsa_indexer_scores + dsa_topk + dsa_sparse_mla_fwd on the same inputs.
 * dsa_prefill_fwd is tuned for many query rows per sequence (prefill, chunked
 * prefill); dsa_decode_fwd for one or a few query rows per sequence over long
 * contexts (split-KV).  Both accept any batch.
 * Short sequences: when every context fits in k (max_kv <= k) the top-k of
 * each row is all of its visible keys, so both entries skip the indexer and
 * the select, write that selection to idx_out, and run the dense masked
 * attention of dsa_dense_mla_fwd (the "MHA with mask" mode of [R]
 * "Стоимость"); out and lse are bit-identical to the three-step path.
 *   out [T, H, Dv] bf16, lse [T, H] fp32, idx_out [T, k] int32 (nullable:
 *   the selected positions, as dsa_topk returns them).
 * Workspace: dsa_workspace_size(DSA_WS_PREFILL or DSA_WS_DECODE, ...). */
dsa_status dsa_prefill_fwd(const dsa_fwd_args *args, uint16_t *out, float *lse,
                           int32_t *idx_out, void *ws, size_t ws_bytes, void *stream);
dsa_status dsa_decode_fwd(const dsa_fwd_args *args, uint16_t *out, float *lse,
                          int32_t *idx_out, void *ws, size_t ws_bytes, void *stream);

/* dsa_decode_fwd without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Same arguments, launches and results as
 * dsa_decode_fwd (bit for bit); the workspace is a static device array of
 * the library, dsa_decode_fwd_noalloc_max_bytes() = 128 MiB, one copy per
 * GPU, held until the process ends (enough for 64 sequences of 128K-token
 * contexts, or 256 of 32K).  A batch whose dsa_workspace_size(DSA_WS_DECODE,
 * ...) exceeds it returns DSA_ERR_WORKSPACE before any launch.  The call
 * allocates nothing: on its first use on a device it looks up that device's
 * copy of the array (hipGetSymbolAddress).  Every call on a GPU shares that
 * GPU's array and leaves its last contents there (the kernels clear what they
 * need cleared): calls that overlap on one GPU (several streams, several host
 * threads) race, so serialise them. */
dsa_status dsa_decode_fwd_noalloc(const dsa_fwd_args *args, uint16_t *out, float *lse,
                                  int32_t *idx_out, void *stream);
size_t dsa_decode_fwd_noalloc_max_bytes(void);

/* Measurement helper (not part of the hot path's data flow): runs the same
 * launches as dsa_prefill_fwd (decode = 0) or dsa_decode_fwd (decode != 0)
 * with a HIP event recorded on `stream` before the first launch and after
 * each one, then WAITS for the last event (a host synchronisation, unlike
 * every other entry point) and reports, per launch in order, the kernel's
 * name and the time between its two events in ms (launch gaps included).
 * Outputs, workspace and errors are those of the entry it runs; `times`
 * [max_times] and `n_times` are host memory; kernel names are static
 * strings.  Events are created and destroyed inside the call.  `items`
 * counts what the library itself tallies for a kernel: for the fused
 * wave select, the candidates it selected over (all rows); for the
 * workgroup select, the rows it selected (every row of a batch of few rows,
 * else those the wave select handed on); for the on-chip recompute, the rows
 * it recomputed; -1 for the others. */
typedef struct {
    const char *kernel;
    float ms;
    int64_t items;
} dsa_kernel_time;
dsa_status dsa_fwd_profile(const dsa_fwd_args *args, int decode, uint16_t *out, float *lse,
                           int32_t *idx_out, void *ws, size_t ws_bytes, void *stream,
                           dsa_kernel_time *times, int max_times, int *n_times);

/* Measurement helper (not part of the hot path's data flow): the rates this
 * GPU attains, under its own clock and power limits, for the work the
 * rooflines price against the spec-sheet peaks: the 16x16x32 bf16 MFMA (the
 * attention's product) and the 16x16x128 FP8 MFMA (the indexer's), each in
 * 8 independent accumulator chains per wave, 16 waves per compute unit; a
 * streaming read and a streaming copy (16-byte non-temporal loads and
 * stores) over `buf`.  `buf` is caller-owned device memory of `bytes` bytes
 * (at least 64 MiB, 16-byte aligned; several times the 256 MB Infinity
 * Cache for a memory-bound figure), used as scratch: its contents are
 * overwritten.  Each loop runs 3 times on `stream`, the fastest run counts;
 * the call WAITS for `stream`.  The copy rate counts the bytes read plus
 * the bytes written.  Events are created and destroyed inside the call. */
typedef struct {
    double bf16_tflops;
    double fp8_tflops;
    double hbm_read_gbs;
    double hbm_copy_gbs;
} dsa_peaks;
dsa_status dsa_measure_peaks(void *buf, size_t bytes, void *stream, dsa_peaks *out);

/* Validation of a selection against the contract of Top-k ([R] "Отбор и
 * основное внимание": the k top-scored visible keys of each query row):
 * every row t of idx [T, k] int32 (device) must hold exactly min(k, n_t)
 * positions, strictly ascending and inside 0..n_t-1 (n_t = the row's visible
 * keys), then -1 in the remaining slots.  Writes the number of rows that do
 * not to *bad_rows (host memory).  The call WAITS for `stream` (it reads the
 * count back); the count lives in a small static device variable of the
 * library, so concurrent calls on one GPU race.  This is the check that
 * DSA_DEBUG_CHECKS=1 runs after every entry that selects. */
dsa_status dsa_check_selection(const dsa_batch *batch, const int32_t *idx, int k, void *stream, int *bad_rows);

/* FP8 quantisation of the indexer queries, the step before the index score
 * ([R] "Молниеносный индексатор": the indexer runs on FP8 values).  Per
 * token t, one scale over its HI x DI values:
 *   s_t = absmax_t / 448 in fp32 (1 for an all-zero token),
 *   q_fp8[t,j,d] = E4M3FN(q[t,j,d] / s_t): the division in fp32 (correctly
 *   rounded), then the nearest E4M3FN code, ties to the even mantissa,
 *   magnitudes above 448 saturate to 448, sign bit from the quotient;
 *   q_scale[t,j] = s_t for every head j.
 *   q [T, HI, DI] fp32 (finite)   q_fp8 [T, HI, DI] uint8 out   q_scale [T, HI] fp32 out
 * HI = 64, DI = 128 (else DSA_ERR_UNSUPPORTED).  All pointers device, 16-byte
 * aligned, caller-owned; the call only enqueues work on `stream`. */
dsa_status dsa_quantize_queries(const float *q, int64_t T, int HI, int DI, uint8_t *q_fp8,
                                float *q_scale, void *stream);

/* Cache append: the R new tokens' indexer keys are quantised as above, one
 * scale per key row (k_scale[row] = absmax/448), and written with their scale
 * to rows dst_rows[r] of the FP8 key cache; their bf16 latent rows are copied
 * to the same rows of the latent cache.  Rows r whose dst_rows[r] lies
 * outside [0, N) are skipped.
 *   k_new [R, DI] fp32 (finite)   kv_new [R, D] bf16 bits (NULL: keys only)
 *   dst_rows [R] int64 device
 *   k_fp8 [N, DI] uint8, k_scale [N] fp32, kv [N, D] bf16 (NULL with kv_new NULL)
 * DI = 128, D = 576 (else DSA_ERR_UNSUPPORTED).  Device pointers, 16-byte
 * aligned; rows of one call must be distinct (else the last write wins). */
dsa_status dsa_append_cache(const float *k_new, const uint16_t *kv_new, int64_t R, int DI, int D,
                            const int64_t *dst_rows, uint8_t *k_fp8, float *k_scale, uint16_t *kv,
                            int64_t N, void *stream);

typedef enum {
    DSA_WS_TOPK = 0,
    DSA_WS_SPARSE_MLA = 1,
    DSA_WS_PREFILL = 2,
    DSA_WS_DECODE = 3,
    DSA_WS_DENSE_MLA = 4,      /* k is ignored (pass any 1..2048) */
    DSA_WS_INDEXER_KL = 5,
    DSA_WS_SPARSE_MLA_BWD = 6,
    DSA_WS_INDEXER_TOPK = 7     /* the layout depends on max_q (>= 16: prefill-shaped) */
} dsa_ws_entry;

/* Workspace bytes the given entry point needs for this batch (host only; reads
 * only the host scalars of the batch).  Returns 0 on invalid arguments. */
size_t dsa_workspace_size(dsa_ws_entry entry, const dsa_batch *batch, int k, int H, int Dv);

const char *dsa_status_string(dsa_status status);
const char *dsa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
