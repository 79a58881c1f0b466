/*
 * dsa_oracle.c — plain, slow, CPU reference of the DeepSeek Sparse Attention
 * (DSA) hot path.  TEST INFRASTRUCTURE ONLY: the GPU library never links,
 * loads or calls this file; only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header, table or
 * constant with the GPU path.
 *
 * Sources (pages of text; cited by title and section, never by line):
 *   [R]  "Техотчёт DeepSeek-V3.2 (2025): разреженное внимание DSA и
 *         масштабирование RL" (ai.flicky.cc), sections
 *         "Молниеносный индексатор" (the index-score equation I_{t,s}) and
 *         "Отбор и основное внимание" (the selection equation u_t, the
 *         MQA-mode remark and the data-flow figure).
 *   [N]  neurosova.ru news item on DeepSeek-V3.2, section
 *         "DeepSeek Sparse Attention" (indexer over all token pairs in low
 *         precision; selector keeps top-k key/value positions; MQA + MLA on
 *         the sparse set).
 *
 * What is computed (everything in double, outputs rounded once at the end):
 *   1. FP8 E4M3FN / bf16 decoding from the bit-level format definitions
 *      (OCP FP8: 1 sign, 4 exponent bits, bias 7, 3 mantissa bits, no
 *      infinities, S.1111.111 is NaN; bf16: the top 16 bits of an IEEE
 *      binary32).  Dequantised value = decode(code) * scale, exact in double.
 *   2. Index score, [R] "Молниеносный индексатор":
 *        I[t,s] = sum_j w[t,j] * max(0, sum_d q[t,j,d] * k[s,d])
 *      for visible s (s <= position of t, s < context length), else -inf.
 *      Also A[t,s] = sum_j |w[t,j]| * max(0, ...), the absolute-term sum used
 *      as the tolerance scale where signed w makes I cancel.
 *   3. Top-k, [R] "Отбор и основное внимание": the k highest I[t,s] over the
 *      visible s, compared as binary32 values (the precision the scores are
 *      stored in), ties to the lower s; all visible s when there are at most k
 *      of them; output in ascending s, padded with -1.
 *   4. Attention over the selected latent rows in MQA mode (one selected set
 *      and one latent row shared by every query head), [R] "Отбор и основное
 *      внимание" and [N]: z_s = scale * <q[t,h,:], kv[s,:]> over all D dims,
 *      o[t,h,c] = sum_s exp(z_s - M) kv[s,c] / sum_s exp(z_s - M) for c < Dv,
 *      lse = M + ln(sum_s exp(z_s - M)), M = max z.  Exact softmax, not online.
 *   5. Dense causal attention: step 4 over every visible s (brute force).
 *   6. FP8 quantisation of a row group, the step before the index score
 *      ([R] "Молниеносный индексатор": the indexer runs on FP8 values): one
 *      scale per group s = absmax / 448 (binary32; 1 for an all-zero group),
 *      y = x / s (binary32), code = the E4M3FN code nearest to y by
 *      exhaustive search over the finite codes, ties to the code with an even
 *      mantissa; |y| above 448 takes 448; the sign bit is that of y.
 *   7. Indexer KL loss, [R] "Как учили индексатор": the target is the main
 *      attention's probabilities (step 4's exact per-head softmax over the key
 *      set) summed over the heads and L1-normalised; the loss is
 *      KL(target || softmax of I) over the same set: every visible key
 *      (dense warm-up) or the selected slots (sparse stage).
 *   8. Backward of step 4 over the same selection: the exact softmax's
 *      backward (dZ = P (dP - delta)), then the two products that use z
 *      (query and key sides) and the one that uses the value (the first Dv
 *      dims of the same latent row), summed over heads per selected row.
 *
 * Batch description shared by every function: B sequences; query rows of
 * sequence b are [cu_q[b], cu_q[b+1]); its cache rows are
 * [cu_kv[b], cu_kv[b+1]); query row cu_q[b]+i sits at absolute position
 * pos0[b]+i and sees sequence-local key positions 0..min(pos, ctx_b-1).
 * All positions in idx / score columns are sequence-local.
 *
 * `rows` (nullable) restricts the work to a list of global query rows;
 * outputs are then indexed by the position in that list.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORA_OK 0
#define ORA_ERR 1

/* ---------------------------------------------------------------- codecs */

/* OCP FP8 E4M3FN: value = (-1)^S * 2^(E-7) * (1 + M/8) for E > 0,
 * (-1)^S * 2^-6 * (M/8) for E == 0; E == 15 && M == 7 is NaN. */
double ora_e4m3_value(uint8_t code)
{
    int sign = (code >> 7) & 1;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double v;
    if (e == 0xF && m == 0x7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -v : v;
}

/* bf16: the 16 most significant bits of an IEEE-754 binary32. */
double ora_bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

void ora_e4m3_decode_all(double *table256)
{
    for (int c = 0; c < 256; c++)
        table256[c] = ora_e4m3_value((uint8_t)c);
}

/* E4M3FN code nearest to y (binary32), by exhaustive search over the finite
 * non-negative codes 0x00..0x7E (their values increase with the code), ties to
 * the even code (even mantissa); values above 448 take 448 (the largest finite
 * code); the sign bit is copied from y.  NaN input is not supported. */
uint8_t ora_e4m3_encode(float y)
{
    const double a = fabs((double)y);
    int best = 0;
    double bd = a;   /* distance to code 0 (value 0) */
    for (int c = 1; c <= 0x7E; c++) {
        const double d = fabs(ora_e4m3_value((uint8_t)c) - a);
        if (d < bd || (d == bd && (c & 1) == 0)) {
            best = c;
            bd = d;
        }
    }
    return (uint8_t)(best | (signbit(y) ? 0x80 : 0));
}

/* Quantises `rows` groups of `cols` binary32 values: scale[r] = absmax/448 of
 * group r in binary32 (1 for an all-zero group), codes[r, i] =
 * ora_e4m3_encode(x[r, i] / scale[r]) with the division in binary32. */
int ora_quant_rows(const float *x, int64_t rows, int64_t cols, uint8_t *codes, float *scale)
{
    if (!x || !codes || !scale || rows < 0 || cols <= 0)
        return ORA_ERR;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        const float *xr = x + r * cols;
        float amax = 0.0f;
        for (int64_t i = 0; i < cols; i++) {
            const float v = fabsf(xr[i]);
            if (v > amax)
                amax = v;
        }
        const float s = amax == 0.0f ? 1.0f : amax / 448.0f;
        scale[r] = s;
        for (int64_t i = 0; i < cols; i++) {
            volatile float y = xr[i] / s;   /* rounded to binary32 here */
            codes[r * cols + i] = ora_e4m3_encode(y);
        }
    }
    return ORA_OK;
}

/* ------------------------------------------------------------ batch rows */

typedef struct {
    int b;          /* sequence */
    int64_t kv0;    /* first cache row of the sequence */
    int64_t ctx;    /* cache rows of the sequence */
    int64_t pos;    /* absolute position of the query */
    int64_t nvis;   /* visible keys: min(pos + 1, ctx), at least 0 */
} ora_row;

static int ora_row_info(int B, const int32_t *cu_q, const int64_t *cu_kv,
                        const int32_t *pos0, int64_t t, ora_row *r)
{
    for (int b = 0; b < B; b++) {
        if (t >= cu_q[b] && t < cu_q[b + 1]) {
            r->b = b;
            r->kv0 = cu_kv[b];
            r->ctx = cu_kv[b + 1] - cu_kv[b];
            r->pos = (int64_t)pos0[b] + (t - cu_q[b]);
            r->nvis = r->pos + 1 < r->ctx ? r->pos + 1 : r->ctx;
            if (r->nvis < 0)
                r->nvis = 0;
            return ORA_OK;
        }
    }
    return ORA_ERR;
}

static int64_t ora_pick_row(const int32_t *rows, int64_t i)
{
    return rows ? (int64_t)rows[i] : i;
}

/* Element type of a value array: 0 = float32, 1 = bf16 bits, 2 = e4m3 codes
 * (the latter with a per-row scale). */
static double ora_load(const void *p, int type, int64_t i)
{
    if (type == 0)
        return (double)((const float *)p)[i];
    if (type == 1)
        return ora_bf16_value(((const uint16_t *)p)[i]);
    return ora_e4m3_value(((const uint8_t *)p)[i]);
}

/* ---------------------------------------------------------------- indexer */

/*
 * Index scores, [R] "Молниеносный индексатор", equation I_{t,s}.
 *   q      [T, HI, DI]  type q_type (0 f32 values, 2 e4m3 codes)
 *   q_scale[T, HI]      dequantisation scale (ignored for f32; may be NULL)
 *   w      [T, HI]      f32 head weights
 *   k      [N, DI]      type k_type
 *   k_scale[N]          dequantisation scale (ignored for f32; may be NULL)
 *   scores [nrows, ld]  f32 out; columns >= ctx_b untouched, masked = -inf
 *   absum  [nrows, ld]  f64 out (nullable): A[t,s], 0 where masked
 */
int ora_indexer(int B, const int32_t *cu_q, const int64_t *cu_kv,
                const int32_t *pos0, const int32_t *rows, int64_t nrows,
                int HI, int DI,
                const void *q, int q_type, const float *q_scale,
                const float *w,
                const void *k, int k_type, const float *k_scale,
                float *scores, double *absum, int64_t ld)
{
    int err = 0;
    #pragma omp parallel
    {
        double *qd = (double *)malloc(sizeof(double) * (size_t)HI * DI);
        double *kd = (double *)malloc(sizeof(double) * (size_t)DI);
        #pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < nrows; i++) {
            ora_row r;
            int64_t t = ora_pick_row(rows, i);
            if (!qd || !kd || ora_row_info(B, cu_q, cu_kv, pos0, t, &r)) {
                #pragma omp atomic write
                err = 1;
                continue;
            }
            for (int j = 0; j < HI; j++) {
                double sq = (q_type == 0 || !q_scale) ? 1.0
                          : (double)q_scale[t * HI + j];
                for (int d = 0; d < DI; d++)
                    qd[j * DI + d] = ora_load(q, q_type, (t * HI + j) * DI + d) * sq;
            }
            float *srow = scores + i * ld;
            double *arow = absum ? absum + i * ld : NULL;
            for (int64_t s = 0; s < r.ctx; s++) {
                if (s >= r.nvis) {
                    srow[s] = -INFINITY;
                    if (arow)
                        arow[s] = 0.0;
                    continue;
                }
                int64_t ks = r.kv0 + s;
                double sk = (k_type == 0 || !k_scale) ? 1.0 : (double)k_scale[ks];
                for (int d = 0; d < DI; d++)
                    kd[d] = ora_load(k, k_type, ks * DI + d) * sk;
                double acc = 0.0, aacc = 0.0;
                for (int j = 0; j < HI; j++) {
                    double dot = 0.0;
                    for (int d = 0; d < DI; d++)
                        dot += qd[j * DI + d] * kd[d];
                    double relu = dot > 0.0 ? dot : 0.0;
                    acc += (double)w[t * HI + j] * relu;
                    aacc += fabs((double)w[t * HI + j]) * relu;
                }
                srow[s] = (float)acc;
                if (arow)
                    arow[s] = aacc;
            }
        }
        free(qd);
        free(kd);
    }
    return err ? ORA_ERR : ORA_OK;
}

/* ------------------------------------------------------------------ top-k */

typedef struct {
    float v;
    int64_t s;
} ora_cand;

/* Order for selection: larger score first; equal scores (compared as
 * binary32 values, so -0 == +0) go to the lower position. */
static int ora_cand_cmp(const void *a, const void *b)
{
    const ora_cand *x = (const ora_cand *)a, *y = (const ora_cand *)b;
    if (x->v > y->v)
        return -1;
    if (x->v < y->v)
        return 1;
    return (x->s > y->s) - (x->s < y->s);
}

static int ora_i64_cmp(const void *a, const void *b)
{
    int64_t x = *(const int64_t *)a, y = *(const int64_t *)b;
    return (x > y) - (x < y);
}

/*
 * Top-k selection, [R] "Отбор и основное внимание" (Top-k(I_{t,:}), k = 2048
 * in production).  scores [nrows, ld] as produced by ora_indexer for the same
 * row list; idx [nrows, k] out: ascending sequence-local positions, -1 pad.
 */
int ora_topk(int B, const int32_t *cu_q, const int64_t *cu_kv,
             const int32_t *pos0, const int32_t *rows, int64_t nrows,
             const float *scores, int64_t ld, int k, int32_t *idx)
{
    int err = 0;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < nrows; i++) {
        ora_row r;
        if (ora_row_info(B, cu_q, cu_kv, pos0, ora_pick_row(rows, i), &r)) {
            #pragma omp atomic write
            err = 1;
            continue;
        }
        int64_t n = r.nvis;
        ora_cand *c = (ora_cand *)malloc(sizeof(ora_cand) * (size_t)(n > 0 ? n : 1));
        int64_t *sel = (int64_t *)malloc(sizeof(int64_t) * (size_t)(k > 0 ? k : 1));
        if (!c || !sel) {
            #pragma omp atomic write
            err = 1;
            free(c);
            free(sel);
            continue;
        }
        for (int64_t s = 0; s < n; s++) {
            c[s].v = scores[i * ld + s];
            c[s].s = s;
        }
        qsort(c, (size_t)n, sizeof(ora_cand), ora_cand_cmp);
        int64_t m = n < k ? n : k;
        for (int64_t j = 0; j < m; j++)
            sel[j] = c[j].s;
        qsort(sel, (size_t)m, sizeof(int64_t), ora_i64_cmp);
        for (int64_t j = 0; j < k; j++)
            idx[i * k + j] = j < m ? (int32_t)sel[j] : -1;
        free(c);
        free(sel);
    }
    return err ? ORA_ERR : ORA_OK;
}

/* -------------------------------------------------------------- attention */

/*
 * Attention of one query row over an explicit list of sequence-local key
 * positions `sel` (length m, entries -1 skipped), MQA mode: every head uses
 * the same latent rows.  Exact softmax in double; every sum runs over the
 * selected rows in list order.  Work buffers (caller-owned):
 *   z [m*H], qd [H*D], kd [D], acc [H*Dv], mx [H], den [H].
 */
static int ora_attend_row(int64_t t, const ora_row *r, const int64_t *sel,
                          int64_t m, int H, int D, int Dv, double scale,
                          const void *q, int q_type, const void *kv, int kv_type,
                          float *o, float *lse, double *z, double *qd,
                          double *kd, double *acc, double *mx, double *den)
{
    for (int h = 0; h < H; h++)
        for (int d = 0; d < D; d++)
            qd[h * D + d] = ora_load(q, q_type, (t * H + h) * (int64_t)D + d);
    /* logits z[j,h] = scale * <q[t,h,:], kv[s_j,:]> */
    int64_t nsel = 0;
    for (int64_t j = 0; j < m; j++) {
        int64_t s = sel[j];
        if (s < 0)
            continue;
        if (s >= r->ctx)
            return ORA_ERR;
        for (int d = 0; d < D; d++)
            kd[d] = ora_load(kv, kv_type, (r->kv0 + s) * D + d);
        for (int h = 0; h < H; h++) {
            double dot = 0.0;
            for (int d = 0; d < D; d++)
                dot += qd[h * D + d] * kd[d];
            z[nsel * H + h] = scale * dot;
        }
        nsel++;
    }
    if (nsel == 0) {
        for (int h = 0; h < H; h++) {
            for (int c = 0; c < Dv; c++)
                o[(int64_t)h * Dv + c] = 0.0f;
            lse[h] = -INFINITY;
        }
        return ORA_OK;
    }
    /* softmax statistics per head */
    for (int h = 0; h < H; h++) {
        double M = -INFINITY;
        for (int64_t j = 0; j < nsel; j++)
            if (z[j * H + h] > M)
                M = z[j * H + h];
        double Z = 0.0;
        for (int64_t j = 0; j < nsel; j++)
            Z += exp(z[j * H + h] - M);
        mx[h] = M;
        den[h] = Z;
    }
    /* o[h,c] = sum_j p[j,h] * kv[s_j, c] / Z[h] for c < Dv */
    for (int64_t x = 0; x < (int64_t)H * Dv; x++)
        acc[x] = 0.0;
    int64_t jj = 0;
    for (int64_t j = 0; j < m; j++) {
        int64_t s = sel[j];
        if (s < 0)
            continue;
        for (int c = 0; c < Dv; c++)
            kd[c] = ora_load(kv, kv_type, (r->kv0 + s) * D + c);
        for (int h = 0; h < H; h++) {
            double p = exp(z[jj * H + h] - mx[h]);
            for (int c = 0; c < Dv; c++)
                acc[h * Dv + c] += p * kd[c];
        }
        jj++;
    }
    for (int h = 0; h < H; h++) {
        for (int c = 0; c < Dv; c++)
            o[(int64_t)h * Dv + c] = (float)(acc[h * Dv + c] / den[h]);
        lse[h] = (float)(mx[h] + log(den[h]));
    }
    return ORA_OK;
}

typedef struct {
    double *z, *qd, *kd, *acc, *mx, *den;
    int64_t *sel;
} ora_attn_ws;

static int ora_attn_ws_alloc(ora_attn_ws *w, int64_t m, int H, int D, int Dv)
{
    if (m < 1)
        m = 1;
    w->z = (double *)malloc(sizeof(double) * (size_t)m * H);
    w->qd = (double *)malloc(sizeof(double) * (size_t)H * D);
    w->kd = (double *)malloc(sizeof(double) * (size_t)D);
    w->acc = (double *)malloc(sizeof(double) * (size_t)H * Dv);
    w->mx = (double *)malloc(sizeof(double) * (size_t)H);
    w->den = (double *)malloc(sizeof(double) * (size_t)H);
    w->sel = (int64_t *)malloc(sizeof(int64_t) * (size_t)m);
    return (w->z && w->qd && w->kd && w->acc && w->mx && w->den && w->sel) ? ORA_OK : ORA_ERR;
}

static void ora_attn_ws_free(ora_attn_ws *w)
{
    free(w->z);
    free(w->qd);
    free(w->kd);
    free(w->acc);
    free(w->mx);
    free(w->den);
    free(w->sel);
}

/*
 * Sparse MQA-mode attention over the selected rows, [R] "Отбор и основное
 * внимание", equation u_t.
 *   q   [T, H, D]  type q_type (0 f32, 1 bf16 bits)
 *   kv  [N, D]     type kv_type; value = first Dv dims of the same row
 *   idx [nrows, k] sequence-local positions, -1 = unused slot
 *   o   [nrows, H, Dv] f32 out;  lse [nrows, H] f32 out (natural log;
 *   -inf and o = 0 when a row selects nothing)
 */
int ora_sparse_attn(int B, const int32_t *cu_q, const int64_t *cu_kv,
                    const int32_t *pos0, const int32_t *rows, int64_t nrows,
                    int H, int D, int Dv, double scale,
                    const void *q, int q_type, const void *kv, int kv_type,
                    const int32_t *idx, int k, float *o, float *lse)
{
    int err = 0;
    #pragma omp parallel
    {
        ora_attn_ws w;
        int ok = ora_attn_ws_alloc(&w, k, H, D, Dv) == ORA_OK;
        #pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < nrows; i++) {
            ora_row r;
            int64_t t = ora_pick_row(rows, i);
            if (!ok || ora_row_info(B, cu_q, cu_kv, pos0, t, &r)) {
                #pragma omp atomic write
                err = 1;
                continue;
            }
            for (int j = 0; j < k; j++)
                w.sel[j] = idx[i * k + j];
            if (ora_attend_row(t, &r, w.sel, k, H, D, Dv, scale, q, q_type, kv,
                               kv_type, o + i * (int64_t)H * Dv, lse + i * H,
                               w.z, w.qd, w.kd, w.acc, w.mx, w.den)) {
                #pragma omp atomic write
                err = 1;
            }
        }
        ora_attn_ws_free(&w);
    }
    return err ? ORA_ERR : ORA_OK;
}

/*
 * Dense causal MQA attention: every visible key of each row (brute force).
 * Same layouts as ora_sparse_attn without idx.
 */
int ora_dense_attn(int B, const int32_t *cu_q, const int64_t *cu_kv,
                   const int32_t *pos0, const int32_t *rows, int64_t nrows,
                   int H, int D, int Dv, double scale,
                   const void *q, int q_type, const void *kv, int kv_type,
                   float *o, float *lse)
{
    int err = 0;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < nrows; i++) {
        ora_row r;
        ora_attn_ws w;
        int64_t t = ora_pick_row(rows, i);
        if (ora_row_info(B, cu_q, cu_kv, pos0, t, &r)) {
            #pragma omp atomic write
            err = 1;
            continue;
        }
        if (ora_attn_ws_alloc(&w, r.nvis, H, D, Dv) == ORA_OK) {
            for (int64_t s = 0; s < r.nvis; s++)
                w.sel[s] = s;
            if (ora_attend_row(t, &r, w.sel, r.nvis, H, D, Dv, scale, q, q_type,
                               kv, kv_type, o + i * (int64_t)H * Dv, lse + i * H,
                               w.z, w.qd, w.kd, w.acc, w.mx, w.den)) {
                #pragma omp atomic write
                err = 1;
            }
        } else {
            #pragma omp atomic write
            err = 1;
        }
        ora_attn_ws_free(&w);
    }
    return err ? ORA_ERR : ORA_OK;
}

/*
 * Indexer KL loss, [R] "Как учили индексатор": the indexer is trained toward
 * the main attention.  Its target p[t,:] is the attention's probabilities
 * summed over all heads and L1-normalised over the key set; the loss of row
 * t is KL(p[t,:] || softmax(I[t,:])) over the same set.  Two stages:
 *   dense warm-up (idx == NULL): the set is every visible key 0..nvis-1;
 *   sparse stage: the selected slots idx[i, 0..k-1] (negative entries are
 *   skipped; a position listed twice is two slots, as in the attention).
 * Steps for one row, in the order the section gives them:
 *   1. z[j,h] = scale * <q[t,h,:], kv[s_j,:]>, and per head the softmax over
 *      the set: P[j,h] = exp(z[j,h] - M_h) / Z_h (the main attention);
 *   2. a[j] = sum_h P[j,h];  p[j] = a[j] / sum_j a[j]   (L1 normalisation);
 *   3. r = softmax over the set of I[t, s_j];
 *   4. kl = sum_j p[j] * (ln p[j] - ln r[j]), with 0 * ln 0 = 0.
 *   q [T,H,D], kv [N,D]: types as in ora_sparse_attn
 *   scores [nrows, ld] f32: I[t, s] of the rows asked for, at column s
 *   kl  [nrows] f64 out (0 for an empty set)
 *   p   [nrows, k] (sparse: per slot, 0 for skipped slots) or [nrows, ld]
 *       (dense: columns 0..nvis-1) f64 out, nullable
 */
int ora_indexer_kl(int B, const int32_t *cu_q, const int64_t *cu_kv,
                   const int32_t *pos0, const int32_t *rows, int64_t nrows,
                   int H, int D, double scale,
                   const void *q, int q_type, const void *kv, int kv_type,
                   const float *scores, int64_t ld, const int32_t *idx, int k,
                   double *kl, double *p)
{
    int err = 0;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < nrows; i++) {
        ora_row r;
        int64_t t = ora_pick_row(rows, i);
        if (ora_row_info(B, cu_q, cu_kv, pos0, t, &r)) {
            #pragma omp atomic write
            err = 1;
            continue;
        }
        const int64_t m = idx ? k : r.nvis;          /* slots of the row */
        const int64_t pw = idx ? k : ld;              /* width of a p row */
        int64_t *pos = (int64_t *)malloc(sizeof(int64_t) * (size_t)(m > 0 ? m : 1));
        double *z = (double *)malloc(sizeof(double) * (size_t)(m > 0 ? m : 1) * H);
        double *a = (double *)malloc(sizeof(double) * (size_t)(m > 0 ? m : 1));
        double *qd = (double *)malloc(sizeof(double) * (size_t)H * D);
        double *kd = (double *)malloc(sizeof(double) * (size_t)D);
        if (!pos || !z || !a || !qd || !kd) {
            #pragma omp atomic write
            err = 1;
        } else {
            int bad = 0;
            for (int64_t j = 0; j < m; j++) {
                pos[j] = idx ? (int64_t)idx[i * k + j] : j;
                if (pos[j] >= r.ctx || pos[j] >= ld)
                    bad = 1;
            }
            if (bad) {
                #pragma omp atomic write
                err = 1;
            } else {
                for (int h = 0; h < H; h++)
                    for (int d = 0; d < D; d++)
                        qd[h * D + d] = ora_load(q, q_type, (t * H + h) * (int64_t)D + d);
                /* step 1: logits and the per-head softmax */
                for (int64_t j = 0; j < m; j++) {
                    if (pos[j] < 0)
                        continue;
                    for (int d = 0; d < D; d++)
                        kd[d] = ora_load(kv, kv_type, (r.kv0 + pos[j]) * D + d);
                    for (int h = 0; h < H; h++) {
                        double dot = 0.0;
                        for (int d = 0; d < D; d++)
                            dot += qd[h * D + d] * kd[d];
                        z[j * H + h] = scale * dot;
                    }
                }
                for (int64_t j = 0; j < m; j++)
                    a[j] = 0.0;
                for (int h = 0; h < H; h++) {
                    double M = -INFINITY, Z = 0.0;
                    for (int64_t j = 0; j < m; j++)
                        if (pos[j] >= 0 && z[j * H + h] > M)
                            M = z[j * H + h];
                    for (int64_t j = 0; j < m; j++)
                        if (pos[j] >= 0)
                            Z += exp(z[j * H + h] - M);
                    /* step 2 (first half): the sum over heads */
                    for (int64_t j = 0; j < m; j++)
                        if (pos[j] >= 0)
                            a[j] += exp(z[j * H + h] - M) / Z;
                }
                /* step 2 (second half): L1 normalisation over the set */
                double asum = 0.0;
                for (int64_t j = 0; j < m; j++)
                    if (pos[j] >= 0)
                        asum += a[j];
                /* step 3: the indexer's softmax over the same set */
                double MI = -INFINITY, ZI = 0.0;
                for (int64_t j = 0; j < m; j++)
                    if (pos[j] >= 0 && (double)scores[i * ld + pos[j]] > MI)
                        MI = (double)scores[i * ld + pos[j]];
                for (int64_t j = 0; j < m; j++)
                    if (pos[j] >= 0)
                        ZI += exp((double)scores[i * ld + pos[j]] - MI);
                const double lnZI = MI + log(ZI);
                /* step 4: the divergence */
                double sum = 0.0;
                for (int64_t j = 0; j < m; j++) {
                    if (pos[j] < 0) {
                        if (p && idx)
                            p[i * pw + j] = 0.0;
                        continue;
                    }
                    const double pj = a[j] / asum;
                    const double lnr = (double)scores[i * ld + pos[j]] - lnZI;
                    if (pj > 0.0)
                        sum += pj * (log(pj) - lnr);
                    if (p)
                        p[i * pw + (idx ? j : pos[j])] = pj;
                }
                kl[i] = asum > 0.0 ? sum : 0.0;
            }
        }
        free(pos);
        free(z);
        free(a);
        free(qd);
        free(kd);
    }
    return err ? ORA_ERR : ORA_OK;
}

/*
 * Backward of the sparse MQA attention (step 4) over the same selection,
 * [R] "Как учили индексатор" (in the sparse stage all parameters learn, so
 * gradients flow through the attention over the selected rows).  Given
 * dout = dL/do [T, H, Dv] (type dout_type), for the rows asked for, in double:
 *   z[j,h]  = scale * <q[t,h,:], kv[s_j,:]>,  P = exact softmax over the slots,
 *   o[h,c]  = sum_j P[j,h] kv[s_j,c]                  (c < Dv),
 *   dP[j,h] = <dout[t,h,:], kv[s_j,:Dv]>,
 *   delta_h = sum_c dout[t,h,c] o[h,c]   (= sum_j P[j,h] dP[j,h]),
 *   dZ[j,h] = P[j,h] (dP[j,h] - delta_h)           (the softmax's backward),
 *   dq[i,h,d]   = scale * sum_j dZ[j,h] kv[s_j,d]             (d < D),
 *   dkv[s_j,d] += scale * sum_h dZ[j,h] q[t,h,d]             (d < D: the key),
 *   dkv[s_j,c] += sum_h P[j,h] dout[t,h,c]                   (c < Dv: the value).
 * Negative idx entries are skipped; a position listed twice is two slots.
 * out (nullable, [T, H, Dv], type out_type): the forward output to take delta
 * from, delta_h = sum_c dout[t,h,c] out[t,h,c] (what a backward that is handed
 * the forward's rounded output computes); NULL: the exact o above.
 *   dq [nrows, H, D] f64 out; dkv [N, D] f64, accumulated (the caller zeroes).
 */
int ora_sparse_attn_bwd(int B, const int32_t *cu_q, const int64_t *cu_kv,
                        const int32_t *pos0, const int32_t *rows, int64_t nrows,
                        int H, int D, int Dv, double scale,
                        const void *q, int q_type, const void *kv, int kv_type,
                        const void *dout, int dout_type, const void *out, int out_type,
                        const int32_t *idx, int k, double *dq, double *dkv)
{
    int err = 0;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < nrows; i++) {
        ora_row r;
        int64_t t = ora_pick_row(rows, i);
        if (ora_row_info(B, cu_q, cu_kv, pos0, t, &r)) {
            #pragma omp atomic write
            err = 1;
            continue;
        }
        const int64_t m = k > 0 ? k : 1;
        double *qd = (double *)malloc(sizeof(double) * (size_t)H * D);
        double *gd = (double *)malloc(sizeof(double) * (size_t)H * Dv);
        double *kd = (double *)malloc(sizeof(double) * (size_t)m * D);
        double *P = (double *)malloc(sizeof(double) * (size_t)m * H);
        double *dZ = (double *)malloc(sizeof(double) * (size_t)m * H);
        double *o = (double *)malloc(sizeof(double) * (size_t)H * Dv);
        double *delta = (double *)malloc(sizeof(double) * (size_t)H);
        double *g = (double *)malloc(sizeof(double) * (size_t)m * D);
        int64_t *pos = (int64_t *)malloc(sizeof(int64_t) * (size_t)m);
        if (!qd || !gd || !kd || !P || !dZ || !o || !delta || !g || !pos) {
            #pragma omp atomic write
            err = 1;
        } else {
            int bad = 0;
            for (int64_t j = 0; j < k; j++) {
                pos[j] = idx[i * k + j];
                if (pos[j] >= r.ctx)
                    bad = 1;
            }
            if (bad) {
                #pragma omp atomic write
                err = 1;
            } else {
                for (int h = 0; h < H; h++) {
                    for (int d = 0; d < D; d++)
                        qd[h * D + d] = ora_load(q, q_type, (t * H + h) * (int64_t)D + d);
                    for (int c = 0; c < Dv; c++)
                        gd[h * Dv + c] = ora_load(dout, dout_type, (t * H + h) * (int64_t)Dv + c);
                }
                for (int64_t j = 0; j < k; j++)
                    if (pos[j] >= 0)
                        for (int d = 0; d < D; d++)
                            kd[j * D + d] = ora_load(kv, kv_type, (r.kv0 + pos[j]) * D + d);
                /* the forward: logits and the exact softmax per head, then o */
                for (int h = 0; h < H; h++) {
                    double M = -INFINITY, Z = 0.0;
                    for (int64_t j = 0; j < k; j++) {
                        if (pos[j] < 0)
                            continue;
                        double dot = 0.0;
                        for (int d = 0; d < D; d++)
                            dot += qd[h * D + d] * kd[j * D + d];
                        P[j * H + h] = scale * dot;        /* z for now */
                        if (P[j * H + h] > M)
                            M = P[j * H + h];
                    }
                    for (int64_t j = 0; j < k; j++)
                        if (pos[j] >= 0)
                            Z += exp(P[j * H + h] - M);
                    for (int64_t j = 0; j < k; j++)
                        P[j * H + h] = pos[j] >= 0 ? exp(P[j * H + h] - M) / Z : 0.0;
                    for (int c = 0; c < Dv; c++) {
                        double acc = 0.0;
                        for (int64_t j = 0; j < k; j++)
                            if (pos[j] >= 0)
                                acc += P[j * H + h] * kd[j * D + c];
                        o[h * Dv + c] = acc;
                    }
                    /* the backward of o = P V, then of the softmax */
                    double dl = 0.0;
                    for (int c = 0; c < Dv; c++)
                        dl += gd[h * Dv + c] *
                              (out ? ora_load(out, out_type, (t * H + h) * (int64_t)Dv + c) : o[h * Dv + c]);
                    delta[h] = dl;
                    for (int64_t j = 0; j < k; j++) {
                        if (pos[j] < 0) {
                            dZ[j * H + h] = 0.0;
                            continue;
                        }
                        double dp = 0.0;
                        for (int c = 0; c < Dv; c++)
                            dp += gd[h * Dv + c] * kd[j * D + c];
                        dZ[j * H + h] = P[j * H + h] * (dp - delta[h]);
                    }
                    /* the backward of z = scale q . kv, query side */
                    for (int d = 0; d < D; d++) {
                        double acc = 0.0;
                        for (int64_t j = 0; j < k; j++)
                            if (pos[j] >= 0)
                                acc += dZ[j * H + h] * kd[j * D + d];
                        dq[(i * H + h) * (int64_t)D + d] = scale * acc;
                    }
                }
                /* key side and value side, per slot (summed over the heads) */
                for (int64_t j = 0; j < k; j++) {
                    if (pos[j] < 0)
                        continue;
                    for (int d = 0; d < D; d++) {
                        double acc = 0.0;
                        for (int h = 0; h < H; h++)
                            acc += dZ[j * H + h] * qd[h * D + d];
                        g[j * D + d] = scale * acc;
                    }
                    for (int c = 0; c < Dv; c++) {
                        double acc = 0.0;
                        for (int h = 0; h < H; h++)
                            acc += P[j * H + h] * gd[h * Dv + c];
                        g[j * D + c] += acc;
                    }
                }
                #pragma omp critical(ora_dkv)
                for (int64_t j = 0; j < k; j++)
                    if (pos[j] >= 0)
                        for (int d = 0; d < D; d++)
                            dkv[(r.kv0 + pos[j]) * D + d] += g[j * D + d];
            }
        }
        free(qd);
        free(gd);
        free(kd);
        free(P);
        free(dZ);
        free(o);
        free(delta);
        free(g);
        free(pos);
    }
    return err ? ORA_ERR : ORA_OK;
}

/* Threads the OpenMP runtime uses for the parallel loops above (reported
 * beside CPU timings). */
int ora_num_threads(void)
{
    return omp_get_max_threads();
}
