/*
 * Lightning-indexer oracle: a plain, slow, obviously correct CPU reference.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file or the library built from it; only the tests, the
 * smoke check and the benchmark's CPU-baseline leg use it.  It shares no
 * code, header, table or helper with the HIP library.
 *
 * What it computes (llama.cpp release b11372, "qwen4exp: halve the indexer
 * score memory" and "qwen4exp: compute the indexer score with the lightning
 * indexer"; vLLM PR #45743, "Tune Triton indexer score decode for
 * spec-decode", kernel section):
 *
 *   score[t][s] = sum over heads h of  w[h] * max(q[t][h][:] . k[s][:], 0)
 *                 + mask[t][s]
 *
 * Each head's dot product is rectified on its own and only then summed (the
 * b11372 notes: every head gets its own product, rectified, then summed in
 * place into one [n_pool, n_tokens] score).  Any 1/sqrt(head_dim) scale is
 * carried in w (the notes on the lightning indexer: the scaled unweighted sum
 * is the indexer with every head weight set to the scale; the vLLM decode
 * kernel drops sm_scale).  Keys are shared by every head.  The f16 mask is
 * additive and enters once, after the head sum; an entry whose mask is -inf,
 * or which lies past the row's visible length, is invisible and scores -inf.
 *
 * Arithmetic: every f16 and f32 input is widened exactly to double and all
 * products and sums are formed in double, in the natural index order.
 *
 * Top-k (the selection step of the vLLM index_topk module): for every row,
 * the k_top visible keys with the largest score, ordered by score descending
 * and, among equal scores, by key index ascending; -inf and NaN are never
 * selected and -0 ties with +0.  Rows with fewer than k_top visible keys are
 * padded with index -1 and value -inf.
 *
 * Block ranking (oracle_topk_blocks_*) follows a reading of the vLLM decode
 * kernel's init_blocks / local_blocks arguments, spelled out above the code.
 *
 * Pins: every function here is checked by tests/test_oracle_pins.py against
 * a hand-derived worked example, closed forms, the pages' scale identity, the
 * "materialise then sum" scheme the pages replaced, a sign-flip identity that
 * reduces to a plain matrix product, and a library sort.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* IEEE 754 binary16 -> double, from the format's definition: 1 sign bit,
 * 5 exponent bits (bias 15), 10 fraction bits. */
static double half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -24);            /* zero or subnormal */
    else if (expo == 31)
        v = frac ? NAN : INFINITY;               /* inf or NaN */
    else
        v = ldexp((double)(frac + 1024), expo - 25);
    return sign ? -v : v;
}

static int half_is_neg_inf(uint16_t h) { return h == 0xfc00; }

/* Widen rows of f16 values to a dense double array [n_rows][d]. */
static double *widen_rows(const uint16_t *src, int64_t n_rows, int64_t row_stride, int d)
{
    double *dst = (double *)malloc(sizeof(double) * (size_t)(n_rows > 0 ? n_rows : 1) * (size_t)d);
    for (int64_t r = 0; r < n_rows; ++r)
        for (int i = 0; i < d; ++i)
            dst[r * d + i] = half_to_double(src[r * row_stride + i]);
    return dst;
}

/* Widen q [T][H][d] (strides q_stride_t, q_stride_h) to dense [T][H][d]. */
static double *widen_queries(const uint16_t *q, int64_t q_stride_t, int64_t q_stride_h,
                             int T, int H, int d)
{
    double *dst = (double *)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1) * (size_t)H * (size_t)d);
    for (int t = 0; t < T; ++t)
        for (int h = 0; h < H; ++h)
            for (int i = 0; i < d; ++i)
                dst[((int64_t)t * H + h) * d + i] =
                    half_to_double(q[(int64_t)t * q_stride_t + (int64_t)h * q_stride_h + i]);
    return dst;
}

/* One visible (token, key) pair: rectify each head's dot product, weight it,
 * sum over heads.  q_t is [H][d], k_s is [d], both already in double. */
static double head_sum(const double *q_t, const double *k_s, const float *w, int H, int d)
{
    double total = 0.0;
    for (int h = 0; h < H; ++h) {
        const double *q_th = q_t + (int64_t)h * d;
        double dot = 0.0;
        for (int i = 0; i < d; ++i)
            dot += q_th[i] * k_s[i];
        double rect = dot > 0.0 ? dot : 0.0;
        total += (double)w[h] * rect;
    }
    return total;
}

/*
 * Contiguous ("prefill") score.
 *   q    f16 [T][H][d] with strides (q_stride_t, q_stride_h, 1) in elements
 *   k    f16 [P][d]    with stride k_stride_s
 *   w    f32 [H]
 *   mask f16 [T][P] with stride mask_stride_t, or NULL (all visible, +0)
 *   vis_len i32 [T]: key s is visible to token t only if s < vis_len[t];
 *        NULL means every s < P
 *   out  f64 [T][P] with stride out_stride_t
 */
void oracle_score_prefill(const uint16_t *q, int64_t q_stride_t, int64_t q_stride_h,
                          const uint16_t *k, int64_t k_stride_s,
                          const float *w,
                          const uint16_t *mask, int64_t mask_stride_t,
                          const int32_t *vis_len,
                          int T, int P, int H, int d,
                          double *out, int64_t out_stride_t)
{
    double *qd = widen_queries(q, q_stride_t, q_stride_h, T, H, d);
    double *kd = widen_rows(k, P, k_stride_s, d);
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
    for (int t = 0; t < T; ++t) {
        for (int s = 0; s < P; ++s) {
            double *o = out + (int64_t)t * out_stride_t + s;
            int visible = 1;
            if (vis_len && s >= vis_len[t])
                visible = 0;
            if (mask && half_is_neg_inf(mask[(int64_t)t * mask_stride_t + s]))
                visible = 0;
            if (!visible) {
                *o = -INFINITY;
                continue;
            }
            double v = head_sum(qd + (int64_t)t * H * d, kd + (int64_t)s * d, w, H, d);
            if (mask)
                v += half_to_double(mask[(int64_t)t * mask_stride_t + s]);
            *o = v;
        }
    }
    free(kd);
    free(qd);
}

/*
 * Paged ("decode") score.  Request r owns query rows r*Q .. r*Q+Q-1 (query j
 * of request r is row r*Q+j) and keys 0 .. seq_lens[r]-1.  Logical key s of
 * request r lives in physical block block_table[r*bt_stride + s/block_size],
 * slot s % block_size, of k_cache [n_blocks][block_size][d].
 *
 * Query j is the (j+1)-th of Q trailing tokens of the request, so it sees the
 * keys before the speculative tail plus the accepted ones up to itself:
 * s < seq_len - Q + 1 + j (for Q = 1: every s < seq_len).
 *
 *   mask f16 [R*Q][max_seq_len] with stride mask_stride_t, or NULL
 *   out  f64 [R*Q][max_seq_len] with stride out_stride_t; keys at or past the
 *        row's visible length score -inf.
 */
void oracle_score_decode(const uint16_t *q, int64_t q_stride_t, int64_t q_stride_h,
                         const uint16_t *k_cache, int block_size,
                         const int32_t *block_table, int64_t bt_stride,
                         const int32_t *seq_lens,
                         int R, int Q, int max_seq_len,
                         const float *w,
                         const uint16_t *mask, int64_t mask_stride_t,
                         int H, int d,
                         double *out, int64_t out_stride_t)
{
    double *qd = widen_queries(q, q_stride_t, q_stride_h, R * Q, H, d);
    for (int r = 0; r < R; ++r) {
        int L = seq_lens[r] < max_seq_len ? seq_lens[r] : max_seq_len;
        if (L < 0)
            L = 0;
        /* fetch the request's keys through its block table */
        double *kd = (double *)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1) * (size_t)d);
        for (int s = 0; s < L; ++s) {
            int64_t phys = block_table[(int64_t)r * bt_stride + s / block_size];
            const uint16_t *k_s = k_cache + (phys * block_size + s % block_size) * (int64_t)d;
            for (int i = 0; i < d; ++i)
                kd[(int64_t)s * d + i] = half_to_double(k_s[i]);
        }
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
        for (int j = 0; j < Q; ++j) {
            for (int s = 0; s < max_seq_len; ++s) {
                int64_t t = (int64_t)r * Q + j;
                int64_t vis = (int64_t)seq_lens[r] - Q + 1 + j;
                double *o = out + t * out_stride_t + s;
                int visible = s < vis && s < L;
                if (visible && mask && half_is_neg_inf(mask[t * mask_stride_t + s]))
                    visible = 0;
                if (!visible) {
                    *o = -INFINITY;
                    continue;
                }
                double v = head_sum(qd + t * H * d, kd + (int64_t)s * d, w, H, d);
                if (mask)
                    v += half_to_double(mask[t * mask_stride_t + s]);
                *o = v;
            }
        }
        free(kd);
    }
    free(qd);
}

/* ---------------------------- top-k ----------------------------------- */

typedef struct {
    double score;
    int32_t index;
} cand_t;

/* Total order: larger score first; equal scores (with -0 == +0) by smaller
 * key index first. */
static int cand_cmp(const void *a, const void *b)
{
    const cand_t *x = (const cand_t *)a, *y = (const cand_t *)b;
    if (x->score > y->score) return -1;
    if (x->score < y->score) return 1;
    return (x->index > y->index) - (x->index < y->index);
}

static void topk_row(const double *row, int n, int k_top, cand_t *scratch,
                     int32_t *idx_out, double *val_out)
{
    int m = 0;
    for (int s = 0; s < n; ++s) {
        double v = row[s];
        if (isnan(v) || (isinf(v) && v < 0))
            continue;                          /* never selectable */
        scratch[m].score = v == 0.0 ? 0.0 : v; /* -0 -> +0 */
        scratch[m].index = s;
        ++m;
    }
    qsort(scratch, (size_t)m, sizeof(cand_t), cand_cmp);
    for (int i = 0; i < k_top; ++i) {
        if (i < m) {
            idx_out[i] = scratch[i].index;
            if (val_out) val_out[i] = row[scratch[i].index];
        } else {
            idx_out[i] = -1;
            if (val_out) val_out[i] = -INFINITY;
        }
    }
}

/*
 * Top-k over double score rows [n_rows][n_cols] (stride score_stride).
 * row_len i32 [n_rows] limits row t to its first row_len[t] columns, or NULL.
 * idx_out i32 [n_rows][k_top], val_out f64 [n_rows][k_top] (nullable).
 */
void oracle_topk_f64(const double *score, int64_t score_stride, int n_rows, int n_cols,
                     const int32_t *row_len, int k_top,
                     int32_t *idx_out, double *val_out)
{
#pragma omp parallel
    {
        cand_t *scratch = (cand_t *)malloc(sizeof(cand_t) * (size_t)(n_cols > 0 ? n_cols : 1));
#pragma omp for schedule(dynamic, 1)
        for (int t = 0; t < n_rows; ++t) {
            int n = n_cols;
            if (row_len && row_len[t] < n) n = row_len[t] < 0 ? 0 : row_len[t];
            topk_row(score + (int64_t)t * score_stride, n, k_top, scratch,
                     idx_out + (int64_t)t * k_top,
                     val_out ? val_out + (int64_t)t * k_top : NULL);
        }
        free(scratch);
    }
}

/* Same selection over f32 score rows (e.g. scores produced elsewhere); each
 * f32 is widened exactly to double, so the order is the f32 order. */
void oracle_topk_f32(const float *score, int64_t score_stride, int n_rows, int n_cols,
                     const int32_t *row_len, int k_top,
                     int32_t *idx_out, float *val_out)
{
#pragma omp parallel
    {
        cand_t *scratch = (cand_t *)malloc(sizeof(cand_t) * (size_t)(n_cols > 0 ? n_cols : 1));
        double *row = (double *)malloc(sizeof(double) * (size_t)(n_cols > 0 ? n_cols : 1));
        double *vals = (double *)malloc(sizeof(double) * (size_t)(k_top > 0 ? k_top : 1));
#pragma omp for schedule(dynamic, 1)
        for (int t = 0; t < n_rows; ++t) {
            int n = n_cols;
            if (row_len && row_len[t] < n) n = row_len[t] < 0 ? 0 : row_len[t];
            const float *src = score + (int64_t)t * score_stride;
            for (int s = 0; s < n; ++s) row[s] = (double)src[s];
            topk_row(row, n, k_top, scratch, idx_out + (int64_t)t * k_top,
                     val_out ? vals : NULL);
            if (val_out)
                for (int i = 0; i < k_top; ++i)
                    val_out[(int64_t)t * k_top + i] = (float)vals[i];
        }
        free(vals);
        free(row);
        free(scratch);
    }
}

/* ---------------------- block ranking (top-k) -------------------------- */

/*
 * Block ranking: the vLLM decode index-score kernel takes init_blocks and
 * local_blocks, and decode "only needs block ordering" (vLLM PR #45743, key
 * source snippets).  The pages leave the two arguments undefined; the reading
 * implemented here: of a row's n candidates, the keys s < init_blocks and the
 * keys s >= n - local_blocks are forced -- always selected when selectable,
 * ranked ahead of every other key, and among themselves by index ascending.
 * The other selectable keys follow by (score descending, index ascending).
 * The first k_top of that order are output, padded with (-1, -inf).
 */
typedef struct {
    double score;
    int32_t index;
    int forced;
} block_cand_t;

static int block_cand_cmp(const void *a, const void *b)
{
    const block_cand_t *x = (const block_cand_t *)a, *y = (const block_cand_t *)b;
    if (x->forced != y->forced)
        return x->forced ? -1 : 1;             /* forced keys first */
    if (!x->forced) {                          /* others by score */
        if (x->score > y->score) return -1;
        if (x->score < y->score) return 1;
    }
    return (x->index > y->index) - (x->index < y->index);
}

static void topk_blocks_row(const double *row, int n, int init_blocks, int local_blocks,
                            int k_top, block_cand_t *scratch, int32_t *idx_out, double *val_out)
{
    int m = 0;
    for (int s = 0; s < n; ++s) {
        double v = row[s];
        if (isnan(v) || (isinf(v) && v < 0))
            continue;                          /* never selectable, forced or not */
        scratch[m].score = v == 0.0 ? 0.0 : v;
        scratch[m].index = s;
        scratch[m].forced = s < init_blocks || (local_blocks > 0 && s >= n - local_blocks);
        ++m;
    }
    qsort(scratch, (size_t)m, sizeof(block_cand_t), block_cand_cmp);
    for (int i = 0; i < k_top; ++i) {
        if (i < m) {
            idx_out[i] = scratch[i].index;
            if (val_out) val_out[i] = row[scratch[i].index];
        } else {
            idx_out[i] = -1;
            if (val_out) val_out[i] = -INFINITY;
        }
    }
}

/*
 * Block ranking over f32 score rows [n_rows][n_cols] (each f32 widened
 * exactly to double).  row_len i32 [n_rows] (nullable) limits row t to its
 * first row_len[t] columns, which are its n candidates.
 */
void oracle_topk_blocks_f32(const float *score, int64_t score_stride, int n_rows, int n_cols,
                            const int32_t *row_len, int init_blocks, int local_blocks, int k_top,
                            int32_t *idx_out, float *val_out)
{
#pragma omp parallel
    {
        block_cand_t *scratch = (block_cand_t *)malloc(sizeof(block_cand_t) * (size_t)(n_cols > 0 ? n_cols : 1));
        double *row = (double *)malloc(sizeof(double) * (size_t)(n_cols > 0 ? n_cols : 1));
        double *vals = (double *)malloc(sizeof(double) * (size_t)(k_top > 0 ? k_top : 1));
#pragma omp for schedule(dynamic, 1)
        for (int t = 0; t < n_rows; ++t) {
            int n = n_cols;
            if (row_len && row_len[t] < n) n = row_len[t] < 0 ? 0 : row_len[t];
            const float *src = score + (int64_t)t * score_stride;
            for (int s = 0; s < n; ++s) row[s] = (double)src[s];
            topk_blocks_row(row, n, init_blocks, local_blocks, k_top, scratch,
                            idx_out + (int64_t)t * k_top, val_out ? vals : NULL);
            if (val_out)
                for (int i = 0; i < k_top; ++i)
                    val_out[(int64_t)t * k_top + i] = (float)vals[i];
        }
        free(vals);
        free(row);
        free(scratch);
    }
}

/* The same over f64 rows (the oracle's own scores). */
void oracle_topk_blocks_f64(const double *score, int64_t score_stride, int n_rows, int n_cols,
                            const int32_t *row_len, int init_blocks, int local_blocks, int k_top,
                            int32_t *idx_out, double *val_out)
{
#pragma omp parallel
    {
        block_cand_t *scratch = (block_cand_t *)malloc(sizeof(block_cand_t) * (size_t)(n_cols > 0 ? n_cols : 1));
#pragma omp for schedule(dynamic, 1)
        for (int t = 0; t < n_rows; ++t) {
            int n = n_cols;
            if (row_len && row_len[t] < n) n = row_len[t] < 0 ? 0 : row_len[t];
            topk_blocks_row(score + (int64_t)t * score_stride, n, init_blocks, local_blocks, k_top, scratch,
                            idx_out + (int64_t)t * k_top, val_out ? val_out + (int64_t)t * k_top : NULL);
        }
        free(scratch);
    }
}

/* Number of threads the OpenMP loops above run with (1 without OpenMP). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
