/*
 * Oracle: a plain, slow CPU reference for fused indexer scoring + exact top-k.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header, table or constant with the HIP
 * library.
 *
 * What it computes (FlashTopK README, section "Quick start", the indexer-score
 * equation and the text under it):
 *
 *     I[t,s] = sigma[s] * sum_{h<32} w[t,h] * ReLU( q[t,h,:] . kv[s,:] )
 *
 * for every key s of the row's half-open window [ks[t], ke[t]); sigma[s] is
 * kv_scales[s], taken as 1 when no scales are given.  Each row then returns
 * the topk keys with the largest score, exactly (README, "What you can do":
 * exact), ordered by score descending, ties going to the smaller key index
 * (README, "What you can do": deterministic tie rule).  Rows whose window
 * holds fewer than topk keys return the whole window and pad the rest with
 * index -1 and value -inf (DeepSelect README, "Variable-length rows": short
 * rows are padded with fill values; -1 / -inf are this library's fill values).
 *
 * Arithmetic: every FP8 (OCP E4M3FN) or BF16 operand is decoded exactly from
 * its bit pattern; the 128-term dot product, the ReLU, the weighted head sum
 * and the sigma scale are all carried out in IEEE binary64, in the plain
 * order h = 0..31, d = 0..127.  The returned value is the binary64 score
 * rounded once to binary32 (round to nearest even), with -0 written as +0.
 * Selection is a full sort of the window (qsort) under the comparator
 * (score desc, index asc); +0 and -0 compare equal.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_FP8_E4M3 0
#define ORACLE_BF16 1
#define ORACLE_HEADS 32
#define ORACLE_DIM 128

/* OCP 8-bit floating point, E4M3 ("fn" flavour: finite only).  Layout
 * s.eeee.mmm, exponent bias 7.  Exponent field 0 encodes subnormals
 * m * 2^-9; 0x7F and 0xFF are NaN; there is no infinity.  Largest finite
 * value is 0x7E = 1.75 * 2^8 = 448. */
double oracle_decode_e4m3fn(uint8_t code)
{
    int sign = (code >> 7) & 1;
    int expo = (code >> 3) & 0xF;
    int mant = code & 0x7;
    double mag;
    if (expo == 0xF && mant == 0x7)
        return NAN;
    if (expo == 0)
        mag = ldexp((double)mant, -9);              /* (m/8) * 2^(1-7) */
    else
        mag = ldexp(8.0 + (double)mant, expo - 10); /* (1+m/8) * 2^(e-7) */
    return sign ? -mag : mag;
}

/* bfloat16: s.eeeeeeee.mmmmmmm, exponent bias 127 (the upper half of an
 * IEEE binary32).  Exponent 0 encodes subnormals m * 2^-133; exponent 255
 * encodes infinity (m == 0) or NaN. */
double oracle_decode_bf16(uint16_t code)
{
    int sign = (code >> 15) & 1;
    int expo = (code >> 7) & 0xFF;
    int mant = code & 0x7F;
    double mag;
    if (expo == 0xFF)
        mag = mant ? NAN : INFINITY;
    else if (expo == 0)
        mag = ldexp((double)mant, -133);             /* (m/128) * 2^(1-127) */
    else
        mag = ldexp(128.0 + (double)mant, expo - 134); /* (1+m/128) * 2^(e-127) */
    return sign ? -mag : mag;
}

static double decode(const void *base, int dtype, int64_t i)
{
    if (dtype == ORACLE_FP8_E4M3)
        return oracle_decode_e4m3fn(((const uint8_t *)base)[i]);
    return oracle_decode_bf16(((const uint16_t *)base)[i]);
}

/* Decode one row of 128 key components. */
static void decode_key(const void *kv, int dtype, int64_t s, double *out)
{
    for (int d = 0; d < ORACLE_DIM; ++d)
        out[d] = decode(kv, dtype, s * ORACLE_DIM + d);
}

/* Decode the heads x 128 query components of row t. */
static void decode_query(const void *q, int dtype, int heads, int64_t t, double *out)
{
    for (int i = 0; i < heads * ORACLE_DIM; ++i)
        out[i] = decode(q, dtype, t * heads * ORACLE_DIM + i);
}

/* The score of one (query, key) pair from already-decoded operands. */
static double score_pair(const double *qrow, const double *key,
                         const float *wrow, int heads, double sigma)
{
    double acc = 0.0;
    for (int h = 0; h < heads; ++h) {
        double x = 0.0;
        for (int d = 0; d < ORACLE_DIM; ++d)
            x += qrow[h * ORACLE_DIM + d] * key[d];
        double r = x > 0.0 ? x : 0.0; /* ReLU per head */
        acc += (double)wrow[h] * r;   /* weighted head sum */
    }
    return sigma * acc;               /* per-key scale */
}

/* Scores of row t for keys s in [s_begin, s_end), written to out[s - s_begin].
 * Any key range is allowed (the window is not consulted).  Returns 0, or -1 if
 * an operand decodes to NaN. */
int oracle_scores_h(const void *q, const void *kv, int dtype, int heads, const float *kv_scales,
                    const float *weights, int64_t t, int64_t s_begin, int64_t s_end,
                    double *out)
{
    if (heads < 1) return -3;
    double *qrow = (double *)malloc(sizeof(double) * heads * ORACLE_DIM);
    double key[ORACLE_DIM];
    int bad = 0;
    if (!qrow) return -2;
    decode_query(q, dtype, heads, t, qrow);
    for (int i = 0; i < heads * ORACLE_DIM; ++i)
        if (isnan(qrow[i])) bad = 1;
    for (int64_t s = s_begin; s < s_end && !bad; ++s) {
        decode_key(kv, dtype, s, key);
        for (int d = 0; d < ORACLE_DIM; ++d)
            if (isnan(key[d])) bad = 1;
        double sigma = kv_scales ? (double)kv_scales[s] : 1.0;
        out[s - s_begin] = score_pair(qrow, key, weights + t * heads, heads, sigma);
    }
    free(qrow);
    return bad ? -1 : 0;
}

int oracle_scores(const void *q, const void *kv, int dtype, const float *kv_scales,
                  const float *weights, int64_t t, int64_t s_begin, int64_t s_end,
                  double *out)
{
    return oracle_scores_h(q, kv, dtype, ORACLE_HEADS, kv_scales, weights, t, s_begin, s_end, out);
}

typedef struct {
    double score;
    int64_t index;
} scored_key;

/* Full order used for selection: larger score first; equal scores (including
 * +0 against -0) keep the smaller key index first. */
static int by_score_then_index(const void *pa, const void *pb)
{
    const scored_key *a = (const scored_key *)pa;
    const scored_key *b = (const scored_key *)pb;
    if (a->score > b->score) return -1;
    if (a->score < b->score) return 1;
    if (a->index < b->index) return -1;
    if (a->index > b->index) return 1;
    return 0;
}

/* One row of the selection.  Writes topk slots of out_idx / out_val (and, when
 * out_score is given, the unrounded binary64 scores, NaN in padding slots).
 * all_scores, when given, receives the binary64 score of every key of the
 * window in key order (length ke - ks).  Returns 0, -1 on NaN operands, -2 on
 * allocation failure. */
static int select_row(const void *q, int dtype, int heads, const float *kv_scales,
                      const float *weights, int64_t t, int32_t ks, int32_t ke, int topk,
                      const double *kv_decoded, int32_t *out_idx, float *out_val,
                      double *out_score, double *all_scores)
{
    int64_t len = (int64_t)ke - (int64_t)ks;
    if (len < 0) len = 0;
    scored_key *keys = (scored_key *)malloc(sizeof(scored_key) * (size_t)(len > 0 ? len : 1));
    double *qrow = (double *)malloc(sizeof(double) * heads * ORACLE_DIM);
    if (!keys || !qrow) { free(keys); free(qrow); return -2; }
    int bad = 0;
    decode_query(q, dtype, heads, t, qrow);
    for (int i = 0; i < heads * ORACLE_DIM; ++i)
        if (isnan(qrow[i])) bad = 1;
    for (int64_t j = 0; j < len; ++j) {
        int64_t s = ks + j;
        const double *key = kv_decoded + s * ORACLE_DIM;
        double sigma = kv_scales ? (double)kv_scales[s] : 1.0;
        keys[j].score = score_pair(qrow, key, weights + t * heads, heads, sigma);
        keys[j].index = s;
        if (isnan(keys[j].score)) bad = 1;
        if (all_scores) all_scores[j] = keys[j].score;
    }
    qsort(keys, (size_t)len, sizeof(scored_key), by_score_then_index);
    for (int j = 0; j < topk; ++j) {
        if (j < len) {
            float v = (float)keys[j].score;
            if (v == 0.0f) v = 0.0f; /* write -0 as +0 */
            out_idx[j] = (int32_t)keys[j].index;
            out_val[j] = v;
            if (out_score) out_score[j] = keys[j].score;
        } else {
            out_idx[j] = -1;
            out_val[j] = -INFINITY;
            if (out_score) out_score[j] = NAN;
        }
    }
    free(keys);
    free(qrow);
    return bad ? -1 : 0;
}

/* Exact top-k for a list of rows.
 *   q        [num_q, heads, 128]  FP8 E4M3FN bytes or BF16 codes (heads = 32 for
 *            oracle_select; the head count is a parameter of oracle_select_h, for
 *            head counts besides 32, e.g. 64: README "Roadmap")
 *   kv       [num_kv, 128]     same dtype
 *   kv_scales[num_kv] fp32 or NULL (all ones)
 *   weights  [num_q, heads] fp32
 *   ks, ke   [num_q] int32, window [ks, ke)
 *   rows     the nrows query rows to process (NULL: rows 0..nrows-1)
 *   out_idx / out_val  [nrows, topk]; out_score [nrows, topk] binary64 or NULL
 *   all_scores [nrows, num_kv] binary64 or NULL: the score of every key of the
 *            row's window at its key position, NaN outside the window
 *   nthreads OpenMP threads (<= 0: runtime default)
 * Returns 0, or a negative code (-1 NaN operand, -2 allocation failure,
 * -3 bad argument). */
int oracle_select_h(const void *q, const void *kv, int dtype, int heads, const float *kv_scales,
                    const float *weights, const int32_t *ks, const int32_t *ke,
                    int64_t num_q, int64_t num_kv, int topk, const int64_t *rows,
                    int64_t nrows, int32_t *out_idx, float *out_val, double *out_score,
                    double *all_scores, int nthreads)
{
    if (topk < 1 || num_q < 0 || num_kv < 0 || nrows < 0 || heads < 1) return -3;
    if (dtype != ORACLE_FP8_E4M3 && dtype != ORACLE_BF16) return -3;
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t t = rows ? rows[r] : r;
        if (t < 0 || t >= num_q) return -3;
        if (ks[t] < 0 || ke[t] > num_kv || (ke[t] > ks[t] && ks[t] >= num_kv)) return -3;
    }
    double *kv_decoded = (double *)malloc(sizeof(double) * (size_t)(num_kv > 0 ? num_kv : 1) * ORACLE_DIM);
    if (!kv_decoded) return -2;
    for (int64_t s = 0; s < num_kv; ++s)
        decode_key(kv, dtype, s, kv_decoded + s * ORACLE_DIM);
    int status = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1) reduction(min : status)
#endif
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t t = rows ? rows[r] : r;
        double *row_all = NULL;
        if (all_scores) {
            row_all = all_scores + r * num_kv;
            for (int64_t s = 0; s < num_kv; ++s) row_all[s] = NAN;
            if (ke[t] > ks[t]) row_all += ks[t];
        }
        int st = select_row(q, dtype, heads, kv_scales, weights, t, ks[t], ke[t], topk,
                            kv_decoded, out_idx + r * topk, out_val + r * topk,
                            out_score ? out_score + r * topk : NULL, row_all);
        if (st < status) status = st;
    }
    free(kv_decoded);
    return status;
}

int oracle_select(const void *q, const void *kv, int dtype, const float *kv_scales,
                  const float *weights, const int32_t *ks, const int32_t *ke,
                  int64_t num_q, int64_t num_kv, int topk, const int64_t *rows,
                  int64_t nrows, int32_t *out_idx, float *out_val, double *out_score,
                  double *all_scores, int nthreads)
{
    return oracle_select_h(q, kv, dtype, ORACLE_HEADS, kv_scales, weights, ks, ke, num_q, num_kv, topk, rows,
                           nrows, out_idx, out_val, out_score, all_scores, nthreads);
}

/* Exact top-k over materialized score rows (DeepSelect README, "Usage" and
 * "Variable-length rows": each row keeps its topk largest values among its
 * first end[r] entries; rows shorter than topk are padded with fill values,
 * here index -1 / value -inf).  Order: value desc, index asc, with +0 and -0
 * equal -- the same order as the indexer selection above.
 *   x        [rows, stride] float32 (dtype 0) or BF16 codes (dtype 1)
 *   ends     [rows] int32 or NULL (every row has cols entries); each end is
 *            clamped to [0, cols]
 *   out_idx / out_val  [rows, topk]: positions in the row and their values
 * Returns 0, -1 on a NaN entry, -2 on allocation failure, -3 bad argument. */
int oracle_topk_rows(const void *x, int dtype, int64_t rows, int64_t cols, int64_t stride,
                     const int32_t *ends, int topk, int32_t *out_idx, float *out_val, int nthreads)
{
    if (topk < 1 || rows < 0 || cols < 0 || stride < cols) return -3;
    if (dtype != 0 && dtype != 1) return -3;
    int status = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1) reduction(min : status)
#endif
    for (int64_t r = 0; r < rows; ++r) {
        int64_t n = cols;
        if (ends) {
            n = ends[r];
            if (n < 0) n = 0;
            if (n > cols) n = cols;
        }
        scored_key *keys = (scored_key *)malloc(sizeof(scored_key) * (size_t)(n > 0 ? n : 1));
        if (!keys) {
            status = -2;
            continue;
        }
        int st = 0;
        for (int64_t j = 0; j < n; ++j) {
            double v;
            if (dtype == 0)
                v = (double)((const float *)x)[r * stride + j];
            else
                v = oracle_decode_bf16(((const uint16_t *)x)[r * stride + j]);
            if (isnan(v)) st = -1;
            keys[j].score = v;
            keys[j].index = j;
        }
        qsort(keys, (size_t)n, sizeof(scored_key), by_score_then_index);
        for (int j = 0; j < topk; ++j) {
            if (j < n) {
                float v = (float)keys[j].score; /* exact: the entries are float32 or BF16 */
                if (v == 0.0f) v = 0.0f;
                out_idx[r * topk + j] = (int32_t)keys[j].index;
                out_val[r * topk + j] = v;
            } else {
                out_idx[r * topk + j] = -1;
                out_val[r * topk + j] = -INFINITY;
            }
        }
        free(keys);
        if (st < status) status = st;
    }
    return status;
}

/* Number of threads an OpenMP parallel region of this library would use. */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
