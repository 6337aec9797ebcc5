/*
 * qli_oracle.c -- plain, slow CPU oracle for the quantized lightning indexer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  The product path
 * (the HIP library under sparse_attention_token_paged_amd/) never calls it
 * and shares no code with it: no header, helper, table or constant.
 *
 * Source of the method ("QLI-README" below): the EngineX-Ascend page
 * "VllmQuantLightningIndexer" (csrc/attention/vllm_quant_lightning_indexer/
 * README.md).  Sections cited by their headings:
 *   [功能说明]   function description: the Top-k formula and its three steps
 *   [参数说明]   parameter table (query, key, scales, weights, lengths,
 *               block_table, sparse_count, sparse_mode, cmp_ratio, stride,
 *               sparse_indices, sparse_values) and the dtype pairing notes
 *   [约束说明]   constraints (D = 128, N = 64 / 1, TND prefix sums,
 *               block_size multiple of 16 up to 1024, NaN order undefined)
 *
 * Precision: integer dots are exact (int64); fp8 dots are exact in fp64
 * (every e4m3 product is a multiple of 2^-18 below 2^18, and 128 of them
 * need fewer than 53 bits); the score formula is evaluated in fp64 in the
 * literal order of the formula.  Readings of points the page leaves open
 * are marked "reading:" where they are applied.
 *
 * Every function here is pinned by tests under tests/ (test_oracle_*.py)
 * against brute force, closed forms, invariants or library routines.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define QLIO_HEADS 64 /* [约束说明]: query N axis is 64 */
#define QLIO_DIM 128  /* [约束说明]: D axis of query and key is 128 */

enum {
    QLIO_OK = 0,
    QLIO_E_ARG = 1,
    QLIO_E_UNSUPPORTED = 2
};

/* ------------------------------------------------------------------ */
/* Element decoding                                                   */
/* ------------------------------------------------------------------ */

/* [参数说明] query/key dtype FLOAT8_e4m3fn.  OCP E4M3FN: 1 sign bit, 4
 * exponent bits with bias 7, 3 mantissa bits; no infinities; the two codes
 * S.1111.111 are NaN; exponent field 0 encodes subnormals m * 2^-9. */
double qlio_e4m3fn_value(uint8_t code)
{
    int s = code >> 7;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double v;
    if (e == 0xF && m == 0x7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);              /* 0.m * 2^(1-7) */
    else
        v = ldexp((double)(8 + m), e - 10);    /* 1.m * 2^(e-7) */
    return s ? -v : v;
}

/* [参数说明] scales / weights dtype FLOAT16: IEEE 754 binary16 (bias 15,
 * 10 mantissa bits, subnormals m * 2^-24). */
double qlio_f16_value(uint16_t bits)
{
    int s = bits >> 15;
    int e = (bits >> 10) & 0x1F;
    int m = bits & 0x3FF;
    double v;
    if (e == 0x1F)
        v = m ? NAN : INFINITY;
    else if (e == 0)
        v = ldexp((double)m, -24);
    else
        v = ldexp((double)(1024 + m), e - 25);
    return s ? -v : v;
}

/* scales / weights dtype FLOAT32: IEEE binary32, widened exactly. */
static double f32_value(const void *base, int64_t i)
{
    float f;
    memcpy(&f, (const char *)base + 4 * i, 4);
    return (double)f;
}

static double scale_value(const void *base, int64_t i, int scale_dtype)
{
    if (scale_dtype == 0) {
        uint16_t h;
        memcpy(&h, (const char *)base + 2 * i, 2);
        return qlio_f16_value(h);
    }
    return f32_value(base, i);
}

/* ------------------------------------------------------------------ */
/* Visibility                                                         */
/* ------------------------------------------------------------------ */

/* Number of compressed key entries that query i (0-based) of a sequence with
 * s1b query tokens and skb original key tokens may see.
 *  [参数说明] cmp_ratio: the key is compressed by cmp_ratio.
 *    reading: actual_seq_lengths_key counts original tokens; only complete
 *    groups are stored, so floor(skb / cmp) entries exist; entry j covers
 *    original tokens [j*cmp, (j+1)*cmp).
 *  [参数说明] sparse_mode 0 (defaultMask): no mask, every stored entry.
 *  [参数说明] sparse_mode 3 (rightDownCausal, lower triangle cut at the
 *    bottom-right corner).  reading: query i sits at original position
 *    skb - s1b + i and sees an entry only when every token of it is at or
 *    before that position, i.e. entries j < floor((pos + 1) / cmp); a
 *    negative count clamps to 0. */
int64_t qlio_visible(int sparse_mode, int cmp_ratio, int64_t skb, int64_t s1b,
                     int64_t i)
{
    int64_t stored = skb / cmp_ratio;
    int64_t upto, v;
    if (sparse_mode == 0)
        return stored;
    upto = skb - s1b + i + 1; /* original tokens at or before the query */
    if (upto <= 0)
        return 0;
    v = upto / cmp_ratio;
    return v < stored ? v : stored;
}

/* Is original token t inside the window of a query at position pos?
 * Written with differences of small numbers only, so that the default
 * 2^63-1 of either bound cannot overflow. */
static int in_window(int64_t t, int64_t pos, int64_t pre_tokens, int64_t next_tokens)
{
    if (t < pos && pos - t > pre_tokens)
        return 0;
    if (t > pos && t - pos > next_tokens)
        return 0;
    return 1;
}

/* Visible range [*lo, return value) of query i, windows included.
 *  [参数说明] pre_tokens / next_tokens: the page marks both as reserved
 *    parameters (only the default 2^63-1 accepted) that say how many tokens
 *    before (after) a query the attention relates to.  reading, for other
 *    values: query i sits at the original position pos = skb - s1b + i (the
 *    same bottom-right alignment as sparse_mode 3, for both modes); token t
 *    is inside its window when pos - pre_tokens <= t <= pos + next_tokens;
 *    an entry is visible when sparse_mode lets the query see it and every
 *    token it covers is inside the window.  The window is an interval, so
 *    the visible entries are consecutive; with the defaults the range is
 *    [0, qlio_visible).  Both bounds are >= 0 (validate). */
int64_t qlio_visible_range(int sparse_mode, int cmp_ratio, int64_t skb, int64_t s1b, int64_t i,
                           int64_t pre_tokens, int64_t next_tokens, int64_t *lo_out)
{
    int64_t n = qlio_visible(sparse_mode, cmp_ratio, skb, s1b, i);
    int64_t pos = skb - s1b + i;
    int64_t j, lo = -1, hi = -1;
    for (j = 0; j < n; j++) {
        int64_t first = j * cmp_ratio, last = (j + 1) * cmp_ratio - 1;
        if (in_window(first, pos, pre_tokens, next_tokens) &&
            in_window(last, pos, pre_tokens, next_tokens)) {
            if (lo < 0)
                lo = j;
            hi = j + 1;
        }
    }
    if (lo < 0)
        lo = hi = 0;
    *lo_out = lo;
    return hi;
}

/* ------------------------------------------------------------------ */
/* Paged key access                                                   */
/* ------------------------------------------------------------------ */

/* [参数说明] key is PA_BSND [num_blocks, block_size, 1, 128] reached through
 * block_table[B, maxBlockNumPerSeq]; "stride" is the step of the key's first
 * axis.  reading: stride counts elements (= bytes for 8-bit keys) between
 * consecutive blocks; key_dequant_scale is a contiguous
 * [num_blocks, block_size, 1] array.  Entry j of batch b lives in block
 * block_table[b][j / block_size] at slot j % block_size. */
typedef struct {
    const uint8_t *key;
    const void *k_scale;
    const int32_t *block_table;
    int block_size;
    int max_blocks;
    int64_t stride;
    int scale_dtype;
} paged_keys;

static const uint8_t *key_row(const paged_keys *pk, int b, int64_t j,
                              double *scale)
{
    int32_t blk = pk->block_table[(int64_t)b * pk->max_blocks + j / pk->block_size];
    int64_t slot = j % pk->block_size;
    *scale = scale_value(pk->k_scale, (int64_t)blk * pk->block_size + slot,
                         pk->scale_dtype);
    return pk->key + (int64_t)blk * pk->stride + slot * QLIO_DIM;
}

/* ------------------------------------------------------------------ */
/* Dot products Q_index . K_index^T                                   */
/* ------------------------------------------------------------------ */

/* The value of every e4m3fn code, filled once from qlio_e4m3fn_value so that
 * the dot loop does not call ldexp per element (same values). */
static double e4m3_value_of[256];

__attribute__((constructor)) static void fill_e4m3_values(void)
{
    int c;
    for (c = 0; c < 256; c++)
        e4m3_value_of[c] = qlio_e4m3fn_value((uint8_t)c);
}

/* [功能说明] step 1: the token's query (g x d) times the key (S_k x d).
 * INT8: exact integer sum.  FLOAT8_e4m3fn: exact in fp64 (see header). */
static double dot_q_k(const uint8_t *q, const uint8_t *k, int qk_dtype)
{
    int d;
    if (qk_dtype == 0) {
        int64_t acc = 0;
        for (d = 0; d < QLIO_DIM; d++)
            acc += (int64_t)(int8_t)q[d] * (int64_t)(int8_t)k[d];
        return (double)acc;
    } else {
        double acc = 0.0;
        for (d = 0; d < QLIO_DIM; d++)
            acc += e4m3_value_of[q[d]] * e4m3_value_of[k[d]];
        return acc;
    }
}

/* ------------------------------------------------------------------ */
/* Problem description (the oracle's own; shares nothing with the library) */
/* ------------------------------------------------------------------ */

typedef struct {
    int qk_dtype;    /* 0 INT8, 1 FLOAT8_e4m3fn */
    int scale_dtype; /* 0 FLOAT16, 1 FLOAT32 */
    int layout;      /* 0 BSND, 1 TND */
    int batch;
    int s1_or_t;
    int sparse_count;
    int sparse_mode;
    int cmp_ratio;
    int64_t pre_tokens;
    int64_t next_tokens;
    const uint8_t *query;
    const void *weights;
    const void *q_scale;
    const int32_t *aslq;
    const int32_t *aslk;
    paged_keys pk;
} oracle_problem;

/* Row r of the output belongs to batch *b with local query index *i among
 * *s1b query tokens of that batch; returns 0 for rows that belong to no
 * query token (BSND rows past actual_seq_lengths_query[b], TND rows past the
 * last prefix sum).
 *  [参数说明] actual_seq_lengths_query: valid query tokens per batch.
 *  [约束说明] TND: actual_seq_lengths_query is required; its length is B and
 *    each element is the prefix sum of the token counts. */
static int locate_row(const oracle_problem *p, int64_t r, int *b, int64_t *i,
                      int64_t *s1b)
{
    if (p->layout == 0) {
        int bb = (int)(r / p->s1_or_t);
        int64_t ii = r % p->s1_or_t;
        int64_t n = p->aslq ? p->aslq[bb] : p->s1_or_t;
        if (ii >= n)
            return 0;
        *b = bb;
        *i = ii;
        *s1b = n;
        return 1;
    } else {
        int bb;
        int64_t start = 0;
        for (bb = 0; bb < p->batch; bb++) {
            int64_t end = p->aslq[bb];
            if (r < end) {
                *b = bb;
                *i = r - start;
                *s1b = end - start;
                return 1;
            }
            start = end;
        }
        return 0;
    }
}

/* Visible range [*lo, return value) of output row r (empty for rows that
 * belong to no query token). */
static int64_t row_range(const oracle_problem *p, int64_t r, int *b, int64_t *lo)
{
    int64_t i, s1b;
    *lo = 0;
    if (!locate_row(p, r, b, &i, &s1b))
        return 0;
    return qlio_visible_range(p->sparse_mode, p->cmp_ratio, p->aslk[*b], s1b, i, p->pre_tokens,
                              p->next_tokens, lo);
}

/* One score, literally as the [功能说明] formula reads:
 *   [1]_{1 x g} @ [ (W @ [1]_{1 x Sk}) (.) ReLU( (ScaleQ @ ScaleK^T) (.) (Q K^T) ) ]
 * i.e. for key j:  sum over heads g (ascending) of
 *   W[g] * max(0, (ScaleQ[g] * ScaleK[j]) * dot[g][j]).
 * Optionally stores dot[g] for g < 64 into dots (stride dot_stride). */
static double score_one(const oracle_problem *p, int64_t r, int b, int64_t j,
                        double *dots, int64_t dot_stride)
{
    double sk, score = 0.0;
    const uint8_t *k = key_row(&p->pk, b, j, &sk);
    int g;
    for (g = 0; g < QLIO_HEADS; g++) {
        const uint8_t *q = p->query + (r * QLIO_HEADS + g) * QLIO_DIM;
        double dot = dot_q_k(q, k, p->qk_dtype);
        double w = scale_value(p->weights, r * QLIO_HEADS + g, p->scale_dtype);
        double sq = scale_value(p->q_scale, r * QLIO_HEADS + g, p->scale_dtype);
        double corr = (sq * sk) * dot;
        double relu = corr > 0.0 ? corr : 0.0;
        score += w * relu;
        if (dots)
            dots[g * dot_stride] = dot;
    }
    return score;
}

/* ------------------------------------------------------------------ */
/* Top-k                                                              */
/* ------------------------------------------------------------------ */

typedef struct {
    double score;
    int64_t idx;
} scored;

/* [功能说明] step 3: keep the Top-k indices.  reading: larger score first;
 * equal scores go to the lower index (a total order, so the result is the
 * stable top-k). */
static int cmp_scored(const void *a, const void *b)
{
    const scored *x = (const scored *)a, *y = (const scored *)b;
    if (x->score > y->score)
        return -1;
    if (x->score < y->score)
        return 1;
    return (x->idx > y->idx) - (x->idx < y->idx);
}

/* Stable top-k of scores[0..n): writes min(k, n) indices (score descending,
 * index ascending among equals) to idx_out and returns that count. */
int64_t qlio_topk(const double *scores, int64_t n, int64_t k, int64_t *idx_out)
{
    int64_t i, m = n < k ? n : k;
    scored *v;
    if (m <= 0)
        return 0;
    v = (scored *)malloc(sizeof(scored) * (size_t)n);
    if (!v)
        return -1;
    for (i = 0; i < n; i++) {
        v[i].score = scores[i];
        v[i].idx = i;
    }
    qsort(v, (size_t)n, sizeof(scored), cmp_scored);
    for (i = 0; i < m; i++)
        idx_out[i] = v[i].idx;
    free(v);
    return m;
}

/* ------------------------------------------------------------------ */
/* Validation (the oracle's own reading of the constraints)           */
/* ------------------------------------------------------------------ */

static int validate(const oracle_problem *p, int num_blocks, int max_blocks)
{
    int b, c;
    if (p->batch < 0 || p->s1_or_t < 0 || p->pk.block_size <= 0)
        return QLIO_E_ARG;
    /* [约束说明] block_size: multiple of 16, at most 1024. */
    if (p->pk.block_size % 16 != 0 || p->pk.block_size > 1024)
        return QLIO_E_ARG;
    /* [参数说明] sparse_count in [1, 2048]; sparse_mode 0 or 3;
     * cmp_ratio in {1, 2, 4, ..., 128}. */
    if (p->sparse_count < 1 || p->sparse_count > 2048)
        return QLIO_E_ARG;
    if (p->sparse_mode != 0 && p->sparse_mode != 3)
        return QLIO_E_ARG;
    /* pre_tokens / next_tokens: the window reading (qlio_visible_range)
     * takes bounds >= 0. */
    if (p->pre_tokens < 0 || p->next_tokens < 0)
        return QLIO_E_ARG;
    for (c = 1; c <= 128 && c != p->cmp_ratio; c *= 2)
        ;
    if (c > 128)
        return QLIO_E_ARG;
    /* [参数说明] notes: INT8 q/k go with FLOAT16 scales; FLOAT8_e4m3fn q/k
     * go with FLOAT32 scales. */
    if (!((p->qk_dtype == 0 && p->scale_dtype == 0) ||
          (p->qk_dtype == 1 && p->scale_dtype == 1)))
        return QLIO_E_UNSUPPORTED;
    if (p->layout != 0 && p->layout != 1)
        return QLIO_E_ARG;
    if (p->pk.stride < (int64_t)p->pk.block_size * QLIO_DIM)
        return QLIO_E_ARG;
    if (p->layout == 1 && !p->aslq)
        return QLIO_E_ARG;
    if (!p->aslk)
        return QLIO_E_ARG;
    for (b = 0; b < p->batch; b++) {
        int64_t stored, need;
        if (p->aslk[b] < 0)
            return QLIO_E_ARG;
        if (p->layout == 0 && p->aslq &&
            (p->aslq[b] < 0 || p->aslq[b] > p->s1_or_t))
            return QLIO_E_ARG;
        if (p->layout == 1 &&
            (p->aslq[b] < 0 || (b > 0 && p->aslq[b] < p->aslq[b - 1]) ||
             p->aslq[b] > p->s1_or_t))
            return QLIO_E_ARG;
        stored = p->aslk[b] / p->cmp_ratio;
        need = (stored + p->pk.block_size - 1) / p->pk.block_size;
        if (need > max_blocks)
            return QLIO_E_ARG;
        {
            int64_t j;
            for (j = 0; j < need; j++) {
                int32_t blk = p->pk.block_table[(int64_t)b * max_blocks + j];
                if (blk < 0 || blk >= num_blocks)
                    return QLIO_E_ARG;
            }
        }
    }
    return QLIO_OK;
}

/* ------------------------------------------------------------------ */
/* Entry points                                                       */
/* ------------------------------------------------------------------ */

static int fill_problem(oracle_problem *p, int qk_dtype, int scale_dtype,
                        int layout, int batch, int s1_or_t, int block_size,
                        int max_blocks, int64_t key_stride, int sparse_count,
                        int sparse_mode, int cmp_ratio, int64_t pre_tokens,
                        int64_t next_tokens, const void *query,
                        const void *key, const void *weights,
                        const void *q_scale, const void *k_scale,
                        const int32_t *aslq, const int32_t *aslk,
                        const int32_t *block_table)
{
    p->qk_dtype = qk_dtype;
    p->scale_dtype = scale_dtype;
    p->layout = layout;
    p->batch = batch;
    p->s1_or_t = s1_or_t;
    p->sparse_count = sparse_count;
    p->sparse_mode = sparse_mode;
    p->cmp_ratio = cmp_ratio;
    p->pre_tokens = pre_tokens;
    p->next_tokens = next_tokens;
    p->query = (const uint8_t *)query;
    p->weights = weights;
    p->q_scale = q_scale;
    p->aslq = aslq;
    p->aslk = aslk;
    p->pk.key = (const uint8_t *)key;
    p->pk.k_scale = k_scale;
    p->pk.block_table = block_table;
    p->pk.block_size = block_size;
    p->pk.max_blocks = max_blocks;
    p->pk.stride = key_stride > 0 ? key_stride : (int64_t)block_size * QLIO_DIM;
    p->pk.scale_dtype = scale_dtype;
    return 0;
}

static int64_t total_rows(const oracle_problem *p)
{
    return p->layout == 0 ? (int64_t)p->batch * p->s1_or_t : (int64_t)p->s1_or_t;
}

/* Visible range of every output row (rows = B*S1 for BSND, T for TND):
 * entries [lo_out[r], hi_out[r]). */
int qlio_row_range(int layout, int batch, int s1_or_t, int sparse_mode,
                   int cmp_ratio, const int32_t *aslq, const int32_t *aslk,
                   int64_t pre_tokens, int64_t next_tokens, int64_t *lo_out,
                   int64_t *hi_out)
{
    oracle_problem p;
    int64_t r, n;
    memset(&p, 0, sizeof(p));
    p.layout = layout;
    p.batch = batch;
    p.s1_or_t = s1_or_t;
    p.sparse_mode = sparse_mode;
    p.cmp_ratio = cmp_ratio;
    p.pre_tokens = pre_tokens;
    p.next_tokens = next_tokens;
    p.aslq = aslq;
    p.aslk = aslk;
    n = total_rows(&p);
    for (r = 0; r < n; r++) {
        int b;
        hi_out[r] = row_range(&p, r, &b, &lo_out[r]);
    }
    return QLIO_OK;
}

/* Visible-entry count of every output row without a window. */
int qlio_row_visible(int layout, int batch, int s1_or_t, int sparse_mode,
                     int cmp_ratio, const int32_t *aslq, const int32_t *aslk,
                     int64_t *vis_out)
{
    oracle_problem p;
    int64_t r, n, lo;
    memset(&p, 0, sizeof(p));
    p.layout = layout;
    p.batch = batch;
    p.s1_or_t = s1_or_t;
    p.sparse_mode = sparse_mode;
    p.cmp_ratio = cmp_ratio;
    p.pre_tokens = INT64_MAX;
    p.next_tokens = INT64_MAX;
    p.aslq = aslq;
    p.aslk = aslk;
    n = total_rows(&p);
    for (r = 0; r < n; r++) {
        int b;
        vis_out[r] = row_range(&p, r, &b, &lo);
    }
    return QLIO_OK;
}

/* The whole operator.
 *  Outputs ([参数说明] sparse_indices INT32 / sparse_values FLOAT32),
 *  shaped [rows, sparse_count]; row r sees entries [lo, hi) (row_range),
 *  vis = hi - lo of them:
 *    sparse_indices[r, 0:n] = top-n entry indices (n = min(k, vis)), in the
 *      order score descending, index ascending; sparse_indices[r, n:k] = -1.
 *    sparse_values[r, 0:n] = the fp32 rounding of those scores; the rest
 *      -INFINITY.  (reading: the page defines sparse_values as the values of
 *      the returned indices.)
 *  Optional: scores[r * score_cols + j] = fp64 score of visible entry j
 *    (entries outside [lo, hi) are left untouched).
 *  nthreads <= 0 uses the OpenMP default. */
int qlio_indexer(int qk_dtype, int scale_dtype, int layout, int batch,
                 int s1_or_t, int num_blocks, int block_size, int max_blocks,
                 int64_t key_stride, int sparse_count, int sparse_mode,
                 int cmp_ratio, int64_t pre_tokens, int64_t next_tokens,
                 const void *query, const void *key,
                 const void *weights, const void *q_scale, const void *k_scale,
                 const int32_t *aslq, const int32_t *aslk,
                 const int32_t *block_table, int32_t *sparse_indices,
                 float *sparse_values, double *scores, int64_t score_cols,
                 int nthreads)
{
    oracle_problem p;
    int64_t r, rows;
    int rc, failed = 0;
    fill_problem(&p, qk_dtype, scale_dtype, layout, batch, s1_or_t,
                 block_size, max_blocks, key_stride, sparse_count, sparse_mode,
                 cmp_ratio, pre_tokens, next_tokens, query, key, weights,
                 q_scale, k_scale, aslq, aslk, block_table);
    rc = validate(&p, num_blocks, max_blocks);
    if (rc != QLIO_OK)
        return rc;
    rows = total_rows(&p);
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
#endif
    for (r = 0; r < rows; r++) {
        int b = 0;
        int64_t lo, hi = row_range(&p, r, &b, &lo), vis = hi - lo, j, n;
        int32_t *oi = sparse_indices + r * sparse_count;
        float *ov = sparse_values ? sparse_values + r * sparse_count : NULL;
        double *sc;
        int64_t *top;
        for (j = 0; j < sparse_count; j++) {
            oi[j] = -1;
            if (ov)
                ov[j] = -INFINITY;
        }
        if (vis <= 0)
            continue;
        sc = (double *)malloc(sizeof(double) * (size_t)vis);
        top = (int64_t *)malloc(sizeof(int64_t) * (size_t)(vis < sparse_count ? vis : sparse_count));
        if (!sc || !top) {
            free(sc);
            free(top);
            failed = 1;
            continue;
        }
        /* sc[e] = score of entry lo + e; the top-k positions map back by + lo */
        for (j = 0; j < vis; j++)
            sc[j] = score_one(&p, r, b, lo + j, NULL, 0);
        n = qlio_topk(sc, vis, sparse_count, top);
        for (j = 0; j < n; j++) {
            oi[j] = (int32_t)(lo + top[j]);
            if (ov)
                ov[j] = (float)sc[top[j]];
        }
        if (scores)
            for (j = 0; j < vis && lo + j < score_cols; j++)
                scores[r * score_cols + lo + j] = sc[j];
        free(sc);
        free(top);
    }
    return failed ? QLIO_E_ARG : QLIO_OK;
}

/* Dots and scores of one output row over entries [j0, j1) of its visible
 * range (pins and parity sampling).  dots: [64, j1 - j0] row-major (fp64,
 * exact integers for INT8); scores: [j1 - j0].  Returns the row's visible
 * count, or -1 if [j0, j1) leaves the visible range. */
int64_t qlio_row_detail(int qk_dtype, int scale_dtype, int layout, int batch,
                        int s1_or_t, int block_size, int max_blocks,
                        int64_t key_stride, int sparse_mode, int cmp_ratio,
                        const void *query, const void *key,
                        const void *weights, const void *q_scale,
                        const void *k_scale, const int32_t *aslq,
                        const int32_t *aslk, const int32_t *block_table,
                        int64_t row, int64_t j0, int64_t j1, double *dots,
                        double *scores)
{
    oracle_problem p;
    int b = 0;
    int64_t vis, lo, j;
    /* the score of an entry does not depend on a window: none is applied */
    fill_problem(&p, qk_dtype, scale_dtype, layout, batch, s1_or_t,
                 block_size, max_blocks, key_stride, 1, sparse_mode, cmp_ratio,
                 INT64_MAX, INT64_MAX, query, key, weights, q_scale, k_scale,
                 aslq, aslk, block_table);
    vis = row_range(&p, row, &b, &lo);
    if (j0 < 0 || j1 < j0 || j1 > vis)
        return -1;
    for (j = j0; j < j1; j++) {
        double s = score_one(&p, row, b, j, dots ? dots + (j - j0) : NULL,
                             j1 - j0);
        if (scores)
            scores[j - j0] = s;
    }
    return vis;
}
