/*
 * CPU oracle for the sparse-index hot path: indexer score, top-k selection and
 * sparse attention over the selected rows.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plainly written reference
 * that the GPU library is checked against.  Only the test suite, the smoke
 * entry point and the benchmark's CPU-baseline leg may load it.  It shares no
 * code, header or constant with the GPU library.
 *
 * Sources (the pages describe the method in prose only):
 *  - IndexCache news article (app.myzaker.com), section "IndexCache": a light
 *    indexer in front of every layer's attention scans the whole context and
 *    picks the important tokens; the main attention then reads only those.
 *  - IndexShare term page (earlyterms.com), opening definition: the indexer's
 *    work is a dot product followed by a top-k.
 *  - IndexShare explainer (yun88.com), section on the hidden cost of sparse
 *    attention: every token keeps only its top-k history positions.
 * The pages name the indexer score only as "dot product + top-k"; this oracle
 * fixes it as
 *     score[t,s] = sum_h w[t,h] * max(0, sum_d q[t,h,d] * k[s,d]),  s <= p_t
 * with one key row per token shared by all indexer heads.
 *
 * Arithmetic: every input is decoded exactly to double, every sum runs in
 * double in ascending index order, and each result is rounded once (scores to
 * fp32, attention outputs to bf16, both round-to-nearest-even).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ decode */

/* bf16 is the upper half of an IEEE-754 binary32 word. */
double oracle_bf16_to_double(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP 8-bit E4M3 ("fn" variant): 1 sign bit, 4 exponent bits with bias 7,
 * 3 mantissa bits, subnormals when the exponent field is 0, no infinities,
 * and exponent 15 with mantissa 7 is NaN.  Largest finite value 448. */
double oracle_fp8e4m3_to_double(uint8_t b)
{
    int sign = (b >> 7) & 1;
    int e = (b >> 3) & 15;
    int m = b & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9); /* m/8 * 2^(1-7) */
    else
        v = ldexp(1.0 + m / 8.0, e - 7);
    return sign ? -v : v;
}

/* Round a double to the nearest bf16 (ties to even) in one step and return
 * its bit pattern.  bf16 keeps 8 significant bits; below 2^-126 the spacing
 * stays 2^-133 (subnormals). */
uint16_t oracle_double_to_bf16(double x)
{
    if (isnan(x))
        return 0x7FC0;
    double ax = fabs(x);
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (ax == 0.0)
        return sign;
    int e;
    frexp(ax, &e);          /* ax = f * 2^e, f in [0.5, 1) */
    int ulp_exp = (e - 1) - 7;
    if (ulp_exp < -133)
        ulp_exp = -133;
    double q = ldexp(ax, -ulp_exp);   /* exact: power-of-two scaling */
    double r = nearbyint(q);          /* default mode: ties to even */
    double y = ldexp(r, ulp_exp);
    if (y >= 0x1p128)                 /* rounds past the largest finite */
        return sign | 0x7F80;
    float f = (float)y;               /* exact: y has <= 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return sign | (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------------- score */

/* One score row: out[s] for s = 0..n-1 (n = p+1 causal keys).
 * q: bf16 bits [H][D]; w: [H]; keys: [n][D] bf16 bits (key_fp8 = 0) or fp8
 * bytes with a per-key scale (key_fp8 = 1), row stride k_ld elements. */
/* Query rows come as bf16, or as fp8 e4m3 with one positive scale per head
 * (q_scale[h]); either way each element is decoded exactly and an fp8 query
 * element stands for fp8 value * scale, the same reading as an fp8 key. */
void oracle_score_row(const void *q, const float *q_scale, int q_fp8,
                      const float *w, const void *keys,
                      const float *k_scale, int key_fp8, int64_t k_ld, int H,
                      int D, int64_t n, float *out)
{
    double *qd = malloc(sizeof(double) * (size_t)H * D);
    double *kd = malloc(sizeof(double) * (size_t)D);
    for (int i = 0; i < H * D; i++)
        qd[i] = q_fp8 ? oracle_fp8e4m3_to_double(((const uint8_t *)q)[i]) * (double)q_scale[i / D]
                      : oracle_bf16_to_double(((const uint16_t *)q)[i]);
    for (int64_t s = 0; s < n; s++) {
        for (int d = 0; d < D; d++) {
            if (key_fp8) {
                const uint8_t *kr = (const uint8_t *)keys + s * k_ld;
                kd[d] = oracle_fp8e4m3_to_double(kr[d]) * (double)k_scale[s];
            } else {
                const uint16_t *kr = (const uint16_t *)keys + s * k_ld;
                kd[d] = oracle_bf16_to_double(kr[d]);
            }
        }
        double score = 0.0;
        for (int h = 0; h < H; h++) {
            double dot = 0.0;
            for (int d = 0; d < D; d++)
                dot += qd[h * D + d] * kd[d];
            double relu = dot > 0.0 ? dot : 0.0;
            score += (double)w[h] * relu;
        }
        float f = (float)score;
        if (f == 0.0f)
            f = 0.0f; /* store +0 for a -0 result */
        out[s] = f;
    }
    free(qd);
    free(kd);
}

/* ------------------------------------------------------------------ select */

typedef struct {
    float v;
    int32_t i;
} scored_t;

/* Larger value first; equal values (and +0 against -0) by lower index. */
static int cmp_desc_value_asc_index(const void *a, const void *b)
{
    const scored_t *x = a, *y = b;
    if (x->v > y->v)
        return -1;
    if (x->v < y->v)
        return 1;
    return (x->i > y->i) - (x->i < y->i);
}

static int cmp_i32(const void *a, const void *b)
{
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

/* Top-k of one row of n scores: the min(k, n) positions with the largest
 * scores, ties to the lower position, returned in ascending position order
 * and padded with -1 up to k entries. */
void oracle_select_row(const float *s, int64_t n, int k, int32_t *out)
{
    scored_t *a = malloc(sizeof(scored_t) * (size_t)(n > 0 ? n : 1));
    for (int64_t i = 0; i < n; i++) {
        a[i].v = s[i];
        a[i].i = (int32_t)i;
    }
    qsort(a, (size_t)n, sizeof(scored_t), cmp_desc_value_asc_index);
    int64_t m = n < k ? n : k;
    for (int64_t j = 0; j < m; j++)
        out[j] = a[j].i;
    qsort(out, (size_t)m, sizeof(int32_t), cmp_i32);
    for (int64_t j = m; j < k; j++)
        out[j] = -1;
    free(a);
}

/* --------------------------------------------------------------- attention */

/* Softmax attention of H query heads over the rows listed in idx[0..k-1]
 * (negative entries skipped).  q: bf16 bits [H][Dqk]; K rows of Dqk bf16 and
 * V rows of Dv bf16 with row strides k_ld / v_ld elements; out: bf16 bits
 * [H][Dv].  A row with no valid index yields zeros. */
void oracle_attn_row(const uint16_t *q, const uint16_t *K, int64_t k_ld,
                     const uint16_t *V, int64_t v_ld, const int32_t *idx, int k,
                     int H, int Dqk, int Dv, double tau, uint16_t *out)
{
    double *logit = malloc(sizeof(double) * (size_t)k);
    double *acc = malloc(sizeof(double) * (size_t)Dv);
    for (int h = 0; h < H; h++) {
        const uint16_t *qh = q + (size_t)h * Dqk;
        double mx = -INFINITY;
        int valid = 0;
        for (int j = 0; j < k; j++) {
            if (idx[j] < 0)
                continue;
            const uint16_t *kr = K + (int64_t)idx[j] * k_ld;
            double dot = 0.0;
            for (int d = 0; d < Dqk; d++)
                dot += oracle_bf16_to_double(qh[d]) * oracle_bf16_to_double(kr[d]);
            logit[j] = tau * dot;
            if (logit[j] > mx)
                mx = logit[j];
            valid++;
        }
        for (int d = 0; d < Dv; d++)
            acc[d] = 0.0;
        double denom = 0.0;
        for (int j = 0; j < k && valid; j++) {
            if (idx[j] < 0)
                continue;
            double p = exp(logit[j] - mx);
            denom += p;
            const uint16_t *vr = V + (int64_t)idx[j] * v_ld;
            for (int d = 0; d < Dv; d++)
                acc[d] += p * oracle_bf16_to_double(vr[d]);
        }
        for (int d = 0; d < Dv; d++)
            out[(size_t)h * Dv + d] = oracle_double_to_bf16(valid ? acc[d] / denom : 0.0);
    }
    free(logit);
    free(acc);
}

/* ------------------------------------------------- multi-row, multi-thread */
/* Rows are independent; each row is computed by one thread exactly as above.
 * Threading changes no arithmetic. */

typedef struct {
    int n_rows;
    const int64_t *pos;      /* [n_rows] absolute position p of each row */
    const void *q_rows;      /* [n_rows][H][D] bf16 bits, or fp8 bytes */
    const float *q_scale;    /* [n_rows][H] when q_fp8, else NULL */
    int q_fp8;
    const float *w_rows;     /* [n_rows][H] */
    const void *keys;        /* [>= max p + 1][k_ld] */
    const float *k_scale;
    int key_fp8;
    int64_t k_ld;
    int H, D, top_k;
    float *scores;           /* [n_rows][s_ld] or NULL */
    int64_t s_ld;
    int32_t *idx;            /* [n_rows][top_k] or NULL */
    int next;                /* shared row counter */
    pthread_mutex_t lock;
} score_job_t;

static int take_row(pthread_mutex_t *lock, int *next, int n)
{
    pthread_mutex_lock(lock);
    int r = *next < n ? (*next)++ : -1;
    pthread_mutex_unlock(lock);
    return r;
}

static void *score_worker(void *arg)
{
    score_job_t *j = arg;
    int64_t maxn = 0;
    for (int r = 0; r < j->n_rows; r++)
        if (j->pos[r] + 1 > maxn)
            maxn = j->pos[r] + 1;
    float *tmp = j->scores ? NULL : malloc(sizeof(float) * (size_t)maxn);
    for (;;) {
        int r = take_row(&j->lock, &j->next, j->n_rows);
        if (r < 0)
            break;
        int64_t n = j->pos[r] + 1;
        float *s = j->scores ? j->scores + (int64_t)r * j->s_ld : tmp;
        const size_t qel = (size_t)r * j->H * j->D;
        oracle_score_row(j->q_fp8 ? (const void *)((const uint8_t *)j->q_rows + qel)
                                  : (const void *)((const uint16_t *)j->q_rows + qel),
                         j->q_fp8 ? j->q_scale + (size_t)r * j->H : NULL, j->q_fp8,
                         j->w_rows + (size_t)r * j->H, j->keys, j->k_scale,
                         j->key_fp8, j->k_ld, j->H, j->D, n, s);
        if (j->idx)
            oracle_select_row(s, n, j->top_k, j->idx + (int64_t)r * j->top_k);
    }
    free(tmp);
    return NULL;
}

static void run_threads(void *(*fn)(void *), void *job, int threads)
{
    if (threads < 1)
        threads = 1;
    pthread_t *t = malloc(sizeof(pthread_t) * (size_t)threads);
    for (int i = 0; i < threads; i++)
        pthread_create(&t[i], NULL, fn, job);
    for (int i = 0; i < threads; i++)
        pthread_join(t[i], NULL);
    free(t);
}

/* Score (and optionally select) a list of rows that share one key array.
 * scores may be NULL (then only idx is produced); idx may be NULL. */
int oracle_score_select_rows(int n_rows, const int64_t *pos,
                             const void *q_rows, const float *q_scale, int q_fp8,
                             const float *w_rows,
                             const void *keys, const float *k_scale,
                             int key_fp8, int64_t k_ld, int H, int D, int top_k,
                             float *scores, int64_t s_ld, int32_t *idx,
                             int threads)
{
    score_job_t j = {n_rows, pos, q_rows, q_scale, q_fp8, w_rows, keys, k_scale, key_fp8,
                     k_ld, H, D, top_k, scores, s_ld, idx, 0,
                     PTHREAD_MUTEX_INITIALIZER};
    run_threads(score_worker, &j, threads);
    return 0;
}

typedef struct {
    int n_rows;
    const float *scores;     /* [n_rows][s_ld] */
    int64_t s_ld;
    const int64_t *n;        /* [n_rows] row lengths */
    int top_k;
    int32_t *idx;            /* [n_rows][top_k] */
    int next;
    pthread_mutex_t lock;
} select_job_t;

static void *select_worker(void *arg)
{
    select_job_t *j = arg;
    for (;;) {
        int r = take_row(&j->lock, &j->next, j->n_rows);
        if (r < 0)
            break;
        oracle_select_row(j->scores + (int64_t)r * j->s_ld, j->n[r], j->top_k,
                          j->idx + (int64_t)r * j->top_k);
    }
    return NULL;
}

/* Select on given score rows (row r has n[r] valid entries). */
int oracle_select_rows(int n_rows, const float *scores, int64_t s_ld,
                       const int64_t *n, int top_k, int32_t *idx, int threads)
{
    select_job_t j = {n_rows, scores, s_ld, n, top_k, idx, 0,
                      PTHREAD_MUTEX_INITIALIZER};
    run_threads(select_worker, &j, threads);
    return 0;
}

typedef struct {
    int n_rows;
    const uint16_t *q_rows;  /* [n_rows][H][Dqk] */
    const uint16_t *K;
    int64_t k_ld;
    const uint16_t *V;
    int64_t v_ld;
    const int32_t *idx;      /* [n_rows][top_k] */
    int top_k, H, Dqk, Dv;
    double tau;
    uint16_t *out;           /* [n_rows][H][Dv] */
    int next;
    pthread_mutex_t lock;
} attn_job_t;

static void *attn_worker(void *arg)
{
    attn_job_t *j = arg;
    for (;;) {
        int r = take_row(&j->lock, &j->next, j->n_rows);
        if (r < 0)
            break;
        oracle_attn_row(j->q_rows + (size_t)r * j->H * j->Dqk, j->K, j->k_ld,
                        j->V, j->v_ld, j->idx + (int64_t)r * j->top_k, j->top_k,
                        j->H, j->Dqk, j->Dv, j->tau,
                        j->out + (size_t)r * j->H * j->Dv);
    }
    return NULL;
}

/* Sparse attention for a list of rows that share one K/V array. */
int oracle_attn_rows(int n_rows, const uint16_t *q_rows, const uint16_t *K,
                     int64_t k_ld, const uint16_t *V, int64_t v_ld,
                     const int32_t *idx, int top_k, int H, int Dqk, int Dv,
                     double tau, uint16_t *out, int threads)
{
    attn_job_t j = {n_rows, q_rows, K, k_ld, V, v_ld, idx, top_k, H, Dqk, Dv,
                    tau, out, 0, PTHREAD_MUTEX_INITIALIZER};
    run_threads(attn_worker, &j, threads);
    return 0;
}
