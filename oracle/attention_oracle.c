/*
 * attention_oracle.c -- plain, slow fp64 CPU oracle of the attention forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library calls, links or loads
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline leg
 * do.  It shares no code, header or constant with the GPU path.
 *
 * What it computes is the plain definition, written out:
 *
 *   Attention(Q,K,V) = softmax(Q K^T * scale) V
 *       -- "FlashAttention (VI)", section "Vấn đề của cơ chế attention tiêu chuẩn",
 *          equation Attention (scale = 1/sqrt(d_k) there; here the caller passes it).
 *
 * following the standard path of "MCU 上 Transformer 模型的 Flash Attention 实现…"
 * §一 (Q x K^T gives an [N,N] score matrix, which then multiplies V) and the
 * two-pass softmax of its §二, first paragraph (pass 1: the row maximum; pass 2:
 * the sum of exp(x - max)).  Scores are materialised for a block of query rows
 * at a time, each row holding all N columns; rows are independent, so the result
 * does not depend on the block size.
 *
 * Readings where the pages are silent:
 *   - causal: key j is visible to query i iff j <= i ("FlashAttention 在昇腾 NPU 上…",
 *     pitfall 1: a generation model must not see the future);
 *   - grouped-query heads: query head h reads key/value head h / (Hq/Hkv), so each
 *     key/value head serves Hq/Hkv consecutive query heads ("深度探索Flash-Attention中
 *     GQA性能调优技术解析", GQA mechanism);
 *   - lse[b,h,i] = m_i + ln(l_i), natural log, in units of scaled scores.
 *
 * With an additive bias (a fused-operator variant: "深度探索Flash-Attention中GQA性能
 * 调优技术解析" and the FlashAttention-3 feature list of "FlashAttention (VI)"), the
 * scores are s_ij = scale * q_i.k_j + bias[b,h,i,j]; a bias of -inf masks the pair.
 * A row whose every score is -inf attends to nothing: o = 0, lse = -inf.
 *
 * Layouts: q, o are [B,Hq,N,d]; k, v are [B,Hkv,N,d]; lse is [B,Hq,N]; all fp64,
 * contiguous, d innermost.  With a row list, o and lse hold only those rows, in
 * list order: o is [B,Hq,nrows,d], lse is [B,Hq,nrows].
 *
 * Queries against a longer key/value sequence (decoding with a key/value cache,
 * oracle_attention_fwd_kv): q, o are [B,Hq,Nq,d], k, v are [B,Hkv,Nk,d], Nq <= Nk
 * when causal.  Reading (the pages only treat square causal attention): the Nq
 * queries are the last Nq of the Nk positions, so query i sees keys
 * j <= i + (Nk - Nq); for Nq = Nk this is the square rule j <= i.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

typedef struct {
    const double *q, *k, *v;
    double *o, *lse, *probs;
    int64_t B, Hq, Hkv, N, d;  /* N: query rows per head                            */
    int64_t Nk;                /* key/value rows per head (N for square attention)  */
    int causal;
    double scale;
    const double *bias;    /* optional additive bias, element (b,h,i,j) at       */
    int64_t sb, sh, si;    /* b*sb + h*sh + i*si + j (strides may be 0)         */
    const int64_t *rows;   /* query rows computed for every (b, h); NULL = all   */
    int64_t nrows;         /* length of the row list (N when rows == NULL)       */
    int64_t chunk;         /* rows per work unit                                 */
    int64_t units_per_bh;
    int64_t nunits;
    int64_t next;
    int failed;
    pthread_mutex_t mu;
} oracle_job;

static int64_t row_index(const oracle_job *J, int64_t r)
{
    return J->rows ? J->rows[r] : r;
}

/* One work unit: query rows [r0, r1) of the row list, for one (b, h). */
static void run_unit(const oracle_job *J, int64_t unit, double *S)
{
    const int64_t bh = unit / J->units_per_bh;
    const int64_t b = bh / J->Hq, h = bh % J->Hq;
    const int64_t group = J->Hq / J->Hkv;
    const int64_t hk = h / group;
    const int64_t N = J->N, Nk = J->Nk, d = J->d;
    const int64_t r0 = (unit % J->units_per_bh) * J->chunk;
    const int64_t r1 = (r0 + J->chunk < J->nrows) ? r0 + J->chunk : J->nrows;

    const double *qh = J->q + (b * J->Hq + h) * N * d;
    const double *kh = J->k + (b * J->Hkv + hk) * Nk * d;
    const double *vh = J->v + (b * J->Hkv + hk) * Nk * d;

    for (int64_t r = r0; r < r1; ++r) {
        const int64_t i = row_index(J, r);
        /* Visible keys: j < jend (query i is position i + Nk - N of the keys). */
        const int64_t jend = J->causal ? i + 1 + (Nk - N) : Nk;
        double *s = S + (r - r0) * Nk;
        const double *qi = qh + i * d;

        /* Scores s_ij = scale * sum_t q_it k_jt (+ bias), the full row materialised. */
        const double *brow = J->bias ? J->bias + b * J->sb + h * J->sh + i * J->si : NULL;
        for (int64_t j = 0; j < jend; ++j) {
            const double *kj = kh + j * d;
            double acc = 0.0;
            for (int64_t t = 0; t < d; ++t)
                acc += qi[t] * kj[t];
            s[j] = J->scale * acc;
            if (brow)
                s[j] += brow[j];
        }

        /* Pass 1: the row maximum over the visible keys. */
        double m = -INFINITY;
        for (int64_t j = 0; j < jend; ++j)
            if (s[j] > m)
                m = s[j];

        /* Pass 2: e_ij = exp(s_ij - m_i), l_i = sum_j e_ij; then P_ij = e_ij / l_i.
         * A row with no finite score (only possible with a bias) has P = 0. */
        double l = 0.0;
        for (int64_t j = 0; j < jend; ++j) {
            s[j] = m == -INFINITY ? 0.0 : exp(s[j] - m);
            l += s[j];
        }
        for (int64_t j = 0; j < jend; ++j)
            s[j] = l > 0.0 ? s[j] / l : 0.0;

        /* O_i = sum_j P_ij v_j. */
        double *oi = J->o ? J->o + (bh * J->nrows + r) * d : NULL;
        if (oi) {
            for (int64_t t = 0; t < d; ++t)
                oi[t] = 0.0;
            for (int64_t j = 0; j < jend; ++j) {
                const double *vj = vh + j * d;
                for (int64_t t = 0; t < d; ++t)
                    oi[t] += s[j] * vj[t];
            }
        }
        if (J->lse)
            J->lse[bh * J->nrows + r] = l > 0.0 ? m + log(l) : -INFINITY;
        if (J->probs) {
            double *pr = J->probs + (bh * J->nrows + r) * Nk;
            for (int64_t j = 0; j < Nk; ++j)
                pr[j] = j < jend ? s[j] : 0.0;
        }
    }
}

static void *worker(void *arg)
{
    oracle_job *J = (oracle_job *)arg;
    double *S = (double *)malloc((size_t)(J->chunk * J->Nk) * sizeof(double));
    if (!S) {
        pthread_mutex_lock(&J->mu);
        J->failed = 1;
        pthread_mutex_unlock(&J->mu);
        return NULL;
    }
    for (;;) {
        pthread_mutex_lock(&J->mu);
        const int64_t u = J->failed ? J->nunits : J->next++;
        pthread_mutex_unlock(&J->mu);
        if (u >= J->nunits)
            break;
        run_unit(J, u, S);
    }
    free(S);
    return NULL;
}

static int run_job(oracle_job *J, int threads)
{
    if (threads <= 0)
        threads = (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (threads < 1)
        threads = 1;

    /* Rows per work unit: enough units to keep every thread busy (about four per
     * thread), and each thread's score block at or below 64 MB. */
    const int64_t heads = J->B * J->Hq;
    const int64_t want = (4LL * threads + heads - 1) / heads;
    int64_t chunk = (J->nrows + want - 1) / want;
    const int64_t cap = (64LL << 20) / (8 * J->Nk);
    if (chunk > cap)
        chunk = cap;
    if (chunk < 1)
        chunk = 1;
    J->chunk = chunk;
    J->units_per_bh = (J->nrows + chunk - 1) / chunk;
    J->nunits = heads * J->units_per_bh;
    J->next = 0;
    J->failed = 0;
    pthread_mutex_init(&J->mu, NULL);

    if (threads > J->nunits)
        threads = (int)J->nunits;

    pthread_t *tid = (pthread_t *)calloc((size_t)threads, sizeof(pthread_t));
    if (!tid)
        return -3;
    int started = 0;
    for (int t = 1; t < threads; ++t) {
        if (pthread_create(&tid[t], NULL, worker, J) != 0)
            break;
        ++started;
    }
    worker(J);
    for (int t = 1; t <= started; ++t)
        pthread_join(tid[t], NULL);
    free(tid);
    pthread_mutex_destroy(&J->mu);
    return J->failed ? -3 : 0;
}

static int check_args(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                      const int64_t *rows, int64_t nrows)
{
    if (B < 1 || Hq < 1 || Hkv < 1 || N < 1 || d < 1 || Hq % Hkv != 0)
        return -2;
    if (rows) {
        if (nrows < 1)
            return -2;
        for (int64_t r = 0; r < nrows; ++r)
            if (rows[r] < 0 || rows[r] >= N)
                return -2;
    }
    return 0;
}

/*
 * o and lse for every (b, h) and every query row in `rows` (all N rows when rows
 * is NULL).  Either output may be NULL.  Returns 0, -1 on a NULL input, -2 on a bad
 * shape or row index, -3 when memory or threads cannot be had.  threads <= 0 uses
 * every online CPU.
 */
int oracle_attention_fwd(const double *q, const double *k, const double *v,
                         double *o, double *lse,
                         int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                         int causal, double scale,
                         const int64_t *rows, int64_t nrows, int threads)
{
    if (!q || !k || !v)
        return -1;
    if (!rows)
        nrows = N;
    int rc = check_args(B, Hq, Hkv, N, d, rows, nrows);
    if (rc)
        return rc;
    oracle_job J;
    memset(&J, 0, sizeof(J));
    J.q = q; J.k = k; J.v = v; J.o = o; J.lse = lse; J.probs = NULL;
    J.B = B; J.Hq = Hq; J.Hkv = Hkv; J.N = N; J.Nk = N; J.d = d;
    J.causal = causal != 0;
    J.scale = scale;
    J.rows = rows;
    J.nrows = nrows;
    return run_job(&J, threads);
}

/*
 * The softmax matrix P itself, [B,Hq,N,N] (zeros where a key is masked), for small
 * problems.  Same arithmetic as oracle_attention_fwd.
 */
int oracle_attention_probs(const double *q, const double *k, double *probs,
                           int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                           int causal, double scale)
{
    if (!q || !k || !probs)
        return -1;
    int rc = check_args(B, Hq, Hkv, N, d, NULL, N);
    if (rc)
        return rc;
    oracle_job J;
    memset(&J, 0, sizeof(J));
    J.q = q; J.k = k; J.v = k; J.o = NULL; J.lse = NULL; J.probs = probs;
    J.B = B; J.Hq = Hq; J.Hkv = Hkv; J.N = N; J.Nk = N; J.d = d;
    J.causal = causal != 0;
    J.scale = scale;
    J.rows = NULL;
    J.nrows = N;
    return run_job(&J, 1);
}

/*
 * As oracle_attention_fwd, with an additive bias on the scaled scores: element
 * (b, h, i, j) of the fp64 array `bias` sits at b*sb + h*sh + i*si + j.
 */
int oracle_attention_fwd_bias(const double *q, const double *k, const double *v,
                              const double *bias, int64_t sb, int64_t sh, int64_t si,
                              double *o, double *lse,
                              int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                              int causal, double scale, int threads)
{
    if (!q || !k || !v || !bias)
        return -1;
    int rc = check_args(B, Hq, Hkv, N, d, NULL, N);
    if (rc)
        return rc;
    oracle_job J;
    memset(&J, 0, sizeof(J));
    J.q = q; J.k = k; J.v = v; J.o = o; J.lse = lse; J.probs = NULL;
    J.bias = bias; J.sb = sb; J.sh = sh; J.si = si;
    J.B = B; J.Hq = Hq; J.Hkv = Hkv; J.N = N; J.Nk = N; J.d = d;
    J.causal = causal != 0;
    J.scale = scale;
    J.rows = NULL;
    J.nrows = N;
    return run_job(&J, threads);
}

/*
 * Queries against a key/value sequence of another length (see the header): q, o
 * [B,Hq,Nq,d], k, v [B,Hkv,Nk,d], lse [B,Hq,Nq]; causal requires Nq <= Nk.  Returns
 * as oracle_attention_fwd.
 */
int oracle_attention_fwd_kv(const double *q, const double *k, const double *v,
                            double *o, double *lse,
                            int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d,
                            int causal, double scale, int threads)
{
    if (!q || !k || !v)
        return -1;
    int rc = check_args(B, Hq, Hkv, Nq, d, NULL, Nq);
    if (rc)
        return rc;
    if (Nk < 1 || (causal && Nq > Nk))
        return -2;
    oracle_job J;
    memset(&J, 0, sizeof(J));
    J.q = q; J.k = k; J.v = v; J.o = o; J.lse = lse; J.probs = NULL;
    J.B = B; J.Hq = Hq; J.Hkv = Hkv; J.N = Nq; J.Nk = Nk; J.d = d;
    J.causal = causal != 0;
    J.scale = scale;
    J.rows = NULL;
    J.nrows = Nq;
    return run_job(&J, threads);
}
