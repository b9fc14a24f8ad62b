/*
 * attention_grad_oracle.c -- plain, slow fp64 CPU oracle of the gradients of
 * attention (the backward pass).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library calls, links or loads
 * this file; only the tests and the benchmark's CPU-baseline leg do.  It shares
 * no code, header or constant with the GPU path.
 *
 * The pages name the backward pass without spelling it out: standard attention
 * keeps the score and probability matrices for the gradient computation
 * ("FlashAttention 在昇腾 NPU 上是怎么省显存的？", the section on what goes wrong
 * with the standard implementation), the v2 operator improves that gradient
 * computation (same page, v1 versus v2), and the training speed-ups reported for
 * FlashAttention need it ("FlashAttention (VI)", experimental results).  What is
 * computed here is therefore the derivative of the definition
 *
 *   O = softmax(S) V,   S = scale * Q K^T   (masked entries: -inf)
 *       -- "FlashAttention (VI)", equation Attention --
 *
 * for a loss L with dL/dO = dO, written out by the chain rule, one query row at
 * a time (P_i = the softmax row, materialised over all visible keys):
 *
 *   dV_j  += P_ij dO_i                                  (O_i = sum_j P_ij V_j)
 *   dP_ij  = dO_i . V_j
 *   dS_ij  = P_ij (dP_ij - sum_k P_ik dP_ik)            (softmax Jacobian)
 *   dQ_i   = scale * sum_j dS_ij K_j
 *   dK_j  += scale * dS_ij Q_i
 *
 * Causal masking and grouped-query heads as in the forward oracle: key j is
 * visible to query i iff j <= i; query head h uses key/value head h / (Hq/Hkv),
 * so dK and dV of a key/value head sum over its Hq/Hkv query heads.
 *
 * Layouts: q, dout, dq are [B,Hq,N,d]; k, v, dk, dv are [B,Hkv,N,d]; all fp64,
 * contiguous, d innermost.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

typedef struct {
    const double *q, *k, *v, *dout;
    double *dq, *dk, *dv;
    int64_t B, Hq, Hkv, N, d;
    int causal;
    double scale;
    int64_t next;
    int failed;
    pthread_mutex_t mu;
} grad_job;

/* One (b, key/value head): every query row of every query head of its group. */
static int grad_unit(const grad_job *J, int64_t unit, double *p, double *dp)
{
    const int64_t b = unit / J->Hkv, hk = unit % J->Hkv;
    const int64_t G = J->Hq / J->Hkv, N = J->N, d = J->d;
    const double *kh = J->k + (b * J->Hkv + hk) * N * d;
    const double *vh = J->v + (b * J->Hkv + hk) * N * d;
    double *dkh = J->dk + (b * J->Hkv + hk) * N * d;
    double *dvh = J->dv + (b * J->Hkv + hk) * N * d;
    memset(dkh, 0, (size_t)(N * d) * sizeof(double));
    memset(dvh, 0, (size_t)(N * d) * sizeof(double));

    for (int64_t h = hk * G; h < (hk + 1) * G; ++h) {
        const double *qh = J->q + (b * J->Hq + h) * N * d;
        const double *gh = J->dout + (b * J->Hq + h) * N * d;
        double *dqh = J->dq + (b * J->Hq + h) * N * d;
        for (int64_t i = 0; i < N; ++i) {
            const int64_t jend = J->causal ? i + 1 : N;
            const double *qi = qh + i * d, *gi = gh + i * d;

            /* The softmax row P_i: scores, maximum, exponentials, normalisation. */
            double m = -INFINITY;
            for (int64_t j = 0; j < jend; ++j) {
                double acc = 0.0;
                for (int64_t t = 0; t < d; ++t)
                    acc += qi[t] * kh[j * d + t];
                p[j] = J->scale * acc;
                if (p[j] > m)
                    m = p[j];
            }
            double l = 0.0;
            for (int64_t j = 0; j < jend; ++j) {
                p[j] = exp(p[j] - m);
                l += p[j];
            }
            for (int64_t j = 0; j < jend; ++j)
                p[j] /= l;

            /* dP_ij = dO_i . V_j, and the row term sum_k P_ik dP_ik. */
            double pdp = 0.0;
            for (int64_t j = 0; j < jend; ++j) {
                double acc = 0.0;
                for (int64_t t = 0; t < d; ++t)
                    acc += gi[t] * vh[j * d + t];
                dp[j] = acc;
                pdp += p[j] * acc;
            }

            double *dqi = dqh + i * d;
            for (int64_t t = 0; t < d; ++t)
                dqi[t] = 0.0;
            for (int64_t j = 0; j < jend; ++j) {
                const double ds = p[j] * (dp[j] - pdp);
                for (int64_t t = 0; t < d; ++t) {
                    dqi[t] += J->scale * ds * kh[j * d + t];
                    dkh[j * d + t] += J->scale * ds * qi[t];
                    dvh[j * d + t] += p[j] * gi[t];
                }
            }
        }
    }
    return 0;
}

static void *grad_worker(void *arg)
{
    grad_job *J = (grad_job *)arg;
    double *p = (double *)malloc((size_t)J->N * sizeof(double));
    double *dp = (double *)malloc((size_t)J->N * sizeof(double));
    if (!p || !dp) {
        pthread_mutex_lock(&J->mu);
        J->failed = 1;
        pthread_mutex_unlock(&J->mu);
        free(p);
        free(dp);
        return NULL;
    }
    const int64_t units = J->B * J->Hkv;
    for (;;) {
        pthread_mutex_lock(&J->mu);
        const int64_t u = J->failed ? units : J->next++;
        pthread_mutex_unlock(&J->mu);
        if (u >= units)
            break;
        grad_unit(J, u, p, dp);
    }
    free(p);
    free(dp);
    return NULL;
}

/* Returns 0, or -2 for bad sizes, -3 when memory runs out. */
int oracle_attention_bwd(const double *q, const double *k, const double *v,
                         const double *dout, double *dq, double *dk, double *dv,
                         int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                         int causal, double scale, int threads)
{
    if (B < 1 || Hq < 1 || Hkv < 1 || N < 1 || d < 1 || Hq % Hkv != 0)
        return -2;
    grad_job J = {q, k, v, dout, dq, dk, dv, B, Hq, Hkv, N, d, causal, scale, 0, 0};
    pthread_mutex_init(&J.mu, NULL);
    if (threads <= 0)
        threads = (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (threads > B * Hkv)
        threads = (int)(B * Hkv);
    if (threads < 1)
        threads = 1;
    pthread_t *tid = (pthread_t *)calloc((size_t)threads, sizeof(pthread_t));
    if (!tid)
        return -3;
    int started = 0;
    for (int t = 1; t < threads; ++t) {
        if (pthread_create(&tid[t], NULL, grad_worker, &J) != 0)
            break;
        ++started;
    }
    grad_worker(&J);
    for (int t = 1; t <= started; ++t)
        pthread_join(tid[t], NULL);
    free(tid);
    pthread_mutex_destroy(&J.mu);
    return J.failed ? -3 : 0;
}
