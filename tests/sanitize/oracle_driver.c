/*
 * Drives every function of the fp64 oracle on small inputs, for a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer: any out-of-bounds access, use of
 * freed memory or undefined arithmetic aborts the run.  The results are checked
 * only loosely (finite values, rows of P summing to 1, the blocked reference
 * agreeing with the two-pass one); the oracle's real pins are the Python tests.
 * Exit status 0 means every call ran clean.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_attention_fwd(const double *q, const double *k, const double *v, double *o, double *lse,
                         int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int causal,
                         double scale, const int64_t *rows, int64_t nrows, int threads);
int oracle_attention_probs(const double *q, const double *k, double *probs, int64_t B, int64_t Hq,
                           int64_t Hkv, int64_t N, int64_t d, int causal, double scale);
int oracle_attention_fwd_bias(const double *q, const double *k, const double *v, const double *bias,
                              int64_t sb, int64_t sh, int64_t si, double *o, double *lse,
                              int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int causal,
                              double scale, int threads);
int oracle_attention_fwd_kv(const double *q, const double *k, const double *v, double *o,
                            double *lse, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk,
                            int64_t d, int causal, double scale, int threads);
int oracle_attention_bwd(const double *q, const double *k, const double *v, const double *dout,
                         double *dq, double *dk, double *dv, int64_t B, int64_t Hq, int64_t Hkv,
                         int64_t N, int64_t d, int causal, double scale, int threads);
int blocked_attention_fwd(const double *q, const double *k, const double *v, double *o, double *lse,
                          int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int causal,
                          double scale, int64_t Br, int64_t Bc);

static uint64_t state = 12345;
static double uniform_pm1(void)     /* a small LCG: inputs only */
{
    state = state * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(state >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}

static double *fill(size_t n)
{
    double *a = (double *)malloc(n * sizeof(double));
    for (size_t i = 0; i < n; ++i)
        a[i] = uniform_pm1();
    return a;
}

static int failures = 0;
#define CHECK(cond, what)                                                   \
    do {                                                                    \
        if (!(cond)) {                                                      \
            fprintf(stderr, "check failed: %s (line %d)\n", what, __LINE__); \
            ++failures;                                                     \
        }                                                                   \
    } while (0)

static int all_finite(const double *a, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(a[i]))
            return 0;
    return 1;
}

int main(void)
{
    const int64_t shapes[][5] = {{1, 1, 1, 1, 8}, {1, 2, 1, 7, 16}, {2, 4, 2, 33, 32}, {1, 3, 3, 64, 64}};
    for (size_t s = 0; s < sizeof(shapes) / sizeof(shapes[0]); ++s) {
        const int64_t B = shapes[s][0], Hq = shapes[s][1], Hkv = shapes[s][2], N = shapes[s][3],
                      d = shapes[s][4];
        const size_t nq = (size_t)(B * Hq * N * d), nkv = (size_t)(B * Hkv * N * d);
        double *q = fill(nq), *k = fill(nkv), *v = fill(nkv), *g = fill(nq);
        double *o = malloc(nq * sizeof(double)), *o2 = malloc(nq * sizeof(double));
        double *lse = malloc((size_t)(B * Hq * N) * sizeof(double));
        double *lse2 = malloc((size_t)(B * Hq * N) * sizeof(double));
        double *p = malloc((size_t)(B * Hq * N * N) * sizeof(double));
        double *dq = malloc(nq * sizeof(double)), *dk = malloc(nkv * sizeof(double)),
               *dv = malloc(nkv * sizeof(double));
        for (int causal = 0; causal < 2; ++causal) {
            CHECK(oracle_attention_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, 0.3, NULL, 0, 3) == 0, "fwd");
            CHECK(all_finite(o, nq) && all_finite(lse, (size_t)(B * Hq * N)), "fwd finite");
            CHECK(blocked_attention_fwd(q, k, v, o2, lse2, B, Hq, Hkv, N, d, causal, 0.3, 5, 3) == 0, "blocked");
            double worst = 0.0;
            for (size_t i = 0; i < nq; ++i)
                worst = fmax(worst, fabs(o[i] - o2[i]));
            CHECK(worst <= 1e-12, "blocked agrees");
            /* A row subset: outputs are compact, [B, Hq, nrows, d] and [B, Hq, nrows]. */
            const int64_t rows[3] = {0, N / 2, N - 1};
            double *or_ = malloc((size_t)(B * Hq * 3 * d) * sizeof(double));
            double *lr = malloc((size_t)(B * Hq * 3) * sizeof(double));
            CHECK(oracle_attention_fwd(q, k, v, or_, lr, B, Hq, Hkv, N, d, causal, 0.3, rows, 3, 2) == 0, "rows");
            for (int64_t bh = 0; bh < B * Hq; ++bh)
                for (int r = 0; r < 3; ++r)
                    CHECK(lr[bh * 3 + r] == lse[bh * N + rows[r]], "row subset equals the full run");
            free(or_);
            free(lr);
            CHECK(oracle_attention_probs(q, k, p, B, Hq, Hkv, N, d, causal, 0.3) == 0, "probs");
            for (int64_t r = 0; r < B * Hq * N; ++r) {
                double sum = 0.0;
                for (int64_t j = 0; j < N; ++j)
                    sum += p[r * N + j];
                CHECK(fabs(sum - 1.0) <= 1e-12, "probability rows sum to 1");
            }
            CHECK(oracle_attention_bwd(q, k, v, g, dq, dk, dv, B, Hq, Hkv, N, d, causal, 0.3, 3) == 0, "bwd");
            CHECK(all_finite(dq, nq) && all_finite(dk, nkv) && all_finite(dv, nkv), "bwd finite");
            /* An additive bias with a masked pair per row (never the diagonal). */
            double *bias = fill((size_t)(Hq * N * N));
            for (int64_t h = 0; h < Hq; ++h)
                for (int64_t i = 0; i < N; ++i)
                    if (i > 0)
                        bias[(h * N + i) * N + (i - 1)] = -INFINITY;
            CHECK(oracle_attention_fwd_bias(q, k, v, bias, 0, N * N, N, o, lse, B, Hq, Hkv, N, d, causal,
                                            0.3, 2) == 0, "bias");
            CHECK(all_finite(o, nq), "bias finite");
            free(bias);
            /* Queries against a longer key sequence: the last rows of q. */
            if (N >= 2) {
                const int64_t nq2 = N / 2;
                double *qs = fill((size_t)(B * Hq * nq2 * d));
                double *os = malloc((size_t)(B * Hq * nq2 * d) * sizeof(double));
                double *ls = malloc((size_t)(B * Hq * nq2) * sizeof(double));
                CHECK(oracle_attention_fwd_kv(qs, k, v, os, ls, B, Hq, Hkv, nq2, N, d, causal, 0.3, 2) == 0, "kv");
                CHECK(all_finite(os, (size_t)(B * Hq * nq2 * d)), "kv finite");
                free(qs); free(os); free(ls);
            }
        }
        /* Rejections. */
        CHECK(oracle_attention_fwd(NULL, k, v, o, lse, B, Hq, Hkv, N, d, 0, 0.3, NULL, 0, 1) < 0, "null");
        CHECK(oracle_attention_fwd(q, k, v, o, lse, B, 3, 2, N, d, 0, 0.3, NULL, 0, 1) < 0, "heads");
        CHECK(oracle_attention_fwd_kv(q, k, v, o, lse, B, Hq, Hkv, N + 1, N, d, 1, 0.3, 1) < 0, "kv causal");
        free(q); free(k); free(v); free(g); free(o); free(o2); free(lse); free(lse2); free(p);
        free(dq); free(dk); free(dv);
    }
    if (failures)
        fprintf(stderr, "%d checks failed\n", failures);
    else
        printf("oracle driver: all calls clean\n");
    return failures ? 1 : 0;
}
