/*
 * A C client of libfa355: plain HIP runtime calls and the C ABI, no Python.
 *
 * It runs one causal grouped-query forward pass (bf16, B = 1, Hq = 4, Hkv = 2,
 * N = 300, d = 128) on inputs whose result has a closed form: with K = 0 every
 * score is 0, so each query row i weighs its visible keys 0..i equally and
 *     O[h, i, :] = mean of V[h / 2, 0..i, :],   lse[h, i] = ln(i + 1).
 * V holds multiples of 1/8 in [-1, 1), exact in bf16.  It then checks that an
 * unsupported head dimension is refused before any launch.  Exit status 0 and the
 * line "fa355 example: ok" mean every value was within tolerance.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "fa355.h"

#define B 1
#define HQ 4
#define HKV 2
#define N 300
#define D 128

#define HIP_OK(call)                                                                    \
    do {                                                                                \
        hipError_t e_ = (call);                                                         \
        if (e_ != hipSuccess) {                                                         \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));           \
            return 2;                                                                   \
        }                                                                               \
    } while (0)

/* bf16 bits of a float that bf16 holds exactly (the top half of its fp32 bits). */
static uint16_t bf16_bits(float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    return (uint16_t)(u >> 16);
}

static float bf16_value(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float x;
    memcpy(&x, &u, 4);
    return x;
}

static float v_value(int j, int c) { return (float)(((j * 7 + c * 3) % 16) - 8) / 8.0f; }

int main(void)
{
    const size_t nq = (size_t)B * HQ * N * D, nkv = (size_t)B * HKV * N * D;
    uint16_t *hq = calloc(nq, 2), *hk = calloc(nkv, 2), *hv = calloc(nkv, 2), *ho = calloc(nq, 2);
    float *hl = calloc((size_t)B * HQ * N, 4);
    if (!hq || !hk || !hv || !ho || !hl)
        return 2;
    for (size_t t = 0; t < nq; ++t)
        hq[t] = bf16_bits((float)((t % 5) + 1) / 4.0f);        /* any Q: K = 0 cancels it */
    for (int h = 0; h < HKV; ++h)
        for (int j = 0; j < N; ++j)
            for (int c = 0; c < D; ++c)
                hv[((size_t)h * N + j) * D + c] = bf16_bits(v_value(j + 11 * h, c));

    void *q, *k, *v, *o;
    float *lse;
    HIP_OK(hipMalloc(&q, nq * 2));
    HIP_OK(hipMalloc(&k, nkv * 2));
    HIP_OK(hipMalloc(&v, nkv * 2));
    HIP_OK(hipMalloc(&o, nq * 2));
    HIP_OK(hipMalloc((void **)&lse, (size_t)B * HQ * N * 4));
    HIP_OK(hipMemcpy(q, hq, nq * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(k, hk, nkv * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(v, hv, nkv * 2, hipMemcpyHostToDevice));
    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));

    const float scale = 0.08838834764831845f;
    int rc = fa_fwd(q, k, v, o, lse, B, HQ, HKV, N, D, 1, scale, FA355_BF16, stream);
    if (rc != FA355_OK) {
        fprintf(stderr, "fa_fwd: %s\n", fa_status_str(rc));
        return 1;
    }
    HIP_OK(hipStreamSynchronize(stream));
    HIP_OK(hipMemcpy(ho, o, nq * 2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(hl, lse, (size_t)B * HQ * N * 4, hipMemcpyDeviceToHost));

    /* O is a mean of values in [-1, 1): rounding to bf16 moves it by at most 2^-9
     * (half an ulp at magnitude < 1), the fp32 accumulation by far less. */
    double worst_o = 0.0, worst_l = 0.0;
    for (int h = 0; h < HQ; ++h)
        for (int i = 0; i < N; ++i) {
            for (int c = 0; c < D; ++c) {
                double mean = 0.0;
                for (int j = 0; j <= i; ++j)
                    mean += v_value(j + 11 * (h / (HQ / HKV)), c);
                mean /= (double)(i + 1);
                const double err = fabs(bf16_value(ho[((size_t)h * N + i) * D + c]) - mean);
                worst_o = err > worst_o ? err : worst_o;
            }
            const double lerr = fabs(hl[(size_t)h * N + i] - log((double)(i + 1)));
            worst_l = lerr > worst_l ? lerr : worst_l;
        }
    printf("max |O - mean V| = %.3g, max |lse - ln(i+1)| = %.3g\n", worst_o, worst_l);

    /* An unsupported head dimension is an error, never a slower path. */
    const int bad = fa_fwd(q, k, v, o, lse, B, HQ, HKV, N, 96, 1, scale, FA355_BF16, stream);
    printf("d = 96: %s\n", fa_status_str(bad));

    HIP_OK(hipStreamDestroy(stream));
    HIP_OK(hipFree(q));
    HIP_OK(hipFree(k));
    HIP_OK(hipFree(v));
    HIP_OK(hipFree(o));
    HIP_OK(hipFree(lse));
    free(hq); free(hk); free(hv); free(ho); free(hl);
    if (worst_o > 0x1p-8 || worst_l > 1e-5 || bad != FA355_ERR_UNSUPPORTED) {
        printf("fa355 example: FAILED\n");
        return 1;
    }
    printf("fa355 example: ok\n");
    return 0;
}
