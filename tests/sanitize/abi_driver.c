/*
 * Drives the C ABI's host code -- argument validation, launch planning, empty
 * calls, status strings -- for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer.  Every call below either is rejected, has nothing to
 * compute, or is fa_fwd_check (planning only): none reaches a HIP call, so no GPU
 * is needed.  Pointers are distinct, aligned fake addresses 64 GiB apart (so the
 * largest tensors do not overlap) that are compared but never dereferenced.  Exit
 * status 0 means every call ran clean and returned the status the header documents.
 */
#include <stdint.h>
#include <stdio.h>

#include "fa355.h"

#define P(i) ((void *)((uintptr_t)1 << 44 | (uintptr_t)(i) << 36))
#define F(i) ((float *)P(i))

static int failures = 0;
#define EXPECT(call, want)                                                             \
    do {                                                                               \
        const int got_ = (call);                                                       \
        if (got_ != (want)) {                                                          \
            fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #call, \
                    got_, (want));                                                     \
            ++failures;                                                                \
        }                                                                              \
    } while (0)

int main(void)
{
    fa355_plan plan;
    /* Planning over a grid of valid shapes: every built tile and dtype. */
    const int dims[] = {64, 128, 256};
    const int ns[] = {1, 31, 33, 511, 4096, 8388351};
    for (int di = 0; di < 3; ++di)
        for (int ni = 0; ni < 6; ++ni)
            for (int dt = FA355_F16; dt <= FA355_BF16; ++dt)
                for (int causal = 0; causal < 2; ++causal) {
                    const int n = dims[di] == 256 && ns[ni] > 4194175 ? 4194175 : ns[ni];
                    EXPECT(fa_fwd_check(P(1), P(2), P(3), P(4), F(5), 1, 4, 2, n, dims[di], causal, 0.1f,
                                        (fa355_dtype)dt, (fa355_dtype)dt, NULL, &plan), FA355_OK);
                    if (plan.grid < 1 || plan.lds_bytes < 1)
                        ++failures;
                }
    const fa355_tuning tiles[] = {{0, 0}, {128, 64}, {64, 64}, {128, 32}, {256, 64}};
    for (int t = 0; t < 5; ++t)
        EXPECT(fa_fwd_check(P(1), P(2), P(3), P(4), NULL, 2, 8, 8, 1000, 128, 1, 0.1f, FA355_BF16, FA355_BF16,
                            &tiles[t], &plan), FA355_OK);
    EXPECT(fa_fwd_check(P(1), P(2), P(3), P(4), NULL, 2, 8, 8, 1000, 128, 1, 0.1f, FA355_BF16, FA355_F32,
                        &tiles[4], &plan), FA355_OK);
    EXPECT(fa_fwd_check(P(1), P(2), P(3), P(4), NULL, 2, 8, 8, 1000, 128, 1, 0.1f, FA355_BF16, FA355_BF16,
                        &(fa355_tuning){96, 64}, &plan), FA355_ERR_UNSUPPORTED);
    EXPECT(fa_fwd_check(P(1), P(2), P(3), P(4), NULL, 1, 1, 1, 128, 64, 0, 0.1f, FA355_F32, FA355_F32,
                        &(fa355_tuning){32, 32}, &plan), FA355_OK);

    /* Rejections, one per documented status. */
    EXPECT(fa_fwd(NULL, P(2), P(3), P(4), F(5), 1, 4, 2, 100, 128, 1, 0.1f, FA355_BF16, NULL), FA355_ERR_NULL);
    EXPECT(fa_fwd(P(1), P(2), P(3), P(4), F(5), 1, 3, 2, 100, 128, 1, 0.1f, FA355_BF16, NULL), FA355_ERR_SHAPE);
    EXPECT(fa_fwd(P(1), P(2), P(3), P(4), F(5), 1, 4, 2, 8388352, 128, 1, 0.1f, FA355_BF16, NULL), FA355_ERR_SHAPE);
    EXPECT(fa_fwd(P(1), P(2), P(3), P(4), F(5), 1, 4, 2, 100, 96, 1, 0.1f, FA355_BF16, NULL), FA355_ERR_UNSUPPORTED);
    EXPECT(fa_fwd(P(1), (char *)P(2) + 2, P(3), P(4), F(5), 1, 4, 2, 100, 128, 1, 0.1f, FA355_BF16, NULL),
           FA355_ERR_ALIGN);
    EXPECT(fa_fwd(P(1), P(2), P(3), P(1), F(5), 1, 4, 2, 100, 128, 1, 0.1f, FA355_BF16, NULL), FA355_ERR_ARG);
    EXPECT(fa_fwd(P(1), P(2), P(3), P(4), F(5), 1, 4, 2, 100, 128, 1, 1.0f / 0.0f, FA355_BF16, NULL), FA355_ERR_ARG);
    EXPECT(fa_fwd_ex(P(1), P(2), P(3), P(4), F(5), 1, 4, 2, 100, 128, 1, 0.1f, FA355_BF16, FA355_F16, NULL, NULL),
           FA355_ERR_UNSUPPORTED);
    EXPECT(fa_bwd(P(1), P(2), P(3), P(4), P(5), F(6), F(7), F(8), F(9), NULL, 1, 4, 2, 100, 128, 1, 0.1f,
                  FA355_BF16, NULL), FA355_ERR_NULL);
    EXPECT(fa_bwd(P(1), P(2), P(3), P(4), P(5), F(6), F(7), F(8), F(9), F(10), 1, 4, 2, 100, 32, 1, 0.1f,
                  FA355_BF16, NULL), FA355_ERR_UNSUPPORTED);
    EXPECT(fa_fwd_split(P(1), P(2), P(3), P(4), F(5), 1, 4, 2, 100, 128, 1, 0.1f, FA355_BF16, 17, F(6), F(7), NULL),
           FA355_ERR_ARG);
    EXPECT(fa_fwd_bias(P(1), P(2), P(3), P(4), F(5), P(6), 0, 0, 96, 1, 4, 2, 100, 128, 1, 0.1f, FA355_BF16, NULL),
           FA355_ERR_ARG);
    EXPECT(fa_fwd_fp8(P(1), P(2), P(3), P(4), F(5), 1, 4, 2, 100, 128, 1, 0.1f, 0.0f, 1.0f, 1.0f, NULL),
           FA355_ERR_ARG);
    EXPECT(fa_fwd_decode(P(1), P(2), P(3), P(4), F(5), 1, 8, 2, 9, 100, 128, 1, 0.1f, FA355_BF16, 4, F(6), F(7),
                         NULL), FA355_ERR_UNSUPPORTED);
    EXPECT(fa_fwd_decode(P(1), P(2), P(3), P(4), F(5), 1, 8, 2, 2, 8388320, 128, 1, 0.1f, FA355_BF16, 4, F(6),
                         F(7), NULL), FA355_ERR_SHAPE);

    /* Sizes whose byte extents would wrap a 64-bit count: too large, not an overlap,
     * and no signed overflow on the way (UBSan checks the arithmetic). */
    const int big = 1 << 30;
    EXPECT(fa_fwd_check(P(1), P(2), P(3), P(4), F(5), big, big, big, 4096, 128, 1, 0.1f, FA355_BF16,
                        FA355_BF16, NULL, &plan), FA355_ERR_SHAPE);
    EXPECT(fa_fwd_check(P(1), P(2), P(3), P(4), F(5), 2147483647, 2147483647, 1, 8388351, 128, 0, 0.1f,
                        FA355_BF16, FA355_F32, NULL, &plan), FA355_ERR_SHAPE);
    EXPECT(fa_fwd_check(P(1), P(2), P(3), P(4), F(5), 2048, 4096, 4096, 8192, 128, 1, 0.1f, FA355_BF16,
                        FA355_BF16, NULL, &plan), FA355_ERR_SHAPE);           /* 2^43 elements */
    EXPECT(fa_fwd_check(P(1), P(2), P(3), P(4), F(5), 256, 4096, 4096, 8192, 128, 1, 0.1f, FA355_BF16,
                        FA355_BF16, NULL, &plan), FA355_ERR_ARG);  /* 2^40: accepted size, 2 TiB overlap */
    EXPECT(fa_fwd(P(1), P(2), P(3), P(4), F(5), big, 8, 8, 4096, 128, 1, 0.1f, FA355_F16, NULL),
           FA355_ERR_SHAPE);
    EXPECT(fa_fwd_split(P(1), P(2), P(3), P(4), F(5), big, 8, 8, 4096, 128, 1, 0.1f, FA355_BF16, 4, F(6),
                        F(7), NULL), FA355_ERR_SHAPE);
    EXPECT(fa_bwd(P(1), P(2), P(3), P(4), P(5), F(6), F(7), F(8), F(9), F(10), big, big, 1, 4096, 128, 1,
                  0.1f, FA355_BF16, NULL), FA355_ERR_SHAPE);
    EXPECT(fa_fwd_fp8(P(1), P(2), P(3), P(4), F(5), big, big, 1, 4096, 128, 1, 0.1f, 1.0f, 1.0f, 1.0f,
                      NULL), FA355_ERR_SHAPE);
    EXPECT(fa_fwd_decode(P(1), P(2), P(3), P(4), F(5), big, 8, 8, 1, 8388000, 128, 1, 0.1f, FA355_BF16, 256,
                         F(6), F(7), NULL), FA355_ERR_SHAPE);
    EXPECT(fa_fwd_bias(P(1), P(2), P(3), P(4), F(5), P(6), 4611686018427387904LL, 0, 128, 2, 4, 2, 100, 128, 1,
                       0.1f, FA355_BF16, NULL), FA355_ERR_SHAPE);
    EXPECT(fa_fwd_bias(P(1), P(2), P(3), P(4), F(5), P(6), 9223372036854775804LL, 9223372036854775804LL, 128,
                       1 << 10, 4, 2, 100, 128, 1, 0.1f, FA355_BF16, NULL), FA355_ERR_SHAPE);
    /* Just under the limits: accepted by planning. */
    EXPECT(fa_fwd_check(P(1), P(2), P(3), P(4), F(5), 64, 64, 8, 65536, 128, 1, 0.1f, FA355_BF16,
                        FA355_BF16, NULL, &plan), FA355_OK);                  /* 2^35 elements */

    /* Empty calls: success, nothing touched, NULL pointers allowed. */
    EXPECT(fa_fwd(NULL, NULL, NULL, NULL, NULL, 0, 4, 2, 100, 128, 1, 0.1f, FA355_BF16, NULL), FA355_OK);
    EXPECT(fa_bwd(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1, 4, 2, 0, 128, 1, 0.1f,
                  FA355_BF16, NULL), FA355_OK);
    EXPECT(fa_fwd_decode(NULL, NULL, NULL, NULL, NULL, 1, 8, 2, 0, 100, 128, 1, 0.1f, FA355_BF16, 4, NULL, NULL,
                         NULL), FA355_OK);
    EXPECT(fa_fwd_check(NULL, NULL, NULL, NULL, NULL, 0, 4, 2, 100, 128, 1, 0.1f, FA355_BF16, FA355_BF16, NULL,
                        &plan), FA355_OK);

    for (int s = -7; s <= 1; ++s)
        if (!fa_status_str(s))
            ++failures;
    if (fa_version() < 1)
        ++failures;
    if (failures)
        fprintf(stderr, "%d checks failed\n", failures);
    else
        printf("abi driver: all calls clean\n");
    return failures ? 1 : 0;
}
