/*
 * A plain C client of libfa2.so: it includes only include/fa2.h and calls the
 * C ABI the way a non-Python caller would. It checks, without a GPU, what the
 * header promises before any HIP call: status names, the launch description of
 * fa2_kernel_config, and the argument errors of fa2_fwd, fa2_fwd_ex and
 * fa2_fwd_varlen. Every call that passes pointers also carries an error that
 * is checked before any device work, so nothing is ever launched.
 * Prints "C CLIENT OK" and returns 0 on success.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "fa2.h"

static int failures = 0;

#define EXPECT(cond)                                                  \
    do {                                                              \
        if (!(cond)) {                                                \
            fprintf(stderr, "line %d: expected %s\n", __LINE__, #cond); \
            ++failures;                                               \
        }                                                             \
    } while (0)

int main(void)
{
    /* fake, 16-byte aligned, far-apart device addresses (never dereferenced) */
    void *q = (void *)(uintptr_t)(1ull << 40), *k = (void *)(uintptr_t)((1ull << 40) + (1ull << 36));
    void *v = (void *)(uintptr_t)((1ull << 40) + (2ull << 36)), *o = (void *)(uintptr_t)((1ull << 40) + (3ull << 36));
    float *lse = (float *)(uintptr_t)((1ull << 40) + (4ull << 36));
    const int *cu = (const int *)(uintptr_t)((1ull << 40) + (5ull << 36));

    for (int s = FA2_OK; s <= FA2_ERR_ARG; ++s) {
        const char *msg = fa2_strerror(s);
        EXPECT(msg != NULL && strlen(msg) > 0);
    }
    EXPECT(strcmp(fa2_strerror(12345), "unknown status") == 0);

    int rows = 0, keys = 0, threads = 0, lds = 0;
    long long blocks = 0;
    EXPECT(fa2_kernel_config(4, 8, 4096, 64, 0, &rows, &keys, &threads, &blocks, &lds) == FA2_OK);
    EXPECT(rows > 0 && threads % 64 == 0 && blocks == 4LL * 8 * ((4096 + rows - 1) / rows) && lds > 0);
    EXPECT(fa2_kernel_config(4, 8, 4096, 64, 0, NULL, NULL, NULL, NULL, NULL) == FA2_OK);
    EXPECT(fa2_kernel_config(1, 1, 128, 96, 0, &rows, &keys, &threads, &blocks, &lds) == FA2_ERR_SHAPE);

    /* fa2_fwd: errors in the documented order, all before any HIP call */
    EXPECT(fa2_fwd(NULL, k, v, o, lse, 1, 1, 128, 64, 0, 0.125f, NULL) == FA2_ERR_NULLPTR);
    EXPECT(fa2_fwd(q, k, v, o, lse, 0, 1, 128, 64, 0, 0.125f, NULL) == FA2_ERR_SHAPE);
    EXPECT(fa2_fwd(q, k, v, o, lse, 1, 1, 128, 64, 2, 0.125f, NULL) == FA2_ERR_SHAPE);
    EXPECT(fa2_fwd(q, k, v, o, lse, 1, 1, 128, 64, 0, -1.0f, NULL) == FA2_ERR_SCALE);
    EXPECT(fa2_fwd((char *)q + 2, k, v, o, lse, 1, 1, 128, 64, 0, 0.125f, NULL) == FA2_ERR_ALIGN);
    EXPECT(fa2_fwd(q, k, v, o, lse, 1, 1, 1 << 29, 64, 0, 0.125f, NULL) == FA2_ERR_OVERFLOW);
    EXPECT(fa2_fwd(q, k, v, q, lse, 1, 1, 128, 64, 1, 0.125f, NULL) == FA2_ERR_ALIAS);

    /* fa2_fwd_ex */
    EXPECT(fa2_fwd_ex(q, k, v, o, lse, 1, 4, 3, 128, 64, -1, -1, 0.0f, 0, 0, 0.125f, NULL) == FA2_ERR_SHAPE);
    EXPECT(fa2_fwd_ex(q, k, v, o, lse, 1, 4, 2, 128, 64, -2, 0, 0.0f, 0, 0, 0.125f, NULL) == FA2_ERR_ARG);
    EXPECT(fa2_fwd_ex(q, k, v, o, lse, 1, 4, 2, 128, 64, -1, -1, 1.0f, 0, 0, 0.125f, NULL) == FA2_ERR_ARG);
    EXPECT(fa2_fwd_ex(q, k, v, q, lse, 1, 4, 2, 128, 64, 16, 0, 0.1f, 7, 3, 0.125f, NULL) == FA2_ERR_ALIAS);

    /* fa2_fwd_varlen */
    EXPECT(fa2_fwd_varlen(q, k, v, o, lse, NULL, 3, 300, 200, 4, 1, 128, -1, -1, 0.0f, 0, 0, 0.125f, NULL) ==
           FA2_ERR_NULLPTR);
    EXPECT(fa2_fwd_varlen(q, k, v, o, lse, cu, 0, 300, 200, 4, 1, 128, -1, -1, 0.0f, 0, 0, 0.125f, NULL) ==
           FA2_ERR_SHAPE);
    EXPECT(fa2_fwd_varlen(q, k, v, o, lse, (const int *)((const char *)cu + 2), 3, 300, 200, 4, 1, 128, -1, -1,
                          0.0f, 0, 0, 0.125f, NULL) == FA2_ERR_ALIGN);
    EXPECT(fa2_fwd_varlen(q, k, v, q, lse, cu, 3, 300, 200, 4, 1, 128, -1, 0, 0.0f, 0, 0, 0.125f, NULL) ==
           FA2_ERR_ALIAS);

    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("C CLIENT OK\n");
    return 0;
}
