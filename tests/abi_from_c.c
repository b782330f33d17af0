/* A plain C99 client of libdemo: includes only include/demo.h and calls the
 * host-side entry points (version, error strings, payload layout, argument
 * validation), none of which launches a kernel.  Prints the layout of one
 * configuration as "key value" lines for the test to check against the
 * oracle's codec; exits nonzero on the first failed expectation. */
#include <stddef.h>
#include <stdio.h>
#include <string.h>

#include "demo.h"

static int failures = 0;

#define EXPECT(cond)                                                  \
    do {                                                              \
        if (!(cond)) {                                                \
            fprintf(stderr, "%s:%d: failed: %s\n", __FILE__, __LINE__, #cond); \
            failures++;                                               \
        }                                                             \
    } while (0)

static demo_cfg base_cfg(void)
{
    demo_cfg c;
    memset(&c, 0, sizeof c);
    c.abi_version = DEMO_ABI_VERSION;
    c.scheme = DEMO_SCHEME_DCT;
    c.chunk = 32;
    c.k = 1;
    c.period = 16;
    c.sign = 1;
    c.value_fmt = DEMO_VAL_TERNARY;
    c.beta = 0.9f;
    c.lr = 1e-3f;
    return c;
}

int main(void)
{
    EXPECT(demo_abi_version() == DEMO_ABI_VERSION);
    EXPECT(sizeof(demo_cfg) == 64);
    EXPECT(offsetof(demo_cfg, beta) == 28 && offsetof(demo_cfg, lr) == 32 && offsetof(demo_cfg, seed) == 40 &&
           offsetof(demo_cfg, step) == 48 && offsetof(demo_cfg, chunk_offset) == 56);
    EXPECT(sizeof(demo_layout) == 64);
    EXPECT(demo_strerror(DEMO_OK) != NULL && demo_strerror(-99) != NULL);

    demo_cfg cfg = base_cfg();
    demo_layout lay;
    const uint64_t n = 639697920u; /* OLMo2-1B half shard */
    EXPECT(demo_payload_layout(&cfg, n, &lay) == DEMO_OK);
    printf("idx_off %llu\nidx_bytes %llu\nnz_off %llu\nneg_off %llu\nplane_bytes %llu\n"
           "val_off %llu\nval_bytes %llu\ntotal_bytes %llu\n",
           (unsigned long long)lay.idx_off, (unsigned long long)lay.idx_bytes,
           (unsigned long long)lay.nz_off, (unsigned long long)lay.neg_off,
           (unsigned long long)lay.plane_bytes, (unsigned long long)lay.val_off,
           (unsigned long long)lay.val_bytes, (unsigned long long)lay.total_bytes);
    EXPECT(lay.total_bytes % 256 == 0 && lay.nz_off % 256 == 0 && lay.neg_off % 256 == 0);

    /* synchronous validation: nothing is launched, no device is touched */
    static float dummy[64] __attribute__((aligned(16)));
    EXPECT(demo_encode(&cfg, n, NULL, dummy, dummy + 16, NULL, NULL) == DEMO_EINVAL);
    EXPECT(demo_encode(&cfg, 0, dummy, dummy + 16, dummy + 32, NULL, NULL) == DEMO_EINVAL);
    EXPECT(demo_encode(&cfg, 64, dummy + 1, dummy + 16, dummy + 32, NULL, NULL) == DEMO_EALIGN);
    demo_cfg bad = base_cfg();
    bad.abi_version = DEMO_ABI_VERSION + 1;
    EXPECT(demo_payload_layout(&bad, n, &lay) == DEMO_EABI);
    bad = base_cfg();
    bad.sign = 0; /* ternary planes carry signs only */
    EXPECT(demo_payload_layout(&bad, n, &lay) == DEMO_EINVAL);
    bad = base_cfg();
    bad.chunk = 64;
    EXPECT(demo_payload_layout(&bad, n, &lay) == DEMO_EUNSUPPORTED);
    EXPECT(demo_decode_apply(&cfg, n, dummy, dummy + 16, 8, 2, NULL) == DEMO_EALIGN);   /* stride not a multiple of 16 */
    EXPECT(demo_decode_apply(&cfg, n, dummy, dummy + 16, 256, 2, NULL) == DEMO_EINVAL); /* stride below the payload size */
    EXPECT(demo_random_select(&cfg, 0, 0, 16, (uint32_t *)dummy, NULL) == DEMO_EINVAL); /* DCT has no shared positions */

    if (failures)
        fprintf(stderr, "%d failure(s)\n", failures);
    return failures ? 1 : 0;
}
