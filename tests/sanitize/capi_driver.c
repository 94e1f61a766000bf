/*
 * Host-side validation of the C ABI (include/pisa.h) under AddressSanitizer and
 * UndefinedBehaviorSanitizer: plans geometries, queries workspace sizes and
 * passes malformed arguments to every entry point, each of which must be
 * rejected on the host with its documented status before anything is queued
 * (no GPU is touched). Test infrastructure (tests/test_sanitizers.py builds
 * capi.hip's host code with the sanitizers and links this driver).
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "pisa.h"

static int fails = 0;
#define EXPECT(call, want)                                                                    \
    do {                                                                                      \
        pisa_status got_ = (call);                                                            \
        if (got_ != (want)) {                                                                 \
            fprintf(stderr, "line %d: %s -> %d, expected %d\n", __LINE__, #call, (int)got_, (int)(want)); \
            fails++;                                                                          \
        }                                                                                     \
    } while (0)

int main(void)
{
    pisa_pyramid p, zero;
    memset(&zero, 0, sizeof(zero));
    size_t n = 0;
    void* fake = (void*)(uintptr_t)(1u << 24);  /* never dereferenced: validation fails first */
    int32_t* fi = (int32_t*)fake;

    /* geometry planning over the supported and unsupported set */
    static const int gs[] = {2, 3, 4, 8, 16, 32};
    static const int cs[] = {8, 16, 32, 64, 128};
    static const int ds[] = {32, 64, 128, 256};
    for (int a = 0; a < 6; a++)
        for (int c = 0; c < 5; c++)
            for (int e = 0; e < 4; e++) {
                pisa_status s = pisa_pyramid_plan(&p, 2, 4, ds[e], cs[c], gs[a], 1000003);
                if (s == PISA_OK) {
                    for (int mode = 0; mode < 3; mode++)
                        EXPECT(pisa_route_prefill_workspace(&p, 1000003, 16, 8, mode, &n), PISA_OK);
                    EXPECT(pisa_route_prefill_workspace(&p, 1000004, 16, 8, 2, &n), PISA_ENOSPACE);
                }
            }
    EXPECT(pisa_pyramid_plan(&p, 0, 4, 128, 64, 4, 1024), PISA_EINVAL);
    EXPECT(pisa_pyramid_plan(&p, 1, 4, 128, 64, 4, 0), PISA_EINVAL);
    EXPECT(pisa_pyramid_plan(NULL, 1, 4, 128, 64, 4, 1024), PISA_EINVAL);

    /* descriptors that were not planned */
    for (int mode = 0; mode < 4; mode++)
        EXPECT(pisa_route_prefill_workspace(&zero, 4096, 16, 8, mode, &n), PISA_EINVAL);
    EXPECT(pisa_build_pyramid(&zero, fake, PISA_BF16, 16, NULL), PISA_EINVAL);

    EXPECT(pisa_pyramid_plan(&p, 1, 4, 128, 64, 4, 4096), PISA_OK);
    p.buf = (float*)(uintptr_t)(1u << 20);
    EXPECT(pisa_route_prefill_workspace(&p, 4096, 16, 8, 7, &n), PISA_EINVAL);
    EXPECT(pisa_build_pyramid(&p, fake, PISA_BF16, 0, NULL), PISA_EINVAL);
    EXPECT(pisa_build_pyramid(&p, fake, PISA_BF16, 4097, NULL), PISA_ENOSPACE);
    EXPECT(pisa_build_pyramid(&p, NULL, PISA_BF16, 16, NULL), PISA_EINVAL);
    EXPECT(pisa_pyramid_append(&p, fake, PISA_BF16, NULL, NULL), PISA_EINVAL);
    EXPECT(pisa_route_prefill(&p, fake, fake, PISA_BF16, 0, 16, 8, 1, 4, 0, fi, NULL, NULL, 0, NULL), PISA_EINVAL);
    EXPECT(pisa_route_prefill(&p, fake, fake, PISA_BF16, 4097, 16, 8, 1, 4, 0, fi, NULL, NULL, 0, NULL), PISA_ENOSPACE);
    EXPECT(pisa_route_prefill(&p, fake, fake, PISA_BF16, 4096, 16, 8, 1, 2, 0, fi, NULL, NULL, 0, NULL), PISA_EINVAL);
    EXPECT(pisa_route_prefill(&p, fake, fake, PISA_BF16, 4096, 16, 2, 1, 4, 0, fi, NULL, NULL, 0, NULL), PISA_EINVAL);
    EXPECT(pisa_route_prefill(&p, fake, fake, PISA_BF16, 4096, 16, 65, 1, 4, 0, fi, NULL, NULL, 0, NULL), PISA_EINVAL);
    EXPECT(pisa_route_prefill(&p, fake, fake, (pisa_dtype)7, 4096, 16, 8, 1, 4, 0, fi, NULL, NULL, 0, NULL), PISA_EINVAL);
    EXPECT(pisa_route_prefill(&p, fake, fake, PISA_BF16, 4096, 16, 8, 1, 4, 9, fi, NULL, NULL, 0, NULL), PISA_EINVAL);
    EXPECT(pisa_route_prefill(&p, fake, fake, PISA_BF16, 4096, 16, 8, 1, 4, 0, fi, NULL, fake, 1, NULL), PISA_ENOSPACE);
    EXPECT(pisa_route_prefill_scored(&p, fake, fake, PISA_BF16, 4096, 16, 8, 1, 4, 2, 3, fi, NULL, NULL, 0, NULL), PISA_EINVAL);
    EXPECT(pisa_route_prefill_scored(&p, fake, fake, PISA_BF16, 4096, 16, 8, 1, 4, 0, 1, fi, NULL, NULL, 0, NULL), PISA_EUNSUPPORTED);
    EXPECT(pisa_route_prefill_noalloc(&p, fake, fake, PISA_BF16, 4097, 16, 8, 1, 4, fi, NULL, NULL), PISA_ENOSPACE);
    EXPECT(pisa_route_prefill_noalloc(&zero, fake, fake, PISA_BF16, 16, 16, 8, 1, 4, fi, NULL, NULL), PISA_EINVAL);
    EXPECT(pisa_route_decode(&p, fake, fake, PISA_BF16, NULL, 16, 8, 4, fi, NULL, NULL), PISA_EINVAL);
    EXPECT(pisa_route_decode(&p, fake, fake, PISA_BF16, (const int64_t*)fake, 16, 2, 4, fi, NULL, NULL), PISA_EINVAL);
    EXPECT(pisa_route_decode_scored(&p, fake, fake, PISA_BF16, (const int64_t*)fake, 16, 8, 4, 3, fi, NULL, NULL), PISA_EINVAL);
    EXPECT(pisa_bsa_select(&p, fake, PISA_BF16, 4096, 16, 17, 1, 4, fi, NULL, NULL), PISA_EUNSUPPORTED);
    EXPECT(pisa_bsa_select(&p, NULL, PISA_BF16, 4096, 16, 8, 1, 4, fi, NULL, NULL), PISA_EINVAL);
    EXPECT(pisa_sparse_attn_workspace(1, 4096, 4096, 16, 4, 128, 64, 8, NULL), PISA_EINVAL);
    EXPECT(pisa_sparse_attn_bwd_workspace(1, 4096, 4096, 16, 3, 128, 64, 8, &n), PISA_EINVAL);
    EXPECT(pisa_selection_quality_workspace(1, 4096, 16, 64, NULL), PISA_EINVAL);
    EXPECT(pisa_time_stage(PISA_STAGE_COUNT, NULL, NULL), PISA_EINVAL);
    for (int s = -3; s <= 1; s++)
        if (!pisa_status_str((pisa_status)s)) fails++;
    if (pisa_abi_version() < 1) fails++;
    if (!pisa_last_error()) fails++;
    printf(fails ? "capi driver: %d FAILED\n" : "capi driver: ok\n", fails);
    return fails != 0;
}
