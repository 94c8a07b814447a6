/*
 * The library's host-side argument checking under AddressSanitizer and
 * UndefinedBehaviorSanitizer (built by tests/sanitize/build.py with the host
 * pass instrumented): every entry point with null and forged handles, null
 * and misaligned pointers, the five workload shapes, and a few thousand
 * seeded configurations with sizes from 0 through far past what the kernels
 * support (sdm_workspace_bytes, sdm_backward_workspace_bytes,
 * sdm_mem_stride_hint, sdm_create and sdm_step_static on rejected shapes).
 * Nothing here reaches a device: every call returns before the first HIP call.
 * Exits 0 when every status is one the header allows; a sanitizer report
 * aborts the run.  Test code only.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "sdm.h"

static unsigned long long g_state = 12345;

static unsigned long long next(void) /* splitmix64 */
{
    unsigned long long z = (g_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* a size drawn from edge values and a wide log-uniform range */
static int draw(void)
{
    static const int edges[] = {0, -1, 1, 2, 7, 8, 15, 16, 31, 32, 63, 64, 65, 128, 255, 256, 480, 640,
                                1023, 1024, 1025, 2048, 3840, 8192, 131072, 1 << 24, 0x7FFFFFFF, -2147483647};
    const unsigned long long r = next();
    if (r % 3 == 0)
        return edges[(r >> 8) % (sizeof edges / sizeof edges[0])];
    return (int)((r >> 8) % (1ull << ((r >> 40) % 21)));
}

static int failures = 0;

#define EXPECT(cond)                                                                                             \
    do {                                                                                                         \
        if (!(cond)) {                                                                                           \
            fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond);                       \
            ++failures;                                                                                          \
        }                                                                                                        \
    } while (0)

static int known(sdm_status s) { return s >= SDM_OK && s <= SDM_ERR_DEVICE; }

int main(void)
{
    /* the five workload shapes are accepted and sized */
    const sdm_config good[] = {
        {1, 1, 256, 32, 64, 32, 8, 16, SDM_F32, SDM_F32, 0},
        {4, 4, 4096, 128, 128, 128, 16, 64, SDM_F32, SDM_F32, 0},
        {4, 1, 8192, 2048, 480, 256, 32, 64, SDM_BF16, SDM_F32, 0},
        {1, 1, 131072, 2048, 480, 256, 32, 64, SDM_BF16, SDM_BF16, 0},
        {8, 1, 16384, 3840, 640, 256, 32, 64, SDM_BF16, SDM_BF16, 0},
    };
    for (size_t i = 0; i < sizeof good / sizeof good[0]; ++i) {
        size_t n = 0;
        EXPECT(sdm_workspace_bytes(&good[i], &n) == SDM_OK && n > 0);
        EXPECT(sdm_backward_workspace_bytes(&good[i], &n) == SDM_OK && n > 0);
        sdm_config p = good[i];
        p.mem_stride = sdm_mem_stride_hint(&p);
        EXPECT(sdm_workspace_bytes(&p, &n) == SDM_OK);
    }
    /* seeded configurations: any status the header names, a message on every error */
    long accepted = 0, rejected = 0;
    for (int it = 0; it < 4000; ++it) {
        sdm_config c;
        c.B = draw(), c.H = draw(), c.T = draw(), c.d = draw(), c.n_sub = draw(), c.dk = draw();
        c.k = draw(), c.W = draw();
        c.in_dtype = (sdm_dtype)(next() % 3), c.state_dtype = (sdm_dtype)(next() % 3);
        c.mem_stride = next() % 2 ? 0 : draw();
        if (next() % 2) { /* keep most fields plausible so the deeper checks run */
            c.B = 1 + (int)(next() % 8), c.H = 1 + (int)(next() % 4), c.T = 1 + (int)(next() % 20000);
            c.d = 8 * (1 + (int)(next() % 600)), c.n_sub = 1 + (int)(next() % 700);
            c.dk = 32 * (1 + (int)(next() % 16)), c.k = 1 + (int)(next() % 64), c.W = 1 + (int)(next() % 64);
            c.in_dtype = (sdm_dtype)(next() % 2), c.state_dtype = (sdm_dtype)(next() % 2);
        }
        size_t n = 0;
        const sdm_status s = sdm_workspace_bytes(&c, &n);
        EXPECT(known(s));
        if (s == SDM_OK) {
            ++accepted;
        } else {
            ++rejected;
            EXPECT(sdm_last_error()[0] != 0);
        }
        EXPECT(known(sdm_backward_workspace_bytes(&c, &n)));
        (void)sdm_mem_stride_hint(&c);
        if (s != SDM_OK) { /* rejected shapes fail before any device call */
            sdm_handle h = (sdm_handle)0x1;
            EXPECT(sdm_create(&c, NULL, &h) == s && h == NULL);
        }
        /* sdm_step_static on pointers that are never dereferenced: only its host checks may run */
        if (s != SDM_OK) {
            void* p = (void*)0x100;
            EXPECT(sdm_step_static(&c, NULL, p, p, p, (const float*)p, (const float*)p, p, p, (float*)p) != SDM_OK);
        }
    }
    printf("seeded configurations: %ld accepted, %ld rejected\n", accepted, rejected);
    EXPECT(accepted > 100 && rejected > 100);

    /* null and forged handles, null and misaligned arguments */
    uint32_t junk[64];
    memset(junk, 0xAB, sizeof junk);
    sdm_handle forged = (sdm_handle)junk;
    EXPECT(sdm_forward(NULL, 0, 0, 0, 0, 0, 0, 0, 0) == SDM_ERR_INVALID_ARG);
    EXPECT(sdm_forward(forged, 0, 0, 0, 0, 0, 0, 0, 0) == SDM_ERR_INVALID_ARG);
    EXPECT(sdm_step(forged, 0, 0, 0, 0, 0, 0, 0, 0) == SDM_ERR_INVALID_ARG);
    EXPECT(sdm_forward_train(forged, 0, 0, 0, 0, 0, 0, 0, 0, 0) == SDM_ERR_INVALID_ARG);
    EXPECT(sdm_backward(forged, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0) == SDM_ERR_INVALID_ARG);
    EXPECT(sdm_project(forged, 64, 0, 0, 0, 0, 0, 0, 0, 0) == SDM_ERR_INVALID_ARG);
    EXPECT(sdm_broadcast_memory(forged, 0, 0) == SDM_ERR_INVALID_ARG);
    EXPECT(sdm_overlap(forged, 0, 0, 0, 0, 4, 0, 0, 0, 0, 0) == SDM_ERR_INVALID_ARG);
    EXPECT(sdm_score(forged, 0, 0, 0) == SDM_ERR_INVALID_ARG);
    EXPECT(sdm_select(forged, 0, 0, 0) == SDM_ERR_INVALID_ARG);
    EXPECT(sdm_address(forged, 0, 0, 0, 0) == SDM_ERR_INVALID_ARG);
    EXPECT(sdm_scan_with(forged, 0, 0, 0, 0, 0, 0, 0, 0, 0) == SDM_ERR_INVALID_ARG);
    EXPECT(sdm_set_timing(forged, 1) == SDM_ERR_INVALID_ARG);
    EXPECT(sdm_get_timing(forged, NULL) == SDM_ERR_INVALID_ARG);
    EXPECT(sdm_destroy(forged) == SDM_ERR_INVALID_ARG);
    EXPECT(sdm_workspace_bytes(NULL, NULL) == SDM_ERR_INVALID_ARG);
    EXPECT(sdm_create(&good[2], NULL, NULL) == SDM_ERR_INVALID_ARG);
    EXPECT(sdm_mem_stride_hint(NULL) == 0);
    EXPECT(sdm_step_static(NULL, NULL, 0, 0, 0, 0, 0, 0, 0, 0) == SDM_ERR_INVALID_ARG);
    EXPECT(sdm_step_static(&good[2], NULL, 0, 0, 0, 0, 0, 0, 0, 0) == SDM_ERR_INVALID_ARG);
    {
        char* p = (char*)0x100;
        EXPECT(sdm_step_static(&good[2], NULL, p + 4, p, p, (const float*)p, (const float*)p, p, p, (float*)p) ==
               SDM_ERR_INVALID_ARG);
    }
    EXPECT(sdm_pattern_probe(NULL, 4, 16, 128, 16, 64, 0, NULL) == SDM_ERR_INVALID_ARG);
    EXPECT(sdm_pattern_probe_mix((void*)0x100, 4, 16, 128, 0, 16, 64, 3, 1, 0, NULL) == SDM_ERR_INVALID_ARG);
    for (int s = -1; s <= 6; ++s)
        EXPECT(sdm_status_str((sdm_status)s) != NULL);
    if (failures)
        fprintf(stderr, "%d expectations failed\n", failures);
    else
        printf("host checks ok\n");
    return failures ? 1 : 0;
}
