/* Host-side checks of libbfly's argument validation and size queries, built
 * with AddressSanitizer and UndefinedBehaviorSanitizer (host code only) by
 * tests/test_sanitize_cpu.py.  Every call here is rejected, or is a pure
 * size query, before any HIP call: no device is needed and none is touched.
 * The pointers are fake, aligned addresses the library never dereferences
 * on these paths. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "bfly.h"

static int failures = 0;
#define EXPECT(cond)                                                         \
    do {                                                                     \
        if (!(cond)) {                                                       \
            fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                                      \
        }                                                                    \
    } while (0)

#define P(a) ((void*)(uintptr_t)(a))
#define F(a) ((float*)(uintptr_t)(a))

static const int64_t huge_rows[] = {INT64_MAX, INT64_MAX - 1, INT64_MIN, -1,
                                    (int64_t)1 << 62, (int64_t)1 << 40, ((int64_t)1 << 34) + 1};
static const int32_t odd_n[] = {INT32_MIN, -4096, -1, 0, 1, 2, 3, 32, 63, 65, 4095, 4097,
                                16384, 1 << 30, INT32_MAX};

static void size_queries(void)
{
    for (size_t i = 0; i < sizeof(odd_n) / sizeof(odd_n[0]); ++i) {
        EXPECT(bfly_coeff_bytes(odd_n[i]) == 0);
        EXPECT(bfly_backward_workspace_bytes(1, odd_n[i]) == 0);
        EXPECT(bfly_calib_workspace_bytes(1, odd_n[i]) == 0);
        EXPECT(bfly_kron_forward_wide_workspace_bytes(1, 5, odd_n[i]) == 0);
        EXPECT(bfly_kron_backward_workspace_bytes(1, 5, odd_n[i]) == 0);
        EXPECT(bfly_calib_step_weight_workspace_bytes(1, 64, odd_n[i]) == 0);
    }
    for (int l = 6; l <= 13; ++l) EXPECT(bfly_coeff_bytes(1 << l) > 0);
    /* rows no device could hold: every query answers 0, with no wrap-around */
    for (size_t i = 0; i < sizeof(huge_rows) / sizeof(huge_rows[0]); ++i) {
        const int64_t r = huge_rows[i];
        EXPECT(bfly_backward_workspace_bytes(r, 4096) == 0);
        EXPECT(bfly_calib_workspace_bytes(r, 4096) == 0);
        EXPECT(bfly_kron_forward_wide_workspace_bytes(r, 43, 256) == 0);
        EXPECT(bfly_kron_backward_workspace_bytes(r, 64, 1024) == 0);
        EXPECT(bfly_calib_step_weight_workspace_bytes(r, 4096, 4096) == 0);
    }
    /* within range, the sizes grow with the rows */
    size_t prev[5] = {0, 0, 0, 0, 0};
    for (int64_t r = 1; r <= ((int64_t)1 << 30); r *= 8) {
        const size_t now[5] = {bfly_backward_workspace_bytes(r, 4096),
                               bfly_calib_workspace_bytes(r, 4096),
                               bfly_kron_forward_wide_workspace_bytes(r, 43, 256),
                               bfly_kron_backward_workspace_bytes(r, 5, 1024),
                               bfly_calib_step_weight_workspace_bytes(r, 4096, 4096)};
        for (int k = 0; k < 5; ++k) {
            EXPECT(now[k] >= prev[k] && now[k] > 0);
            prev[k] = now[k];
        }
    }
    EXPECT(bfly_calib_step_weight_workspace_bytes(1, 15, 4096) == 0);
    EXPECT(bfly_calib_step_weight_workspace_bytes(1, 65552, 4096) == 0);
    EXPECT(bfly_calib_step_weight_workspace_bytes(1, 65536, 4096) > 0);
    EXPECT(bfly_kron_forward_wide_workspace_bytes(1, 65, 256) == 0);
    EXPECT(bfly_kron_forward_wide_workspace_bytes(1, 64, 2048) == 0);
}

static void rejected_calls(void)
{
    const size_t big = (size_t)1 << 40;
    /* prepare */
    EXPECT(bfly_prepare(NULL, 4096, P(0x30000), big, NULL) == BFLY_ERR_NULL);
    EXPECT(bfly_prepare(F(0x60000), 4095, P(0x30000), big, NULL) == BFLY_ERR_SIZE);
    EXPECT(bfly_prepare(F(0x60000), 32, P(0x30000), big, NULL) == BFLY_ERR_UNSUPPORTED);
    EXPECT(bfly_prepare(F(0x60000), 4096, P(0x30000), 16, NULL) == BFLY_ERR_WORKSPACE);
    EXPECT(bfly_prepare(F(0x60000), 4096, P(0x30008), big, NULL) == BFLY_ERR_ALIGN);
    EXPECT(bfly_prepare_hadamard(INT32_MIN, P(0x30000), big, NULL) == BFLY_ERR_SIZE);
    /* forward and forward_quant */
    for (size_t i = 0; i < sizeof(huge_rows) / sizeof(huge_rows[0]); ++i) {
        const int64_t r = huge_rows[i];
        const bfly_status want = r < 0 ? BFLY_ERR_SIZE : BFLY_ERR_UNSUPPORTED;
        EXPECT(bfly_forward(P(0x10000), BFLY_BF16, P(0x20000), BFLY_BF16, r, 4096, NULL,
                            P(0x90000), NULL, 0, NULL) == want);
        EXPECT(bfly_forward_quant(P(0x10000), BFLY_BF16, NULL, BFLY_BF16, P(0x30000), P(0x40000),
                                  NULL, r, 4096, NULL, P(0x90000), 4, 128, BFLY_SYM_ABSMAX, NULL,
                                  0, NULL) == want);
        EXPECT(bfly_forward_quant_noalloc(P(0x10000), BFLY_BF16, NULL, BFLY_BF16, P(0x30000),
                                          P(0x40000), NULL, r, 4096, F(0x60000), 4, 128,
                                          BFLY_SYM_ABSMAX, NULL) == want);
        EXPECT(bfly_backward(F(0x10000), F(0x20000), NULL, F(0x30000), F(0x40000), r, 4096,
                             F(0x60000), NULL, P(0x80000), big, NULL) == want);
        EXPECT(bfly_kron_forward(P(0x10000), BFLY_BF16, P(0x20000), BFLY_BF16, NULL, NULL, NULL,
                                 r, 5, 1024, NULL, P(0x90000), F(0x70000), 0, 0, BFLY_SYM_ABSMAX,
                                 NULL, 0, NULL) == want);
        EXPECT(bfly_kron_forward_wide(P(0x10000), BFLY_BF16, P(0x20000), BFLY_BF16, NULL, NULL,
                                      NULL, r, 43, 256, NULL, P(0x90000), F(0x70000), 0, 0,
                                      BFLY_SYM_ABSMAX, P(0x80000), big, NULL) == want);
        EXPECT(bfly_kron_backward(F(0x10000), F(0x20000), F(0x30000), F(0x40000), r, 5, 1024,
                                  F(0x60000), NULL, F(0x70000), P(0x80000), big, NULL) == want);
        EXPECT(bfly_quant_matmul(P(0x10000), BFLY_BF16, P(0x30000), P(0x40000), P(0x50000),
                                 P(0x20000), BFLY_F32, r, 11008,
                                 4096, 2, 128, BFLY_ASYM_MINMAX, NULL) == want);
    }
    EXPECT(bfly_forward(NULL, BFLY_BF16, P(0x20000), BFLY_BF16, 1, 4096, NULL, P(0x90000), NULL,
                        0, NULL) == BFLY_ERR_NULL);
    EXPECT(bfly_forward(P(0x10000), (bfly_dtype)7, P(0x20000), BFLY_BF16, 1, 4096, NULL,
                        P(0x90000), NULL, 0, NULL) == BFLY_ERR_DTYPE);
    EXPECT(bfly_forward(P(0x10001), BFLY_BF16, P(0x20000), BFLY_BF16, 1, 4096, NULL, P(0x90000),
                        NULL, 0, NULL) == BFLY_ERR_ALIGN);
    EXPECT(bfly_forward(P(0x10000), BFLY_BF16, P(0x20000), BFLY_BF16, 1, 4096, F(0x60000), NULL,
                        P(0x80000), 64, NULL) == BFLY_ERR_WORKSPACE);
    EXPECT(bfly_forward(P(0x10000), BFLY_BF16, P(0x20000), BFLY_BF16, 1, 16384, NULL, P(0x90000),
                        NULL, 0, NULL) == BFLY_ERR_UNSUPPORTED);
    for (int32_t g = -8; g <= 1024; g += 8) {
        const int valid = g >= 8 && g <= 512 && (g & (g - 1)) == 0;
        /* x misaligned: a valid group gets as far as the alignment check */
        const bfly_status s = bfly_forward_quant(P(0x10001), BFLY_BF16, NULL, BFLY_BF16,
                                                 P(0x30000), P(0x40000), NULL, 1, 4096, NULL,
                                                 P(0x90000), 4, g, BFLY_SYM_ABSMAX, NULL, 0, NULL);
        EXPECT(s == (valid ? BFLY_ERR_ALIGN : BFLY_ERR_QUANT));
    }
    EXPECT(bfly_forward_quant(P(0x10000), BFLY_BF16, NULL, BFLY_BF16, P(0x30000), P(0x40000),
                              P(0x50000), 1, 4096, NULL, P(0x90000), 4, 128, BFLY_SYM_ABSMAX, NULL,
                              0, NULL) == BFLY_ERR_QUANT);
    EXPECT(bfly_forward_quant(P(0x10000), BFLY_BF16, NULL, BFLY_BF16, P(0x30000), P(0x40000),
                              NULL, 1, 4096, NULL, P(0x90000), 3, 128, BFLY_SYM_ABSMAX, NULL, 0,
                              NULL) == BFLY_ERR_QUANT);
    /* calibration steps */
    bfly_calib_config cc = {4, 128, 16, 0.1f, 1e-3f, 0.9f, 0.999f, 1e-8f};
    EXPECT(bfly_calib_step(F(0x10000), INT64_MAX, 4096, F(0x20000), F(0x30000), F(0x40000), 1,
                           &cc, F(0x50000), P(0x80000), big, NULL) == BFLY_ERR_UNSUPPORTED);
    EXPECT(bfly_calib_step(F(0x10000), 0, 4096, F(0x20000), F(0x30000), F(0x40000), 1, &cc,
                           F(0x50000), P(0x80000), big, NULL) == BFLY_ERR_SIZE);
    cc.bins = 33;
    EXPECT(bfly_calib_step(F(0x10000), 8, 4096, F(0x20000), F(0x30000), F(0x40000), 1, &cc,
                           F(0x50000), P(0x80000), big, NULL) == BFLY_ERR_QUANT);
    bfly_calib_weight_config wc = {2, 64, BFLY_ASYM_MINMAX, 16, 0.1f, 1e-3f, 0.9f, 0.999f, 1e-8f};
    EXPECT(bfly_calib_step_weight(F(0x10000), INT64_MAX, P(0x20000), BFLY_BF16, 64, 4096,
                                  F(0x30000), F(0x40000), F(0x50000), 1, &wc, F(0x60000),
                                  P(0x80000), big, NULL) == BFLY_ERR_UNSUPPORTED);
    EXPECT(bfly_calib_step_weight(F(0x10000), 8, P(0x20000), (bfly_dtype)-1, 64, 4096,
                                  F(0x30000), F(0x40000), F(0x50000), 1, &wc, F(0x60000),
                                  P(0x80000), big, NULL) == BFLY_ERR_DTYPE);
    wc.bins = 12;
    EXPECT(bfly_calib_step_weight(F(0x10000), 8, P(0x20000), BFLY_BF16, 64, 4096, F(0x30000),
                                  F(0x40000), F(0x50000), 1, &wc, F(0x60000), P(0x80000), big,
                                  NULL) == BFLY_ERR_QUANT);
    /* diagnostics */
    for (int s = -3; s < 12; ++s) EXPECT(bfly_status_string((bfly_status)s) != NULL);
    EXPECT(bfly_time_next_forward(P(0x1000), NULL) == BFLY_ERR_NULL);
    EXPECT(bfly_time_next_forward(NULL, NULL) == BFLY_OK);
    EXPECT(bfly_last_hip_error() == 0);
}

int main(void)
{
    size_queries();
    rejected_calls();
    if (failures) {
        fprintf(stderr, "%d failed checks\n", failures);
        return 1;
    }
    printf("abi_san: all checks passed\n");
    return 0;
}
