/*
 * Host-side check of the C ABI under AddressSanitizer and UndefinedBehavior-
 * Sanitizer (built and run by tests/test_abi_cpu.py, no GPU needed): every
 * call here either validates its arguments or reports static information
 * and returns before any GPU work. Exits 0 when every status is the one the
 * header documents; a sanitizer report aborts with a non-zero status.
 */
#include <stdio.h>
#include <string.h>

#include "smconv.h"

static int failures = 0;

#define EXPECT(expr, want)                                                                \
    do {                                                                                  \
        long long got_ = (long long)(expr);                                               \
        if (got_ != (long long)(want)) {                                                  \
            fprintf(stderr, "%s:%d: %s = %lld, want %lld\n", __FILE__, __LINE__, #expr,  \
                    got_, (long long)(want));                                             \
            ++failures;                                                                   \
        }                                                                                 \
    } while (0)

static void free_only(void* ctx, void* p, void* s) {
    (void)ctx;
    (void)p;
    (void)s;
}

int main(void) {
    smc_map* h = NULL;
    smc_map_info_t info;
    int32_t order[27], groups[27];
    double ms[SMC_STAGE_COUNT];
    int64_t calls[SMC_STAGE_COUNT];
    EXPECT(smc_version() >= 100, 1);
    EXPECT(strcmp(smc_status_string(SMC_OK), "ok"), 0);
    EXPECT(strcmp(smc_status_string(999), "unknown status"), 0);
    EXPECT(smc_weight_packed_bytes(3, 128, 128), 2 * 27 * 8 * 4 * 64 * 16); /* + 64-column tiles */
    EXPECT(smc_weight_packed_bytes(3, 64, 64), 2 * 27 * 4 * 2 * 64 * 16); /* two packings */
    EXPECT(smc_weight_packed_bytes(3, 136, 128), 27 * 8 * 5 * 64 * 16);
    EXPECT(smc_weight_packed_bytes(3, 0, 5), 0);
    EXPECT(smc_weight_packed_bytes(4, 16, 16), 0);
    EXPECT(smc_map_create(NULL), SMC_ERR_ARG);
    EXPECT(smc_map_create(&h), SMC_OK);
    /* build arguments: kernel size, ncols, n, route, handle */
    EXPECT(smc_map_build(h, NULL, 0, 4, NULL, 0, 4, 0, 0, NULL), SMC_ERR_UNSUPPORTED);
    EXPECT(smc_map_build(h, NULL, 0, 4, NULL, 0, 5, 0, SMC_BUILD_NO_PAIRS, NULL),
           SMC_ERR_UNSUPPORTED);
    EXPECT(smc_map_build(h, NULL, 0, 2, NULL, 0, 3, 0, 0, NULL), SMC_ERR_ARG);
    EXPECT(smc_map_build(h, NULL, -1, 4, NULL, 0, 3, 0, 0, NULL), SMC_ERR_ARG);
    EXPECT(smc_map_build(h, NULL, 5, 4, NULL, 0, 3, 0, 0, NULL), SMC_ERR_ARG);
    EXPECT(smc_map_build(h, NULL, 0, 4, NULL, 0, 3, 7, 0, NULL), SMC_ERR_ARG);
    EXPECT(strstr(smc_last_error(), "route") != NULL, 1);
    EXPECT(smc_map_build(NULL, NULL, 0, 4, NULL, 0, 3, 0, 0, NULL), SMC_ERR_ARG);
    EXPECT(smc_map_build_strided(h, NULL, 0, 4, NULL, 0, 5, 2, 0, 0, NULL), SMC_ERR_UNSUPPORTED);
    EXPECT(smc_map_build_strided(h, NULL, 0, 4, NULL, 0, 3, 3, 0, 0, NULL), SMC_ERR_UNSUPPORTED);
    /* a handle never built */
    EXPECT(smc_map_info(h, &info), SMC_ERR_STATE);
    EXPECT(smc_map_info(h, NULL), SMC_ERR_ARG);
    EXPECT(smc_map_rows(NULL, NULL, NULL), SMC_ERR_ARG);
    EXPECT(smc_map_rows(h, NULL, NULL), SMC_ERR_STATE);
    EXPECT(smc_map_sync(h), SMC_ERR_STATE);
    EXPECT(smc_map_export(h, NULL, NULL, NULL, NULL, NULL, NULL), SMC_ERR_STATE);
    EXPECT(smc_map_export_out_coords(h, NULL), SMC_ERR_STATE);
    EXPECT(smc_map_calibrate(h, 1, order, groups), SMC_ERR_STATE);
    EXPECT(smc_map_calibrate(h, 1, NULL, groups), SMC_ERR_ARG);
    EXPECT(smc_conv_forward(h, NULL, 16, NULL, 16, NULL, 0, NULL), SMC_ERR_STATE);
    EXPECT(smc_conv_forward_noalloc(h, NULL, 16, NULL, 16, NULL, 0, NULL), SMC_ERR_STATE);
    EXPECT(smc_conv_forward(NULL, NULL, 16, NULL, 16, NULL, 0, NULL), SMC_ERR_ARG);
    /* orders: a repeated tap, a group index out of range, the centre not last */
    for (int j = 0; j < 27; ++j) {
        order[j] = 26 - j;
        groups[j] = 0;
    }
    EXPECT(smc_map_set_order(h, order, groups), SMC_OK);
    order[3] = order[4];
    EXPECT(smc_map_set_order(h, order, NULL), SMC_ERR_ARG);
    groups[0] = 7;
    EXPECT(smc_map_set_order(h, NULL, groups), SMC_ERR_ARG);
    groups[0] = 1;
    EXPECT(smc_map_set_order(h, NULL, groups), SMC_ERR_ARG);
    /* timers, the test hook and the probes */
    EXPECT(smc_timing_enable(h, 1), SMC_OK);
    EXPECT(smc_timing_read(h, ms, calls, 1), SMC_OK);
    EXPECT(calls[SMC_STAGE_MAP], 0);
    EXPECT(smc_timing_enable(NULL, 1), SMC_ERR_ARG);
    EXPECT(smc_test_force_lookback_timeout(NULL, 1), SMC_ERR_ARG);
    EXPECT(smc_test_force_lookback_timeout(h, 0), SMC_OK);
    EXPECT(smc_probe_mfma_bf16(0, NULL, 0, NULL, NULL), SMC_ERR_ARG);
    EXPECT(smc_probe_copy(NULL, NULL, 16, NULL), SMC_ERR_ARG);
    EXPECT(smc_weight_pack(NULL, 3, 16, 16, NULL, NULL), SMC_ERR_ARG);
    /* allocator pair: both or neither */
    EXPECT(smc_set_allocator(NULL, free_only, NULL), SMC_ERR_ARG);
    EXPECT(smc_set_allocator(NULL, NULL, NULL), SMC_OK);
    EXPECT(smc_map_destroy(h), SMC_OK);
    EXPECT(smc_map_destroy(NULL), SMC_OK);
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("abi host check ok\n");
    return 0;
}
