/* Plain C99 client of the C ABI: include/adacomp.h must compile as C, and the
 * host-only calls must work through it without any GPU.  Prints one line per
 * check and exits non-zero on the first failure. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../../include/adacomp.h"

static int fail(const char* what) {
    printf("FAIL %s\n", what);
    return 1;
}

int main(void) {
    adacomp_segment segs[3];
    memset(segs, 0, sizeof segs);
    segs[0].offset = 0;    segs[0].numel = 100000; segs[0].bin_len = 500;
    segs[1].offset = 100000; segs[1].numel = 4097; segs[1].bin_len = 50; segs[1].flags = ADACOMP_SEG_LS;
    segs[2].offset = 104100; segs[2].numel = 3;    segs[2].bin_len = 32768;
    adacomp_plan_info info;
    memset(&info, 0, sizeof info);
    if (adacomp_plan_query(segs, 3, &info) != ADACOMP_OK) return fail("plan_query");
    if (info.nseg != 3 || info.total_numel != 104100 || info.span != 104104) return fail("info sizes");
    if (info.total_bins != 200 + 82 + 1) return fail("total_bins");
    if (info.header_bytes != 32 + 16 * 3) return fail("header_bytes");
    /* shapes 0 (L_T 500, 50) and 2 (L_T 32768): two tile passes, one finish */
    if (info.compress_launches != 3) return fail("compress_launches");
    printf("OK plan_query nseg=%u bins=%llu capacity=%llu launches=%llu\n", info.nseg,
           (unsigned long long)info.total_bins, (unsigned long long)info.message_capacity,
           (unsigned long long)info.compress_launches);
    {   /* past the small-table span, within the two-kernel finish's limits */
        adacomp_segment big;
        memset(&big, 0, sizeof big);
        big.numel = ADACOMP_SMALL_TABLE_MAX_SPAN + 4;
        big.bin_len = 500;
        adacomp_plan_info bi;
        if (adacomp_plan_query(&big, 1, &bi) != ADACOMP_OK) return fail("plan_query big");
        if (bi.ntiles > ADACOMP_CHUNK_FINISH_MAX_TILES || bi.compress_launches != 3)
            return fail("two-kernel finish launches");
    }
    adacomp_plan* plan = NULL;
    if (adacomp_plan_create_ex(segs, 3, ADACOMP_PLAN_SEPARATE_FINISH | ADACOMP_PLAN_SINGLE_LAUNCH,
                               &plan) != ADACOMP_ERR_INVALID_ARGUMENT || plan != NULL)
        return fail("exclusive plan flags");
    segs[1].flags = 2;
    if (adacomp_plan_query(segs, 3, &info) != ADACOMP_ERR_INVALID_ARGUMENT) return fail("flags 2");
    segs[1].flags = 0;
    segs[1].offset = 99996;
    if (adacomp_plan_query(segs, 3, &info) != ADACOMP_ERR_OVERLAP) return fail("overlap");
    if (adacomp_plan_query(NULL, 0, &info) != ADACOMP_ERR_INVALID_ARGUMENT) return fail("null table");
    if (strcmp(adacomp_status_str(ADACOMP_ERR_CAPACITY), "buffer smaller than the plan requires") != 0)
        return fail("status_str");
    if (adacomp_compress(NULL, NULL, NULL, 0, NULL, 0, NULL, 0, NULL, NULL) != ADACOMP_ERR_INVALID_ARGUMENT)
        return fail("compress null plan");
    if (adacomp_decode_accumulate(NULL, NULL, 0, NULL, 0, 0, NULL, 0, NULL) != ADACOMP_ERR_INVALID_ARGUMENT)
        return fail("decode null plan");
    uint64_t bytes = 0;
    if (adacomp_decode_sgd_workspace_bytes(NULL, 1, &bytes) != ADACOMP_ERR_INVALID_ARGUMENT)
        return fail("sgd workspace null plan");
    adacomp_sgd sgd = {0.1f, 0.9f, 0.0f, 1.0f};
    adacomp_adam adam = {1e-3f, 0.9f, 0.999f, 1e-8f, 0.0f, 1.0f, 1u};
    if (adacomp_decode_sgd(NULL, NULL, 1, NULL, NULL, 0, &sgd, NULL, 0, NULL) != ADACOMP_ERR_INVALID_ARGUMENT)
        return fail("sgd null plan");
    if (adacomp_decode_adam(NULL, NULL, 1, NULL, NULL, NULL, 0, &adam, NULL, 0, NULL) != ADACOMP_ERR_INVALID_ARGUMENT)
        return fail("adam null plan");
    adacomp_timer* t = NULL;
    if (adacomp_timer_create(&t) != ADACOMP_OK || t == NULL) return fail("timer_create");
    double ms[ADACOMP_NUM_STAGES];
    uint64_t n[ADACOMP_NUM_STAGES];
    if (adacomp_timer_read(t, ms, n, ADACOMP_NUM_STAGES) != ADACOMP_OK) return fail("timer_read");
    for (int i = 0; i < ADACOMP_NUM_STAGES; ++i)
        if (n[i] != 0 || ms[i] != 0.0) return fail("fresh timer not empty");
    if (adacomp_timer_destroy(t) != ADACOMP_OK) return fail("timer_destroy");
    printf("OK host-only calls\n");
    return 0;
}
