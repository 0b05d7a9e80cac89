/* A plain C11 consumer of include/moe.h, linked against libmoe_layout.so.
 *
 * It needs no GPU: it reports what the C compiler makes of the public
 * structs and constants (sizes, field offsets, values) as one JSON object,
 * and runs the host-only part of the documented call sequence (workspace
 * size, context creation on a caller-chosen address, workspace offsets,
 * tuning round trip, destruction) plus its error paths. The Python test
 * compares the report with the ctypes declarations of the binding. The
 * workspace address is never dereferenced: moe_create only carves offsets.
 */
#include "moe.h"

#include <stddef.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static int failures = 0;

static void expect(int cond, const char *what) {
    if (!cond) {
        ++failures;
        fprintf(stderr, "FAIL: %s\n", what);
    }
}

#define FIELD(type, f) printf("%s\"%s\": [%zu, %zu]", first ? "" : ", ", #f, \
                              offsetof(type, f), sizeof(((type *)0)->f)); first = 0

static void report_layouts(void) {
    int first;
    printf("\"moe_config\": {\"sizeof\": %zu, \"fields\": {", sizeof(moe_config));
    first = 1;
    FIELD(moe_config, num_max_tokens_per_rank);
    FIELD(moe_config, hidden);
    FIELD(moe_config, num_experts);
    FIELD(moe_config, topk);
    FIELD(moe_config, dtype);
    FIELD(moe_config, flags);
    printf("}}, ");

    printf("\"moe_buffers_desc\": {\"sizeof\": %zu, \"fields\": {", sizeof(moe_buffers_desc));
    first = 1;
    FIELD(moe_buffers_desc, workspace_bytes);
    FIELD(moe_buffers_desc, nmax4);
    FIELD(moe_buffers_desc, max_rows);
    FIELD(moe_buffers_desc, row_bytes);
    FIELD(moe_buffers_desc, max_tiles);
    FIELD(moe_buffers_desc, tile_slots);
    FIELD(moe_buffers_desc, counts);
    FIELD(moe_buffers_desc, offsets);
    FIELD(moe_buffers_desc, row_map);
    FIELD(moe_buffers_desc, src_map);
    FIELD(moe_buffers_desc, s_e);
    FIELD(moe_buffers_desc, x_e);
    FIELD(moe_buffers_desc, y);
    FIELD(moe_buffers_desc, block_hist);
    FIELD(moe_buffers_desc, map_ids);
    FIELD(moe_buffers_desc, map_scores);
    FIELD(moe_buffers_desc, map_n_experts);
    FIELD(moe_buffers_desc, g_e);
    FIELD(moe_buffers_desc, g_s);
    FIELD(moe_buffers_desc, g_x);
    printf("}}, ");

    printf("\"moe_tuning\": {\"sizeof\": %zu, \"fields\": {", sizeof(moe_tuning));
    first = 1;
    FIELD(moe_tuning, dispatch_segments);
    FIELD(moe_tuning, combine_segments);
    FIELD(moe_tuning, dispatch_nontemporal);
    FIELD(moe_tuning, combine_nontemporal);
    FIELD(moe_tuning, dispatch_block_waves);
    FIELD(moe_tuning, combine_block_waves);
    FIELD(moe_tuning, combine_store_nontemporal);
    FIELD(moe_tuning, layout_launches);
    FIELD(moe_tuning, dispatch_store_burst);
    FIELD(moe_tuning, combine_backward_store);
    FIELD(moe_tuning, dispatch_x_nontemporal);
    printf("}}, ");
}

static void report_constants(void) {
    printf("\"constants\": {\"MOE_OK\": %d, \"MOE_ERR_INVALID_ARG\": %d, "
           "\"MOE_ERR_CAPACITY\": %d, \"MOE_ERR_WORKSPACE\": %d, \"MOE_ERR_HIP\": %d, "
           "\"MOE_ERR_STATE\": %d, \"MOE_ERR_UNSUPPORTED\": %d, \"MOE_ERR_SCRATCH\": %d, "
           "\"MOE_FLAG_BACKWARD\": %d, \"MOE_MAX_EXPERTS\": %d, \"MOE_MAX_TOPK\": %d, "
           "\"MOE_WORKSPACE_ALIGN\": %d, \"MOE_F32\": %d, \"MOE_BF16\": %d, "
           "\"MOE_NOALLOC_SCRATCH_BYTES\": %d, \"MOE_WEIGHTS_ROW_MAJOR\": %d, "
           "\"MOE_WEIGHTS_TILED\": %d}, ",
           MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_CAPACITY, MOE_ERR_WORKSPACE, MOE_ERR_HIP,
           MOE_ERR_STATE, MOE_ERR_UNSUPPORTED, MOE_ERR_SCRATCH, MOE_FLAG_BACKWARD,
           MOE_MAX_EXPERTS, MOE_MAX_TOPK, MOE_WORKSPACE_ALIGN, (int)MOE_F32, (int)MOE_BF16,
           MOE_NOALLOC_SCRATCH_BYTES, MOE_WEIGHTS_ROW_MAJOR, MOE_WEIGHTS_TILED);
}

/* Every carved buffer lies inside the workspace and starts on the
 * workspace alignment. */
static void check_offsets(const moe_buffers_desc *d, int backward) {
    const int64_t off[] = {d->counts, d->offsets, d->row_map, d->src_map, d->s_e,
                           d->x_e,    d->y,       d->block_hist, d->map_ids,
                           d->map_scores, d->map_n_experts};
    for (size_t i = 0; i < sizeof(off) / sizeof(off[0]); ++i) {
        expect(off[i] >= 0 && off[i] < d->workspace_bytes, "offset inside the workspace");
        expect(off[i] % MOE_WORKSPACE_ALIGN == 0, "offset aligned");
    }
    expect(d->x_e + d->max_rows * d->row_bytes <= d->workspace_bytes, "x_e fits");
    if (backward) {
        expect(d->g_e + d->max_rows * d->row_bytes <= d->workspace_bytes, "g_e fits");
        expect(d->g_x + d->nmax4 * d->row_bytes <= d->workspace_bytes, "g_x fits");
    }
}

static void run_usage(void) {
    /* The DeepSeek-V3-shaped layer, forward and with backward buffers. */
    for (int backward = 0; backward <= 1; ++backward) {
        moe_config cfg = {.num_max_tokens_per_rank = 4096, .hidden = 7168, .num_experts = 256,
                          .topk = 8, .dtype = MOE_BF16,
                          .flags = backward ? MOE_FLAG_BACKWARD : 0};
        size_t bytes = 0;
        expect(moe_workspace_bytes(&cfg, &bytes) == MOE_OK, "workspace bytes");
        /* 4096 tokens x 8 slots x 7168 bf16 of expert rows at least. */
        expect(bytes >= (size_t)4096 * 8 * 7168 * 2, "workspace holds x_e");

        void *ws = (void *)(uintptr_t)(MOE_WORKSPACE_ALIGN * 4096);
        moe_ctx *ctx = NULL;
        expect(moe_create(&cfg, ws, bytes - 1, &ctx) == MOE_ERR_WORKSPACE && ctx == NULL,
               "short workspace refused");
        expect(moe_create(&cfg, (char *)ws + 16, bytes, &ctx) == MOE_ERR_WORKSPACE &&
                   ctx == NULL,
               "misaligned workspace refused");
        expect(moe_create(&cfg, ws, bytes, &ctx) == MOE_OK && ctx != NULL, "create");
        if (!ctx) continue;

        moe_buffers_desc d;
        memset(&d, 0, sizeof(d));
        expect(moe_workspace_offsets(ctx, &d) == MOE_OK, "offsets");
        expect(d.workspace_bytes == (int64_t)bytes, "desc workspace bytes");
        expect(d.nmax4 == 4096 && d.max_rows == 4096 * 8 && d.row_bytes == 7168 * 2,
               "desc sizes");
        check_offsets(&d, backward);

        moe_tuning t, back;
        expect(moe_get_tuning(ctx, &t) == MOE_OK, "get tuning");
        expect(moe_set_tuning(ctx, &t) == MOE_OK, "set tuning");
        expect(moe_get_tuning(ctx, &back) == MOE_OK, "get tuning again");
        expect(memcmp(&t, &back, sizeof(t)) == 0, "tuning round trip");

        /* A dispatch before any layout is a call-order error and a capacity
         * above the configured maximum a capacity error, both reported
         * before anything is enqueued; an empty batch needs no data. */
        int32_t *counts = (int32_t *)((char *)ws + d.counts);
        expect(moe_dispatch(ctx, NULL, NULL, NULL, counts, 0, 0, NULL) == MOE_ERR_STATE,
               "dispatch before layout refused");
        expect(moe_dispatch(ctx, NULL, NULL, NULL, counts, 0, 4097, NULL) == MOE_ERR_CAPACITY,
               "capacity above the maximum refused");
        expect(moe_dispatch(ctx, NULL, NULL, NULL, counts + 1, 0, 0, NULL) ==
                   MOE_ERR_INVALID_ARG,
               "counts other than the context's refused");
        expect(moe_destroy(ctx) == MOE_OK, "destroy");
    }

    /* Configuration errors. */
    moe_config bad = {.num_max_tokens_per_rank = 4096, .hidden = 7168,
                      .num_experts = MOE_MAX_EXPERTS + 1, .topk = 8, .dtype = MOE_BF16,
                      .flags = 0};
    size_t bytes = 0;
    const int st = moe_workspace_bytes(&bad, &bytes);
    expect(st < 0, "too many experts refused");
    expect(moe_strerror(st) != NULL && strlen(moe_strerror(st)) > 0, "strerror");
    bad.num_experts = 256;
    bad.topk = MOE_MAX_TOPK + 1;
    expect(moe_workspace_bytes(&bad, &bytes) < 0, "top-k above the maximum refused");
    expect(moe_workspace_bytes(NULL, &bytes) == MOE_ERR_INVALID_ARG, "null config refused");

    /* Capacity helpers. */
    expect(moe_round_up4(0) == 0 && moe_round_up4(5) == 8 && moe_round_up4(8) == 8,
           "round_up4");
    expect(moe_ceil_div(7, 2) == 4 && moe_ceil_div(0, 3) == 0, "ceil_div");
    expect(moe_check_capacity(3, 5, 8) == MOE_OK, "capacity relation holds");
    expect(moe_check_capacity(6, 5, 8) == MOE_ERR_CAPACITY, "T above ntpr refused");
    expect(moe_check_capacity(3, 9, 8) == MOE_ERR_CAPACITY, "ntpr above nmax refused");
}

int main(void) {
    printf("{");
    report_layouts();
    report_constants();
    run_usage();
    printf("\"failures\": %d}\n", failures);
    return failures == 0 ? 0 : 1;
}
