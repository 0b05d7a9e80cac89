// Drives every entry point of include/moe.h through the host code, with the
// kernel launchers stubbed out: valid calls, every documented error path and
// many configurations, so AddressSanitizer / UndefinedBehaviorSanitizer see
// all host-side arithmetic (sizes, carve-up, offsets, checks). Device
// pointers are fake, aligned addresses that are never dereferenced.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <initializer_list>

#include "moe.h"

namespace moe { extern int g_launches; }

static int failures = 0;
#define EXPECT(cond)                                                              \
    do {                                                                          \
        if (!(cond)) {                                                            \
            std::fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__,     \
                         __LINE__, #cond);                                        \
            ++failures;                                                           \
        }                                                                         \
    } while (0)

static void* fake(uintptr_t at) { return reinterpret_cast<void*>(at); }

static void one_config(int32_t nmax, int32_t D, int32_t E, int32_t K, int32_t dtype,
                       int32_t flags) {
    moe_config cfg = {nmax, D, E, K, dtype, flags};
    size_t bytes = 0;
    EXPECT(moe_workspace_bytes(&cfg, &bytes) == MOE_OK && bytes > 0);
    moe_ctx* ctx = nullptr;
    void* ws = fake(uintptr_t(1) << 40);
    EXPECT(moe_create(&cfg, ws, bytes - 1, &ctx) == MOE_ERR_WORKSPACE);
    EXPECT(moe_create(&cfg, fake((uintptr_t(1) << 40) + 16), bytes, &ctx) == MOE_ERR_WORKSPACE);
    EXPECT(moe_create(&cfg, ws, bytes, &ctx) == MOE_OK && ctx);
    moe_buffers_desc d;
    EXPECT(moe_workspace_offsets(ctx, &d) == MOE_OK);
    EXPECT(d.workspace_bytes == int64_t(bytes));
    EXPECT(d.counts >= 0 && d.offsets > d.counts && d.x_e > 0 && d.y > 0);
    const uintptr_t base = uintptr_t(1) << 40;
    const int32_t* counts = reinterpret_cast<const int32_t*>(base + d.counts);
    const int32_t* row_map = reinterpret_cast<const int32_t*>(base + d.row_map);
    void* p = fake(uintptr_t(1) << 41);
    const int32_t ntpr = nmax;
    for (int32_t T : {0, 1, ntpr / 2, ntpr}) {
        EXPECT(moe_layout(ctx, static_cast<const int32_t*>(p), T, ntpr, nullptr) == MOE_OK);
        EXPECT(moe_dispatch(ctx, p, static_cast<const float*>(p), static_cast<const int32_t*>(p),
                            counts, T, ntpr, nullptr) == MOE_OK);
        EXPECT(moe_dispatch_scaled(ctx, p, static_cast<const float*>(p),
                                   static_cast<const int32_t*>(p), counts, T, ntpr,
                                   nullptr) == MOE_OK);
        EXPECT(moe_layout_dispatch(ctx, p, static_cast<const float*>(p),
                                   static_cast<const int32_t*>(p), T, ntpr, nullptr) == MOE_OK);
        if (T > 0)
            EXPECT(moe_layout_dispatch(ctx, nullptr, static_cast<const float*>(p),
                                       static_cast<const int32_t*>(p), T, ntpr, nullptr) ==
                   MOE_ERR_INVALID_ARG);
        void* y = nullptr;
        EXPECT(moe_combine(ctx, p, row_map, static_cast<const float*>(p), T, ntpr, nullptr, &y) ==
               MOE_OK);
        EXPECT(moe_combine(ctx, p, row_map, nullptr, T, ntpr, nullptr, &y) == MOE_OK);
        void *ge = nullptr, *gx = nullptr;
        float* gs = nullptr;
        const int want = (flags & MOE_FLAG_BACKWARD) ? MOE_OK : MOE_ERR_UNSUPPORTED;
        EXPECT(moe_combine_backward(ctx, p, p, row_map, static_cast<const float*>(p), nullptr,
                                    T, ntpr, nullptr, &ge, &gs) == want);
        EXPECT(moe_combine_backward(ctx, p, p, row_map, static_cast<const float*>(p),
                                    static_cast<const int32_t*>(p), T, ntpr, nullptr, &ge,
                                    &gs) == want);
        EXPECT(moe_dispatch_backward(ctx, p, row_map, T, ntpr, nullptr, &gx) == want);
        int32_t *ids = nullptr, *nexp = nullptr;
        float* sc = nullptr;
        EXPECT(moe_topk_from_routing_map(ctx, static_cast<const uint8_t*>(p),
                                         static_cast<const float*>(p), T, nullptr, &ids, &sc,
                                         &nexp) == MOE_OK);
    }
    // call order and capacity errors
    EXPECT(moe_layout(ctx, static_cast<const int32_t*>(p), 3, 8 > nmax ? nmax : 8, nullptr) ==
           MOE_OK);
    EXPECT(moe_dispatch(ctx, p, static_cast<const float*>(p), static_cast<const int32_t*>(p),
                        counts, 2, 8 > nmax ? nmax : 8, nullptr) == MOE_ERR_STATE);
    EXPECT(moe_layout(ctx, static_cast<const int32_t*>(p), nmax + 1, nmax + 1, nullptr) ==
           MOE_ERR_CAPACITY);
    EXPECT(moe_layout(ctx, static_cast<const int32_t*>(p), -1, nmax, nullptr) ==
           MOE_ERR_CAPACITY);
    EXPECT(moe_layout_dispatch(ctx, p, static_cast<const float*>(p),
                               static_cast<const int32_t*>(p), nmax + 1, nmax + 1, nullptr) ==
           MOE_ERR_CAPACITY);
    EXPECT(moe_layout_dispatch(nullptr, p, static_cast<const float*>(p),
                               static_cast<const int32_t*>(p), 0, 0, nullptr) ==
           MOE_ERR_INVALID_ARG);
    EXPECT(moe_dispatch(ctx, p, static_cast<const float*>(p), static_cast<const int32_t*>(p),
                        counts + 1, 0, nmax, nullptr) != MOE_OK);
    moe_tuning t;
    EXPECT(moe_get_tuning(ctx, &t) == MOE_OK);
    t.dispatch_segments = 3;
    t.combine_block_waves = 2;
    EXPECT(moe_set_tuning(ctx, &t) == MOE_OK);
    t.dispatch_segments = 99;
    EXPECT(moe_set_tuning(ctx, &t) != MOE_OK);
    // both layout forms and both dispatch store forms, forced, then bad values
    for (int32_t lf : {1, 2, -1}) {
        for (int32_t sb : {1, 2}) {
            EXPECT(moe_get_tuning(ctx, &t) == MOE_OK);
            t.layout_launches = lf;
            t.dispatch_store_burst = sb;
            EXPECT(moe_set_tuning(ctx, &t) == MOE_OK);
            EXPECT(moe_layout(ctx, static_cast<const int32_t*>(p), ntpr, ntpr, nullptr) == MOE_OK);
            EXPECT(moe_dispatch(ctx, p, static_cast<const float*>(p),
                                static_cast<const int32_t*>(p), counts, ntpr, ntpr,
                                nullptr) == MOE_OK);
        }
    }
    EXPECT(moe_get_tuning(ctx, &t) == MOE_OK);
    t.layout_launches = 3;
    EXPECT(moe_set_tuning(ctx, &t) == MOE_ERR_INVALID_ARG);
    t.layout_launches = 0;
    t.dispatch_store_burst = -1;
    EXPECT(moe_set_tuning(ctx, &t) == MOE_ERR_INVALID_ARG);
    EXPECT(moe_destroy(ctx) == MOE_OK);
}

int main() {
    // configurations: small, ragged, DSV3-like, maximal E and K, prefill-sized
    const int32_t cfgs[][6] = {
        {64, 128, 8, 2, MOE_F32, 0},           {5, 8, 1, 1, MOE_BF16, 0},
        {4096, 7168, 256, 8, MOE_BF16, 0},     {4096, 7168, 256, 8, MOE_BF16, MOE_FLAG_BACKWARD},
        {300, 64, 1024, 16, MOE_BF16, MOE_FLAG_BACKWARD}, {32768, 7168, 256, 8, MOE_BF16, 0},
        {13, 36, 3, 5, MOE_F32, MOE_FLAG_BACKWARD},
    };
    for (const auto& c : cfgs) one_config(c[0], c[1], c[2], c[3], c[4], c[5]);

    // invalid configurations
    const int32_t bad[][6] = {
        {0, 128, 8, 2, MOE_F32, 0},   {64, 3, 8, 2, MOE_F32, 0},    {64, 128, 0, 2, MOE_F32, 0},
        {64, 128, 1025, 2, MOE_F32, 0}, {64, 128, 8, 0, MOE_F32, 0}, {64, 128, 8, 17, MOE_F32, 0},
        {64, 128, 8, 2, 7, 0},        {64, 128, 8, 2, MOE_F32, 4},  {0x7FFFFFF0, 64, 8, 16, MOE_F32, 0},
    };
    for (const auto& c : bad) {
        moe_config cfg = {c[0], c[1], c[2], c[3], c[4], c[5]};
        size_t bytes = 0;
        EXPECT(moe_workspace_bytes(&cfg, &bytes) != MOE_OK);
    }
    EXPECT(moe_workspace_bytes(nullptr, nullptr) != MOE_OK);
    EXPECT(moe_destroy(nullptr) == MOE_OK);

    // capacity helpers
    EXPECT(moe_ceil_div(10, 4) == 3 && moe_ceil_div(-1, 4) == -1 && moe_ceil_div(1, 0) == -1);
    EXPECT(moe_round_up4(5) == 8 && moe_round_up4(0) == 0 && moe_round_up4(-2) == -1);
    EXPECT(moe_num_max_tokens_pretrain(2, 4097, 2, 1) == 2 * 2049);
    EXPECT(moe_num_max_tokens_infer(32768, 1, 1) == 32768);
    EXPECT(moe_validate_num_max(100, 99) == MOE_OK && moe_validate_num_max(0, 0) != MOE_OK);
    EXPECT(moe_check_capacity(3, 4, 8) == MOE_OK && moe_check_capacity(5, 4, 8) != MOE_OK);
    for (int s = -8; s <= 0; ++s) EXPECT(moe_strerror(s) != nullptr);

    // layout without a context (static scratch above 32768 slots)
    {
        void* q = fake(uintptr_t(1) << 41);
        const int32_t* ids = static_cast<const int32_t*>(q);
        int32_t* o = static_cast<int32_t*>(q);
        const int32_t sizes[][4] = {  // T, ntpr, E, K
            {0, 0, 8, 2}, {61, 64, 8, 2}, {4096, 4096, 256, 8}, {8191, 8192, 128, 8},
            {32768, 32768, 256, 8}, {131072, 131072, 1024, 8}, {0, 524288, 256, 8},
        };
        for (const auto& c : sizes)
            EXPECT(moe_layout_noalloc(c[0] ? ids : nullptr, c[0], c[1], c[2], c[3], o, o, o, o,
                                      nullptr) == MOE_OK);
        EXPECT(moe_layout_noalloc(ids, 0, 131076, 1024, 8, o, o, o, o, nullptr) == MOE_ERR_SCRATCH);
        EXPECT(moe_layout_noalloc(ids, 0, 524292, 256, 8, o, o, o, o, nullptr) == MOE_ERR_SCRATCH);
        EXPECT(moe_layout_noalloc(ids, 9, 8, 8, 2, o, o, o, o, nullptr) == MOE_ERR_CAPACITY);
        EXPECT(moe_layout_noalloc(ids, 8, 8, 8, 2, o, o, nullptr, o, nullptr) ==
               MOE_ERR_INVALID_ARG);
        EXPECT(moe_layout_noalloc(nullptr, 8, 8, 8, 2, o, o, o, o, nullptr) == MOE_ERR_INVALID_ARG);
        EXPECT(moe_layout_noalloc(ids, 8, 8, 0, 2, o, o, o, o, nullptr) == MOE_ERR_INVALID_ARG);
    }

    // expert step
    void* p = fake(uintptr_t(1) << 41);
    const int32_t* off = static_cast<const int32_t*>(p);
    for (int lay : {MOE_WEIGHTS_ROW_MAJOR, MOE_WEIGHTS_TILED})
        for (int tile : {0, 64, 128}) {
            EXPECT(moe_grouped_gemm(p, p, off, 256, 32768, 7168, 4096, p, tile, lay, nullptr) ==
                   MOE_OK);
            EXPECT(moe_grouped_gemm(p, p, off, 5, 37, 72, 200, p, tile, lay, nullptr) == MOE_OK);
        }
    EXPECT(moe_grouped_gemm(p, p, off, 256, 32768, 7168, 4096, p, 0, 2, nullptr) != MOE_OK);
    EXPECT(moe_grouped_gemm(p, p, off, 256, 32768, 7166, 4096, p, 0, 0, nullptr) != MOE_OK);
    EXPECT(moe_grouped_gemm(p, p, off, 256, int64_t(1) << 31, 64, 64, p, 0, 0, nullptr) != MOE_OK);
    EXPECT(moe_tiled_weights_bytes(256, 4096, 7168) == int64_t(256) * 4096 * 7168 * 2);
    EXPECT(moe_tiled_weights_bytes(5, 200, 72) == int64_t(5) * 224 * 128 * 2);
    EXPECT(moe_tiled_weights_bytes(0, 8, 8) == -1);
    EXPECT(moe_tile_expert_weights(p, 256, 4096, 7168, p, nullptr) == MOE_OK);
    EXPECT(moe_tile_expert_weights(p, 1024, 16384, 16384, p, nullptr) == MOE_OK);
    EXPECT(moe_tile_expert_weights(nullptr, 4, 64, 64, p, nullptr) != MOE_OK);

    std::printf("host driver: %d launches stubbed, %d failures\n", moe::g_launches, failures);
    return failures == 0 ? 0 : 1;
}
