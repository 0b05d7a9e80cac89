/* Runs every function of the CPU oracle (oracle/moe_oracle.c) on small
 * seeded inputs -- ragged sizes, T = 0, tokens without an expert, duplicate
 * ids, K > E -- so AddressSanitizer / UndefinedBehaviorSanitizer check its
 * indexing. Also asserts the layout's basic invariants. Test infrastructure. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int64_t orc_ceil_div(int64_t a, int64_t b);
int64_t orc_round_up4(int64_t n);
int64_t orc_num_max_pretrain(int64_t, int64_t, int64_t, int64_t);
int64_t orc_num_max_infer(int64_t, int64_t, int64_t);
int orc_validate_num_max(int64_t, int64_t);
int orc_check_capacity(int64_t, int64_t, int64_t);
int64_t orc_layout(const int32_t *ids, int64_t T, int64_t ntpr, int32_t E, int32_t K,
                   int32_t *counts, int32_t *offsets, int32_t *row_map, int32_t *src);
void orc_dispatch(const void *x, int64_t row_bytes, const float *scores, int32_t K,
                  const int32_t *src, int64_t total, void *x_e, float *s_e, int nthreads);
void orc_dispatch_rows(const void *x, int64_t row_bytes, const float *scores, int32_t K,
                       const int32_t *src, const int64_t *rows, int64_t n, void *out_x,
                       float *out_s);
uint16_t orc_f32_to_bf16(float f);
void orc_combine(const void *y_e, int dtype, int64_t D, const int32_t *row_map,
                 const float *scores, int64_t T, int32_t K, void *y, int nthreads);
void orc_combine_tokens(const void *y_e, int dtype, int64_t D, const int32_t *row_map,
                        const float *scores, int32_t K, const int64_t *tokens, int64_t n,
                        void *out);
void orc_combine_backward(const void *g, const void *y_e, int dtype, int64_t D,
                          const int32_t *row_map, const float *scores, int64_t T, int32_t K,
                          void *g_e, double *grad_s, int nthreads);
void orc_dispatch_backward(const void *h, int dtype, int64_t D, const int32_t *row_map,
                           int64_t T, int32_t K, void *gx, int nthreads);
void orc_topk_from_routing_map(const uint8_t *map, const float *probs, int64_t T, int32_t E,
                               int32_t K, int32_t *ids, float *scores, int32_t *n_experts);
void orc_dispatch_scaled(const void *x, int dtype, int64_t D, const float *scores, int32_t K,
                         const int32_t *src, int64_t total, void *x_e, int nthreads);
void orc_grouped_gemm(const uint16_t *x_e, const uint16_t *w, const int32_t *offsets, int32_t E,
                      int64_t Kd, int64_t N, double *out, int nthreads);
void orc_grouped_gemm_at(const uint16_t *x_e, const uint16_t *w, const int32_t *offsets,
                         int32_t E, int64_t Kd, int64_t N, const int64_t *rows,
                         const int64_t *cols, int64_t count, double *out, int nthreads);
uint16_t orc_f64_to_bf16(double v);
void orc_f64_to_bf16_n(const double *v, int64_t n, uint16_t *out);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void)      /* splitmix64, upper half */
{
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return (uint32_t)((z ^ (z >> 31)) >> 32);
}
static float rndf(void) { return (float)(rnd() % 2001) / 1000.0f - 1.0f; }

static int failures = 0;
#define EXPECT(c) do { if (!(c)) { fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, #c); ++failures; } } while (0)

static void run_case(int64_t T, int64_t ntpr, int32_t E, int32_t K, int64_t D, int dtype)
{
    int64_t n4 = orc_round_up4(ntpr);
    int64_t slots = n4 * K;
    int64_t elem = dtype == 0 ? 4 : 2;
    int32_t *ids = malloc(sizeof(int32_t) * (size_t)(T * K + 1));
    float *scores = malloc(sizeof(float) * (size_t)(T * K + 1));
    for (int64_t i = 0; i < T * K; ++i) {
        uint32_t r = rnd() % 10;
        ids[i] = r == 0 ? -1 : (r == 1 ? E + (int32_t)(rnd() % 3) : (int32_t)(rnd() % (uint32_t)E));
        scores[i] = rndf();
    }
    int32_t *counts = malloc(sizeof(int32_t) * (size_t)E);
    int32_t *offsets = malloc(sizeof(int32_t) * (size_t)(E + 1));
    int32_t *row_map = malloc(sizeof(int32_t) * (size_t)(slots + 1));
    int32_t *src = malloc(sizeof(int32_t) * (size_t)(slots + 1));
    int64_t total = orc_layout(ids, T, ntpr, E, K, counts, offsets, row_map, src);
    EXPECT(total >= 0 && total <= T * K);
    int64_t sum = 0;
    for (int32_t e = 0; e < E; ++e) sum += counts[e];
    EXPECT(sum == total && offsets[E] == total);
    for (int64_t i = T * K; i < slots; ++i) EXPECT(row_map[i] == -1);

    uint8_t *x = malloc((size_t)(T * D * elem + 1));
    for (int64_t i = 0; i < T * D * elem; ++i) x[i] = (uint8_t)(rnd() & 0x3F);  /* finite values */
    uint8_t *x_e = malloc((size_t)(total * D * elem + 1));
    float *s_e = malloc(sizeof(float) * (size_t)(total + 1));
    orc_dispatch(x, D * elem, scores, K, src, total, x_e, s_e, 2);
    if (total > 0) {
        int64_t rows[2] = {0, total - 1};
        uint8_t *ox = malloc((size_t)(2 * D * elem));
        float os[2];
        orc_dispatch_rows(x, D * elem, scores, K, src, rows, 2, ox, os);
        EXPECT(memcmp(ox, x_e, (size_t)(D * elem)) == 0);
        free(ox);
    }
    uint8_t *y = malloc((size_t)(T * D * elem + 1));
    orc_combine(x_e, dtype, D, row_map, scores, T, K, y, 2);
    if (T > 0) {
        int64_t tok[1] = {T - 1};
        uint8_t *oy = malloc((size_t)(D * elem));
        orc_combine_tokens(x_e, dtype, D, row_map, scores, K, tok, 1, oy);
        EXPECT(memcmp(oy, y + (T - 1) * D * elem, (size_t)(D * elem)) == 0);
        free(oy);
    }
    uint8_t *g_e = calloc((size_t)(total * D * elem + 1), 1);
    double *g_s = malloc(sizeof(double) * (size_t)(T * K + 1));
    orc_combine_backward(y, x_e, dtype, D, row_map, scores, T, K, g_e, g_s, 2);
    uint8_t *gx = malloc((size_t)(T * D * elem + 1));
    orc_dispatch_backward(g_e, dtype, D, row_map, T, K, gx, 2);
    orc_dispatch_scaled(x, dtype, D, scores, K, src, total, x_e, 2);

    /* routing map form of the same routing */
    uint8_t *map = calloc((size_t)(T * E + 1), 1);
    float *probs = calloc((size_t)(T * E + 1), sizeof(float));
    for (int64_t t = 0; t < T; ++t)
        for (int32_t k = 0; k < K; ++k) {
            int32_t e = ids[t * K + k];
            if (e >= 0 && e < E) { map[t * E + e] = 1; probs[t * E + e] = scores[t * K + k]; }
        }
    int32_t *mids = malloc(sizeof(int32_t) * (size_t)(T * K + 1));
    float *msc = malloc(sizeof(float) * (size_t)(T * K + 1));
    int32_t *nexp = malloc(sizeof(int32_t) * (size_t)(T + 1));
    orc_topk_from_routing_map(map, probs, T, E, K, mids, msc, nexp);

    /* expert step over the dispatched rows (bf16 bits of small values) */
    int64_t Kd = 8 * (1 + rnd() % 5), N = 8 * (1 + rnd() % 4);
    uint16_t *xb = malloc(sizeof(uint16_t) * (size_t)(total * Kd + 1));
    uint16_t *wb = malloc(sizeof(uint16_t) * (size_t)(E * N * Kd + 1));
    for (int64_t i = 0; i < total * Kd; ++i) xb[i] = orc_f32_to_bf16(rndf());
    for (int64_t i = 0; i < E * N * Kd; ++i) wb[i] = orc_f32_to_bf16(rndf());
    double *out = malloc(sizeof(double) * (size_t)(total * N + 1));
    orc_grouped_gemm(xb, wb, offsets, E, Kd, N, out, 2);
    if (total > 0) {
        int64_t r[2] = {0, total - 1}, c[2] = {0, N - 1};
        double at[2];
        orc_grouped_gemm_at(xb, wb, offsets, E, Kd, N, r, c, 2, at, 1);
        EXPECT(at[0] == out[0] && at[1] == out[(total - 1) * N + N - 1]);
    }
    uint16_t *ob = malloc(sizeof(uint16_t) * (size_t)(total * N + 1));
    orc_f64_to_bf16_n(out, total * N, ob);

    free(ids); free(scores); free(counts); free(offsets); free(row_map); free(src);
    free(x); free(x_e); free(s_e); free(y); free(g_e); free(g_s); free(gx);
    free(map); free(probs); free(mids); free(msc); free(nexp);
    free(xb); free(wb); free(out); free(ob);
}

int main(void)
{
    EXPECT(orc_ceil_div(7, 2) == 4 && orc_ceil_div(-1, 2) == -1 && orc_round_up4(13) == 16);
    EXPECT(orc_num_max_pretrain(1, 32768, 1, 1) == 32768 && orc_num_max_infer(100, 2, 2) == 25);
    EXPECT(orc_validate_num_max(8, 8) == 0 && orc_check_capacity(3, 4, 4) == 0);
    EXPECT(orc_check_capacity(5, 4, 8) != 0);
    const double special[] = {0.0, -0.0, 1.0 + 1.0 / 256, 1e-45, 3.4e38, -3.5e38, 1e300};
    for (unsigned i = 0; i < sizeof special / sizeof special[0]; ++i) (void)orc_f64_to_bf16(special[i]);
    /* T, ntpr, E, K, D, dtype */
    const int64_t cases[][6] = {
        {0, 4, 8, 2, 8, 0},   {1, 1, 1, 1, 8, 1},    {13, 13, 8, 3, 12, 0}, {61, 64, 8, 2, 16, 0},
        {5, 8, 2, 4, 16, 1},  /* K > E: duplicate ids */
        {77, 80, 16, 16, 24, 1}, {200, 203, 1024, 8, 8, 1}, {3, 7, 5, 5, 40, 0},
    };
    for (unsigned i = 0; i < sizeof cases / sizeof cases[0]; ++i)
        run_case(cases[i][0], cases[i][1], (int32_t)cases[i][2], (int32_t)cases[i][3],
                 cases[i][4], (int)cases[i][5]);
    printf("oracle driver: %d failures\n", failures);
    return failures == 0 ? 0 : 1;
}
