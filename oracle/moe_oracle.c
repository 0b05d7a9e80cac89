/*
 * CPU oracle for MoE token routing layout, dispatch and combine.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may include, link
 * or call this file: only the tests, the smoke check and the benchmark's
 * CPU-baseline leg use it. It shares no code, header or constant with the
 * HIP library and is built with plain gcc (-O2 -ffp-contract=off, no
 * fast-math), so every floating-point operation below is the one written.
 *
 * Every function is the plain definition of what the method computes, written
 * out in the order the pages describe; nothing is blocked, fused or reordered.
 * Sources (web pages, by title and section):
 *   [TT]  "Unify expert parallel token dispatcher API" (torchtitan PR 3970):
 *         "API design" (the dispatch signature and the capacity relation
 *         T <= num_tokens_per_rank <= num_max_tokens_per_rank),
 *         "Capacity derivation" (pretraining and vLLM inference formulas, and
 *         the validation of an explicit maximum).
 *   [NA]  "fix(moe): equalize and align per-rank token counts for HybridEP
 *         dispatch" (NeMo Automodel PR 3641): "Problem" (4-token alignment),
 *         "Fix" (pad to the aligned extent; padded rows route to no expert
 *         with zero probability; combine slices the padding off), "Testing"
 *         (identity experts: each token's output depends only on its routing).
 *   [UC]  "ep: graph-safe worst-token HT dispatch+combine" (uccl PR 18):
 *         "Internode" items 2 and 3 (device-side per-expert counts; the true
 *         total comes from a device-side prefix sum).
 * Readings where the pages are silent (all listed in the design notes):
 *   - rows of one expert are ordered by ascending flattened index t*K+k;
 *   - "no expert" is any id outside [0,E), the sentinel being -1;
 *   - the combine accumulates in fp32 with fused multiply-add, slots in
 *     ascending k order, starting from +0.0; a no-expert slot's score is
 *     never read;
 *   - bf16 output rounds to nearest even; every NaN becomes 0x7FC0.
 *
 * Floating-point ids: dtype 0 = fp32, 1 = bf16 (stored as uint16 bits).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_NONE (-1)

/* ---------------------------------------------------------------------- */
/* Capacity ([TT] "API design", "Capacity derivation"; [NA] "Problem", "Fix") */

/* ceil(a / b) for a >= 0, b >= 1; -1 for arguments outside that domain. */
int64_t orc_ceil_div(int64_t a, int64_t b)
{
    if (a < 0 || b < 1) return -1;
    return (a + b - 1) / b;
}

/* Smallest multiple of 4 that is >= n (n >= 0); -1 if n < 0. */
int64_t orc_round_up4(int64_t n)
{
    if (n < 0) return -1;
    return 4 * orc_ceil_div(n, 4);
}

/* Pretraining: local_batch_size * ceil_div(seq_len, cp * tp). */
int64_t orc_num_max_pretrain(int64_t local_batch, int64_t seq_len,
                             int64_t cp, int64_t tp)
{
    if (local_batch < 0 || cp < 1 || tp < 1) return -1;
    int64_t per_shard = orc_ceil_div(seq_len, cp * tp);
    if (per_shard < 0) return -1;
    return local_batch * per_shard;
}

/* vLLM inference: ceil_div(max_num_batched_tokens, cp * tp). */
int64_t orc_num_max_infer(int64_t max_num_batched_tokens, int64_t cp, int64_t tp)
{
    if (cp < 1 || tp < 1) return -1;
    return orc_ceil_div(max_num_batched_tokens, cp * tp);
}

/* An explicitly configured maximum must be positive (else 1) and at least
 * the derived requirement (else 2); 0 when valid. */
int orc_validate_num_max(int64_t configured, int64_t derived)
{
    if (configured <= 0) return 1;
    if (configured < derived) return 2;
    return 0;
}

/* The capacity relation of [TT] "API design", with a positive maximum:
 * 0 <= T <= ntpr <= nmax and nmax >= 1. Rounding both capacities up to a
 * multiple of 4 ([NA] "Fix") keeps round_up4(ntpr) <= round_up4(nmax).
 * 0 when it holds, 1 otherwise. */
int orc_check_capacity(int64_t T, int64_t ntpr, int64_t nmax)
{
    if (nmax < 1 || T < 0) return 1;
    if (T > ntpr || ntpr > nmax) return 1;
    return 0;
}

/* ---------------------------------------------------------------------- */
/* Layout ([TT] "API design": per-expert token counts; [UC] "Internode" 2, 3;
 * [NA] "Fix": padded rows route to no expert)                            */

/* Expert of flattened slot i = t*K + k, or ORC_NONE. Rows t >= T are the
 * padding of the current capacity: they route to no expert and their ids
 * are never read. */
static int32_t orc_expert_of(const int32_t *ids, int64_t T, int32_t E,
                             int32_t K, int64_t i)
{
    if (i / K >= T) return ORC_NONE;
    int32_t e = ids[i];
    if (e < 0 || e >= E) return ORC_NONE;
    return e;
}

/*
 * Stable counting sort of the flattened slots by expert.
 *   counts[e]    = number of slots routed to e                (E entries)
 *   offsets[e]   = exclusive prefix sum of counts; offsets[E] = total
 *   row_map[t*K+k] = row of slot (t,k) in the expert-major buffer, -1 for
 *                  no expert, for every t < round_up4(ntpr)
 *   src[row]     = t*K + k of the slot stored at that row, rows [0,total)
 * Returns total, or -1 if 0 <= T <= ntpr fails ([TT] "API design").
 */
int64_t orc_layout(const int32_t *ids, int64_t T, int64_t ntpr, int32_t E,
                   int32_t K, int32_t *counts, int32_t *offsets,
                   int32_t *row_map, int32_t *src)
{
    if (E < 1 || K < 1) return -1;
    /* [TT] "API design": T <= num_tokens_per_rank; the padding of [NA]
     * "Fix" only adds rows past ntpr, it never admits more tokens. */
    if (T < 0 || ntpr < 0 || T > ntpr) return -1;
    int64_t n = orc_round_up4(ntpr) * K;

    for (int32_t e = 0; e < E; ++e) counts[e] = 0;
    for (int64_t i = 0; i < n; ++i) {
        int32_t e = orc_expert_of(ids, T, E, K, i);
        if (e != ORC_NONE) counts[e] += 1;
    }

    offsets[0] = 0;
    for (int32_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];

    /* cursor[e] walks expert e's segment; slots are visited in ascending
     * t, then k, so equal experts keep their flattened order. */
    int32_t *cursor = (int32_t *)malloc((size_t)E * sizeof(int32_t));
    if (!cursor) return -1;
    for (int32_t e = 0; e < E; ++e) cursor[e] = offsets[e];
    for (int64_t i = 0; i < n; ++i) {
        int32_t e = orc_expert_of(ids, T, E, K, i);
        if (e == ORC_NONE) {
            row_map[i] = -1;
        } else {
            int32_t r = cursor[e]++;
            row_map[i] = r;
            src[r] = (int32_t)i;
        }
    }
    free(cursor);
    return offsets[E];
}

/* ---------------------------------------------------------------------- */
/* Dispatch ([TT] "API design", "Backend behavior": the permuted output of
 * one dispatch; [NA] "Fix")                                              */

/* Row r of the expert-major buffers: x_e[r] = x[t], s_e[r] = scores[t][k]
 * where (t,k) is the slot stored at r. Bit copies. */
static void orc_dispatch_row(const uint8_t *x, int64_t row_bytes,
                             const float *scores, int32_t K,
                             const int32_t *src, int64_t r,
                             uint8_t *xe_row, float *se_val)
{
    int64_t slot = src[r];
    int64_t t = slot / K;
    memcpy(xe_row, x + t * row_bytes, (size_t)row_bytes);
    memcpy(se_val, scores + slot, sizeof(float));
}

/* All rows [0,total). nthreads > 1 splits rows over OpenMP threads. */
void orc_dispatch(const void *x, int64_t row_bytes, const float *scores,
                  int32_t K, const int32_t *src, int64_t total,
                  void *x_e, float *s_e, int nthreads)
{
    const uint8_t *xb = (const uint8_t *)x;
    uint8_t *xeb = (uint8_t *)x_e;
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (int64_t r = 0; r < total; ++r)
        orc_dispatch_row(xb, row_bytes, scores, K, src, r,
                         xeb + r * row_bytes, s_e + r);
}

/* Only the listed rows, written densely to out_x[n][row_bytes], out_s[n]. */
void orc_dispatch_rows(const void *x, int64_t row_bytes, const float *scores,
                       int32_t K, const int32_t *src, const int64_t *rows,
                       int64_t n, void *out_x, float *out_s)
{
    for (int64_t j = 0; j < n; ++j)
        orc_dispatch_row((const uint8_t *)x, row_bytes, scores, K, src, rows[j],
                         (uint8_t *)out_x + j * row_bytes, out_s + j);
}

/* ---------------------------------------------------------------------- */
/* Combine ([NA] "Fix": combine slices the padding off; "Testing": with
 * identity experts a token's output depends only on its own routing)      */

static float orc_bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round to nearest, ties to even; any NaN becomes the quiet NaN 0x7FC0. */
uint16_t orc_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if (isnan(f)) return 0x7FC0;
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

static float orc_load_elem(const void *buf, int dtype, int64_t idx)
{
    if (dtype == 0) return ((const float *)buf)[idx];
    return orc_bf16_to_f32(((const uint16_t *)buf)[idx]);
}

/* y_row = sum over k = 0..K-1 with row_map[t][k] >= 0 of
 *         scores[t][k] * y_e[row_map[t][k]], in fp32 with fused multiply-add,
 *         ascending k, from +0.0; stored in the element dtype. */
static void orc_combine_token(const void *y_e, int dtype, int64_t D,
                              const int32_t *row_map, const float *scores,
                              int32_t K, int64_t t, void *y_row)
{
    for (int64_t d = 0; d < D; ++d) {
        float acc = 0.0f;
        for (int32_t k = 0; k < K; ++k) {
            int32_t r = row_map[t * K + k];
            if (r < 0) continue;
            float v = orc_load_elem(y_e, dtype, (int64_t)r * D + d);
            acc = fmaf(scores[t * K + k], v, acc);
        }
        if (dtype == 0)
            ((float *)y_row)[d] = acc;
        else
            ((uint16_t *)y_row)[d] = orc_f32_to_bf16(acc);
    }
}

/* Tokens [0,T): y is [T][D] in the element dtype. */
void orc_combine(const void *y_e, int dtype, int64_t D, const int32_t *row_map,
                 const float *scores, int64_t T, int32_t K, void *y,
                 int nthreads)
{
    int64_t elem = dtype == 0 ? 4 : 2;
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (int64_t t = 0; t < T; ++t)
        orc_combine_token(y_e, dtype, D, row_map, scores, K, t,
                          (uint8_t *)y + t * D * elem);
}

/* Only the listed tokens, written densely to out[n][D]. */
void orc_combine_tokens(const void *y_e, int dtype, int64_t D,
                        const int32_t *row_map, const float *scores, int32_t K,
                        const int64_t *tokens, int64_t n, void *out)
{
    int64_t elem = dtype == 0 ? 4 : 2;
    for (int64_t j = 0; j < n; ++j)
        orc_combine_token(y_e, dtype, D, row_map, scores, K, tokens[j],
                          (uint8_t *)out + j * D * elem);
}

/* ---------------------------------------------------------------------- */
/* Backward ([NA] "Testing": the unequal-count run must reproduce the
 * equal-count run bitwise in forward and backward). The derivatives of the
 * forward definitions above:
 *   combine: y[t] = sum_k s[t][k] * y_e[r(t,k)]
 *     dL/dy_e[r(t,k)] = s[t][k] * dL/dy[t]
 *     dL/ds[t][k]     = <dL/dy[t], y_e[r(t,k)]>        (0 for no expert)
 *   dispatch: x_e[r(t,k)] = x[t]
 *     dL/dx[t] = sum_k dL/dx_e[r(t,k)]                  (+0.0 if none)
 * Precision: the scaled copy is one fp32 product rounded to the element
 * dtype; the gather-sum is fp32, slots in ascending k, from +0.0; the dot
 * product is the exact value computed in fp64 (its fp32 evaluation order
 * on the GPU is not fixed by the definition).                          */

static void orc_store_elem(void *buf, int dtype, int64_t idx, float v)
{
    if (dtype == 0)
        ((float *)buf)[idx] = v;
    else
        ((uint16_t *)buf)[idx] = orc_f32_to_bf16(v);
}

/* g [T][D], y_e [rows][D] (element dtype), row_map [T][K], scores [T][K].
 * Writes g_e rows r(t,k) (other rows untouched) and grad_s [T][K] (fp64). */
void orc_combine_backward(const void *g, const void *y_e, int dtype, int64_t D,
                          const int32_t *row_map, const float *scores,
                          int64_t T, int32_t K, void *g_e, double *grad_s,
                          int nthreads)
{
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t k = 0; k < K; ++k) {
            int32_t r = row_map[t * K + k];
            if (r < 0) {
                grad_s[t * K + k] = 0.0;
                continue;
            }
            float s = scores[t * K + k];
            double dot = 0.0;
            for (int64_t d = 0; d < D; ++d) {
                float gv = orc_load_elem(g, dtype, t * D + d);
                float yv = orc_load_elem(y_e, dtype, (int64_t)r * D + d);
                dot += (double)gv * (double)yv;
                orc_store_elem(g_e, dtype, (int64_t)r * D + d, s * gv);
            }
            grad_s[t * K + k] = dot;
        }
    }
}

/* h [rows][D] (element dtype), row_map [T][K]: gx [T][D]. */
void orc_dispatch_backward(const void *h, int dtype, int64_t D,
                           const int32_t *row_map, int64_t T, int32_t K,
                           void *gx, int nthreads)
{
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t d = 0; d < D; ++d) {
            float acc = 0.0f;
            for (int32_t k = 0; k < K; ++k) {
                int32_t r = row_map[t * K + k];
                if (r < 0) continue;
                acc = acc + orc_load_elem(h, dtype, (int64_t)r * D + d);
            }
            orc_store_elem(gx, dtype, t * D + d, acc);
        }
    }
}

/* ---------------------------------------------------------------------- */
/* Input and weighting variants ([NA] "Fix": HybridEP's dispatcher takes a
 * boolean routing map [T][E] with probabilities [T][E]; padded rows are
 * all-False with zero probabilities).                                    */

/* Top-k form of a routing map: slot k of token t is the k-th expert e in
 * ascending order with map[t][e] != 0, score probs[t][e]; slots past the
 * token's experts get id -1 and score 0. n_experts[t] = number of experts
 * in the row (a row with more than K keeps its K lowest). */
void orc_topk_from_routing_map(const uint8_t *map, const float *probs, int64_t T,
                               int32_t E, int32_t K, int32_t *ids, float *scores,
                               int32_t *n_experts)
{
    for (int64_t t = 0; t < T; ++t) {
        int32_t n = 0;
        for (int32_t e = 0; e < E; ++e) {
            if (!map[t * E + e]) continue;
            if (n < K) {
                ids[t * K + n] = e;
                memcpy(&scores[t * K + n], &probs[t * E + e], sizeof(float));
            }
            ++n;
        }
        for (int32_t k = n; k < K; ++k) {
            ids[t * K + k] = -1;
            scores[t * K + k] = 0.0f;
        }
        n_experts[t] = n;
    }
}

/* Dispatch with the scores applied: x_e[r] = s[t][k] * x[t], one fp32
 * product rounded to the element dtype, for rows [0,total). */
void orc_dispatch_scaled(const void *x, int dtype, int64_t D, const float *scores,
                         int32_t K, const int32_t *src, int64_t total, void *x_e,
                         int nthreads)
{
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (int64_t r = 0; r < total; ++r) {
        int64_t slot = src[r];
        int64_t t = slot / K;
        float s = scores[slot];
        for (int64_t d = 0; d < D; ++d)
            orc_store_elem(x_e, dtype, r * D + d, s * orc_load_elem(x, dtype, t * D + d));
    }
}

/* ---------------------------------------------------------------------- */
/* Expert step between dispatch and combine ([UC] "Tests": layout, dispatch,
 * expert and combine run as one captured graph, checked against an analytic
 * oracle; "Internode" item 2: the expert step takes its per-expert row counts
 * from device memory). Reading: each expert is one linear map, its weight
 * stored as N rows of Kd elements (a linear layer's [out][in] layout).     */

static double orc_bf16_to_f64(uint16_t h)
{
    return (double)orc_bf16_to_f32(h);
}

/* Dot product of row r of x_e with row n of expert e's weight, in fp64. */
static double orc_expert_dot(const uint16_t *x_e, const uint16_t *w, int32_t e,
                             int64_t Kd, int64_t N, int64_t r, int64_t n)
{
    const uint16_t *xr = x_e + r * Kd;
    const uint16_t *wr = w + ((int64_t)e * N + n) * Kd;
    double acc = 0.0;
    for (int64_t d = 0; d < Kd; ++d)
        acc += orc_bf16_to_f64(xr[d]) * orc_bf16_to_f64(wr[d]);
    return acc;
}

/*
 * x_e [rows][Kd] bf16, w [E][N][Kd] bf16, offsets [E+1] (exclusive prefix sum
 * of the per-expert row counts). For every expert e and every row r with
 * offsets[e] <= r < offsets[e+1]:
 *     out[r][n] = sum over d of x_e[r][d] * w[e][n][d]      (fp64)
 * Rows outside every segment are not written.
 */
void orc_grouped_gemm(const uint16_t *x_e, const uint16_t *w, const int32_t *offsets,
                      int32_t E, int64_t Kd, int64_t N, double *out, int nthreads)
{
    if (nthreads < 1) nthreads = 1;
    for (int32_t e = 0; e < E; ++e) {
        int64_t r0 = offsets[e], r1 = offsets[e + 1];
#pragma omp parallel for num_threads(nthreads) schedule(static)
        for (int64_t r = r0; r < r1; ++r)
            for (int64_t n = 0; n < N; ++n)
                out[r * N + n] = orc_expert_dot(x_e, w, e, Kd, N, r, n);
    }
}

/* The same values at count chosen positions (rows[i], cols[i]); a row that
 * lies in no segment gives NaN. For outputs too large to form whole. */
void orc_grouped_gemm_at(const uint16_t *x_e, const uint16_t *w, const int32_t *offsets,
                         int32_t E, int64_t Kd, int64_t N, const int64_t *rows,
                         const int64_t *cols, int64_t count, double *out, int nthreads)
{
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        int32_t owner = -1;
        for (int32_t e = 0; e < E; ++e)
            if (offsets[e] <= rows[i] && rows[i] < offsets[e + 1]) owner = e;
        out[i] = owner < 0 ? NAN : orc_expert_dot(x_e, w, owner, Kd, N, rows[i], cols[i]);
    }
}

/* fp64 to bf16 bits in one rounding (nearest, ties to even; the detour
 * through fp32 would round twice). NaN becomes 0x7FC0; magnitudes that
 * round past the largest finite bf16 become infinity. */
uint16_t orc_f64_to_bf16(double v)
{
    if (isnan(v)) return 0x7FC0;
    double a = fabs(v), r;
    if (a == 0.0 || isinf(a)) {
        r = a;
    } else {
        int ex;
        frexp(a, &ex);                  /* a = m * 2^ex, 0.5 <= m < 1 */
        int qe = ex - 8;                /* 8 significant bits */
        if (qe < -133) qe = -133;       /* spacing of bf16 subnormals */
        r = ldexp(nearbyint(ldexp(a, -qe)), qe);
        if (r >= 0x1p128) r = INFINITY;
    }
    float f = (float)copysign(r, v);    /* exact: r is a bf16 value */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

void orc_f64_to_bf16_n(const double *v, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f64_to_bf16(v[i]);
}
