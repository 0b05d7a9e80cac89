/*
 * moe.h - C ABI of the MI355X (gfx950) MoE token layout / dispatch / combine
 * library (libmoe_layout.so).
 *
 * The library does the local, single-GPU work of expert-parallel token
 * dispatch: it sorts a batch's top-k routing into an expert-major layout,
 * permutes hidden-state rows and their routing scores into a persistent
 * expert-major buffer, and gathers expert outputs back into token order as a
 * score-weighted sum. Sources (web pages, by title and section):
 *   [TT] "Unify expert parallel token dispatcher API" (torchtitan PR 3970):
 *        "API design" (dispatch signature; lifetime maximum vs current
 *        capacity; T <= num_tokens_per_rank <= num_max_tokens_per_rank;
 *        storage allocated once, never grown, stable addresses for graph
 *        capture), "Capacity derivation".
 *   [NA] "fix(moe): equalize and align per-rank token counts for HybridEP
 *        dispatch" (NeMo Automodel PR 3641): "Problem" (counts must be a
 *        multiple of 4), "Fix" (padded rows route to no expert with zero
 *        probability; combine slices the padding off; no extra copies).
 *   [UC] "ep: graph-safe worst-token HT dispatch+combine" (uccl PR 18):
 *        "Internode" items 1-3 (no host handshake, per-expert counts on the
 *        device, the true total from a device-side prefix sum), "Intranode"
 *        (no host-visible counter shared between calls).
 *
 * Conventions for every entry point:
 *   - Pointers named d_* are HIP device memory on the current device; all
 *     other pointers are host memory. Element types are fixed: ids int32,
 *     scores float32, hidden states fp32 or bf16 (config dtype).
 *   - Matrices are row-major and contiguous: ids and scores [T][K], hidden
 *     states [T][hidden].
 *   - Device pointers to hidden-state rows (x, expert outputs and their
 *     gradients) must be 16-byte aligned, int32 and float32 arrays 4-byte
 *     aligned (every torch allocation is; a view that starts at an element
 *     offset may not be): MOE_ERR_INVALID_ARG otherwise.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Device work is enqueued on it asynchronously; no call synchronizes,
 *     allocates device memory, sets memory or copies device-to-host, so the
 *     moe_layout -> moe_dispatch -> (expert) -> moe_combine sequence can be
 *     captured into a hipGraph and replayed.
 *   - Every call returns an int status: MOE_OK (0) or a negative MOE_ERR_*.
 *     All argument checks run on the host before anything is enqueued; on an
 *     error nothing was enqueued. MOE_ERR_HIP means a launch failed.
 *   - Expert ids outside [0, num_experts) (the sentinel -1 included) mean
 *     "no expert": the slot gets no row and its score is never read.
 *   - Calls on one context must be ordered on one stream; two streams using
 *     one context at once race on its buffers.
 */
#ifndef MOE_LAYOUT_MOE_H
#define MOE_LAYOUT_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define MOE_OK               0
#define MOE_ERR_INVALID_ARG (-1) /* null pointer, bad size, unsupported dtype */
#define MOE_ERR_CAPACITY    (-2) /* capacity relation of [TT] "API design" fails */
#define MOE_ERR_WORKSPACE   (-3) /* workspace too small or misaligned */
#define MOE_ERR_HIP         (-4) /* a HIP launch reported an error */
#define MOE_ERR_STATE       (-5) /* dispatch/combine without a matching layout */
#define MOE_ERR_UNSUPPORTED (-6) /* backward call without MOE_FLAG_BACKWARD; moe_layout_dispatch
                                    on a context that got no counter slot */
#define MOE_ERR_SCRATCH     (-7) /* moe_layout_noalloc: the call needs more than the static
                                    scratch (MOE_NOALLOC_SCRATCH_BYTES) */

/* moe_config.flags */
#define MOE_FLAG_BACKWARD   1    /* also carve the backward buffers g_e, g_s, g_x */

/* Limits checked at create. */
#define MOE_MAX_EXPERTS   1024
#define MOE_MAX_TOPK      16
#define MOE_WORKSPACE_ALIGN 256

typedef enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Lifetime configuration ([TT] "API design": the dispatcher configuration
 * carries num_max_tokens_per_rank).
 *   num_max_tokens_per_rank  >= 1; buffers hold round_up4 of it tokens
 *   hidden                   D >= 1, with D * element size a multiple of 16
 *   num_experts              E, 1..MOE_MAX_EXPERTS
 *   topk                     K, 1..MOE_MAX_TOPK
 *   dtype                    moe_dtype of hidden states (x, expert output, y)
 *   flags                    0 or MOE_FLAG_BACKWARD
 * round_up4(num_max_tokens_per_rank) * topk must fit in int32. */
typedef struct moe_config {
    int32_t num_max_tokens_per_rank;
    int32_t hidden;
    int32_t num_experts;
    int32_t topk;
    int32_t dtype;
    int32_t flags;
} moe_config;

/* Byte offsets (into the workspace) and sizes of the persistent buffers,
 * for callers that view them, e.g. as torch tensors. Every offset is a
 * multiple of MOE_WORKSPACE_ALIGN.
 *   counts      int32 [E]            tokens routed to each expert
 *   offsets     int32 [E+1]          exclusive prefix sum; offsets[E] = total
 *   row_map     int32 [nmax4][K]     row of slot (t,k) in x_e, -1 = none;
 *                                    rows [0, round_up4(ntpr)) written by layout
 *   src_map     int32 [nmax4*K]      t*K+k of the slot at each row; [0,total)
 *   s_e         f32   [nmax4*K]      score of each dispatched row; [0,total)
 *   x_e         dtype [nmax4*K][D]   expert-major hidden states; [0,total)
 *   y           dtype [nmax4][D]     combined output; rows [0,T) of a call
 *   block_hist  int32 [max_tiles][round_up4(E)] layout scratch (per-tile
 *                                    histograms)
 *   map_ids, map_scores  int32 / f32 [nmax4][K]  top-k form of a routing map
 *   map_n_experts        int32 [nmax4]          experts per routing-map row
 * With MOE_FLAG_BACKWARD (offsets are -1 without it):
 *   g_e         dtype [nmax4*K][D]   dL/dy_e from moe_combine_backward
 *   g_s         f32   [nmax4][K]     dL/dscores from moe_combine_backward
 *   g_x         dtype [nmax4][D]     dL/dx from moe_dispatch_backward
 * nmax4 = round_up4(num_max_tokens_per_rank). */
typedef struct moe_buffers_desc {
    int64_t workspace_bytes;
    int64_t nmax4;
    int64_t max_rows;      /* nmax4 * K */
    int64_t row_bytes;     /* D * element size */
    int64_t max_tiles;     /* layout tiles at full capacity (smallest tile) */
    int64_t tile_slots;    /* (t,k) slots of the smallest layout tile */
    int64_t counts, offsets, row_map, src_map, s_e, x_e, y;
    int64_t block_hist;
    int64_t map_ids, map_scores, map_n_experts;
    int64_t g_e, g_s, g_x;
} moe_buffers_desc;

/* Opaque per-workspace context; host memory only. */
typedef struct moe_ctx moe_ctx;

/* Bytes of device workspace a context with this configuration needs.
 * Pure host. MOE_ERR_CAPACITY when num_max_tokens_per_rank < 1,
 * MOE_ERR_INVALID_ARG for any other invalid field or a NULL pointer. */
int moe_workspace_bytes(const moe_config *cfg, size_t *bytes);

/* Create a context over a caller-owned device workspace of `bytes` bytes
 * (>= moe_workspace_bytes, aligned to MOE_WORKSPACE_ALIGN). The buffers are
 * carved from it once, at fixed addresses; no call ever allocates or grows
 * them ([TT] "API design"). The caller keeps the workspace alive until
 * moe_destroy and frees it afterwards. Pure host; *out receives the context
 * (NULL on error). Errors: as moe_workspace_bytes for the configuration;
 * MOE_ERR_WORKSPACE for a short or misaligned workspace; MOE_ERR_INVALID_ARG
 * for a NULL workspace or when the host-side context cannot be allocated. */
int moe_create(const moe_config *cfg, void *d_workspace, size_t bytes, moe_ctx **out);

/* Free the host-side context (not the workspace). NULL is accepted. */
int moe_destroy(moe_ctx *ctx);

/* Fill *out with the buffer offsets and sizes of this context. Pure host. */
int moe_workspace_offsets(const moe_ctx *ctx, moe_buffers_desc *out);

/* Routing layout ([TT] "API design": per-expert token counts; [UC]
 * "Internode" 2 and 3). From d_topk_ids [T][K] computes into the context:
 *   counts[e], offsets[0..E] (offsets[E] = total valid slots, on the device),
 *   row_map[t][k] for t < round_up4(num_tokens_per_rank): the row of slot
 *     (t,k) in the expert-major buffer, rows of one expert ordered by
 *     ascending t*K+k; -1 for no expert and for padding rows t >= T,
 *   src_map[row] = t*K+k for rows [0,total).
 * Requires 0 <= T <= num_tokens_per_rank <= num_max_tokens_per_rank
 * (MOE_ERR_CAPACITY otherwise). Only ids rows [0,T) are read; d_topk_ids may
 * be NULL when T == 0. Records (T, round_up4(num_tokens_per_rank)) on the
 * host as the context's current layout. */
int moe_layout(moe_ctx *ctx, const int32_t *d_topk_ids, int32_t T,
               int32_t num_tokens_per_rank, void *stream);

/* moe_layout for callers that cannot allocate device memory: code running
 * under graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * No context and no workspace: the caller passes the ids and the four output
 * buffers; the per-tile histograms the two-launch form needs live in a
 * static device array of MOE_NOALLOC_SCRATCH_BYTES per device, which the
 * library holds until the process ends. No device memory is allocated or
 * freed. Results are those of moe_layout bit for bit:
 *   d_topk_ids  int32 [T][K] (may be NULL when T == 0)
 *   d_counts    int32 [num_experts]         written
 *   d_offsets   int32 [num_experts + 1]     written; d_offsets[E] = total
 *   d_row_map   int32 [round_up4(num_tokens_per_rank)][K]  written
 *   d_src_map   int32 [>= total] (at most T*K); rows [0, total) written
 * Requires 0 <= T <= num_tokens_per_rank (MOE_ERR_CAPACITY), 1 <= num_experts
 * <= MOE_MAX_EXPERTS, 1 <= topk <= MOE_MAX_TOPK and
 * round_up4(num_tokens_per_rank) * topk < 2^31 - 512 (MOE_ERR_INVALID_ARG).
 * Scratch limit: up to 32768 slots (round_up4(num_tokens_per_rank) * topk)
 * the layout is one launch and uses no scratch; above, it uses
 * ceil(slots / tile) * round_up4(num_experts) * 4 bytes (tile = 512 slots up
 * to 65536 slots, 1024 above), and a call needing more than
 * MOE_NOALLOC_SCRATCH_BYTES returns MOE_ERR_SCRATCH (e.g. beyond 4194304
 * slots at 256 experts, 1048576 at 1024). Every call on one device shares
 * that device's array, so calls that overlap on one device race: order them
 * on one stream. The first call on each device that needs the scratch looks
 * up its device address (a host-side query, done once); make that call
 * outside graph capture. */
#define MOE_NOALLOC_SCRATCH_BYTES (4 << 20)
int moe_layout_noalloc(const int32_t *d_topk_ids, int32_t T, int32_t num_tokens_per_rank,
                       int32_t num_experts, int32_t topk, int32_t *d_counts,
                       int32_t *d_offsets, int32_t *d_row_map, int32_t *d_src_map,
                       void *stream);

/* Dispatch ([TT] "API design" signature; [NA] "Fix"). Permutes the hidden
 * states into the context's expert-major buffer using the row map of the
 * preceding moe_layout on this context:
 *   x_e[row_map[t][k]] = x[t] (bit copy), s_e[row_map[t][k]] = scores[t][k]
 * for t < T and every slot with an expert. Padding rows [T,
 * round_up4(num_tokens_per_rank)) are never copied.
 *   d_x         [T][D] hidden states (config dtype)
 *   d_topk_scores [T][K] float32; d_topk_ids [T][K] int32 (the ids the
 *               layout was built from; the kernels use the row map instead)
 *   d_counts    must be the context's own counts buffer (as written by
 *               moe_layout); any other pointer is MOE_ERR_INVALID_ARG
 * T and num_tokens_per_rank must equal those of the most recent moe_layout
 * call on this context (MOE_ERR_STATE otherwise). Rows [0, offsets[E]) of x_e
 * and s_e are written; the rest is left as it was. */
int moe_dispatch(moe_ctx *ctx, const void *d_x, const float *d_topk_scores,
                 const int32_t *d_topk_ids, const int32_t *d_counts, int32_t T,
                 int32_t num_tokens_per_rank, void *stream);

/* moe_layout followed by moe_dispatch in two launches (the separate calls
 * take three above 32768 slots, two up to it), with the same results bit for
 * bit: counts, offsets, row_map, src_map, x_e and
 * s_e exactly as those two calls write them ([TT] "Backend behavior": the
 * fused-permute output is sized from the current capacity; [UC] "Internode"
 * 2 and 3: the counts and the total stay on the device). The count launch's
 * last workgroup to finish scans the per-tile expert histograms into each
 * tile's first row per expert; the dispatch workgroups rank their tokens'
 * slots within their tile, record the rows and copy the hidden states. Each
 * dispatch workgroup holds one whole token row when a row spans at least 4
 * wavefronts, unless moe_set_tuning set dispatch_block_waves. No
 * workgroup waits on another. The last workgroup is found with a completion
 * counter that lives in a static device array (one slot per context, taken
 * at moe_create and given back at moe_destroy; MOE_ERR_UNSUPPORTED when all
 * 1024 slots were taken) and is back at zero after every launch, so the call
 * is graph-capturable like the others. Arguments and capacity checks are
 * those of moe_layout plus moe_dispatch (no d_counts: the context's own is
 * used). Records the context's current layout like moe_layout, so
 * moe_combine follows as usual. Two calls on one context must not overlap
 * (as for every entry point); destroy a context only after its work ended. */
int moe_layout_dispatch(moe_ctx *ctx, const void *d_x, const float *d_topk_scores,
                        const int32_t *d_topk_ids, int32_t T, int32_t num_tokens_per_rank,
                        void *stream);

/* Dispatch with the scores applied (the weighting moved from the combine to
 * the dispatch; [NA] "Fix": the dispatcher's inputs are hidden states,
 * routing map and probabilities). Same arguments, checks and rows as
 * moe_dispatch, but
 *   x_e[row_map[t][k]] = scores[t][k] * x[t]
 * as one fp32 product rounded to the element type (bf16: to nearest even).
 * s_e still receives the scores. Pair it with moe_combine(d_topk_scores =
 * NULL) so the weights are not applied twice. */
int moe_dispatch_scaled(moe_ctx *ctx, const void *d_x, const float *d_topk_scores,
                        const int32_t *d_topk_ids, const int32_t *d_counts, int32_t T,
                        int32_t num_tokens_per_rank, void *stream);

/* Routing-map input format ([NA] "Fix": HybridEP's dispatcher takes a
 * boolean routing map [T][E] and probabilities [T][E]; padded rows are
 * all-False with zero probabilities). Writes the top-k form into the
 * context: for t < T, slot k of token t is the k-th expert e, ascending, with
 * d_routing_map[t][e] != 0 and score d_probs[t][e]; the remaining slots get
 * id -1 and score 0 (no expert). n_experts[t] is the row's number of experts;
 * a row with more than K keeps its K lowest (n_experts[t] > K reports it on
 * the device, with no host round trip).
 *   d_routing_map  uint8 [T][E] (torch.bool works), d_probs float32 [T][E]
 *   *d_topk_ids_out, *d_topk_scores_out  receive map_ids / map_scores
 *                  ([nmax4][K], rows [0,T) written), ready for moe_layout,
 *                  moe_dispatch and moe_combine
 *   *d_n_experts_out receives map_n_experts ([nmax4], rows [0,T))
 * Requires 0 <= T <= num_max_tokens_per_rank (MOE_ERR_CAPACITY). */
int moe_topk_from_routing_map(moe_ctx *ctx, const uint8_t *d_routing_map, const float *d_probs,
                              int32_t T, void *stream, int32_t **d_topk_ids_out,
                              float **d_topk_scores_out, int32_t **d_n_experts_out);

/* Combine ([NA] "Fix" and "Testing"). For t < T:
 *   y[t] = sum over k = 0..K-1 with d_row_map[t][k] >= 0 of
 *          scores[t][k] * y_expert[d_row_map[t][k]]
 * accumulated in fp32 with fused multiply-add in ascending k from +0.0 and
 * stored in the config dtype (bf16 rounds to nearest even; NaN -> 0x7FC0).
 * A slot with row -1 is skipped and its score is never read; a token with no
 * expert gets +0.0. Rows >= T (the padding) are not computed.
 *   d_y_expert  expert outputs in the expert-major layout,
 *               [>= round_up4(num_tokens_per_rank) * K][D] (the worst-case
 *               total, known on the host; only rows [0,total) are read).
 *               The context's x_e serves for an identity expert.
 *   d_row_map   [>= T][K] row map, normally the context's; when it is the
 *               context's, T and num_tokens_per_rank must match the most
 *               recent moe_layout (MOE_ERR_STATE otherwise)
 *   d_topk_scores [T][K] float32, or NULL for unit weights (after
 *               moe_dispatch_scaled, which already applied the scores)
 *   *d_y_out    receives the device address of y ([nmax4][D], rows [0,T)
 *               valid until the next combine on this context).
 * Rows of d_row_map outside [0, round_up4(num_tokens_per_rank) * K) are
 * treated as no expert. */
int moe_combine(moe_ctx *ctx, const void *d_y_expert, const int32_t *d_row_map,
                const float *d_topk_scores, int32_t T, int32_t num_tokens_per_rank,
                void *stream, void **d_y_out);

/* Backward of moe_combine ([NA] "Testing": forward and backward of the
 * dispatcher are checked bitwise against the equal-count run). For t < T and
 * every slot with d_row_map[t][k] = r >= 0:
 *   g_e[r]       = scores[t][k] * d_grad_y[t]   (one fp32 product, rounded to
 *                                               the element type)
 *   g_s[t][k]    = <d_grad_y[t], d_y_expert[r]> (fp32, fixed reduction order)
 * and g_s[t][k] = +0.0 for a slot without an expert. With d_total, the rows
 * g_e[*d_total .. round_up4(num_tokens_per_rank) * K) are set to +0.0: no slot
 * reaches them, so their gradient is zero (*d_total is read on the device,
 * clamped to [0, round_up4(num_tokens_per_rank) * K]; [UC] "Internode" 3:
 * the true total stays on the device). Other rows of g_e are not written.
 *   d_grad_y       [T][D] gradient of the combine output
 *   d_y_expert     the expert outputs the forward combine read,
 *                  [>= round_up4(num_tokens_per_rank) * K][D]
 *   d_row_map, d_topk_scores, T, num_tokens_per_rank: as for moe_combine
 *                  (the same MOE_ERR_STATE rule for the context's row map)
 *   d_total        int32 in device memory: the number of rows the slots of
 *                  d_row_map reach (offsets[E] of the layout that made it,
 *                  e.g. the context's offsets + E, or a copy of it), or NULL
 *                  to leave the rows past the slots' rows unwritten
 *   *d_grad_y_expert_out  receives the address of g_e ([nmax4*K][D])
 *   *d_grad_scores_out    receives the address of g_s ([nmax4][K]; rows [0,T))
 * Needs MOE_FLAG_BACKWARD (MOE_ERR_UNSUPPORTED otherwise). */
int moe_combine_backward(moe_ctx *ctx, const void *d_grad_y, const void *d_y_expert,
                         const int32_t *d_row_map, const float *d_topk_scores,
                         const int32_t *d_total, int32_t T, int32_t num_tokens_per_rank,
                         void *stream, void **d_grad_y_expert_out,
                         float **d_grad_scores_out);

/* Backward of moe_dispatch: for t < T,
 *   g_x[t] = sum over k = 0..K-1 with d_row_map[t][k] >= 0 of
 *            d_grad_x_expert[d_row_map[t][k]]
 * in fp32, ascending k, from +0.0, rounded to the element type (+0.0 for a
 * token without an expert).
 *   d_grad_x_expert  gradient of the dispatched rows,
 *                    [>= round_up4(num_tokens_per_rank) * K][D]
 *   d_row_map, T, num_tokens_per_rank: as for moe_combine
 *   *d_grad_x_out    receives the address of g_x ([nmax4][D]; rows [0,T))
 * Needs MOE_FLAG_BACKWARD (MOE_ERR_UNSUPPORTED otherwise). */
int moe_dispatch_backward(moe_ctx *ctx, const void *d_grad_x_expert, const int32_t *d_row_map,
                          int32_t T, int32_t num_tokens_per_rank, void *stream,
                          void **d_grad_x_out);

/* Weight layouts the expert step reads. */
#define MOE_WEIGHTS_ROW_MAJOR 0 /* [num_experts][n_out][k_in] bf16 */
#define MOE_WEIGHTS_TILED     1 /* the output of moe_tile_expert_weights */

/* Expert step between dispatch and combine ([UC] "Tests": layout, dispatch,
 * expert and combine captured in one graph; "Internode" item 2: the expert
 * step takes its per-expert row counts from device memory, with no host
 * handshake). Each expert applies one linear map to its segment of the
 * expert-major rows (a grouped GEMM): for every e and every row r with
 * offsets[e] <= r < offsets[e+1],
 *   out[r][n] = sum over d < k_in of x_expert[r][d] * weights[e][n][d]
 * bf16 inputs, fp32 accumulation (matrix cores; summation order not
 * specified, the same for both layouts), rounded once to bf16 (nearest
 * even). Rows outside every segment are not written. Needs no context and
 * no workspace.
 *   d_x_expert  bf16 [max_rows][k_in]  (x_e of moe_dispatch when k_in = hidden)
 *   d_weights   weight_layout MOE_WEIGHTS_ROW_MAJOR: bf16
 *               [num_experts][n_out][k_in] (expert e's weight as n_out rows
 *               of k_in: a linear layer's [out][in] layout);
 *               MOE_WEIGHTS_TILED: the same weights rewritten once by
 *               moe_tile_expert_weights (faster: read straight into the
 *               matrix-core operand registers)
 *   d_offsets   int32 [num_experts + 1] in device memory, read only by the
 *               kernel: a non-decreasing prefix sum from 0 with
 *               offsets[num_experts] <= max_rows (the context's offsets
 *               after moe_layout satisfy this with max_rows =
 *               round_up4(num_tokens_per_rank) * K). Other values cannot
 *               make the kernel access memory outside the three buffers
 *               (segments are clamped to [0, max_rows)), but the rows
 *               written are then unspecified.
 *   max_rows    rows the launch covers (0 <= max_rows <= INT32_MAX;
 *               0 enqueues nothing)
 *   k_in, n_out multiples of 8, >= 8
 *   d_out       bf16 [max_rows][n_out]; must not overlap the inputs
 *   row_tile    rows per tile: 64, 128, or 0 for the library's choice
 *               (results do not depend on it)
 *   weight_layout  MOE_WEIGHTS_ROW_MAJOR or MOE_WEIGHTS_TILED; tiled weights
 *               must come from moe_tile_expert_weights with the same
 *               num_experts, n_out and k_in (the kernel trusts their size)
 * d_x_expert, d_weights and d_out must be 16-byte aligned, d_offsets
 * 4-byte aligned. 1 <= num_experts <= MOE_MAX_EXPERTS. A launch needs at
 * most INT32_MAX workgroups (ceil(n_out/F) * (ceil(max_rows/row_tile) +
 * num_experts), F = 128 row-major / 512 tiled features per workgroup).
 * Violations: MOE_ERR_INVALID_ARG. */
int moe_grouped_gemm(const void *d_x_expert, const void *d_weights, const int32_t *d_offsets,
                     int32_t num_experts, int64_t max_rows, int32_t k_in, int32_t n_out,
                     void *d_out, int32_t row_tile, int32_t weight_layout, void *stream);

/* Bytes of the tiled form of [num_experts][n_out][k_in] bf16 weights:
 * num_experts * ceil(n_out/32)*32 * ceil(k_in/64)*64 * 2 (zero padded), or
 * -1 for sizes moe_grouped_gemm does not take. Pure host. */
int64_t moe_tiled_weights_bytes(int32_t num_experts, int32_t n_out, int32_t k_in);

/* Rewrites row-major expert weights into the tiled layout (a one-time
 * permutation with zero padding; the weights are static): for feature
 * block b (32 features), k step t (64 elements), instruction s (0..3) and
 * lane l (0..63), 16-byte chunk ((((e*NB + b)*S + t)*4 + s)*64 + l) holds
 * weights[e][32b + l%32][64t + 32(l/32) + 8s .. +8], zeros past n_out or
 * k_in (NB = ceil(n_out/32), S = ceil(k_in/64)).
 *   d_weights  bf16 [num_experts][n_out][k_in], device, 16-byte aligned
 *   d_tiled    moe_tiled_weights_bytes(...) bytes, device, 16-byte aligned,
 *              not overlapping d_weights
 * Same size limits as moe_grouped_gemm; MOE_ERR_INVALID_ARG otherwise. */
int moe_tile_expert_weights(const void *d_weights, int32_t num_experts, int32_t n_out,
                            int32_t k_in, void *d_tiled, void *stream);

/* Launch shape tuning (optional). moe_create picks every default from the
 * context's sizes (measured on MI355X); moe_get_tuning reports them. Each
 * token row is split into `segments` wavefront work items (1..16) and
 * `block_waves` wavefronts (1..16) form a workgroup (dispatch by default:
 * one token row per workgroup; 4 wavefronts when the expert buffer exceeds
 * 1 GiB, 16 when it is at most 128 MiB; combine by default: 16 wavefronts,
 * one token row when the output y exceeds the last-level cache); 0 keeps the
 * current value. A
 * nonzero *_nontemporal marks dispatch's expert-buffer stores / combine's
 * expert-output loads / combine's output stores as streaming (not kept in
 * cache); for the last one -1 keeps the current value. layout_launches 1 runs moe_layout as one launch (every
 * workgroup counts the whole batch, then ranks its tile), 2 as two (count,
 * then offsets and rank), -1 chooses by size (one launch up to 32768
 * slots, the default), 0 keeps the current value. dispatch_store_burst 1
 * issues each wavefront's K row stores back to back, 2 issues each after the
 * previous one has completed (the default), 0 keeps the current value; it
 * applies to the default one-chunk-per-lane shape. combine_backward_store 1
 * writes moe_combine_backward's dL/dy_e rows with streaming stores, 2 with
 * ordinary ones, 0 keeps the current value; by default they stream when the
 * context's dL/dy_e buffer is larger than 1 GiB (four times the 256 MB
 * last-level cache). dispatch_x_nontemporal 1 makes dispatch read the rows
 * of x with streaming loads (the bit copy with ordinary stores: moe_dispatch
 * and moe_layout_dispatch), 2 with ordinary ones, 0 keeps the current value;
 * by default they stream when the context's expert buffer is larger than
 * the last-level cache and at most four times it.
 * Results do not depend on any of these. Pure host. */
typedef struct moe_tuning {
    int32_t dispatch_segments;
    int32_t combine_segments;
    int32_t dispatch_nontemporal;
    int32_t combine_nontemporal;
    int32_t dispatch_block_waves;
    int32_t combine_block_waves;
    int32_t combine_store_nontemporal;  /* streaming stores of y; -1 keeps */
    int32_t layout_launches;            /* 1, 2, or -1 (by size); 0 keeps */
    int32_t dispatch_store_burst;       /* 1 back to back, 2 paced; 0 keeps */
    int32_t combine_backward_store;     /* 1 streaming, 2 ordinary; 0 keeps */
    int32_t dispatch_x_nontemporal;     /* 1 streaming, 2 ordinary; 0 keeps */
} moe_tuning;
int moe_set_tuning(moe_ctx *ctx, const moe_tuning *tuning);
int moe_get_tuning(const moe_ctx *ctx, moe_tuning *out);

/* Capacity helpers ([TT] "Capacity derivation"; [NA] "Fix"). Pure host.
 * Invalid arguments (negative sizes, degrees < 1) return -1. */
int64_t moe_ceil_div(int64_t a, int64_t b);                 /* a >= 0, b >= 1 */
int64_t moe_round_up4(int64_t n);                           /* n >= 0 */
/* local_batch_size * ceil_div(seq_len, cp * tp) */
int64_t moe_num_max_tokens_pretrain(int64_t local_batch, int64_t seq_len,
                                    int64_t cp, int64_t tp);
/* ceil_div(max_num_batched_tokens, cp * tp) */
int64_t moe_num_max_tokens_infer(int64_t max_num_batched_tokens, int64_t cp,
                                 int64_t tp);
/* An explicitly configured maximum must be positive and >= the derived
 * requirement: MOE_OK, or MOE_ERR_CAPACITY. */
int moe_validate_num_max(int64_t configured, int64_t derived);
/* The capacity relation 0 <= T <= ntpr <= nmax, nmax >= 1: MOE_OK or
 * MOE_ERR_CAPACITY. */
int moe_check_capacity(int64_t T, int64_t num_tokens_per_rank,
                       int64_t num_max_tokens_per_rank);

/* Static description of a status code. */
const char *moe_strerror(int status);

#ifdef __cplusplus
}
#endif
#endif /* MOE_LAYOUT_MOE_H */
