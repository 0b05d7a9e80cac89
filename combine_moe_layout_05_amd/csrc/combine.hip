// Combine gather-reduce on gfx950: for each token, the score-weighted sum of
// the expert-output rows its slots were dispatched to, back in token order.
//
// What is computed ("fix(moe): equalize and align per-rank token counts for
// HybridEP dispatch", sections "Fix" and "Testing": combine returns the
// token-ordered output and slices the padding off; with identity experts a
// token's output depends only on its own routing):
//   y[t] = sum_{k=0..K-1, row_map[t][k] >= 0} scores[t][k] * y_e[row_map[t][k]]
// (with scores == nullptr every weight is 1: the gather-sum that is the
// backward of dispatch, dL/dx[t] = sum_k dL/dx_e[row_map[t][k]])
// in fp32, fused multiply-add in ascending k, starting from +0.0, stored in
// the element type (bf16 rounds to nearest even; NaN becomes 0x7FC0). A slot
// without an expert is skipped and its score is not read. Only t < T is
// computed; padding rows are never materialized.
//
// Bound by HBM reads (K rows read per row written). One wavefront per
// (token, row segment); the workgroup's row-map entries and scores are staged
// in LDS with one coalesced load and each wavefront moves its token's K rows
// and scores into SGPRs. Each lane owns one 16-byte chunk per iteration and
// issues its K row loads
// back to back, as streaming loads by default (each row is read once). With
// the default launch shape a segment is exactly one chunk per lane, so a
// wavefront is: K loads, K fused multiply-adds per element, one store. For
// longer segments, when every slot of the token has an expert, the loop is
// double-buffered: the next chunk's K loads are issued before the current
// chunk is reduced and stored. No-expert slots load the token's first valid
// row instead (always written, finite) and skip it in the sum, which keeps
// every load unconditional. Output stores are ordinary, or streaming when the
// output buffer is larger than the last-level cache (single-chunk shape).
#include "moe_kernels.h"
#include "moe_lanes.h"

namespace moe {
namespace {

// One wavefront per (token, row segment). SINGLE: the segment is exactly one
// 16-byte chunk per lane, so no loop and no second buffer (fewer registers,
// more wavefronts resident); otherwise the segment is walked chunk by chunk.
// NT: streaming loads of the expert outputs. NTS (SINGLE only): streaming
// stores of y.
template <int K, bool BF16, bool NT, bool SINGLE, bool NTS>
__global__ __launch_bounds__(kMaxBlockThreads)
void combine_kernel(const v4i* __restrict__ y_e, const int32_t* __restrict__ row_map,
                    const float* __restrict__ scores, int32_t T, int32_t chunks,
                    int32_t segments, int32_t seg_chunks, int64_t row_limit,
                    v4i* __restrict__ y) {
    using L = Lanes<BF16>;
    // Row-map entries and scores of the workgroup's tokens: one coalesced load
    // into LDS, then a barrier. Rows outside [0, row_limit) count as no
    // expert, and such a slot's score is never loaded.
    __shared__ int32_t tile_rows[kMaxBlockWaves * K];
    __shared__ float tile_scores[kMaxBlockWaves * K];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int block_waves = static_cast<int>(blockDim.x) >> 6;
    const int64_t item0 = int64_t(blockIdx.x) * block_waves;
    const int64_t t_first = item0 / segments;
    int64_t t_last = (item0 + block_waves - 1) / segments;
    if (t_last > int64_t(T) - 1) t_last = int64_t(T) - 1;
    const int staged = static_cast<int>(t_last - t_first + 1) * K;
    if (tid < staged) {
        const int32_t r = row_map[t_first * K + tid];
        const bool ok = r >= 0 && r < row_limit;
        tile_rows[tid] = ok ? r : -1;
        tile_scores[tid] = ok ? (scores ? scores[t_first * K + tid] : 1.0f) : 0.0f;
    }
    __syncthreads();

    const int64_t item = item0 + wave;
    const int64_t t = item / segments;
    if (t >= T) return;
    const int seg = static_cast<int>(item - t * segments);
    const int lt = static_cast<int>(t - t_first);

    int32_t row[K];
    float s[K];
    int32_t fallback = -1;
    bool all_valid = true;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        row[k] = __builtin_amdgcn_readfirstlane(tile_rows[lt * K + k]);
        s[k] = __int_as_float(
            __builtin_amdgcn_readfirstlane(__float_as_int(tile_scores[lt * K + k])));
        if (fallback < 0 && row[k] >= 0) fallback = row[k];
        all_valid = all_valid && row[k] >= 0;
    }

    const int32_t c_begin = seg * seg_chunks;
    const int32_t c_end = min(c_begin + seg_chunks, chunks);
    v4i* dst = y + t * chunks;

    if (fallback < 0) {  // no slot reaches an expert: +0.0
        const v4i zero = {0, 0, 0, 0};
        for (int32_t c = c_begin + lane; c < c_end; c += 64) dst[c] = zero;
        return;
    }

    const v4i* src[K];
#pragma unroll
    for (int k = 0; k < K; ++k) src[k] = y_e + int64_t(row[k] >= 0 ? row[k] : fallback) * chunks;

    // Reduce one loaded chunk: every slot, or only the slots with an expert.
    auto reduce = [&](const v4i (&b)[K], bool every) {
        float acc[L::N];
#pragma unroll
        for (int e = 0; e < L::N; ++e) acc[e] = 0.0f;
#pragma unroll
        for (int k = 0; k < K; ++k)
            if (every || row[k] >= 0) L::fma_into(acc, s[k], b[k]);
        return L::pack(acc);
    };

    if constexpr (SINGLE) {
        // Lanes past the segment end (a short last segment) load its last
        // chunk and do not store.
        const int32_t c = c_begin + lane;
        const int32_t cl = min(c, c_end - 1);
        v4i b[K];
#pragma unroll
        for (int k = 0; k < K; ++k) b[k] = fetch<NT>(src[k] + cl);
        const v4i out = all_valid ? reduce(b, true) : reduce(b, false);
        if (c < c_end) {
            if constexpr (NTS)
                __builtin_nontemporal_store(out, dst + c);
            else
                dst[c] = out;
        }
        return;
    } else {
        const int32_t iters = (c_end - c_begin + 63) / 64;   // one chunk per lane each
        auto load = [&](v4i (&b)[K], int32_t i) {
            const int32_t c = min(c_begin + i * 64 + lane, c_end - 1);
#pragma unroll
            for (int k = 0; k < K; ++k) b[k] = fetch<NT>(src[k] + c);
        };
        auto emit = [&](const v4i (&b)[K], int32_t i, bool every) {
            const v4i out = reduce(b, every);
            const int32_t c = c_begin + i * 64 + lane;
            if (c < c_end) dst[c] = out;
        };
        if (all_valid) {
            // Every slot has an expert: the next chunk's loads are in flight
            // while this one is reduced and stored.
            // Every chunk is loaded once: the loop runs while a chunk i + 2
            // exists to prefetch, and the one or two chunks left run after it.
            v4i b0[K], b1[K];
            load(b0, 0);
            int32_t i = 0;
            for (; i + 2 < iters; i += 2) {
                load(b1, i + 1);
                emit(b0, i, true);
                load(b0, i + 2);
                emit(b1, i + 1, true);
            }
            if (i + 1 < iters) {
                load(b1, i + 1);
                emit(b0, i, true);
                emit(b1, i + 1, true);
            } else {
                emit(b0, i, true);
            }
            return;
        }
        for (int32_t i = 0; i < iters; ++i) {
            v4i b[K];
            load(b, i);
            emit(b, i, false);
        }
    }
}

template <int K, bool BF16>
hipError_t launch_k(const CombineArgs& a, int32_t segments, int32_t seg_chunks,
                    hipStream_t stream) {
    const int64_t items = int64_t(a.T) * segments;
    const int64_t blocks = (items + a.block_waves - 1) / a.block_waves;
    const bool single = seg_chunks == 64;
    const bool nts = a.store_nontemporal;
    auto kernel = a.nontemporal
        ? (single ? (nts ? combine_kernel<K, BF16, true, true, true>
                         : combine_kernel<K, BF16, true, true, false>)
                  : combine_kernel<K, BF16, true, false, false>)
        : (single ? (nts ? combine_kernel<K, BF16, false, true, true>
                         : combine_kernel<K, BF16, false, true, false>)
                  : combine_kernel<K, BF16, false, false, false>);
    hipLaunchKernelGGL(kernel, dim3(static_cast<uint32_t>(blocks)), dim3(64 * a.block_waves), 0, stream,
                       static_cast<const v4i*>(a.y_e), a.row_map, a.scores, a.T, a.chunks,
                       segments, seg_chunks, a.row_limit, static_cast<v4i*>(a.y));
    return hipGetLastError();
}

template <bool BF16>
hipError_t launch_dtype(const CombineArgs& a, int32_t segments, int32_t seg_chunks,
                        hipStream_t stream) {
    switch (a.K) {
#define MOE_COMBINE_CASE(k) \
    case k: return launch_k<k, BF16>(a, segments, seg_chunks, stream);
        MOE_COMBINE_CASE(1) MOE_COMBINE_CASE(2) MOE_COMBINE_CASE(3) MOE_COMBINE_CASE(4)
        MOE_COMBINE_CASE(5) MOE_COMBINE_CASE(6) MOE_COMBINE_CASE(7) MOE_COMBINE_CASE(8)
        MOE_COMBINE_CASE(9) MOE_COMBINE_CASE(10) MOE_COMBINE_CASE(11) MOE_COMBINE_CASE(12)
        MOE_COMBINE_CASE(13) MOE_COMBINE_CASE(14) MOE_COMBINE_CASE(15) MOE_COMBINE_CASE(16)
#undef MOE_COMBINE_CASE
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
    if (a.T <= 0) return hipSuccess;
    const int32_t seg_chunks = segment_chunks(a.chunks, a.segments);
    const int32_t segments = (a.chunks + seg_chunks - 1) / seg_chunks;
    return a.bf16 ? launch_dtype<true>(a, segments, seg_chunks, stream)
                  : launch_dtype<false>(a, segments, seg_chunks, stream);
}

}  // namespace moe
