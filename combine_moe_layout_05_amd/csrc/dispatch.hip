// Dispatch scatter on gfx950: copy each token's hidden-state row to the
// expert-major rows its routing slots were given by the layout, and the
// slot's score beside it.
//
// What is computed ("Unify expert parallel token dispatcher API", sections
// "API design" and "Backend behavior": dispatch writes a permuted, per-expert
// output into storage allocated once at the lifetime maximum; "fix(moe):
// equalize and align per-rank token counts for HybridEP dispatch", section
// "Fix": padded rows route to no expert and cost no copy):
//   x_e[row_map[t][k]] = x[t]            (bit copy of the row)
//   s_e[row_map[t][k]] = scores[t][k]
// for t < T and every slot with row >= 0.
//
// The work is pure data movement bound by HBM writes (K row writes per row
// read). One wavefront takes one (token, row segment) item: it loads the
// segment once, 16 bytes per lane so each wavefront access is a contiguous
// 1 KiB run, and stores it K times. With the default launch shape a segment
// is exactly one 16-byte chunk per lane, so a workgroup's wavefronts cover
// neighbouring 1 KiB pieces of one token row. The workgroup's row-map entries
// are staged in LDS with one coalesced load; each wavefront moves its K rows
// into SGPRs, so destination addresses are scalar and the per-slot "has an
// expert" test is a scalar branch. (Measured on MI355X: staging behind a
// workgroup barrier beats per-wavefront scalar loads of the row map by ~9 %,
// because the barrier lines the wavefronts up on neighbouring pieces.)
#include "moe_kernels.h"
#include "moe_lanes.h"

namespace moe {
namespace {

constexpr int kDispatchUnroll = 4;   // 16-byte chunks per lane in flight

template <bool NT>
__device__ __forceinline__ void put(v4i* p, v4i v) {
    if constexpr (NT)
        __builtin_nontemporal_store(v, p);
    else
        *p = v;
}

// Row transform of a dispatch: a bit copy, or the slot's score applied (one
// fp32 product rounded to the element type).
enum RowMode { kCopy = 0, kScaleF32 = 1, kScaleBF16 = 2 };

template <int MODE>
__device__ __forceinline__ v4i transform(float s, v4i v) {
    if constexpr (MODE == kCopy)
        return v;
    else
        return Lanes<MODE == kScaleBF16>::scale(s, v);
}

// One wavefront per (token, row segment). SINGLE: the segment is exactly one
// 16-byte chunk per lane (the default launch shape); otherwise the segment is
// copied in groups of U chunks per lane, then one chunk at a time.
template <int K, bool NT, bool SINGLE, int MODE>
__global__ __launch_bounds__(kMaxBlockThreads)
void dispatch_kernel(const v4i* __restrict__ x, const float* __restrict__ scores,
                     const int32_t* __restrict__ row_map, int32_t T, int32_t chunks,
                     int32_t segments, int32_t seg_chunks, int64_t max_rows,
                     v4i* __restrict__ x_e, float* __restrict__ s_e) {
    constexpr int U = kDispatchUnroll;
    // Row-map entries of the workgroup's tokens: one coalesced load, then a
    // barrier. The barrier also starts the workgroup's wavefronts together, so
    // they store neighbouring 1 KiB pieces of the same rows at the same time.
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
        const bool ok = r >= 0 && r < max_rows;
        tile_rows[tid] = ok ? r : -1;
        if constexpr (MODE != kCopy) tile_scores[tid] = ok ? scores[t_first * K + tid] : 0.0f;
    }
    __syncthreads();

    const int64_t item = item0 + wave;
    const int64_t t = item / segments;
    if (t >= T) return;
    const int seg = static_cast<int>(item - t * segments);
    const int32_t* rows = tile_rows + (t - t_first) * K;
    int32_t row[K];
    float s[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        row[k] = __builtin_amdgcn_readfirstlane(rows[k]);
        s[k] = 0.0f;
        if constexpr (MODE != kCopy)
            s[k] = __int_as_float(__builtin_amdgcn_readfirstlane(
                __float_as_int(tile_scores[(t - t_first) * K + k])));
    }

    const int32_t c_begin = seg * seg_chunks;
    const int32_t c_end = min(c_begin + seg_chunks, chunks);
    const v4i* src = x + t * chunks;

    // Lane k < K of the first segment also moves slot k's score.
    auto move_score = [&]() {
        if (seg == 0 && lane < K) {
            const int32_t r = rows[lane];
            if (r >= 0) s_e[r] = scores[t * K + lane];
        }
    };

    if constexpr (SINGLE) {
        const int32_t c = c_begin + lane;
        const bool in = c < c_end;
        v4i v;
        if (in) v = src[c];
        move_score();
        if (in) {
#pragma unroll
            for (int k = 0; k < K; ++k)
                if (row[k] >= 0) put<NT>(x_e + int64_t(row[k]) * chunks + c, transform<MODE>(s[k], v));
        }
    } else {
        move_score();
        int32_t c0 = c_begin;
        // Whole groups: every lane has U chunks in range.
        for (; c0 + 64 * U <= c_end; c0 += 64 * U) {
            v4i v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) v[u] = src[c0 + u * 64 + lane];
#pragma unroll
            for (int k = 0; k < K; ++k) {
                if (row[k] < 0) continue;
                v4i* dst = x_e + int64_t(row[k]) * chunks + c0 + lane;
#pragma unroll
                for (int u = 0; u < U; ++u) put<NT>(dst + u * 64, transform<MODE>(s[k], v[u]));
            }
        }
        // Tail: one chunk per lane at a time, the last possibly partial.
        for (; c0 < c_end; c0 += 64) {
            const int32_t c = c0 + lane;
            if (c >= c_end) break;
            const v4i v = src[c];
#pragma unroll
            for (int k = 0; k < K; ++k)
                if (row[k] >= 0) put<NT>(x_e + int64_t(row[k]) * chunks + c, transform<MODE>(s[k], v));
        }
    }
}

template <int K>
hipError_t launch_k(const DispatchArgs& a, int32_t segments, int32_t seg_chunks,
                    hipStream_t stream) {
    const int64_t items = int64_t(a.T) * segments;
    const int64_t blocks = (items + a.block_waves - 1) / a.block_waves;
    const bool single = seg_chunks == 64;
    decltype(&dispatch_kernel<K, false, true, kCopy>) kernel;
    if (a.scaled) {  // streaming stores are not offered with the scores applied
        kernel = a.bf16 ? (single ? dispatch_kernel<K, false, true, kScaleBF16>
                                  : dispatch_kernel<K, false, false, kScaleBF16>)
                        : (single ? dispatch_kernel<K, false, true, kScaleF32>
                                  : dispatch_kernel<K, false, false, kScaleF32>);
    } else {
        kernel = a.nontemporal ? (single ? dispatch_kernel<K, true, true, kCopy>
                                         : dispatch_kernel<K, true, false, kCopy>)
                               : (single ? dispatch_kernel<K, false, true, kCopy>
                                         : dispatch_kernel<K, false, false, kCopy>);
    }
    hipLaunchKernelGGL(kernel, dim3(static_cast<uint32_t>(blocks)), dim3(64 * a.block_waves), 0,
                       stream, static_cast<const v4i*>(a.x), a.scores, a.row_map, a.T,
                       a.chunks, segments, seg_chunks, a.max_rows, static_cast<v4i*>(a.x_e),
                       a.s_e);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t stream) {
    if (a.T <= 0) return hipSuccess;
    const int32_t seg_chunks = segment_chunks(a.chunks, a.segments);
    const int32_t segments = (a.chunks + seg_chunks - 1) / seg_chunks;
    switch (a.K) {
#define MOE_DISPATCH_CASE(k) \
    case k: return launch_k<k>(a, segments, seg_chunks, stream);
        MOE_DISPATCH_CASE(1) MOE_DISPATCH_CASE(2) MOE_DISPATCH_CASE(3) MOE_DISPATCH_CASE(4)
        MOE_DISPATCH_CASE(5) MOE_DISPATCH_CASE(6) MOE_DISPATCH_CASE(7) MOE_DISPATCH_CASE(8)
        MOE_DISPATCH_CASE(9) MOE_DISPATCH_CASE(10) MOE_DISPATCH_CASE(11) MOE_DISPATCH_CASE(12)
        MOE_DISPATCH_CASE(13) MOE_DISPATCH_CASE(14) MOE_DISPATCH_CASE(15) MOE_DISPATCH_CASE(16)
#undef MOE_DISPATCH_CASE
        default: return hipErrorInvalidValue;
    }
}

}  // namespace moe
