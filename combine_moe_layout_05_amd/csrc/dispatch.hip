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
// 1 KiB run, and stores it K times. The workgroup's row-map entries (at most
// 4 tokens x K) are staged in LDS with one coalesced load and read back as
// wavefront-uniform scalars, so the destination addresses live in SGPRs.
#include "moe_kernels.h"

namespace moe {
namespace {

typedef int32_t v4i __attribute__((ext_vector_type(4)));

template <int U, bool NT>
__global__ __launch_bounds__(kMoveThreads)
void dispatch_kernel(const v4i* __restrict__ x, const float* __restrict__ scores,
                     const int32_t* __restrict__ row_map, int32_t T, int32_t K,
                     int32_t chunks, int32_t segments, int32_t seg_chunks,
                     int64_t max_rows, v4i* __restrict__ x_e, float* __restrict__ s_e) {
    __shared__ int32_t tile_rows[kMoveWaves * kMaxTopk];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    const int64_t item0 = int64_t(blockIdx.x) * kMoveWaves;
    const int64_t t_first = item0 / segments;
    int64_t t_last = (item0 + kMoveWaves - 1) / segments;
    if (t_last > int64_t(T) - 1) t_last = int64_t(T) - 1;
    const int staged = static_cast<int>(t_last - t_first + 1) * K;
    if (tid < staged) {
        const int32_t r = row_map[t_first * K + tid];
        tile_rows[tid] = (r >= 0 && r < max_rows) ? r : -1;
    }
    __syncthreads();

    const int64_t item = item0 + wave;
    const int64_t t = item / segments;
    if (t >= T) return;
    const int seg = static_cast<int>(item - t * segments);
    const int32_t* rows = tile_rows + (t - t_first) * K;

    if (seg == 0 && lane < K) {
        const int32_t r = rows[lane];
        if (r >= 0) s_e[r] = scores[t * K + lane];
    }

    const int32_t c_begin = seg * seg_chunks;
    const int32_t c_end = min(c_begin + seg_chunks, chunks);
    const v4i* src = x + t * chunks;
    for (int32_t c0 = c_begin; c0 < c_end; c0 += 64 * U) {
        v4i v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int32_t c = c0 + u * 64 + lane;
            if (c < c_end) v[u] = src[c];
        }
        for (int k = 0; k < K; ++k) {
            const int32_t r = __builtin_amdgcn_readfirstlane(rows[k]);
            if (r < 0) continue;
            v4i* dst = x_e + int64_t(r) * chunks;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int32_t c = c0 + u * 64 + lane;
                if (c < c_end) {
                    if constexpr (NT)
                        __builtin_nontemporal_store(v[u], dst + c);
                    else
                        dst[c] = v[u];
                }
            }
        }
    }
}

template <int U, bool NT>
hipError_t launch(const DispatchArgs& a, int32_t segments, int32_t seg_chunks,
                  hipStream_t stream) {
    const int64_t items = int64_t(a.T) * segments;
    const int64_t blocks = (items + kMoveWaves - 1) / kMoveWaves;
    hipLaunchKernelGGL((dispatch_kernel<U, NT>), dim3(static_cast<uint32_t>(blocks)),
                       dim3(kMoveThreads), 0, stream, static_cast<const v4i*>(a.x), a.scores,
                       a.row_map, a.T, a.K, a.chunks, segments, seg_chunks, a.max_rows,
                       static_cast<v4i*>(a.x_e), a.s_e);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t stream) {
    if (a.T <= 0) return hipSuccess;
    const int32_t seg_chunks = segment_chunks(a.chunks, a.segments);
    const int32_t segments = (a.chunks + seg_chunks - 1) / seg_chunks;
    return a.nontemporal ? launch<4, true>(a, segments, seg_chunks, stream)
                         : launch<4, false>(a, segments, seg_chunks, stream);
}

}  // namespace moe
