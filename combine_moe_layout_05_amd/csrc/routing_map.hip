// Routing-map input format on gfx950: turn a boolean routing map [T][E] with
// probabilities [T][E] into the top-k form [T][K] the layout takes.
//
// What is computed ("fix(moe): equalize and align per-rank token counts for
// HybridEP dispatch", section "Fix": HybridEP's dispatcher takes a routing
// map and probabilities, and padded rows are all-False with zero
// probability): slot k of token t is the k-th expert e, in ascending order,
// with map[t][e] != 0, and its score is probs[t][e] (bit copy); slots past the
// token's experts get id -1 and score 0, so an all-False row routes nowhere.
// n_experts[t] is the number of experts in the row; a row with more than K
// keeps its K lowest (n_experts[t] > K tells the caller, on the device).
//
// One wavefront per token: each pass reads 64 map bytes (one per lane), a
// ballot marks the experts present, and a lane's slot is the running count
// plus the experts below it in the ballot, so slots come out in expert order
// without atomics.
#include "moe_kernels.h"

namespace moe {
namespace {

constexpr int kMapThreads = 256;

__global__ __launch_bounds__(kMapThreads)
void topk_from_map_kernel(const uint8_t* __restrict__ map, const float* __restrict__ probs,
                          int32_t T, int32_t E, int32_t K, int32_t* __restrict__ ids,
                          float* __restrict__ scores, int32_t* __restrict__ n_experts) {
    const int lane = __lane_id();
    const int64_t t = int64_t(blockIdx.x) * (kMapThreads / 64) + (threadIdx.x >> 6);
    if (t >= T) return;
    const uint8_t* row = map + t * E;
    const float* prow = probs + t * E;
    const uint64_t below = (uint64_t(1) << lane) - 1;
    int32_t n = 0;
    for (int32_t e0 = 0; e0 < E; e0 += 64) {
        const int32_t e = e0 + lane;
        const bool on = e < E && row[e] != 0;
        const uint64_t m = __ballot(on);
        if (on) {
            const int32_t pos = n + __popcll(m & below);
            if (pos < K) {
                ids[t * K + pos] = e;
                scores[t * K + pos] = prow[e];
            }
        }
        n += __popcll(m);
    }
    for (int32_t k = n + lane; k < K; k += 64) {
        ids[t * K + k] = -1;
        scores[t * K + k] = 0.0f;
    }
    if (lane == 0) n_experts[t] = n;
}

}  // namespace

hipError_t launch_topk_from_map(const TopkFromMapArgs& a, hipStream_t stream) {
    if (a.T <= 0) return hipSuccess;
    const int64_t blocks = (int64_t(a.T) + kMapThreads / 64 - 1) / (kMapThreads / 64);
    hipLaunchKernelGGL(topk_from_map_kernel, dim3(static_cast<uint32_t>(blocks)),
                       dim3(kMapThreads), 0, stream, a.map, a.probs, a.T, a.E, a.K, a.ids,
                       a.scores, a.n_experts);
    return hipGetLastError();
}

}  // namespace moe
