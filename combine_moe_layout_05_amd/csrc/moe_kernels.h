// Internal declarations shared by the HIP kernels and the host API of
// libmoe_layout.so. Not part of the public C ABI (include/moe.h).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace moe {

// Layout: one workgroup of 4 wavefronts sorts a tile of 1024 (t,k) slots;
// each lane holds 4 slots, one per 64-slot chunk of its wavefront's
// 256-slot run.
constexpr int kLayoutThreads = 256;
constexpr int kLayoutWaves = kLayoutThreads / 64;
constexpr int kLayoutSlotsPerLane = 4;
constexpr int kLayoutTile = kLayoutThreads * kLayoutSlotsPerLane;
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopk = 16;

// Dispatch and combine: one (token, row segment) work item per wavefront,
// 16-byte accesses per lane, 1..16 wavefronts per workgroup (a launch-time
// choice; kernels read it from blockDim).
constexpr int kMaxBlockWaves = 16;
constexpr int kMaxBlockThreads = kMaxBlockWaves * 64;
constexpr int kMaxSegments = 16;
// MI355X last-level (Infinity) cache: outputs larger than this cannot stay
// cached for their consumer anyway.
constexpr int64_t kLastLevelCacheBytes = int64_t(256) << 20;

static_assert(kMaxExperts % kLayoutThreads == 0, "experts split evenly over layout threads");

// Number of layout tiles covering n slots.
inline int64_t layout_tiles(int64_t slots) {
    return (slots + kLayoutTile - 1) / kLayoutTile;
}

// Experts rounded up to a multiple of 4: the row stride of the per-tile
// histograms, so rows can be read as 16-byte vectors.
inline int32_t padded_experts(int32_t E) { return (E + 3) & ~3; }

// Bits needed to tell experts 0..E-1 apart (0 for E == 1).
inline int expert_bits(int32_t E) {
    int b = 0;
    while ((int64_t(1) << b) < E) ++b;
    return b;
}

// Chunks of 16 bytes per segment work item, a multiple of 64 so that each
// wavefront access covers a whole 1 KiB run.
inline int32_t segment_chunks(int32_t chunks, int32_t segments) {
    const int32_t waves_of_chunks = (chunks + 63) / 64;
    const int32_t per_seg = (waves_of_chunks + segments - 1) / segments;
    return per_seg * 64;
}

struct LayoutArgs {
    const int32_t* ids;     // [T][K]
    int64_t nvalid;         // T*K slots that may hold an expert
    int64_t nslots;         // round_up4(ntpr)*K slots written to row_map
    int32_t E;
    int32_t* block_hist;    // [tiles][E]
    int32_t* counts;        // [E]
    int32_t* offsets;       // [E+1]
    int32_t* row_map;       // [nslots]
    int32_t* src_map;       // [total]
};
hipError_t launch_layout(const LayoutArgs& a, hipStream_t stream);

struct DispatchArgs {
    const void* x;          // [T][row_bytes]
    const float* scores;    // [T][K]
    const int32_t* row_map; // [T][K]
    int32_t T;
    int32_t K;
    int32_t chunks;         // row_bytes / 16
    int64_t max_rows;       // rows of x_e / s_e
    void* x_e;
    float* s_e;
    int32_t segments;
    int32_t block_waves;    // wavefronts per workgroup, 1..16
    bool nontemporal;
    bool scaled;            // x_e[r] = scores[t][k] * x[t] instead of a bit copy
    bool bf16;              // element type (used when scaled)
};
hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t stream);

struct CombineArgs {
    const void* y_e;        // [>= total][row_bytes]
    const int32_t* row_map; // [T][K]
    const float* scores;    // [T][K]
    int32_t T;
    int32_t K;
    int32_t chunks;         // row_bytes / 16
    int64_t row_limit;      // rows >= this (or < 0) count as no expert
    bool bf16;
    void* y;                // [T][row_bytes]
    int32_t segments;
    int32_t block_waves;    // wavefronts per workgroup, 1..16
    bool nontemporal;       // streaming loads of the expert outputs
    bool store_nontemporal; // streaming stores of y
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t stream);

struct CombineBackwardArgs {
    const void* grad_y;     // [T][row_bytes]
    const void* y_e;        // [>= row_limit][row_bytes]
    const int32_t* row_map; // [T][K]
    const float* scores;    // [T][K]
    int32_t T;
    int32_t K;
    int32_t chunks;         // row_bytes / 16
    int64_t row_limit;      // rows >= this (or < 0) count as no expert
    bool bf16;
    void* grad_y_e;         // rows r(t,k) written
    float* grad_s;          // [T][K]
};
hipError_t launch_combine_backward(const CombineBackwardArgs& a, hipStream_t stream);

struct TopkFromMapArgs {
    const uint8_t* map;     // [T][E], nonzero = routed
    const float* probs;     // [T][E]
    int32_t T;
    int32_t E;
    int32_t K;
    int32_t* ids;           // [T][K]
    float* scores;          // [T][K]
    int32_t* n_experts;     // [T]
};
hipError_t launch_topk_from_map(const TopkFromMapArgs& a, hipStream_t stream);

}  // namespace moe
