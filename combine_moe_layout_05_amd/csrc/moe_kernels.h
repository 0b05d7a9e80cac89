// Internal declarations shared by the HIP kernels and the host API of
// libmoe_layout.so. Not part of the public C ABI (include/moe.h).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace moe {

// Layout: one workgroup of 4 wavefronts sorts a tile of 256*R (t,k) slots;
// each lane holds R slots, one per 64-slot chunk of its wavefront's run.
// R is chosen per call: 2 (512-slot tiles) up to kLayoutSmallSlots slots, 4
// (1024-slot tiles) above (measured on MI355X: more, smaller tiles win while
// the tile count is small; past that the per-tile offset sums dominate).
constexpr int kLayoutThreads = 256;
constexpr int kLayoutWaves = kLayoutThreads / 64;
constexpr int kLayoutMinSlotsPerLane = 2;
constexpr int kLayoutMaxSlotsPerLane = 4;
constexpr int64_t kLayoutSmallSlots = 65536;
// The largest tile count any call can use: the smallest tile.
constexpr int kLayoutTile = kLayoutThreads * kLayoutMinSlotsPerLane;
inline int layout_slots_per_lane(int64_t slots) {
    return slots <= kLayoutSmallSlots ? kLayoutMinSlotsPerLane : kLayoutMaxSlotsPerLane;
}
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

// Number of layout tiles covering n slots with R slots per lane; without R,
// the most any call can use.
inline int64_t layout_tiles(int64_t slots, int slots_per_lane) {
    const int64_t tile = int64_t(kLayoutThreads) * slots_per_lane;
    return (slots + tile - 1) / tile;
}
inline int64_t layout_tiles(int64_t slots) {
    return layout_tiles(slots, kLayoutMinSlotsPerLane);
}

// Single-launch layout: workgroups of 16 wavefronts, each owning a tile of
// 1024*R slots (R = 1, 2 or 4, chosen by the slot count) and each counting
// every slot of the batch itself. Chosen automatically up to
// kLayoutSingleMaxSlots slots. Measured on MI355X: 7.1 us against 8.9 us for
// the two launches at 16384 slots, 8.1 against 10.0 at 32768; at 65536 the
// repeated counting (LDS adds, about 1 us per 16384 slots) makes it 10.9
// against 9.5.
constexpr int kLayoutSingleThreads = 1024;
constexpr int64_t kLayoutSingleMaxSlots = 32768;
inline int layout_single_slots_per_lane(int64_t slots) {
    return slots <= 32768 ? 1 : (slots <= 65536 ? 2 : 4);
}
static_assert(kMaxExperts <= kLayoutSingleThreads, "one expert per thread in the single-launch scan");

// Experts rounded up to a multiple of 4: the row stride of the per-tile
// histograms, so rows can be read as 16-byte vectors.
inline int32_t padded_experts(int32_t E) { return (E + 3) & ~3; }

// Whether a layout of nslots slots runs as the single launch: forced by
// launches (1: single, 2: two launches) or, with 0, chosen by size.
inline bool layout_single_launch(int64_t nslots, int32_t launches) {
    return launches == 1 || (launches == 0 && nslots <= kLayoutSingleMaxSlots);
}
// Bytes of per-tile histograms (block_hist) such a layout uses: none for the
// single launch, one row of round_up4(E) int32 per tile for the two launches.
inline int64_t layout_hist_bytes(int64_t nslots, int32_t E, int32_t launches) {
    if (layout_single_launch(nslots, launches)) return 0;
    return layout_tiles(nslots, layout_slots_per_lane(nslots)) * padded_experts(E) * 4;
}

// Static scratch of moe_layout_noalloc, per device: the per-tile histograms
// of the two-launch layout (4 MiB: e.g. 4096 tiles of 256 experts, 1024 of
// 1024 experts).
constexpr int64_t kNoallocScratchBytes = int64_t(4) << 20;
// Device address of this device's scratch array (looked up once per device
// with hipGetSymbolAddress; the device is the current one).
hipError_t noalloc_scratch(void** out);

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
    int32_t launches = 0;   // 1: single launch, 2: count + rank, 0: by size
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
    bool store_burst = false;  // single-chunk copies: K stores back to back
    bool load_nontemporal = false;  // streaming loads of x
};
hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t stream);

// Layout fused into dispatch, two launches (the separate calls take three
// above kLayoutSingleMaxSlots slots, two up to it). The count launch's last
// workgroup to finish (found with a per-context completion
// counter, kept in a static device array so it starts at zero) turns the
// tile histograms in block_hist into each tile's first row per expert and
// writes counts and offsets; dispatch then ranks each of its tokens' slots
// among the earlier slots of the same tile, writes row_map and src_map, and
// copies the rows. Results equal moe_layout followed by moe_dispatch.
constexpr int kFusedCounterSlots = 1024;
struct FusedLayoutDispatchArgs {
    LayoutArgs layout;      // block_hist ends up holding each tile's first rows
    DispatchArgs dispatch;  // row_map is written here, not read
    const int32_t* ids;     // [T][K]
    int32_t counter_slot;   // 0 .. kFusedCounterSlots-1, one per context
};
hipError_t launch_layout_dispatch(const FusedLayoutDispatchArgs& a, hipStream_t stream);
// The count launch of the fused path (defined with the layout kernels);
// tile_slots receives the tile size it used.
hipError_t launch_layout_count_scan(const LayoutArgs& a, int32_t counter_slot, int32_t* tile_slots,
                                    hipStream_t stream);

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
    const int32_t* total_rows = nullptr;  // device; rows [*total_rows, row_limit) of
                                          // grad_y_e get +0.0 (nullptr: not written)
    bool store_nontemporal = false;       // streaming stores of grad_y_e
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

// Expert step (grouped GEMM): workgroups of the launch for max_rows rows,
// E experts, N output features, row tiles of row_tile rows and feature tiles
// of `features`: every (feature tile, row tile) pair the worst routing can
// need, rounded up to whole chunks of tiles per XCD.
// Tile numbers are dealt to the 8 XCDs in chunks of kGemmXcdChunk
// consecutive tiles, round-robin. Each XCD then gets a share of every large
// expert instead of a few whole experts, which evens out the HBM traffic the
// XCDs draw, while a chunk still keeps a block of one expert's tiles together
// in one L2. Measured on MI355X (256 experts, 7168 -> 4096, interleaved on
// one box): 4096 tokens 3.46-3.49 ms with chunks of 32 against 3.54-3.56
// with one contiguous run of tile numbers per XCD, 3.51 with chunks of 16,
// 3.59 with 64; 32768 tokens 13.91-14.08 against 14.01-14.21 ms with 16
// (uniform routing) and 13.90-13.97 against 14.08-14.13 ms (Zipf), with
// about a tenth less L2-miss traffic (each row tile is fetched by fewer
// chunks); contiguous runs there 14.9-15.2 ms.
constexpr int32_t kGemmXcdChunk = 32;
inline int64_t grouped_gemm_grid(int64_t max_rows, int32_t E, int32_t N, int32_t row_tile,
                                 int32_t features) {
    const int64_t ftiles = (int64_t(N) + features - 1) / features;
    const int64_t tiles = ftiles * ((max_rows + row_tile - 1) / row_tile + E);
    // Whole chunks per XCD, so the dealt tile numbers cover [0, grid).
    const int64_t unit = 8 * int64_t(kGemmXcdChunk);
    return (tiles + unit - 1) / unit * unit;
}
constexpr int kGemmRowTileSmall = 64;
constexpr int kGemmRowTileLarge = 128;
// Wavefronts per workgroup and 32-feature blocks per wavefront: row-major
// weights are staged through LDS per wavefront (one block each); tiled
// weights go straight to registers, two blocks per wavefront, so each row
// fragment read from LDS feeds two matrix-core products.
constexpr int kGemmWavesRowMajor = 4;
constexpr int kGemmWavesTiled = 8;
constexpr int kGemmBlocksTiled = 2;
// Output features per workgroup tile.
constexpr int32_t gemm_tile_features(bool tiled) {
    return tiled ? 32 * kGemmWavesTiled * kGemmBlocksTiled : 32 * kGemmWavesRowMajor;
}

struct GroupedGemmArgs {
    const void* x_e;        // [max_rows][Kd] bf16
    const void* w;          // [E][N][Kd] bf16, or the tiled form of it
    const int32_t* offsets; // [E+1], device
    int32_t E;
    int64_t max_rows;       // <= INT32_MAX
    int32_t Kd;             // multiple of 8
    int32_t N;              // multiple of 8
    int32_t row_tile;       // kGemmRowTileSmall or kGemmRowTileLarge
    bool tiled;             // w is in the tiled layout
    void* out;              // [max_rows][N] bf16
};
hipError_t launch_grouped_gemm(const GroupedGemmArgs& a, hipStream_t stream);

// Tiled weight layout: [E][ceil(N/32)][ceil(Kd/64)][4][64] chunks of 16 bytes.
inline int64_t tiled_weights_bytes(int32_t E, int32_t N, int32_t Kd) {
    return int64_t(E) * ((int64_t(N) + 31) / 32) * ((int64_t(Kd) + 63) / 64) * 256 * 16;
}
struct TileWeightsArgs {
    const void* src;        // [E][N][Kd] bf16
    int32_t E;
    int32_t N;              // multiple of 8
    int32_t Kd;             // multiple of 8
    void* dst;              // tiled_weights_bytes(E, N, Kd) bytes
};
hipError_t launch_tile_weights(const TileWeightsArgs& a, hipStream_t stream);

}  // namespace moe
