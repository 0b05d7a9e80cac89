// Host-only stand-ins for the kernel launchers of libmoe_layout.so, so the
// host side (argument checks, workspace carve-up, call-order state) can be
// built and run under AddressSanitizer / UndefinedBehaviorSanitizer without
// a GPU. Each stub checks that the arguments the host code computed are
// self-consistent and counts the call; nothing touches the pointers.
#include <cstdio>
#include <cstdlib>

#include "moe_kernels.h"

namespace moe {

int g_launches = 0;

static void require(bool ok, const char* what) {
    if (!ok) {
        std::fprintf(stderr, "stub: inconsistent launch arguments: %s\n", what);
        std::abort();
    }
}

hipError_t launch_layout(const LayoutArgs& a, hipStream_t) {
    require(a.E >= 1 && a.nvalid >= 0 && a.nslots >= a.nvalid, "layout sizes");
    require(a.launches >= 0 && a.launches <= 2, "layout launches");
    // The two-launch form needs its per-tile histograms.
    require(layout_hist_bytes(a.nslots, a.E, a.launches) == 0 || a.block_hist != nullptr,
            "layout histograms");
    ++g_launches;
    return hipSuccess;
}

// Stand-in for the static device scratch: a fake, aligned address that is
// never dereferenced.
hipError_t noalloc_scratch(void** out) {
    *out = reinterpret_cast<void*>(uintptr_t(1) << 42);
    return hipSuccess;
}
hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t) {
    require(a.T >= 0 && a.K >= 1 && a.chunks >= 1 && a.segments >= 1 && a.block_waves >= 1 &&
                a.block_waves <= kMaxBlockWaves,
            "dispatch shape");
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_layout_dispatch(const FusedLayoutDispatchArgs& a, hipStream_t) {
    require(a.layout.E >= 1 && a.layout.nvalid >= 0 && a.layout.nslots >= a.layout.nvalid &&
                a.counter_slot >= 0 && a.counter_slot < kFusedCounterSlots &&
                a.dispatch.T >= 0 && a.dispatch.K >= 1 && a.dispatch.chunks >= 1 &&
                a.dispatch.segments >= 1 && a.dispatch.block_waves >= 1 &&
                a.dispatch.block_waves <= kMaxBlockWaves &&
                a.layout.nvalid == int64_t(a.dispatch.T) * a.dispatch.K && a.ids == a.layout.ids,
            "fused layout+dispatch shape");
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_combine(const CombineArgs& a, hipStream_t) {
    require(a.T >= 0 && a.K >= 1 && a.chunks >= 1 && a.segments >= 1 && a.block_waves >= 1 &&
                a.block_waves <= kMaxBlockWaves && a.row_limit >= 0,
            "combine shape");
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_combine_backward(const CombineBackwardArgs& a, hipStream_t) {
    require(a.T >= 0 && a.K >= 1 && a.chunks >= 1, "combine backward shape");
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_topk_from_map(const TopkFromMapArgs& a, hipStream_t) {
    require(a.T >= 0 && a.E >= 1 && a.K >= 1, "routing map shape");
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_grouped_gemm(const GroupedGemmArgs& a, hipStream_t) {
    require(a.E >= 1 && a.max_rows >= 1 && a.Kd % 8 == 0 && a.N % 8 == 0 &&
                (a.row_tile == kGemmRowTileSmall || a.row_tile == kGemmRowTileLarge),
            "grouped gemm shape");
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_tile_weights(const TileWeightsArgs& a, hipStream_t) {
    require(a.E >= 1 && a.Kd % 8 == 0 && a.N % 8 == 0, "tile shape");
    ++g_launches;
    return hipSuccess;
}

}  // namespace moe
