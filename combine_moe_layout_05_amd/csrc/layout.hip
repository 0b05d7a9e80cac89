// Routing layout on gfx950: per-expert counts, their exclusive prefix sum and
// a stable row map, all kept on the device.
//
// What is computed ("Unify expert parallel token dispatcher API", section
// "API design": per-expert token counts feed dispatch; "ep: graph-safe
// worst-token HT dispatch+combine", "Internode" items 2 and 3: counts and the
// true total stay on the device; "fix(moe): equalize and align per-rank token
// counts for HybridEP dispatch", section "Fix": padded rows route to no
// expert):
//   counts[e]  = #{(t,k) : t < T, ids[t][k] == e}
//   offsets[e] = sum of counts below e, offsets[E] = total
//   row_map[t*K+k] = offsets[e] + #{earlier slots (by t*K+k) with expert e},
//                    or -1 (no expert, or padding t >= T)
//   src_map[row]   = t*K+k
//
// Three launches, no atomics on global memory and no host round trip:
//   1. count: each workgroup histograms a 1024-slot tile into LDS and writes
//      its row of block_hist[tile][e].
//   2. scan: one workgroup; thread e scans block_hist[.][e] over tiles into
//      block_base (exclusive, per expert) and then the workgroup scans the
//      per-expert totals into offsets.
//   3. rank: each workgroup re-reads its tile and ranks every slot among the
//      earlier slots of the same expert; the order is fixed by the slot
//      index alone, so the result is deterministic under any skew.
// Within a wavefront, slots with the same expert are found with a ballot per
// expert-id bit (a lane's peers are the lanes whose id agrees on every bit);
// the lowest peer updates the wavefront's LDS histogram once per group, so a
// hot expert costs one LDS update per 64 slots, not 64.
#include "moe_kernels.h"

namespace moe {
namespace {

__device__ __forceinline__ uint64_t lanes_below() {
    return (uint64_t(1) << __lane_id()) - 1;
}

// Mask of the active wavefront lanes whose valid key equals this lane's.
// Must be called by all 64 lanes together.
__device__ __forceinline__ uint64_t peer_mask(int32_t key, bool valid, int bits) {
    uint64_t m = __ballot(valid);
    for (int b = 0; b < bits; ++b) {
        const bool bit = (key >> b) & 1;
        const uint64_t v = __ballot(bit);
        m &= bit ? v : ~v;
    }
    return m;
}

// Expert of slot i, or -1 for padding slots and ids outside [0,E).
__device__ __forceinline__ int32_t slot_expert(const int32_t* __restrict__ ids,
                                               int64_t i, int64_t nvalid, int32_t E) {
    if (i >= nvalid) return -1;
    const int32_t e = ids[i];
    return (static_cast<uint32_t>(e) < static_cast<uint32_t>(E)) ? e : -1;
}

__global__ __launch_bounds__(kLayoutThreads)
void layout_count_kernel(const int32_t* __restrict__ ids, int64_t nvalid,
                         int32_t E, int bits, int32_t* __restrict__ block_hist) {
    __shared__ int32_t hist[kMaxExperts];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    for (int e = tid; e < E; e += kLayoutThreads) hist[e] = 0;
    __syncthreads();

    const int64_t base = int64_t(blockIdx.x) * kLayoutTile + wave * (64 * kLayoutSlotsPerLane);
    int32_t ex[kLayoutSlotsPerLane];
#pragma unroll
    for (int j = 0; j < kLayoutSlotsPerLane; ++j)
        ex[j] = slot_expert(ids, base + j * 64 + lane, nvalid, E);

    const uint64_t below = lanes_below();
#pragma unroll
    for (int j = 0; j < kLayoutSlotsPerLane; ++j) {
        const bool valid = ex[j] >= 0;
        const uint64_t peers = peer_mask(ex[j], valid, bits);
        if (valid && (peers & below) == 0) atomicAdd(&hist[ex[j]], __popcll(peers));
    }
    __syncthreads();
    int32_t* out = block_hist + int64_t(blockIdx.x) * E;
    for (int e = tid; e < E; e += kLayoutThreads) out[e] = hist[e];
}

__global__ __launch_bounds__(kScanThreads)
void layout_scan_kernel(const int32_t* __restrict__ block_hist, int32_t tiles, int32_t E,
                        int32_t* __restrict__ block_base, int32_t* __restrict__ counts,
                        int32_t* __restrict__ offsets) {
    __shared__ int32_t wave_sum[kScanThreads / 64];
    const int e = threadIdx.x;
    const int lane = e & 63;
    const int wave = e >> 6;

    // Per expert, exclusive scan over tiles (tile order = slot order).
    int32_t run = 0;
    if (e < E) {
        int32_t b = 0;
        for (; b + 8 <= tiles; b += 8) {
            int32_t v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = block_hist[int64_t(b + u) * E + e];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                block_base[int64_t(b + u) * E + e] = run;
                run += v[u];
            }
        }
        for (; b < tiles; ++b) {
            const int32_t v = block_hist[int64_t(b) * E + e];
            block_base[int64_t(b) * E + e] = run;
            run += v;
        }
    }

    // Inclusive scan of the per-expert totals across the workgroup.
    int32_t incl = run;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int32_t up = __shfl_up(incl, d, 64);
        if (lane >= d) incl += up;
    }
    if (lane == 63) wave_sum[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        int32_t w = lane < kScanThreads / 64 ? wave_sum[lane] : 0;
#pragma unroll
        for (int d = 1; d < kScanThreads / 64; d <<= 1) {
            const int32_t up = __shfl_up(w, d, 64);
            if (lane >= d) w += up;
        }
        if (lane < kScanThreads / 64) wave_sum[lane] = w;
    }
    __syncthreads();
    if (wave > 0) incl += wave_sum[wave - 1];
    if (e < E) {
        counts[e] = run;
        offsets[e] = incl - run;
        if (e == E - 1) offsets[E] = incl;
    }
}

__global__ __launch_bounds__(kLayoutThreads)
void layout_rank_kernel(const int32_t* __restrict__ ids, int64_t nvalid, int64_t nslots,
                        int32_t E, int bits, const int32_t* __restrict__ offsets,
                        const int32_t* __restrict__ block_base,
                        int32_t* __restrict__ row_map, int32_t* __restrict__ src_map) {
    __shared__ int32_t wave_hist[kLayoutWaves][kMaxExperts];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    for (int e = tid; e < E; e += kLayoutThreads) {
#pragma unroll
        for (int w = 0; w < kLayoutWaves; ++w) wave_hist[w][e] = 0;
    }
    __syncthreads();

    const int64_t base = int64_t(blockIdx.x) * kLayoutTile + wave * (64 * kLayoutSlotsPerLane);
    int32_t ex[kLayoutSlotsPerLane];
    int32_t local[kLayoutSlotsPerLane];
#pragma unroll
    for (int j = 0; j < kLayoutSlotsPerLane; ++j)
        ex[j] = slot_expert(ids, base + j * 64 + lane, nvalid, E);

    // Rank within this wavefront's run, chunk by chunk in slot order. All
    // peers read the expert's running count before the lowest peer advances
    // it; a wavefront's LDS operations complete in program order.
    int32_t* mine = wave_hist[wave];
    const uint64_t below = lanes_below();
#pragma unroll
    for (int j = 0; j < kLayoutSlotsPerLane; ++j) {
        const bool valid = ex[j] >= 0;
        const uint64_t peers = peer_mask(ex[j], valid, bits);
        const int32_t before = valid ? mine[ex[j]] : 0;
        local[j] = before + __popcll(peers & below);
        if (valid && (peers & below) == 0) mine[ex[j]] = before + __popcll(peers);
        __builtin_amdgcn_wave_barrier();
    }
    __syncthreads();

    // Turn the per-wavefront counts into each wavefront's first row per expert.
    const int32_t* tile_base = block_base + int64_t(blockIdx.x) * E;
    for (int e = tid; e < E; e += kLayoutThreads) {
        int32_t run = offsets[e] + tile_base[e];
#pragma unroll
        for (int w = 0; w < kLayoutWaves; ++w) {
            const int32_t c = wave_hist[w][e];
            wave_hist[w][e] = run;
            run += c;
        }
    }
    __syncthreads();

#pragma unroll
    for (int j = 0; j < kLayoutSlotsPerLane; ++j) {
        const int64_t i = base + j * 64 + lane;
        if (i >= nslots) continue;
        if (ex[j] >= 0) {
            const int32_t r = mine[ex[j]] + local[j];
            row_map[i] = r;
            // r < total <= nslots by construction; the bound only keeps a
            // logic error from writing outside the buffer.
            if (r >= 0 && r < nslots) src_map[r] = static_cast<int32_t>(i);
        } else {
            row_map[i] = -1;
        }
    }
}

}  // namespace

hipError_t launch_layout(const LayoutArgs& a, hipStream_t stream) {
    const int64_t tiles = layout_tiles(a.nslots);
    const int bits = expert_bits(a.E);
    if (tiles > 0) {
        hipLaunchKernelGGL(layout_count_kernel, dim3(static_cast<uint32_t>(tiles)),
                           dim3(kLayoutThreads), 0, stream, a.ids, a.nvalid, a.E, bits,
                           a.block_hist);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL(layout_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream,
                       a.block_hist, static_cast<int32_t>(tiles), a.E, a.block_base,
                       a.counts, a.offsets);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (tiles > 0) {
        hipLaunchKernelGGL(layout_rank_kernel, dim3(static_cast<uint32_t>(tiles)),
                           dim3(kLayoutThreads), 0, stream, a.ids, a.nvalid, a.nslots, a.E,
                           bits, a.offsets, a.block_base, a.row_map, a.src_map);
        err = hipGetLastError();
    }
    return err;
}

}  // namespace moe
