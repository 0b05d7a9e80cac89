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
// One launch up to kLayoutSingleMaxSlots slots (layout_single_kernel: each
// workgroup counts the whole batch into LDS, then ranks its own tile), two
// above it; either way no atomics on global memory and no host round trip.
// The two-launch form:
//   1. count: each workgroup histograms a tile of 512 or 1024 slots (chosen
//      per call by the slot count) into LDS and writes
//      its row of block_hist[tile][e].
//   2. rank: each workgroup first turns the tile histograms into the global
//      offsets (sum over all tiles, exclusive scan over experts) and its own
//      per-expert base (sum over earlier tiles); workgroup 0 also writes
//      counts and offsets. It then re-reads its tile and ranks every slot
//      among the earlier slots of the same expert. The order is fixed by the
//      slot index alone, so the result is deterministic under any skew.
// Within a wavefront, slots with the same expert are found with a ballot per
// expert-id bit (a lane's peers are the lanes whose id agrees on every bit);
// the lowest peer updates the LDS histogram (the workgroup's when counting,
// the wavefront's when ranking) once per group, so a hot expert costs one LDS
// update per 64 slots, not 64.
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

// The id of slot i, loaded without a branch (the index is clamped into the
// batch), so the load's wait comes at the value's first use rather than
// right after it; slot_expert_of then discards padding slots. No load at all
// for an empty batch, whose id array may be absent.
__device__ __forceinline__ int32_t load_slot_id(const int32_t* __restrict__ ids, int64_t i,
                                                int64_t nvalid) {
    if (nvalid <= 0) return -1;
    return ids[i < nvalid ? i : nvalid - 1];
}

// Expert of slot i given its loaded id, or -1 for padding slots and ids
// outside [0,E).
__device__ __forceinline__ int32_t slot_expert_of(int32_t id, int64_t i, int64_t nvalid, int32_t E) {
    return (i < nvalid && static_cast<uint32_t>(id) < static_cast<uint32_t>(E)) ? id : -1;
}

// Histogram rows are padded to E4 = round_up(E, 4) entries (zeros past E) so
// they can be read as 16-byte vectors.
template <int R>
__global__ __launch_bounds__(kLayoutThreads)
void layout_count_kernel(const int32_t* __restrict__ ids, int64_t nvalid,
                         int32_t E, int32_t E4, int bits, int32_t* __restrict__ block_hist) {
    __shared__ int32_t hist[kMaxExperts];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    for (int e = tid; e < E4; e += kLayoutThreads) hist[e] = 0;
    __syncthreads();

    const int64_t base = int64_t(blockIdx.x) * (kLayoutThreads * R) + wave * (64 * R);
    int32_t ex[R];
#pragma unroll
    for (int j = 0; j < R; ++j) ex[j] = load_slot_id(ids, base + j * 64 + lane, nvalid);
#pragma unroll
    for (int j = 0; j < R; ++j) ex[j] = slot_expert_of(ex[j], base + j * 64 + lane, nvalid, E);

    const uint64_t below = lanes_below();
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const bool valid = ex[j] >= 0;
        const uint64_t peers = peer_mask(ex[j], valid, bits);
        if (valid && (peers & below) == 0) atomicAdd(&hist[ex[j]], __popcll(peers));
    }
    __syncthreads();
    int32_t* out = block_hist + int64_t(blockIdx.x) * E4;
    for (int e = tid; e < E4; e += kLayoutThreads) out[e] = hist[e];
}

// Experts owned by one thread in the offset scan (consecutive).
constexpr int kExpertsPerThread = kMaxExperts / kLayoutThreads;
// At most this many threads share one quad of experts in the tile sums.
constexpr int kMaxSlices = 16;
typedef int32_t v4i __attribute__((ext_vector_type(4)));

template <int R>
__global__ __launch_bounds__(kLayoutThreads)
void layout_rank_kernel(const int32_t* __restrict__ ids, int64_t nvalid, int64_t nslots,
                        int32_t E, int32_t E4, int bits, int32_t tiles,
                        const int32_t* __restrict__ block_hist, int32_t* __restrict__ counts,
                        int32_t* __restrict__ offsets, int32_t* __restrict__ row_map,
                        int32_t* __restrict__ src_map) {
    __shared__ int32_t wave_hist[kLayoutWaves][kMaxExperts];
    __shared__ int32_t tile_first[kMaxExperts];
    __shared__ int32_t part_tot[kMaxExperts];
    __shared__ int32_t part_pre[kMaxExperts];
    __shared__ int32_t wave_sum[kLayoutWaves];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int32_t blk = static_cast<int32_t>(blockIdx.x);
    // This wavefront's slots, loaded first so that the load overlaps the
    // tile sums below: slots base + j*64 + lane.
    const int64_t base = int64_t(blockIdx.x) * (kLayoutThreads * R) + wave * (64 * R);
    int32_t ex[R];
#pragma unroll
    for (int j = 0; j < R; ++j) ex[j] = load_slot_id(ids, base + j * 64 + lane, nvalid);

    // Per expert: the total over all tiles and the part in tiles before this
    // one. Thread (quad q, slice sl) sums experts 4q..4q+3 over tiles
    // sl, sl+S, ... with 16-byte loads; the S slices of a quad are then added
    // in LDS (integer adds, so the order does not matter).
    const int quads = E4 / 4;
    int S = kLayoutThreads / quads;
    if (S > kMaxSlices) S = kMaxSlices;
    for (int e = tid; e < E4; e += kLayoutThreads) {
        part_tot[e] = 0;
        part_pre[e] = 0;
#pragma unroll
        for (int w = 0; w < kLayoutWaves; ++w) wave_hist[w][e] = 0;
    }
    __syncthreads();
    {
        const int q = tid % quads;
        const int sl = tid / quads;
        if (sl < S) {
            v4i tot4 = {0, 0, 0, 0};
            v4i pre4 = {0, 0, 0, 0};
            const v4i* h = reinterpret_cast<const v4i*>(block_hist) + q;
#pragma unroll 8
            for (int32_t b = sl; b < tiles; b += S) {
                const v4i v = h[int64_t(b) * quads];
                tot4 += v;
                if (b < blk) pre4 += v;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (tot4[j]) atomicAdd(&part_tot[4 * q + j], tot4[j]);
                if (pre4[j]) atomicAdd(&part_pre[4 * q + j], pre4[j]);
            }
        }
    }
    __syncthreads();
    const int e0 = tid * kExpertsPerThread;
    int32_t tot[kExpertsPerThread];
    int32_t pre[kExpertsPerThread];
#pragma unroll
    for (int j = 0; j < kExpertsPerThread; ++j) {
        const bool in = e0 + j < E4;
        tot[j] = in ? part_tot[e0 + j] : 0;
        pre[j] = in ? part_pre[e0 + j] : 0;
    }
    // Exclusive scan of the totals over experts (thread order = expert order).
    int32_t mine_sum = 0;
#pragma unroll
    for (int j = 0; j < kExpertsPerThread; ++j) mine_sum += tot[j];
    int32_t incl = mine_sum;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int32_t up = __shfl_up(incl, d, 64);
        if (lane >= d) incl += up;
    }
    if (lane == 63) wave_sum[wave] = incl;
    __syncthreads();
    int32_t run = incl - mine_sum;
    for (int w = 0; w < wave; ++w) run += wave_sum[w];
#pragma unroll
    for (int j = 0; j < kExpertsPerThread; ++j) {
        const int e = e0 + j;
        if (e < E) {
            tile_first[e] = run + pre[j];
            if (blk == 0) {
                counts[e] = tot[j];
                offsets[e] = run;
            }
        }
        run += tot[j];
    }
    if (blk == 0 && tid == kLayoutThreads - 1) {
        int32_t total = 0;
        for (int w = 0; w < kLayoutWaves; ++w) total += wave_sum[w];
        offsets[E] = total;
    }

    int32_t local[R];
#pragma unroll
    for (int j = 0; j < R; ++j) ex[j] = slot_expert_of(ex[j], base + j * 64 + lane, nvalid, E);

    // Rank within this wavefront's run, chunk by chunk in slot order. All
    // peers read the expert's running count before the lowest peer advances
    // it; a wavefront's LDS operations complete in program order.
    int32_t* mine = wave_hist[wave];
    const uint64_t below = lanes_below();
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const bool valid = ex[j] >= 0;
        const uint64_t peers = peer_mask(ex[j], valid, bits);
        const int32_t before = valid ? mine[ex[j]] : 0;
        local[j] = before + __popcll(peers & below);
        if (valid && (peers & below) == 0) mine[ex[j]] = before + __popcll(peers);
        __builtin_amdgcn_wave_barrier();
    }
    __syncthreads();

    // Turn the per-wavefront counts into each wavefront's first row per expert.
    for (int e = tid; e < E; e += kLayoutThreads) {
        int32_t run = tile_first[e];
#pragma unroll
        for (int w = 0; w < kLayoutWaves; ++w) {
            const int32_t c = wave_hist[w][e];
            wave_hist[w][e] = run;
            run += c;
        }
    }
    __syncthreads();

#pragma unroll
    for (int j = 0; j < R; ++j) {
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

// Single-launch layout. Workgroup b owns the tile of 1024*R slots starting at
// b*1024*R. It first counts every slot of the batch into LDS, split into the
// slots before its tile and the rest (one LDS integer add per slot; integer
// adds commute, so the totals do not depend on their order). The exclusive
// scan of the totals over experts gives the offsets (workgroup 0 writes
// counts and offsets), and offsets plus the count before the tile give the
// tile's first row per expert. The tile is then ranked as in
// layout_rank_kernel: each wavefront ranks its run of R chunks in slot order
// against a per-wavefront LDS running count, and per-expert prefixes over the
// wavefronts give the final rows. Every workgroup reads the whole id array
// (from L2 after the first), which bounds the batch size this form is used
// for; no workgroup waits for another.
template <int R>
__global__ __launch_bounds__(kLayoutSingleThreads)
void layout_single_kernel(const int32_t* __restrict__ ids, int64_t nvalid, int64_t nslots,
                          int32_t E, int bits, int32_t* __restrict__ counts,
                          int32_t* __restrict__ offsets, int32_t* __restrict__ row_map,
                          int32_t* __restrict__ src_map) {
    constexpr int kWaves = kLayoutSingleThreads / 64;
    constexpr int64_t kTile = int64_t(kLayoutSingleThreads) * R;
    // Count copies: lane l adds into copy l % 8, rows 2c (slots before the
    // tile) and 2c + 1 (the rest) of kCntStride words each, so the lanes of
    // one instruction that share an expert (a hot expert, or the same k-slot
    // of neighbouring tokens) mostly hit different words, and the odd stride
    // puts an expert's word in different LDS banks across the copies. Ids
    // outside [0, E) add into word E of the row, which is never read, so the
    // count needs no branch per slot. The rank step then uses the same words
    // as per-wavefront rank counts, wavefront w at [w * kMaxExperts, ...).
    constexpr int kCopies = 8;
    constexpr int kCntStride = kMaxExperts + 1;
    constexpr int kCntWords = 2 * kCopies * kCntStride;
    constexpr int kRankWords = kWaves * kMaxExperts;
    __shared__ int32_t wave_hist[kCntWords > kRankWords ? kCntWords : kRankWords];
    __shared__ int32_t before[kMaxExperts];   // count before the tile, then the tile's first row
    __shared__ int32_t rest[kMaxExperts];     // count from the tile on
    __shared__ int32_t wave_sum[kWaves];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t tile0 = int64_t(blockIdx.x) * kTile;

    // The tile's own slots for the rank step, loaded first so that their
    // latency overlaps the count: wavefront w holds slots
    // tile0 + w*64*R + j*64 + lane.
    const int64_t base = tile0 + wave * (64 * R);
    int32_t ex[R];
#pragma unroll
    for (int j = 0; j < R; ++j) ex[j] = load_slot_id(ids, base + j * 64 + lane, nvalid);

    int32_t* cnt = wave_hist;
    int32_t* my_cnt = cnt + (lane % kCopies) * 2 * kCntStride;
    for (int e = tid; e < E; e += kLayoutSingleThreads) {
#pragma unroll
        for (int w = 0; w < 2 * kCopies; ++w) cnt[w * kCntStride + e] = 0;
    }
    __syncthreads();

    // Count every slot. The body is read as 16-byte quads of ids, thread tid
    // taking quads tid, tid + 1024, ..., eight loads in flight (addresses
    // clamped into the batch) before their adds; only whole quads past the
    // batch are skipped. With 16-byte aligned ids a quad lies on one side of
    // the tile start, so its row is chosen once. The slots before the first
    // 16-byte boundary and after the last whole quad are read one by one.
    {
        auto add = [&](int32_t e, int64_t i) {
            if (static_cast<uint32_t>(e) < static_cast<uint32_t>(E))
                atomicAdd(&my_cnt[(i < tile0 ? 0 : kCntStride) + e], 1);
        };
        const int64_t mis = static_cast<int64_t>((reinterpret_cast<uintptr_t>(ids) >> 2) & 3);
        const int64_t head = mis == 0 ? 0 : (4 - mis < nvalid ? 4 - mis : nvalid);
        const int32_t nq = static_cast<int32_t>((nvalid - head) / 4);
        const int64_t tail0 = head + 4 * int64_t(nq);
        if (tid < head) add(ids[tid], tid);
        if (tail0 + tid < nvalid) add(ids[tail0 + tid], tail0 + tid);
        const v4i* quads = reinterpret_cast<const v4i*>(ids + head);
        const uint32_t uE = static_cast<uint32_t>(E);
        const int64_t tq = tile0 - head;  // the tile start, in slots from the first quad
        constexpr int kU = 8;
        constexpr int kStep = kLayoutSingleThreads;
        for (int32_t j0 = tid; j0 < nq; j0 += kU * kStep) {
            v4i v[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int32_t j = j0 + u * kStep;
                v[u] = quads[j < nq ? j : nq - 1];
            }
            if (head == 0) {
#pragma unroll
                for (int u = 0; u < kU; ++u) {
                    const int32_t j = j0 + u * kStep;
                    int32_t* row = my_cnt + (4 * int64_t(j) < tq ? 0 : kCntStride);
                    if (j < nq) {
#pragma unroll
                        for (int c = 0; c < 4; ++c)
                            atomicAdd(&row[min(static_cast<uint32_t>(v[u][c]), uE)], 1);
                    }
                }
            } else {
#pragma unroll
                for (int u = 0; u < kU; ++u) {
                    const int32_t j = j0 + u * kStep;
                    if (j < nq) {
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            int32_t* row = my_cnt + (4 * int64_t(j) + c < tq ? 0 : kCntStride);
                            atomicAdd(&row[min(static_cast<uint32_t>(v[u][c]), uE)], 1);
                        }
                    }
                }
            }
        }
    }
    __syncthreads();
    for (int e = tid; e < E; e += kLayoutSingleThreads) {
        int32_t b = 0, r = 0;
#pragma unroll
        for (int c = 0; c < kCopies; ++c) {
            b += cnt[(2 * c) * kCntStride + e];
            r += cnt[(2 * c + 1) * kCntStride + e];
        }
        before[e] = b;
        rest[e] = r;
    }
    __syncthreads();
    for (int e = tid; e < E; e += kLayoutSingleThreads) {
#pragma unroll
        for (int w = 0; w < kWaves; ++w) wave_hist[w * kMaxExperts + e] = 0;
    }
    // (the barrier after the scan below orders these stores before the rank step)

    // Exclusive scan of the totals over experts, one expert per thread
    // (E <= kMaxExperts == kLayoutSingleThreads).
    const int32_t mine_tot = tid < E ? before[tid] + rest[tid] : 0;
    int32_t incl = mine_tot;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int32_t up = __shfl_up(incl, d, 64);
        if (lane >= d) incl += up;
    }
    if (lane == 63) wave_sum[wave] = incl;
    __syncthreads();
    int32_t run = incl - mine_tot;
    for (int w = 0; w < wave; ++w) run += wave_sum[w];
    if (tid < E) {
        before[tid] += run;          // the tile's first row for expert tid
        if (blockIdx.x == 0) {
            counts[tid] = mine_tot;
            offsets[tid] = run;
        }
    }
    if (blockIdx.x == 0 && tid == kLayoutSingleThreads - 1) offsets[E] = run + mine_tot;

    // Rank this tile's slots (loaded into ex[] above).
#pragma unroll
    for (int j = 0; j < R; ++j) ex[j] = slot_expert_of(ex[j], base + j * 64 + lane, nvalid, E);
    int32_t local[R];
    int32_t* mine = wave_hist + wave * kMaxExperts;
    const uint64_t below = lanes_below();
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const bool valid = ex[j] >= 0;
        const uint64_t peers = peer_mask(ex[j], valid, bits);
        const int32_t prior = valid ? mine[ex[j]] : 0;
        local[j] = prior + __popcll(peers & below);
        if (valid && (peers & below) == 0) mine[ex[j]] = prior + __popcll(peers);
        __builtin_amdgcn_wave_barrier();
    }
    __syncthreads();

    // Per-wavefront counts -> each wavefront's first row per expert.
    for (int e = tid; e < E; e += kLayoutSingleThreads) {
        int32_t r = before[e];
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const int32_t c = wave_hist[w * kMaxExperts + e];
            wave_hist[w * kMaxExperts + e] = r;
            r += c;
        }
    }
    __syncthreads();

#pragma unroll
    for (int j = 0; j < R; ++j) {
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

// Completion counters of the fused count launch, one per context and device:
// zero when the code object loads, and the last workgroup of every launch
// puts its counter back to zero.
__device__ uint32_t g_fused_done[kFusedCounterSlots];

// Count launch of the layout fused into dispatch. Every workgroup histograms
// its tile (as layout_count_kernel) and marks its tile's padding slots as
// routing nowhere. The last workgroup to finish then turns the histograms,
// in place, into each tile's first row per expert: offsets[e] plus the
// count of expert e in all earlier tiles; it also writes counts and
// offsets. Nothing waits: the workgroup that sees the counter reach
// gridDim.x - 1 is the one that continues. Thread (quad q, slice sl) owns
// experts 4q..4q+3 over the contiguous tile range of slice sl, summed with
// 16-byte loads; slice sums go through LDS.
template <int R>
__global__ __launch_bounds__(kLayoutThreads)
void layout_count_scan_kernel(const int32_t* __restrict__ ids, int64_t nvalid, int64_t nslots,
                              int32_t E, int32_t E4, int bits, int32_t tiles, int32_t slot,
                              int32_t* __restrict__ block_hist, int32_t* __restrict__ counts,
                              int32_t* __restrict__ offsets, int32_t* __restrict__ row_map) {
    __shared__ int32_t hist[kMaxExperts];
    __shared__ int32_t part[kMaxExperts];   // slice sums, [S][E4] (S * E4 <= 4 * kLayoutThreads)
    __shared__ int32_t first[kMaxExperts];  // offsets, then slice bases
    __shared__ int32_t wave_sum[kLayoutWaves];
    __shared__ int last;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    constexpr int kTile = kLayoutThreads * R;

    if (static_cast<int32_t>(blockIdx.x) < tiles) {
        for (int e = tid; e < E4; e += kLayoutThreads) hist[e] = 0;
        __syncthreads();
        const int64_t base = int64_t(blockIdx.x) * kTile + wave * (64 * R);
        int32_t ex[R];
#pragma unroll
        for (int j = 0; j < R; ++j) ex[j] = load_slot_id(ids, base + j * 64 + lane, nvalid);
#pragma unroll
        for (int j = 0; j < R; ++j) ex[j] = slot_expert_of(ex[j], base + j * 64 + lane, nvalid, E);
        const uint64_t below = lanes_below();
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const bool valid = ex[j] >= 0;
            const uint64_t peers = peer_mask(ex[j], valid, bits);
            if (valid && (peers & below) == 0) atomicAdd(&hist[ex[j]], __popcll(peers));
        }
        __syncthreads();
        int32_t* out = block_hist + int64_t(blockIdx.x) * E4;
        for (int e = tid; e < E4; e += kLayoutThreads) out[e] = hist[e];
        // Padding slots of this tile (t >= T) route nowhere.
        const int64_t t0 = int64_t(blockIdx.x) * kTile;
        const int64_t t1 = t0 + kTile < nslots ? t0 + kTile : nslots;
        for (int64_t i = (t0 > nvalid ? t0 : nvalid) + tid; i < t1; i += kLayoutThreads)
            row_map[i] = -1;
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) last = atomicAdd(&g_fused_done[slot], 1u) == gridDim.x - 1;
    __syncthreads();
    if (!last) return;
    __threadfence();

    const int quads = E4 / 4;
    int S = kLayoutThreads / quads;
    if (S > kMaxSlices) S = kMaxSlices;
    const int q = tid % quads;
    const int sl = tid / quads;
    const int32_t per = (tiles + S - 1) / S;
    const int32_t b_lo = sl < S ? min(sl * per, tiles) : tiles;
    const int32_t b_hi = min(b_lo + per, tiles);
    v4i* h = reinterpret_cast<v4i*>(block_hist) + q;
    if (sl < S) {
        v4i sum = {0, 0, 0, 0};
#pragma unroll 8
        for (int32_t b = b_lo; b < b_hi; ++b) sum += h[int64_t(b) * quads];
#pragma unroll
        for (int j = 0; j < 4; ++j) part[sl * E4 + 4 * q + j] = sum[j];
    }
    __syncthreads();

    // Totals per expert and their exclusive scan (thread order = expert order).
    const int e0 = tid * kExpertsPerThread;
    int32_t tot[kExpertsPerThread];
    int32_t mine_sum = 0;
#pragma unroll
    for (int j = 0; j < kExpertsPerThread; ++j) {
        tot[j] = 0;
        if (e0 + j < E4)
            for (int k = 0; k < S; ++k) tot[j] += part[k * E4 + e0 + j];
        mine_sum += tot[j];
    }
    int32_t incl = mine_sum;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int32_t up = __shfl_up(incl, d, 64);
        if (lane >= d) incl += up;
    }
    if (lane == 63) wave_sum[wave] = incl;
    __syncthreads();
    int32_t run = incl - mine_sum;
    for (int w = 0; w < wave; ++w) run += wave_sum[w];
#pragma unroll
    for (int j = 0; j < kExpertsPerThread; ++j) {
        const int e = e0 + j;
        if (e < E4) first[e] = run;
        if (e < E) {
            counts[e] = tot[j];
            offsets[e] = run;
        }
        run += tot[j];
    }
    if (tid == kLayoutThreads - 1) offsets[E] = run;
    __syncthreads();

    // Each tile's first row per expert, written over its histogram.
    if (sl < S) {
        v4i r;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            r[j] = first[4 * q + j];
            for (int k = 0; k < sl; ++k) r[j] += part[k * E4 + 4 * q + j];
        }
#pragma unroll 8
        for (int32_t b = b_lo; b < b_hi; ++b) {
            const v4i v = h[int64_t(b) * quads];
            h[int64_t(b) * quads] = r;
            r += v;
        }
    }
    if (tid == 0) atomicExch(&g_fused_done[slot], 0u);
}

template <int R>
hipError_t launch_r(const LayoutArgs& a, hipStream_t stream) {
    const int64_t tiles = layout_tiles(a.nslots, R);
    const int bits = expert_bits(a.E);
    const int32_t E4 = padded_experts(a.E);
    if (tiles > 0) {
        hipLaunchKernelGGL(layout_count_kernel<R>, dim3(static_cast<uint32_t>(tiles)),
                           dim3(kLayoutThreads), 0, stream, a.ids, a.nvalid, a.E, E4, bits,
                           a.block_hist);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    // At least one workgroup, so counts and offsets are written even for an
    // empty capacity.
    const uint32_t grid = static_cast<uint32_t>(tiles > 0 ? tiles : 1);
    hipLaunchKernelGGL(layout_rank_kernel<R>, dim3(grid), dim3(kLayoutThreads), 0, stream, a.ids,
                       a.nvalid, a.nslots, a.E, E4, bits, static_cast<int32_t>(tiles), a.block_hist,
                       a.counts, a.offsets, a.row_map, a.src_map);
    return hipGetLastError();
}

template <int R>
hipError_t launch_count_scan_r(const LayoutArgs& a, int32_t slot, hipStream_t stream) {
    const int64_t tiles = layout_tiles(a.nslots, R);
    // At least one workgroup, so counts and offsets are written even for an
    // empty capacity.
    const uint32_t grid = static_cast<uint32_t>(tiles > 0 ? tiles : 1);
    hipLaunchKernelGGL(layout_count_scan_kernel<R>, dim3(grid), dim3(kLayoutThreads), 0, stream,
                       a.ids, a.nvalid, a.nslots, a.E, padded_experts(a.E), expert_bits(a.E),
                       static_cast<int32_t>(tiles), slot, a.block_hist, a.counts, a.offsets,
                       a.row_map);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_layout_count_scan(const LayoutArgs& a, int32_t counter_slot, int32_t* tile_slots,
                                    hipStream_t stream) {
    if (counter_slot < 0 || counter_slot >= kFusedCounterSlots) return hipErrorInvalidValue;
    const int R = layout_slots_per_lane(a.nslots);
    *tile_slots = kLayoutThreads * R;
    return R == kLayoutMinSlotsPerLane
               ? launch_count_scan_r<kLayoutMinSlotsPerLane>(a, counter_slot, stream)
               : launch_count_scan_r<kLayoutMaxSlotsPerLane>(a, counter_slot, stream);
}

template <int R>
hipError_t launch_single_r(const LayoutArgs& a, hipStream_t stream) {
    const int64_t tile = int64_t(kLayoutSingleThreads) * R;
    const int64_t tiles = (a.nslots + tile - 1) / tile;
    // At least one workgroup, so counts and offsets are written even for an
    // empty capacity.
    const uint32_t grid = static_cast<uint32_t>(tiles > 0 ? tiles : 1);
    hipLaunchKernelGGL(layout_single_kernel<R>, dim3(grid), dim3(kLayoutSingleThreads), 0, stream,
                       a.ids, a.nvalid, a.nslots, a.E, expert_bits(a.E), a.counts, a.offsets,
                       a.row_map, a.src_map);
    return hipGetLastError();
}

hipError_t launch_layout(const LayoutArgs& a, hipStream_t stream) {
    if (layout_single_launch(a.nslots, a.launches)) {
        switch (layout_single_slots_per_lane(a.nslots)) {
            case 1: return launch_single_r<1>(a, stream);
            case 2: return launch_single_r<2>(a, stream);
            default: return launch_single_r<4>(a, stream);
        }
    }
    return layout_slots_per_lane(a.nslots) == kLayoutMinSlotsPerLane
               ? launch_r<kLayoutMinSlotsPerLane>(a, stream)
               : launch_r<kLayoutMaxSlotsPerLane>(a, stream);
}

}  // namespace moe
