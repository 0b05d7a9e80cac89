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

// The copy of one wavefront's item: its K rows from the staged row map, the
// row chunk(s) stored K times, and (first segment) the slots' scores. BURST
// (single-chunk shape only): the K stores issue back to back.
// A chunk of a token row of x: ordinary load, or streaming (NTX) so that x,
// read exactly once, does not take cache space from the expert rows written
// next to it. A template parameter: with a runtime flag the compiler merges
// the two loads of one address into a single ordinary load.
template <bool NTX>
__device__ __forceinline__ v4i load_x(const v4i* p) {
    if constexpr (NTX)
        return __builtin_nontemporal_load(p);
    else
        return *p;
}

template <int K, bool NT, bool SINGLE, int MODE, bool BURST, bool NTX>
__device__ __forceinline__ void copy_rows(const float* __restrict__ scores,
                                          int32_t chunks, v4i* __restrict__ x_e,
                                          float* __restrict__ s_e, const int32_t* tile_rows,
                                          const float* tile_scores, int64_t t, int64_t t_first,
                                          int seg, int32_t c_begin, int32_t c_end,
                                          const v4i* src, v4i early, float early_score,
                                          int lane) {
    constexpr int U = kDispatchUnroll;
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

    // Lane k < K of the first segment also moves slot k's score (after the
    // row stores, which it would otherwise hold up). In the single-chunk
    // shape the score was loaded with the row chunk, at kernel entry.
    auto move_score = [&]() {
        if (seg == 0 && lane < K) {
            const int32_t r = rows[lane];
            if (r >= 0) s_e[r] = SINGLE ? early_score : scores[t * K + lane];
        }
    };

    // Each slot's store sits behind its own "has an expert" branch, and the
    // compiler waits for all outstanding memory operations before each one
    // (stores count in the same counter as loads), so a wavefront's K stores
    // go out one after another. BURST waits for the loaded chunk once: the
    // empty asm statement below redefines the chunk's registers after an
    // explicit wait, so the compiler sees them ready and issues the K stores
    // back to back. Measured on MI355X, pacing is the faster default: dispatch
    // 79.0 vs 80.8 us at the DSV3 shape, 788 vs 809 us at the 32k-token
    // shape, 21.7 vs 20.4-21.4 us at 2048 tokens of 4 KiB with the step no
    // faster; back to back wins only at 8192 tokens of 8 KiB (95.0 vs
    // 96.7 us).
    if constexpr (SINGLE) {
        const int32_t c = c_begin + lane;
        if (c < c_end) {
            if constexpr (BURST) asm volatile("s_waitcnt vmcnt(0)" : "+v"(early));
#pragma unroll
            for (int k = 0; k < K; ++k)
                if (row[k] >= 0)
                    put<NT>(x_e + int64_t(row[k]) * chunks + c, transform<MODE>(s[k], early));
        }
        move_score();
    } else {
        int32_t c0 = c_begin;
        // Whole groups: every lane has U chunks in range.
        for (; c0 + 64 * U <= c_end; c0 += 64 * U) {
            v4i v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) v[u] = load_x<NTX>(src + c0 + u * 64 + lane);
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
            const v4i v = load_x<NTX>(src + c);
#pragma unroll
            for (int k = 0; k < K; ++k)
                if (row[k] >= 0) put<NT>(x_e + int64_t(row[k]) * chunks + c, transform<MODE>(s[k], v));
        }
        move_score();
    }
}

// Rows of the layout fused into dispatch (RANK): where slot i's row comes
// from. first_rows[tile][e] is the first row of expert e in the slot tile
// (offsets[e] plus the expert's count in all earlier tiles); the slot's row
// adds the number of earlier slots of its tile with the same expert.
struct RankArgs {
    const int32_t* ids;         // [T][K]
    int32_t E;
    int32_t E4;                 // row stride of first_rows
    int32_t tile_slots;
    const int32_t* first_rows;  // [tiles][E4]
    int32_t* row_map;           // written: [T][K]
    int32_t* src_map;           // written: [total]
};

// One wavefront per (token, row segment). SINGLE: the segment is exactly one
// 16-byte chunk per lane (the default launch shape); otherwise the segment is
// copied in groups of U chunks per lane, then one chunk at a time. RANK: the
// workgroup computes its tokens' rows (and writes them to row_map and
// src_map) instead of reading row_map.
template <int K, bool NT, bool SINGLE, int MODE, bool RANK, bool BURST, bool NTX>
__global__ __launch_bounds__(kMaxBlockThreads)
void dispatch_kernel(const v4i* __restrict__ x, const float* __restrict__ scores,
                     const int32_t* __restrict__ row_map, int32_t T, int32_t chunks,
                     int32_t segments, int32_t seg_chunks, int64_t max_rows,
                     v4i* __restrict__ x_e, float* __restrict__ s_e, RankArgs rk) {
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

    // This wavefront's item. In the single-chunk shape its chunk of the token
    // row does not depend on the rows, so it is loaded before the staging and
    // arrives while the rows are found.
    const int64_t item = item0 + wave;
    const int64_t t = item / segments;
    const bool live = t < T;
    const int seg = static_cast<int>(item - t * segments);
    const int32_t c_begin = seg * seg_chunks;
    const int32_t c_end = min(c_begin + seg_chunks, chunks);
    const v4i* src = x + t * chunks;
    v4i early = {0, 0, 0, 0};
    float early_score = 0.0f;
    if constexpr (SINGLE) {
        const int32_t c = c_begin + lane;
        if (live && c < c_end) early = load_x<NTX>(src + c);
        if (live && seg == 0 && lane < K) early_score = scores[t * K + lane];
    }
    // RANK: the row this thread records in row_map / src_map after the copy
    // (stores issued here would hold up the copy's first wait).
    int64_t rec_slot = -1;
    int32_t rec_row = -1;

    if constexpr (RANK) {
        // Slot s_first + j of the workgroup: its expert, then the count of
        // earlier slots of its tile with that expert (a ballot per 64 slots
        // of the range from the first staged slot's tile start to the last
        // staged slot), then its row.
        __shared__ int32_t slot_e[kMaxBlockWaves * K];
        __shared__ int32_t slot_cnt[kMaxBlockWaves * K];
        const int64_t s_first = t_first * K;
        const int64_t lo = s_first / rk.tile_slots * rk.tile_slots;
        const int64_t hi = s_first + staged - 1;
        // The first chunk of the scan range of this wavefront, loaded up front.
        const int64_t i_first = lo + int64_t(wave) * 64 + lane;
        const int32_t id_first = i_first < hi ? rk.ids[i_first] : -1;
        int32_t slot_first_row = 0;
        if (tid < staged) {
            const int64_t sj = s_first + tid;
            int32_t e = rk.ids[sj];
            e = static_cast<uint32_t>(e) < static_cast<uint32_t>(rk.E) ? e : -1;
            if (e >= 0) slot_first_row = rk.first_rows[sj / rk.tile_slots * rk.E4 + e];
            slot_e[tid] = e;
            slot_cnt[tid] = 0;
        }
        __syncthreads();
        for (int64_t c0 = lo + int64_t(wave) * 64; c0 < hi; c0 += int64_t(block_waves) * 64) {
            const int64_t i = c0 + lane;
            const int32_t id = c0 == lo + int64_t(wave) * 64 ? id_first : (i < hi ? rk.ids[i] : -1);
            for (int j = 0; j < staged; ++j) {
                const int32_t ej = slot_e[j];
                if (ej < 0) continue;
                const int64_t sj = s_first + j;
                const bool m = id == ej && i < sj && i >= sj / rk.tile_slots * rk.tile_slots;
                const uint64_t b = __ballot(m);
                if (lane == 0 && b != 0) atomicAdd(&slot_cnt[j], __popcll(b));
            }
        }
        __syncthreads();
        if (tid < staged) {
            const int64_t sj = s_first + tid;
            const int32_t e = slot_e[tid];
            const int32_t r = e >= 0 ? slot_first_row + slot_cnt[tid] : -1;
            const bool ok = r >= 0 && r < max_rows;
            tile_rows[tid] = ok ? r : -1;
            if constexpr (MODE != kCopy) tile_scores[tid] = ok ? scores[sj] : 0.0f;
            // The workgroup holding the token's first segment records its rows.
            if ((t_first + tid / K) * segments >= item0) {
                rec_slot = sj;
                rec_row = ok ? r : -1;
            }
        }
    } else if (tid < staged) {
        const int32_t r = row_map[t_first * K + tid];
        const bool ok = r >= 0 && r < max_rows;
        tile_rows[tid] = ok ? r : -1;
        if constexpr (MODE != kCopy) tile_scores[tid] = ok ? scores[t_first * K + tid] : 0.0f;
    }
    __syncthreads();

    if (live)
        copy_rows<K, NT, SINGLE, MODE, BURST, NTX>(scores, chunks, x_e, s_e, tile_rows, tile_scores, t,
                                              t_first, seg, c_begin, c_end, src, early,
                                              early_score, lane);
    if constexpr (RANK) {
        if (rec_slot >= 0) {
            rk.row_map[rec_slot] = rec_row;
            if (rec_row >= 0) rk.src_map[rec_row] = static_cast<int32_t>(rec_slot);
        }
    }
}


template <int K, bool RANK, bool BURST>
hipError_t launch_kb(const DispatchArgs& a, const RankArgs& rk, int32_t segments,
                     int32_t seg_chunks, hipStream_t stream) {
    const int64_t items = int64_t(a.T) * segments;
    const int64_t blocks = (items + a.block_waves - 1) / a.block_waves;
    const bool single = seg_chunks == 64;
    decltype(&dispatch_kernel<K, false, true, kCopy, RANK, BURST, false>) kernel;
    // BURST only changes the single-chunk copy; the multi-chunk copy has one
    // instantiation (BURST = false). Streaming loads of x (NTX) are offered
    // with the bit copy and ordinary stores.
    if (a.scaled) {  // streaming stores are not offered with the scores applied
        kernel = a.bf16 ? (single ? dispatch_kernel<K, false, true, kScaleBF16, RANK, BURST, false>
                                  : dispatch_kernel<K, false, false, kScaleBF16, RANK, false, false>)
                        : (single ? dispatch_kernel<K, false, true, kScaleF32, RANK, BURST, false>
                                  : dispatch_kernel<K, false, false, kScaleF32, RANK, false, false>);
    } else if (a.nontemporal) {
        kernel = single ? dispatch_kernel<K, true, true, kCopy, RANK, BURST, false>
                        : dispatch_kernel<K, true, false, kCopy, RANK, false, false>;
    } else if (a.load_nontemporal) {
        kernel = single ? dispatch_kernel<K, false, true, kCopy, RANK, BURST, true>
                        : dispatch_kernel<K, false, false, kCopy, RANK, false, true>;
    } else {
        kernel = single ? dispatch_kernel<K, false, true, kCopy, RANK, BURST, false>
                        : dispatch_kernel<K, false, false, kCopy, RANK, false, false>;
    }
    hipLaunchKernelGGL(kernel, dim3(static_cast<uint32_t>(blocks)), dim3(64 * a.block_waves), 0,
                       stream, static_cast<const v4i*>(a.x), a.scores, a.row_map, a.T,
                       a.chunks, segments, seg_chunks, a.max_rows, static_cast<v4i*>(a.x_e),
                       a.s_e, rk);
    return hipGetLastError();
}

template <int K, bool RANK>
hipError_t launch_k(const DispatchArgs& a, const RankArgs& rk, int32_t segments,
                    int32_t seg_chunks, hipStream_t stream) {
    const bool burst = seg_chunks == 64 && a.store_burst;
    return burst ? launch_kb<K, RANK, true>(a, rk, segments, seg_chunks, stream)
                 : launch_kb<K, RANK, false>(a, rk, segments, seg_chunks, stream);
}

template <bool RANK>
hipError_t launch_any(const DispatchArgs& a, const RankArgs& rk, hipStream_t stream) {
    if (a.T <= 0) return hipSuccess;
    const int32_t seg_chunks = segment_chunks(a.chunks, a.segments);
    const int32_t segments = (a.chunks + seg_chunks - 1) / seg_chunks;
    switch (a.K) {
#define MOE_DISPATCH_CASE(k) \
    case k: return launch_k<k, RANK>(a, rk, segments, seg_chunks, stream);
        MOE_DISPATCH_CASE(1) MOE_DISPATCH_CASE(2) MOE_DISPATCH_CASE(3) MOE_DISPATCH_CASE(4)
        MOE_DISPATCH_CASE(5) MOE_DISPATCH_CASE(6) MOE_DISPATCH_CASE(7) MOE_DISPATCH_CASE(8)
        MOE_DISPATCH_CASE(9) MOE_DISPATCH_CASE(10) MOE_DISPATCH_CASE(11) MOE_DISPATCH_CASE(12)
        MOE_DISPATCH_CASE(13) MOE_DISPATCH_CASE(14) MOE_DISPATCH_CASE(15) MOE_DISPATCH_CASE(16)
#undef MOE_DISPATCH_CASE
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t stream) {
    return launch_any<false>(a, RankArgs{}, stream);
}

hipError_t launch_layout_dispatch(const FusedLayoutDispatchArgs& a, hipStream_t stream) {
    int32_t tile_slots = 0;
    hipError_t err = launch_layout_count_scan(a.layout, a.counter_slot, &tile_slots, stream);
    if (err != hipSuccess) return err;
    RankArgs rk;
    rk.ids = a.ids;
    rk.E = a.layout.E;
    rk.E4 = padded_experts(a.layout.E);
    rk.tile_slots = tile_slots;
    rk.first_rows = a.layout.block_hist;
    rk.row_map = a.layout.row_map;
    rk.src_map = a.layout.src_map;
    return launch_any<true>(a.dispatch, rk, stream);
}

}  // namespace moe
