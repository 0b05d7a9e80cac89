// Expert step between dispatch and combine on gfx950: a grouped GEMM over the
// expert-major rows, driven by the per-expert offsets in device memory.
//
// What is computed (the uccl page, "Tests": layout, dispatch, expert and
// combine run as one captured graph; "Internode" item 2: the expert step
// reads its per-expert row counts from the device, never from the host): for
// every expert e and row r in [offsets[e], offsets[e+1]),
//     out[r][n] = sum over d of x_e[r][d] * w[e][n][d]
// with bf16 inputs, fp32 accumulation on the matrix cores and one rounding of
// the sum to bf16 (nearest even). Rows outside every segment are not written.
//
// Work split. A tile is (expert, F output features, up to BT rows of the
// expert's segment), F = 32 per 32-feature block of each wavefront. Within an
// expert, tiles go in
// blocks of up to 8 row tiles: all feature tiles of a block, each with the
// block's row tiles fastest. Workgroups are dealt to the 8 XCDs round-robin,
// so tile numbers are handed out in chunks of kGemmXcdChunk (32) consecutive
// tiles, XCD x taking every eighth chunk; the workgroups an XCD runs at once
// then cover a few row tiles x feature tiles of one expert,
// which share each weight tile and each row tile through that XCD's L2 (with
// a plain feature-major order a large expert re-fetches its rows once per
// feature tile). The grid covers the most tiles any routing can need,
// ceil(max_rows / BT) + E row tiles per feature tile (rounded up to whole
// chunks per XCD); wavefront 0 of each workgroup finds its tile from the
// offsets (a scan of the per-expert tile counts over the 64 lanes) and
// workgroups without a tile exit.
//
// Inside a tile, wavefront w owns FB blocks of 32 features, [32 FB w,
// 32 FB (w + 1)), and all BT rows: v_mfma_f32_32x32x16_bf16 with the weight
// rows as the A operand and the token rows as B. Within a step of 64 k, lane half h supplies k = 32h + 8s +
// j (s the instruction, j the element) for both operands: any pairing of k
// slots gives the same sum. An MFMA fragment puts consecutive lanes on
// different rows, and loads in that layout run at about a third of the rate
// of loads where every 4 consecutive lanes read one contiguous 64-byte piece
// (measured on MI355X from L2-resident data), so:
//   - token rows, which every wavefront reads, are loaded coalesced (8 lanes
//     per 128-byte step of a row) into a shared LDS buffer (double
//     buffered, one barrier per step) and read back as fragments;
//   - weights in the row-major layout [E][N][k_in] are loaded the same way
//     into a per-wavefront LDS slot (4 wavefronts, 128 features per tile);
//   - weights in the tiled layout (moe_tile_expert_weights: each 64-lane A
//     fragment stored as one contiguous KiB) are loaded straight into the
//     fragment registers: 8 wavefronts of two feature blocks (512 features
//     per tile) share each row tile, so the rows are re-read 4x less often,
//     and each row fragment read from LDS feeds both blocks' products.
//     Measured on MI355X (256 experts, 7168 -> 4096, interleaved on one box
//     through the C ABI, bitwise-equal outputs): 13.98-14.13 against
//     14.60-14.75 ms at 32768 tokens (uniform routing), 13.93-13.97 against
//     14.32-14.38 ms (Zipf), 3.41-3.42 against 3.45 ms at 4096 tokens,
//     compared with 16 wavefronts of one block; the two-block wavefront needs
//     up to 256 VGPRs, so a SIMD holds 2 of them instead of 4.
// 16-byte chunks sit in LDS at a position XOR-swizzled by the row index, so
// fragment reads are free of bank conflicts. Loads run kStages steps ahead
// in a register ring, weights and rows of a step issued together; the loop
// body has no branch (a branch there makes the compiler's wait counts
// conservative, which drains the pipeline every group).
#include "moe_kernels.h"
#include "moe_lanes.h"

#include <type_traits>

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kStages = 2;          // steps of loads in flight (more costs occupancy)
constexpr int kStepChunks = 8;      // 64 bf16 of k per step = 8 chunks of 16 bytes
constexpr int kXcds = 8;            // MI355X: 8 XCDs, each with its own L2

__device__ __forceinline__ bf16x8 as_bf16x8(v4i v) { return __builtin_bit_cast(bf16x8, v); }

// LDS position of 16-byte chunk c of row r within the row's 128 bytes is
// c ^ swz(r): any 16 consecutive rows at one chunk index land in 16 distinct
// 16-byte bank groups (and any 8 in 8), so the fragment reads, one chunk
// index per 32 rows, are free of bank conflicts.
__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

// Rows [s0, s1) of expert e, clamped into [0, max_rows).
__device__ __forceinline__ void segment(const int32_t* offsets, int32_t e, int32_t max_rows,
                                        int32_t& s0, int32_t& s1) {
    int32_t a = offsets[e], b = offsets[e + 1];
    a = a < 0 ? 0 : (a > max_rows ? max_rows : a);
    b = b < a ? a : (b > max_rows ? max_rows : b);
    s0 = a;
    s1 = b;
}

template <int BT, int WAVES, int FB, bool TILED>
__global__ __launch_bounds__(WAVES * 64)
void grouped_gemm_kernel(const v4i* __restrict__ x_e, const v4i* __restrict__ w,
                         const int32_t* __restrict__ offsets, int32_t E, int32_t max_rows,
                         int32_t chunks, int32_t N, int32_t ftiles,
                         uint8_t* __restrict__ out) {
    constexpr int kThreads = WAVES * 64;
    constexpr int kFeatures = WAVES * 32 * FB;
    constexpr int U = BT / 32;                                        // 32-row sub-tiles
    static_assert(U == 2 || U == 4, "row tile of 64 or 128");
    static_assert(TILED || FB == 1, "row-major weights: one block per wavefront");
    constexpr int UX = (BT * kStepChunks + kThreads - 1) / kThreads;  // row chunks per thread
    // Row buffer plus one dummy chunk per lane for threads past the tile.
    __shared__ v4i xs[2][BT * kStepChunks + 64];
    __shared__ v4i ws[TILED ? 1 : WAVES][32 * kStepChunks];          // row-major weight slots
    __shared__ int32_t info[4];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    if (wave == 0) {
        const int per = (E + 63) / 64;
        const int e_lo = min(E, lane * per);
        const int e_hi = min(E, e_lo + per);
        int64_t local = 0;
        for (int e = e_lo; e < e_hi; ++e) {
            int32_t s0, s1;
            segment(offsets, e, max_rows, s0, s1);
            local += int64_t((s1 - s0 + BT - 1) / BT) * ftiles;
        }
        int64_t incl = local;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int64_t v = __shfl_up(incl, d, 64);
            if (lane >= d) incl += v;
        }
        const int64_t total = __shfl(incl, 63, 64);
        // Workgroup b runs on XCD b % kXcds (round-robin dispatch). XCD x
        // takes chunks x, x + 8, x + 16, ... of kGemmXcdChunk tiles each (the
        // grid holds whole chunks per XCD, so every tile number is dealt).
        const int64_t idx = blockIdx.x / kXcds;
        const int64_t x = blockIdx.x % kXcds;
        const int64_t u =
            ((idx / kGemmXcdChunk) * kXcds + x) * kGemmXcdChunk + idx % kGemmXcdChunk;
        if (lane == 0 && u >= total) info[0] = -1;
        int64_t base = incl - local;
        if (u >= base && u < incl) {
            for (int e = e_lo; e < e_hi; ++e) {
                int32_t s0, s1;
                segment(offsets, e, max_rows, s0, s1);
                const int32_t mt = (s1 - s0 + BT - 1) / BT;
                const int64_t n = int64_t(mt) * ftiles;
                if (u < base + n) {
                    // Within the expert: blocks of up to 8 row tiles; in a
                    // block, feature tiles, then its row tiles.
                    const int32_t rem = static_cast<int32_t>(u - base);
                    const int32_t mb = rem / (ftiles * 8);
                    const int32_t in = rem - mb * ftiles * 8;
                    const int32_t mbe = min(8, mt - mb * 8);
                    const int32_t r0 = s0 + (mb * 8 + in % mbe) * BT;
                    info[0] = e;
                    info[1] = (in / mbe) * kFeatures;
                    info[2] = r0;
                    info[3] = min(BT, s1 - r0);
                    break;
                }
                base += n;
            }
        }
    }
    __syncthreads();
    const int32_t e = info[0];
    if (e < 0) return;
    const int32_t f0 = info[1];
    const int32_t row0 = info[2];
    const int32_t nrows = info[3];

    const int h = lane >> 5;
    const int i = lane & 31;
    const int32_t steps_all = (chunks + kStepChunks - 1) / kStepChunks;

    // Weights. Tiled: [E][ceil(N/32)][steps][4][64 lanes] chunks, this
    // wavefront's FB 32-feature blocks (clamped into range; the extra features
    // are never stored). Row-major: lane l loads rows (l >> 3) + 8j, chunk
    // l & 7 of the wavefront's 32 rows (features past N read row N-1).
    const v4i* wt[FB] = {};
    const v4i* wrow[4];
    int32_t wslot[4];
    v4i* wbuf = ws[TILED ? 0 : wave];
    if constexpr (TILED) {
        const int32_t nb = (N + 31) / 32;
#pragma unroll
        for (int b = 0; b < FB; ++b) {
            const int32_t blk = min(f0 / 32 + wave * FB + b, nb - 1);
            wt[b] = w + ((int64_t(e) * nb + blk) * steps_all) * 4 * 64 + lane;
        }
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = (lane >> 3) + 8 * j;
            const int c = lane & 7;
            wrow[j] = w + (int64_t(e) * N + min(f0 + wave * 32 + r, N - 1)) * chunks + c;
            wslot[j] = r * kStepChunks + (c ^ swz(r));
        }
    }
    // Token rows: thread chunk q = tid + kThreads*j of the BT x 8 step tile
    // (rows past the segment read its last row and are never stored; threads
    // past the tile load a real row too and write the dummy slot).
    const v4i* xrow[UX];
    int32_t xc[UX];
    int32_t xslot[UX];
#pragma unroll
    for (int j = 0; j < UX; ++j) {
        const int q = tid + kThreads * j;
        const int r = min(q >> 3, BT - 1);
        const int c = q & 7;
        xrow[j] = x_e + int64_t(row0 + min(r, nrows - 1)) * chunks + c;
        xc[j] = c;
        xslot[j] = q < BT * kStepChunks ? r * kStepChunks + (c ^ swz(r))
                                        : BT * kStepChunks + lane;
    }
    // The tile's 32-row sub-tiles that hold rows of the segment (1..U): the
    // loop is instantiated for each count and chosen once per workgroup, so
    // short segments issue no matrix-core work for absent rows and the loop
    // body stays branch-free.
    auto run = [&](auto sub) {
        constexpr int UU = decltype(sub)::value;
        f32x16 acc[FB][UU];
#pragma unroll
        for (int b = 0; b < FB; ++b)
#pragma unroll
            for (int u = 0; u < UU; ++u)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[b][u][r] = 0.0f;

        // One step: rows (and row-major weights) of the step, already in
        // registers, to LDS; then the 4 x UU x FB matrix-core products.
        auto mma_step = [&](int buf_id, const v4i (&wv)[FB][4], const v4i (&xv)[UX], auto&& after_barrier) {
            v4i* buf = xs[buf_id];
#pragma unroll
            for (int j = 0; j < UX; ++j) buf[xslot[j]] = xv[j];
            if constexpr (!TILED) {
#pragma unroll
                for (int j = 0; j < 4; ++j) wbuf[wslot[j]] = wv[0][j];
            }
            __syncthreads();
            after_barrier();
            // Row fragments are read one product ahead: product (s, u) runs
            // while the LDS read for the next one is in flight. Without this
            // the compiler, short of registers, reuses one register quad for
            // every fragment and waits for each read just before its product.
            auto bread = [&](int s, int u) {
                const int r = u * 32 + i;
                return as_bf16x8(buf[r * kStepChunks + ((4 * h + s) ^ swz(r))]);
            };
            bf16x8 bcur = bread(0, 0);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                bf16x8 a[FB];
#pragma unroll
                for (int b = 0; b < FB; ++b) {
                    if constexpr (TILED)
                        a[b] = as_bf16x8(wv[b][s]);
                    else
                        a[b] = as_bf16x8(wbuf[i * kStepChunks + ((4 * h + s) ^ swz(i))]);
                }
#pragma unroll
                for (int u = 0; u < UU; ++u) {
                    const int nu = u + 1 < UU ? u + 1 : 0;
                    const int ns = u + 1 < UU ? s : s + 1;
                    bf16x8 bnext = bcur;
                    if (ns < 4) bnext = bread(ns, nu);
#pragma unroll
                    for (int b = 0; b < FB; ++b)
                        acc[b][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[b], bcur, acc[b][u], 0, 0, 0);
                    bcur = bnext;
                }
            }
            if constexpr (TILED) {
                // Scheduling groups that keep that order: two LDS reads
                // before the first products, then one read per FB products
                // (mask 0x100: LDS reads, 0x008: matrix-core instructions).
                // With tiled weights the step's only LDS reads are the 4 * UU
                // row fragments. Measured on MI355X at 32768 tokens x 7168 ->
                // 4096 (one block per wavefront): 13.9 against 14.2-14.4 ms,
                // results bitwise equal.
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
                for (int q = 0; q < 4 * UU - 2; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x008, FB, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 2 * FB, 0);
            }
        };

        const int32_t full = chunks / kStepChunks;
        v4i wr[kStages][FB][4];
        v4i xr[kStages][UX];
        auto load_w = [&](int32_t step, v4i (&dst)[FB][4]) {
#pragma unroll
            for (int b = 0; b < FB; ++b)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if constexpr (TILED)
                        dst[b][j] = wt[b][(step * 4 + j) * 64];
                    else
                        dst[b][j] = wrow[j][step * kStepChunks];
                }
        };
        auto load_x = [&](int32_t step, v4i (&dst)[UX]) {
#pragma unroll
            for (int j = 0; j < UX; ++j) dst[j] = xrow[j][step * kStepChunks];
        };
        // The loop body runs whole groups of kStages steps with no branch in it;
        // the 0..kStages-1 steps left over run after it from the loaded ring.
        int32_t done = 0;
        if (full > 0) {
#pragma unroll
            for (int p = 0; p < kStages; ++p) {
                load_x(min(p, full - 1), xr[p]);
                load_w(min(p, full - 1), wr[p]);
            }
            int32_t s0 = 0;
            for (; s0 + kStages <= full; s0 += kStages) {
#pragma unroll
                for (int p = 0; p < kStages; ++p) {
                    const int32_t ahead = min(s0 + p + kStages, full - 1);
                    mma_step((s0 + p) & 1, wr[p], xr[p], [&] { load_x(ahead, xr[p]); });
                    load_w(ahead, wr[p]);
                }
            }
#pragma unroll
            for (int p = 0; p < kStages - 1; ++p)
                if (s0 + p < full) mma_step((s0 + p) & 1, wr[p], xr[p], [] {});
            done = full;
        }
        // The last, partial step (k_in not a multiple of 64): row chunks past
        // the row read as zero; row-major weight chunks too, tiled weights are
        // zero there already.
        if (done * kStepChunks < chunks) {
            const int32_t c0 = done * kStepChunks;
            const int32_t last = chunks - 1;
            const v4i zero = {0, 0, 0, 0};
            v4i wv[FB][4], xv[UX];
#pragma unroll
            for (int b = 0; b < FB; ++b)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if constexpr (TILED) {
                        wv[b][j] = wt[b][(done * 4 + j) * 64];
                    } else {
                        const int32_t c = c0 + (lane & 7);
                        const v4i v = wrow[j][min(c, last) - (lane & 7)];
                        wv[b][j] = c <= last ? v : zero;
                    }
                }
#pragma unroll
            for (int j = 0; j < UX; ++j) {
                const int32_t c = c0 + xc[j];
                const v4i v = xrow[j][min(c, last) - xc[j]];
                xv[j] = c <= last ? v : zero;
            }
            mma_step(done & 1, wv, xv, [] {});
        }

        // acc[b][u][4q + t] is out[row u*32 + i][feature 32(FB w + b) + 8q +
        // 4h + t].
#pragma unroll
        for (int b = 0; b < FB; ++b)
#pragma unroll
            for (int u = 0; u < UU; ++u) {
                const int r = u * 32 + i;
                if (r >= nrows) continue;
                uint8_t* orow = out + (int64_t(row0 + r) * N) * 2;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int32_t col = f0 + (wave * FB + b) * 32 + 8 * q + 4 * h;
                    if (col >= N) continue;
                    const f32x16& c = acc[b][u];
                    uint2 v;
                    v.x = f32_to_bf16_bits(c[4 * q]) | (f32_to_bf16_bits(c[4 * q + 1]) << 16);
                    v.y = f32_to_bf16_bits(c[4 * q + 2]) | (f32_to_bf16_bits(c[4 * q + 3]) << 16);
                    *reinterpret_cast<uint2*>(orow + int64_t(col) * 2) = v;
                }
            }
    };
    const int usub = (nrows + 31) / 32;
    if (usub <= 1)
        run(std::integral_constant<int, 1>{});
    else if constexpr (U == 2)
        run(std::integral_constant<int, 2>{});
    else if (usub == 2)
        run(std::integral_constant<int, 2>{});
    else if (usub == 3)
        run(std::integral_constant<int, 3>{});
    else
        run(std::integral_constant<int, U>{});
}

// Tiled weight layout: chunk ((((e * NB + b) * S + t) * 4 + s) * 64 + l) holds
// w[e][32b + (l & 31)][64t + 32(l >> 5) + 8s .. + 8] -- the A fragment of
// lane l for instruction s of step t of feature block b -- or zeros where
// the feature or the k index is past the matrix (NB = ceil(N/32), S =
// ceil(k_in/64)). One thread per 16-byte output chunk.
__global__ __launch_bounds__(256)
void tile_weights_kernel(const v4i* __restrict__ src, int32_t N, int32_t chunks, int32_t NB,
                         int32_t S, int64_t total, v4i* __restrict__ dst) {
    const int64_t q = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (q >= total) return;
    const int l = static_cast<int>(q & 63);
    const int s = static_cast<int>((q >> 6) & 3);
    const int64_t rest = q >> 8;
    const int32_t t = static_cast<int32_t>(rest % S);
    const int64_t eb = rest / S;
    const int32_t b = static_cast<int32_t>(eb % NB);
    const int64_t e = eb / NB;
    const int32_t row = 32 * b + (l & 31);
    const int32_t c = 8 * t + 4 * (l >> 5) + s;
    v4i v = {0, 0, 0, 0};
    if (row < N && c < chunks) v = src[(e * N + row) * chunks + c];
    dst[q] = v;
}

template <int BT, int WAVES, int FB, bool TILED>
hipError_t launch_bt(const GroupedGemmArgs& a, hipStream_t stream) {
    constexpr int32_t kFeatures = WAVES * 32 * FB;
    static_assert(kFeatures == gemm_tile_features(TILED), "tile width as the host sizes it");
    const int64_t grid = grouped_gemm_grid(a.max_rows, a.E, a.N, BT, kFeatures);
    hipLaunchKernelGGL((grouped_gemm_kernel<BT, WAVES, FB, TILED>), dim3(static_cast<uint32_t>(grid)),
                       dim3(WAVES * 64), 0, stream, static_cast<const v4i*>(a.x_e),
                       static_cast<const v4i*>(a.w), a.offsets, a.E,
                       static_cast<int32_t>(a.max_rows), a.Kd / 8, a.N,
                       static_cast<int32_t>((a.N + kFeatures - 1) / kFeatures),
                       static_cast<uint8_t*>(a.out));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_grouped_gemm(const GroupedGemmArgs& a, hipStream_t stream) {
    if (a.max_rows <= 0) return hipSuccess;
    if (a.tiled) {
        switch (a.row_tile) {
            case 64: return launch_bt<64, kGemmWavesTiled, kGemmBlocksTiled, true>(a, stream);
            case 128: return launch_bt<128, kGemmWavesTiled, kGemmBlocksTiled, true>(a, stream);
            default: return hipErrorInvalidValue;
        }
    }
    switch (a.row_tile) {
        case 64: return launch_bt<64, kGemmWavesRowMajor, 1, false>(a, stream);
        case 128: return launch_bt<128, kGemmWavesRowMajor, 1, false>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_tile_weights(const TileWeightsArgs& a, hipStream_t stream) {
    const int64_t NB = (int64_t(a.N) + 31) / 32;
    const int64_t S = (int64_t(a.Kd) + 63) / 64;
    const int64_t total = int64_t(a.E) * NB * S * 256;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(tile_weights_kernel, dim3(static_cast<uint32_t>((total + 255) / 256)),
                       dim3(256), 0, stream, static_cast<const v4i*>(a.src), a.N, a.Kd / 8,
                       static_cast<int32_t>(NB), static_cast<int32_t>(S), total,
                       static_cast<v4i*>(a.dst));
    return hipGetLastError();
}

}  // namespace moe
