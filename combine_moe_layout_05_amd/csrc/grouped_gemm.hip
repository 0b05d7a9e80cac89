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
// Work split. A tile is (expert, 128 output features, up to BT rows of the
// expert's segment). Within an expert, tiles go in blocks of up to 8 row
// tiles: all feature tiles of a block, each with the block's row tiles
// fastest. Workgroups are dealt to the 8 XCDs round-robin, so each XCD is
// given a contiguous run of tile numbers; the ~64 workgroups an XCD runs at
// once then cover about 8 row tiles x 8 feature tiles of one expert, which
// share each weight tile and each row tile through that XCD's L2 (with a
// plain feature-major order a large expert re-fetches its rows once per
// feature tile). The grid covers the most tiles any routing can need,
// ceil(max_rows / BT) + E row tiles per feature tile (rounded up to a
// multiple of 8); wavefront 0 of each workgroup finds its tile from the
// offsets (a scan of the per-expert tile counts over the 64 lanes) and
// workgroups without a tile exit.
//
// Inside a tile, wavefront w owns features [32w, 32w + 32) and all BT rows:
// v_mfma_f32_32x32x16_bf16 with the weight rows as the A operand and the
// token rows as B. An MFMA fragment puts consecutive lanes on different rows,
// and loads in that layout run at about a third of the rate of loads where
// every 4 consecutive lanes read one contiguous 64-byte piece (measured on
// MI355X from L2-resident data). So both operands are loaded coalesced (8
// lanes per 128-byte step of a row) and re-laid out through LDS: the token
// rows, which all four wavefronts read, into a shared buffer (double
// buffered, one barrier per step); each wavefront's weight rows into its own
// slot. 16-byte chunks sit in LDS at a position XOR-swizzled by the row
// index, so fragment reads are free of bank conflicts. Loads run kStages
// steps of 64 k ahead in a register ring, weights and rows of a step issued
// together, so waiting for a step's rows never waits for later weights.
// Within a step, lane half h supplies k = 32h + 8s + j (s the instruction, j
// the element) for both operands: any pairing of k slots gives the same sum.
#include "moe_kernels.h"
#include "moe_lanes.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kGemmThreads = 256;
constexpr int kStages = 2;          // steps of loads in flight (more costs occupancy)
constexpr int kStepChunks = 8;   // 64 bf16 of k per step = 8 chunks of 16 bytes
constexpr int kXcds = 8;         // MI355X: 8 XCDs, each with its own L2

__device__ __forceinline__ bf16x8 as_bf16x8(v4i v) { return __builtin_bit_cast(bf16x8, v); }

// LDS position of 16-byte chunk c of row r within the row's 128 bytes is
// c ^ swz(r): any 16 consecutive rows at one chunk index land in 16 distinct
// 16-byte bank groups (and any 8 in 8), so the B-fragment reads, one chunk
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

template <int BT>
__global__ __launch_bounds__(kGemmThreads)
void grouped_gemm_kernel(const v4i* __restrict__ x_e, const v4i* __restrict__ w,
                         const int32_t* __restrict__ offsets, int32_t E, int32_t max_rows,
                         int32_t chunks, int32_t N, int32_t ftiles, uint8_t* __restrict__ out) {
    constexpr int U = BT / 32;                       // 32-row sub-tiles
    __shared__ v4i xs[2][BT * kStepChunks];
    __shared__ v4i ws[4][32 * kStepChunks];      // one weight slot per wavefront
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
        // Workgroup b runs on XCD b % kXcds (round-robin dispatch); XCD x
        // takes the tile run [x * run, (x + 1) * run), so tiles that share a
        // weight tile or a row tile meet in one L2.
        const int64_t total = __shfl(incl, 63, 64);
        const int64_t run = (total + kXcds - 1) / kXcds;
        const int64_t idx = blockIdx.x / kXcds;
        const int64_t u = (blockIdx.x % kXcds) * run + idx;
        if (lane == 0 && (idx >= run || u >= total)) info[0] = -1;
        int64_t base = incl - local;
        if (idx < run && u >= base && u < incl) {
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
                    info[1] = (in / mbe) * 128;
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
    // Weight rows are loaded coalesced (8 lanes cover one row's 128-byte
    // step, an instruction 8 rows) and staged through the wavefront's own
    // LDS slot into the A-fragment layout: the fragment layout itself (32
    // rows per instruction) costs the vector memory path about 3x more per
    // byte. Lane l loads rows (l >> 3) + 8j, chunk l & 7; features past N
    // read row N-1 (never stored).
    const v4i* wrow[4];
    int32_t wslot[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = (lane >> 3) + 8 * j;
        const int c = lane & 7;
        wrow[j] = w + (int64_t(e) * N + min(f0 + wave * 32 + r, N - 1)) * chunks + c;
        wslot[j] = r * kStepChunks + (c ^ swz(r));
    }
    v4i* wbuf = ws[wave];
    // This thread's token-row chunks: q = tid + 256j of the BT x 8 step tile
    // (rows past the segment read its last row; never stored).
    const v4i* xrow[U];
    int32_t xslot[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
        const int q = tid + kGemmThreads * j;
        const int r = q >> 3;
        const int c = q & 7;
        xrow[j] = x_e + int64_t(row0 + min(r, nrows - 1)) * chunks + c;
        xslot[j] = r * kStepChunks + (c ^ swz(r));
    }
    f32x16 acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[u][r] = 0.0f;

    // One step: rows of the step (already in registers) to LDS, then the
    // 4 x U matrix-core products against the step's weight fragments.
    auto mma_step = [&](int buf_id, const v4i (&wv)[4], const v4i (&xv)[U], auto&& after_barrier) {
        v4i* buf = xs[buf_id];
#pragma unroll
        for (int j = 0; j < U; ++j) buf[xslot[j]] = xv[j];
#pragma unroll
        for (int j = 0; j < 4; ++j) wbuf[wslot[j]] = wv[j];
        __syncthreads();
        after_barrier();
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const bf16x8 a = as_bf16x8(wbuf[i * kStepChunks + ((4 * h + s) ^ swz(i))]);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int r = u * 32 + i;
                const bf16x8 b = as_bf16x8(buf[r * kStepChunks + ((4 * h + s) ^ swz(r))]);
                acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[u], 0, 0, 0);
            }
        }
    };

    // Whole steps: every load is issued unconditionally, kStages steps ahead
    // (the step index is clamped to the last whole step, a scalar, so the
    // loop body has no divergent branches between the loads and their use).
    const int32_t full = chunks / kStepChunks;
    v4i wr[kStages][4];
    v4i xr[kStages][U];
    auto load_w = [&](int32_t step, v4i (&dst)[4]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) dst[j] = wrow[j][step * kStepChunks];
    };
    auto load_x = [&](int32_t step, v4i (&dst)[U]) {
#pragma unroll
        for (int j = 0; j < U; ++j) dst[j] = xrow[j][step * kStepChunks];
    };
    // The loop body runs whole groups of kStages steps with no branch in it
    // (a branch there makes the wait counts conservative, which drains the
    // pipeline every group); the 0..kStages-1 steps left over run after it
    // from the already loaded ring.
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
    // The last, partial step (k_in not a multiple of 64): chunks past the
    // row read as zero in both operands.
    if (done * kStepChunks < chunks) {
        const int32_t c0 = done * kStepChunks;
        const int32_t last = chunks - 1;
        v4i wv[4], xv[U];
        const v4i zero = {0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int32_t c = c0 + (lane & 7);
            const v4i v = wrow[j][min(c, last) - (lane & 7)];
            wv[j] = c <= last ? v : zero;
        }
#pragma unroll
        for (int j = 0; j < U; ++j) {
            const int32_t c = c0 + ((tid + kGemmThreads * j) & 7);
            const v4i v = xrow[j][min(c, last) - ((tid + kGemmThreads * j) & 7)];
            xv[j] = c <= last ? v : zero;
        }
        mma_step(done & 1, wv, xv, [] {});
    }

    // acc[u][4q + t] is out[row u*32 + i][feature 32w + 8q + 4h + t].
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int r = u * 32 + i;
        if (r >= nrows) continue;
        uint8_t* orow = out + (int64_t(row0 + r) * N) * 2;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int32_t col = f0 + wave * 32 + 8 * q + 4 * h;
            if (col >= N) continue;
            uint2 v;
            v.x = f32_to_bf16_bits(acc[u][4 * q]) | (f32_to_bf16_bits(acc[u][4 * q + 1]) << 16);
            v.y = f32_to_bf16_bits(acc[u][4 * q + 2]) | (f32_to_bf16_bits(acc[u][4 * q + 3]) << 16);
            *reinterpret_cast<uint2*>(orow + int64_t(col) * 2) = v;
        }
    }
}

template <int BT>
hipError_t launch_bt(const GroupedGemmArgs& a, hipStream_t stream) {
    const int64_t grid = grouped_gemm_grid(a.max_rows, a.E, a.N, BT);
    hipLaunchKernelGGL((grouped_gemm_kernel<BT>), dim3(static_cast<uint32_t>(grid)),
                       dim3(kGemmThreads), 0, stream, static_cast<const v4i*>(a.x_e),
                       static_cast<const v4i*>(a.w), a.offsets, a.E,
                       static_cast<int32_t>(a.max_rows), a.Kd / 8,
                       a.N, static_cast<int32_t>((a.N + 127) / 128),
                       static_cast<uint8_t*>(a.out));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_grouped_gemm(const GroupedGemmArgs& a, hipStream_t stream) {
    if (a.max_rows <= 0) return hipSuccess;
    switch (a.row_tile) {
        case 64: return launch_bt<64>(a, stream);
        case 128: return launch_bt<128>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace moe
