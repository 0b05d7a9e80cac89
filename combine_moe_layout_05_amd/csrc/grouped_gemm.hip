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
// expert's segment); tiles are numbered expert by expert, row tiles fastest,
// so row tiles that share a weight tile run side by side and share it in
// cache. The grid covers the most tiles any routing can need,
// ceil(max_rows / BT) + E row tiles per feature tile; wavefront 0 of each
// workgroup finds its tile from the offsets (a scan of the per-expert tile
// counts over the 64 lanes) and workgroups past the last tile exit.
//
// Inside a tile, wavefront w owns features [32w, 32w + 32) and all BT rows:
// v_mfma_f32_32x32x16_bf16 with the weight rows as the A operand and the
// token rows as B. The weight rows are read once per tile, straight into the
// A fragments (they are not shared, so they skip LDS); the token rows, which
// all four wavefronts need, go through LDS in 16-byte chunks whose position
// within a 128-byte row is XOR-swizzled by the row index. Both are loaded
// kStages steps of 64 k ahead into a register ring, weights and rows of a
// step issued together, so waiting for a step's rows never waits for later
// weights. Within a step, lane half h supplies k = 32h + 8s + j (s the
// instruction, j the element) for both operands: any pairing of k slots
// gives the same sum, and this one makes a lane's weight loads contiguous.
#include "moe_kernels.h"
#include "moe_lanes.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kGemmThreads = 256;
constexpr int kStages = 4;          // even: the LDS buffer is the step's parity
constexpr int kStepChunks = 8;   // 64 bf16 of k per step = 8 chunks of 16 bytes

__device__ __forceinline__ bf16x8 as_bf16x8(v4i v) { return __builtin_bit_cast(bf16x8, v); }

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
        const int64_t u = blockIdx.x;
        const int64_t total = __shfl(incl, 63, 64);
        if (lane == 0 && u >= total) info[0] = -1;
        int64_t base = incl - local;
        if (u >= base && u < incl) {
            for (int e = e_lo; e < e_hi; ++e) {
                int32_t s0, s1;
                segment(offsets, e, max_rows, s0, s1);
                const int32_t mt = (s1 - s0 + BT - 1) / BT;
                const int64_t n = int64_t(mt) * ftiles;
                if (u < base + n) {
                    const int32_t rem = static_cast<int32_t>(u - base);
                    const int32_t r0 = s0 + (rem % mt) * BT;
                    info[0] = e;
                    info[1] = (rem / mt) * 128;
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

    const int32_t steps = (chunks + kStepChunks - 1) / kStepChunks;
    const int h = lane >> 5;
    const int i = lane & 31;
    // This lane's weight row (features past N read row N-1; never stored).
    const int32_t f = min(f0 + wave * 32 + i, N - 1);
    const v4i* wrow = w + (int64_t(e) * N + f) * chunks;
    // This thread's token-row chunks: q = tid + 256j of the BT x 8 step tile
    // (rows past the segment read its last row; never stored).
    const v4i* xrow[U];
    int32_t xc[U];
    int32_t xslot[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
        const int q = tid + kGemmThreads * j;
        const int r = q >> 3;
        const int c = q & 7;
        xrow[j] = x_e + int64_t(row0 + min(r, nrows - 1)) * chunks;
        xc[j] = c;
        xslot[j] = r * kStepChunks + (c ^ (r & 7));
    }
    // Every load is issued unconditionally (no divergent branches between
    // the loads and their use): a chunk index past the row reads the row's
    // last chunk and the value is replaced by zero, so steps past the end
    // (the rounding of the loop to whole groups of kStages) add nothing.
    const int32_t last = chunks - 1;
    auto pick = [](bool ok, v4i v) {
        v4i o;
#pragma unroll
        for (int t = 0; t < 4; ++t) o[t] = ok ? v[t] : 0;
        return o;
    };
    auto load_w = [&](int32_t step, v4i (&dst)[4]) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int32_t c = step * kStepChunks + 4 * h + s;
            dst[s] = pick(c <= last, wrow[min(c, last)]);
        }
    };
    auto load_x = [&](int32_t step, v4i (&dst)[U]) {
#pragma unroll
        for (int j = 0; j < U; ++j) {
            const int32_t c = step * kStepChunks + xc[j];
            dst[j] = pick(c <= last, xrow[j][min(c, last)]);
        }
    };

    v4i wr[kStages][4];
    v4i xr[kStages][U];
#pragma unroll
    for (int p = 0; p < kStages; ++p) {
        load_x(p, xr[p]);
        load_w(p, wr[p]);
    }
    f32x16 acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[u][r] = 0.0f;

    for (int32_t s0 = 0; s0 < steps; s0 += kStages) {
#pragma unroll
        for (int p = 0; p < kStages; ++p) {
            const int32_t step = s0 + p;
            v4i* buf = xs[p & 1];            // kStages is even: p & 1 == step & 1
#pragma unroll
            for (int j = 0; j < U; ++j) buf[xslot[j]] = xr[p][j];
            __syncthreads();
            load_x(step + kStages, xr[p]);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const bf16x8 a = as_bf16x8(wr[p][s]);
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int r = u * 32 + i;
                    const bf16x8 b = as_bf16x8(buf[r * kStepChunks + ((4 * h + s) ^ (r & 7))]);
                    acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[u], 0, 0, 0);
                }
            }
            load_w(step + kStages, wr[p]);
        }
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
