// Backward of the combine on gfx950.
//
// What is computed (the derivatives of the combine y[t] = sum_k s[t][k] *
// y_e[r(t,k)]; "fix(moe): equalize and align per-rank token counts for
// HybridEP dispatch", section "Testing", checks forward and backward of the
// dispatcher bitwise against the equal-count run):
//   dL/dy_e[r(t,k)] = s[t][k] * dL/dy[t]      one fp32 product, rounded to
//                                             the element type
//   dL/ds[t][k]     = <dL/dy[t], y_e[r(t,k)]> fp32 fused multiply-adds
// for every slot with an expert; a no-expert slot gets dL/ds = +0.0 and no
// row. Rows of dL/dy_e from the true total up to the current capacity's last
// row reached no token, so their gradient is +0.0; with a device pointer to
// that total they are written as such (the total stays on the device:
// "ep: graph-safe worst-token HT dispatch+combine", "Internode" item 3).
//
// One workgroup per token, W = ceil(chunks/64) wavefronts (at most 16): each
// lane owns 16-byte chunks lane + 64*wave + 64*W*i of the row, so the
// workgroup reads dL/dy[t] once, reads the K expert rows (streaming loads,
// all issued before use; a no-expert slot reads the token's first valid row
// and skips it), writes the K scaled rows, and reduces the K dot products:
// in element order within a lane, then a fixed butterfly over the 64 lanes,
// then the wavefronts in order. The reduction order is fixed, so results are
// deterministic; it differs from plain left-to-right order, which stays
// within the fp32 summation error bound of the dot product. The launch has
// kTailBlocks more workgroups than tokens; they store zeros into the rows
// [*total_rows, row_limit), a row per workgroup per turn. With NTS the dL/dy_e
// rows are written with streaming stores (the context picks them for buffers
// far beyond the last-level cache); results are the same bits either way.
#include "moe_kernels.h"
#include "moe_lanes.h"

#include <type_traits>

namespace moe {
namespace {

// Workgroups of the launch that zero the rows past the true total.
constexpr int32_t kTailBlocks = 512;

template <bool NTS>
__device__ __forceinline__ void put_row(v4i* p, v4i v) {
    if constexpr (NTS)
        __builtin_nontemporal_store(v, p);
    else
        *p = v;
}

template <int K, bool BF16, bool NTS>
__global__ __launch_bounds__(kMaxBlockThreads)
void combine_backward_kernel(const v4i* __restrict__ grad_y, const v4i* __restrict__ y_e,
                             const int32_t* __restrict__ row_map,
                             const float* __restrict__ scores, int32_t T, int32_t chunks,
                             int64_t row_limit, const int32_t* __restrict__ total_rows,
                             v4i* __restrict__ grad_y_e, float* __restrict__ grad_s) {
    using L = Lanes<BF16>;
    __shared__ int32_t tok_rows[K];
    __shared__ float tok_scores[K];
    __shared__ float partial[kMaxBlockWaves][K];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int waves = static_cast<int>(blockDim.x) >> 6;
    const int64_t t = blockIdx.x;

    if (t >= T) {
        // Rows [total, row_limit) were reached by no slot. The total is
        // clamped to [0, row_limit], so a wrong value cannot move the stores
        // outside the current capacity's rows.
        if (!total_rows) return;
        int64_t lo = *total_rows;
        lo = lo < 0 ? 0 : (lo > row_limit ? row_limit : lo);
        const v4i zero = {0, 0, 0, 0};
        for (int64_t r = lo + (t - T); r < row_limit; r += kTailBlocks) {
            v4i* dst = grad_y_e + r * chunks;
            for (int32_t c = tid; c < chunks; c += static_cast<int32_t>(blockDim.x))
                put_row<NTS>(dst + c, zero);
        }
        return;
    }

    if (tid < K) {
        // Both loads are issued before either is used.
        const int32_t r = row_map[t * K + tid];
        const float sv = scores[t * K + tid];
        const bool ok = r >= 0 && r < row_limit;
        tok_rows[tid] = ok ? r : -1;
        tok_scores[tid] = ok ? sv : 0.0f;
    }
    __syncthreads();
    int32_t row[K];
    float s[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        row[k] = __builtin_amdgcn_readfirstlane(tok_rows[k]);
        s[k] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(tok_scores[k])));
    }

    float dot[K];
#pragma unroll
    for (int k = 0; k < K; ++k) dot[k] = 0.0f;
    int32_t fallback = -1;
    bool all_valid = true;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        if (fallback < 0 && row[k] >= 0) fallback = row[k];
        all_valid = all_valid && row[k] >= 0;
    }
    if (fallback >= 0) {
        // No-expert slots read the token's first valid row instead (written,
        // finite) and skip it, so every load is unconditional.
        const v4i* src[K];
#pragma unroll
        for (int k = 0; k < K; ++k)
            src[k] = y_e + int64_t(row[k] >= 0 ? row[k] : fallback) * chunks;
        const v4i* g = grad_y + t * chunks;
        // All K scaled rows are computed into registers, stored back to back,
        // and only then do the dot products wait for the expert rows. Holding
        // the K scaled chunks takes the kernel to about 90 VGPRs, 5
        // wavefronts per SIMD: one 14-wavefront workgroup per CU at 7168
        // bf16, two 8-wavefront ones at 4096. Measured on MI355X in a
        // backward pass at 4096 tokens of 7168: 174-176 against 182-193 us
        // for the store-then-dot-per-slot form at 7 wavefronts per SIMD;
        // neither the store order alone nor one workgroup per CU forced by
        // LDS gives it, and the other shapes are unchanged.
        auto pass = [&](auto every) {
            for (int32_t c = wave * 64 + lane; c < chunks; c += waves * 64) {
                const v4i gv = g[c];
                v4i yv[K];
#pragma unroll
                for (int k = 0; k < K; ++k) yv[k] = fetch<true>(src[k] + c);
                v4i scaled[K];
#pragma unroll
                for (int k = 0; k < K; ++k) scaled[k] = L::scale(s[k], gv);
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    if (!decltype(every)::value && row[k] < 0) continue;
                    put_row<NTS>(grad_y_e + int64_t(row[k]) * chunks + c, scaled[k]);
                }
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    if (!decltype(every)::value && row[k] < 0) continue;
                    dot[k] = L::dot_into(dot[k], gv, yv[k]);
                }
            }
        };
        if (all_valid)
            pass(std::true_type{});
        else
            pass(std::false_type{});
    }

    // Lanes, then wavefronts, in a fixed order.
#pragma unroll
    for (int k = 0; k < K; ++k) {
        float v = dot[k];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
        if (lane == 0) partial[wave][k] = v;
    }
    __syncthreads();
    if (tid < K) {
        float sum = 0.0f;
        for (int w = 0; w < waves; ++w) sum += partial[w][tid];
        grad_s[t * K + tid] = tok_rows[tid] >= 0 ? sum : 0.0f;
    }
}

template <int K, bool BF16>
hipError_t launch_k(const CombineBackwardArgs& a, hipStream_t stream) {
    int32_t waves = (a.chunks + 63) / 64;
    if (waves > kMaxBlockWaves) waves = kMaxBlockWaves;
    // Token workgroups first, then the tail workgroups (only when asked for).
    const int64_t blocks = int64_t(a.T) + (a.total_rows ? kTailBlocks : 0);
    auto kernel = a.store_nontemporal ? combine_backward_kernel<K, BF16, true>
                                      : combine_backward_kernel<K, BF16, false>;
    hipLaunchKernelGGL(kernel, dim3(static_cast<uint32_t>(blocks)),
                       dim3(64 * waves), 0, stream, static_cast<const v4i*>(a.grad_y),
                       static_cast<const v4i*>(a.y_e), a.row_map, a.scores, a.T, a.chunks,
                       a.row_limit, a.total_rows, static_cast<v4i*>(a.grad_y_e), a.grad_s);
    return hipGetLastError();
}

template <bool BF16>
hipError_t launch_dtype(const CombineBackwardArgs& a, hipStream_t stream) {
    switch (a.K) {
#define MOE_CB_CASE(k) \
    case k: return launch_k<k, BF16>(a, stream);
        MOE_CB_CASE(1) MOE_CB_CASE(2) MOE_CB_CASE(3) MOE_CB_CASE(4)
        MOE_CB_CASE(5) MOE_CB_CASE(6) MOE_CB_CASE(7) MOE_CB_CASE(8)
        MOE_CB_CASE(9) MOE_CB_CASE(10) MOE_CB_CASE(11) MOE_CB_CASE(12)
        MOE_CB_CASE(13) MOE_CB_CASE(14) MOE_CB_CASE(15) MOE_CB_CASE(16)
#undef MOE_CB_CASE
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_combine_backward(const CombineBackwardArgs& a, hipStream_t stream) {
    if (a.T <= 0 && !a.total_rows) return hipSuccess;
    return a.bf16 ? launch_dtype<true>(a, stream) : launch_dtype<false>(a, stream);
}

}  // namespace moe
