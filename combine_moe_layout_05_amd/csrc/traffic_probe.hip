// Traffic reference kernels for the benchmark (libmoe_traffic_probe.so).
// Not part of the library's C ABI and not on the hot path: bench.py runs
// them beside the combine so that its rate can be compared with the rate
// the same HBM traffic reaches without any arithmetic.
//
//   probe_gather_copy  the combine's exact traffic and launch shape (one
//                      wavefront per 1 KiB piece of a token row, 16
//                      wavefronts per workgroup, the row map staged in LDS,
//                      streaming loads of the K rows of the token), storing
//                      the XOR of the K pieces instead of their weighted sum;
//                      with store = 0 the same reads and no store
//   probe_stream       plain streaming traffic over one buffer: 0 = read
//                      (eight 1 KiB pieces per wavefront), 1 = write
//                      (1 KiB per wavefront), 2 = the combine's read:write
//                      byte ratio in sequential order (eight consecutive
//                      1 KiB reads, one 1 KiB write into a second buffer),
//                      3 = dispatch's read:write byte ratio in sequential
//                      order (one 1 KiB read, written to eight consecutive
//                      KiB of a second buffer)
//
// Reads are kept alive by comparing the loaded data with three words of
// `sink` that the caller sets to values the data never takes; a kernel that
// only reads then stores nothing.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef int32_t v4i __attribute__((ext_vector_type(4)));

constexpr int kWaves = 16;

template <int K, bool STORE>
__global__ __launch_bounds__(kWaves * 64)
void gather_copy_kernel(const v4i* __restrict__ rows, const int32_t* __restrict__ row_map,
                        int32_t T, int32_t chunks, int32_t segments, int64_t row_limit,
                        v4i* __restrict__ dst, int32_t* __restrict__ sink) {
    __shared__ int32_t tile_rows[kWaves * K];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t item0 = int64_t(blockIdx.x) * kWaves;
    const int64_t t_first = item0 / segments;
    int64_t t_last = (item0 + kWaves - 1) / segments;
    if (t_last > int64_t(T) - 1) t_last = int64_t(T) - 1;
    const int staged = static_cast<int>(t_last - t_first + 1) * K;
    if (tid < staged) {
        const int32_t r = row_map[t_first * K + tid];
        tile_rows[tid] = (r >= 0 && r < row_limit) ? r : -1;
    }
    __syncthreads();
    const int64_t item = item0 + wave;
    const int64_t t = item / segments;
    if (t >= T) return;
    const int seg = static_cast<int>(item - t * segments);
    const int lt = static_cast<int>(t - t_first);
    const int32_t c = seg * 64 + lane;
    const int32_t cl = c < chunks ? c : chunks - 1;
    int32_t fallback = -1;
    int32_t row[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        row[k] = __builtin_amdgcn_readfirstlane(tile_rows[lt * K + k]);
        if (fallback < 0 && row[k] >= 0) fallback = row[k];
    }
    v4i acc = {0, 0, 0, 0};
    if (fallback >= 0) {
        v4i b[K];
#pragma unroll
        for (int k = 0; k < K; ++k)
            b[k] = __builtin_nontemporal_load(rows + int64_t(row[k] >= 0 ? row[k] : fallback) * chunks + cl);
        // as the combine: a no-expert slot loads the token's first valid row
        // (so every load is unconditional) and is left out of the result
#pragma unroll
        for (int k = 0; k < K; ++k)
            if (row[k] >= 0) acc ^= b[k];
    }
    if constexpr (STORE) {
        if (c < chunks) dst[t * chunks + c] = acc;
    } else if (acc[0] == sink[1] && acc[1] == sink[2] && acc[2] == sink[3]) {
        sink[0] = acc[3];
    }
}

// kind 0: read; 1: write; 2: sequential 8:1 read:write mix; 3: sequential
// 1:8 mix. One kernel per kind, so traces and counters name them apart.
template <int KIND>
__global__ __launch_bounds__(1024)
void stream_kernel(const v4i* __restrict__ a, v4i* __restrict__ b, int64_t n_chunks,
                   int32_t* __restrict__ sink) {
    const int lane = threadIdx.x & 63;
    const int64_t w = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
    if constexpr (KIND == 1) {
        const int64_t c = w * 64 + lane;
        if (c < n_chunks) b[c] = v4i{static_cast<int32_t>(c), 1, 2, 3};
        return;
    }
    if constexpr (KIND == 3) {
        const int64_t c = w * 64 + lane;
        if (c < n_chunks) {
            const v4i v = a[c];
#pragma unroll
            for (int i = 0; i < 8; ++i) b[(w * 8 + i) * 64 + lane] = v;
        }
        return;
    }
    v4i acc = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t c = (w * 8 + i) * 64 + lane;
        if (c < n_chunks) acc ^= __builtin_nontemporal_load(a + c);
    }
    if constexpr (KIND == 2) {
        const int64_t c = w * 64 + lane;
        if (c * 8 < n_chunks) b[c] = acc;
    } else if (acc[0] == sink[1] && acc[1] == sink[2] && acc[2] == sink[3]) {
        sink[0] = acc[3];
    }
}

template <int K>
hipError_t launch_gather(const void* rows, const int32_t* row_map, int32_t T, int32_t chunks,
                         int64_t row_limit, void* dst, int32_t* sink, int store,
                         hipStream_t stream) {
    const int32_t segments = (chunks + 63) / 64;
    const int64_t blocks = (int64_t(T) * segments + kWaves - 1) / kWaves;
    auto kernel = store ? gather_copy_kernel<K, true> : gather_copy_kernel<K, false>;
    hipLaunchKernelGGL(kernel, dim3(static_cast<uint32_t>(blocks)), dim3(kWaves * 64), 0, stream,
                       static_cast<const v4i*>(rows), row_map, T, chunks, segments, row_limit,
                       static_cast<v4i*>(dst), sink);
    return hipGetLastError();
}

}  // namespace

extern "C" {

// rows: [>= row_limit][chunks * 16 bytes]; row_map: [T][K] int32 (rows
// outside [0, row_limit) are skipped, as the combine skips them); dst:
// [T][chunks * 16 bytes]; sink: 4 int32 in device memory. 1 <= K <= 16.
// Returns a hipError_t value (0 = launched).
int probe_gather_copy(const void* rows, const int32_t* row_map, int32_t T, int32_t K,
                      int32_t chunks, int64_t row_limit, void* dst, int32_t* sink, int store,
                      void* stream) {
    if (T <= 0) return 0;
    if (chunks < 1 || !rows || !row_map || !sink || (store && !dst)) return hipErrorInvalidValue;
    hipStream_t st = static_cast<hipStream_t>(stream);
    switch (K) {
#define PROBE_CASE(k) \
    case k: return launch_gather<k>(rows, row_map, T, chunks, row_limit, dst, sink, store, st);
        PROBE_CASE(1) PROBE_CASE(2) PROBE_CASE(3) PROBE_CASE(4) PROBE_CASE(5) PROBE_CASE(6)
        PROBE_CASE(7) PROBE_CASE(8) PROBE_CASE(9) PROBE_CASE(10) PROBE_CASE(11) PROBE_CASE(12)
        PROBE_CASE(13) PROBE_CASE(14) PROBE_CASE(15) PROBE_CASE(16)
#undef PROBE_CASE
        default: return hipErrorInvalidValue;
    }
}

// kind 0: read `bytes` of a; 1: write `bytes` of b; 2: read `bytes` of a and
// write bytes / 8 of b (sequential); 3: read `bytes` of a and write 8 x bytes
// of b (sequential). bytes: a multiple of 16 (of 128 for 2, of 1024 for 3).
int probe_stream(int kind, const void* a, void* b, int64_t bytes, int32_t* sink, void* stream) {
    const int64_t unit = kind == 2 ? 128 : (kind == 3 ? 1024 : 16);
    if (kind < 0 || kind > 3 || bytes <= 0 || bytes % unit != 0 || !sink)
        return hipErrorInvalidValue;
    if ((kind != 1 && !a) || (kind != 0 && !b)) return hipErrorInvalidValue;
    const int64_t n = bytes / 16;
    const int64_t waves = (kind == 1 || kind == 3) ? (n + 63) / 64 : (n + 511) / 512;
    const int64_t blocks = (waves + 15) / 16;
    auto kernel = kind == 0 ? stream_kernel<0>
                : kind == 1 ? stream_kernel<1>
                : kind == 2 ? stream_kernel<2> : stream_kernel<3>;
    hipLaunchKernelGGL(kernel, dim3(static_cast<uint32_t>(blocks)), dim3(1024), 0,
                       static_cast<hipStream_t>(stream), static_cast<const v4i*>(a),
                       static_cast<v4i*>(b), n, sink);
    return hipGetLastError();
}

}  // extern "C"
