// Element helpers for the 16-byte chunks the data-movement kernels work on:
// a chunk is 4 fp32 or 8 bf16 elements. Internal to libmoe_layout.so.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace moe {

typedef int32_t v4i __attribute__((ext_vector_type(4)));

// bf16 <-> fp32 by bit manipulation: widening is exact; narrowing rounds to
// nearest even, with every NaN mapped to the quiet NaN 0x7FC0.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Per-chunk arithmetic in fp32:
//   fma_into(acc, s, v):  acc[i] = fma(s, v[i], acc[i])
//   pack(acc):            acc rounded to the element type
//   scale(s, v):          s * v[i], one fp32 product rounded to the element type
//   dot_into(acc, a, b):  acc = fma(a[i], b[i], acc) for i in element order
template <bool BF16>
struct Lanes;

template <>
struct Lanes<false> {  // 4 fp32 per 16-byte chunk
    static constexpr int N = 4;
    __device__ static void fma_into(float (&acc)[N], float s, v4i v) {
#pragma unroll
        for (int i = 0; i < N; ++i) acc[i] = __builtin_fmaf(s, __int_as_float(v[i]), acc[i]);
    }
    __device__ static v4i pack(const float (&acc)[N]) {
        v4i o;
#pragma unroll
        for (int i = 0; i < N; ++i) o[i] = __float_as_int(acc[i]);
        return o;
    }
    __device__ static v4i scale(float s, v4i v) {
        v4i o;
#pragma unroll
        for (int i = 0; i < N; ++i) o[i] = __float_as_int(s * __int_as_float(v[i]));
        return o;
    }
    __device__ static float dot_into(float acc, v4i a, v4i b) {
#pragma unroll
        for (int i = 0; i < N; ++i) acc = __builtin_fmaf(__int_as_float(a[i]), __int_as_float(b[i]), acc);
        return acc;
    }
};

template <>
struct Lanes<true> {  // 8 bf16 per 16-byte chunk, element 2i in the low half
    static constexpr int N = 8;
    __device__ static void fma_into(float (&acc)[N], float s, v4i v) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t w = static_cast<uint32_t>(v[i]);
            acc[2 * i] = __builtin_fmaf(s, bf16_lo(w), acc[2 * i]);
            acc[2 * i + 1] = __builtin_fmaf(s, bf16_hi(w), acc[2 * i + 1]);
        }
    }
    __device__ static v4i pack(const float (&acc)[N]) {
        v4i o;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            o[i] = static_cast<int32_t>(f32_to_bf16_bits(acc[2 * i]) |
                                        (f32_to_bf16_bits(acc[2 * i + 1]) << 16));
        return o;
    }
    __device__ static v4i scale(float s, v4i v) {
        v4i o;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t w = static_cast<uint32_t>(v[i]);
            o[i] = static_cast<int32_t>(f32_to_bf16_bits(s * bf16_lo(w)) |
                                        (f32_to_bf16_bits(s * bf16_hi(w)) << 16));
        }
        return o;
    }
    __device__ static float dot_into(float acc, v4i a, v4i b) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t wa = static_cast<uint32_t>(a[i]);
            const uint32_t wb = static_cast<uint32_t>(b[i]);
            acc = __builtin_fmaf(bf16_lo(wa), bf16_lo(wb), acc);
            acc = __builtin_fmaf(bf16_hi(wa), bf16_hi(wb), acc);
        }
        return acc;
    }
};

template <bool NT>
__device__ __forceinline__ v4i fetch(const v4i* p) {
    if constexpr (NT)
        return __builtin_nontemporal_load(p);
    else
        return *p;
}

}  // namespace moe
