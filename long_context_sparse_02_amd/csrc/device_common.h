// Device-side types and helpers shared by the gfx950 kernels of libgsa.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

__device__ __forceinline__ float neg_inf() { return __int_as_float(0xff800000u); }

// Order-preserving map of an fp32 score to uint32 (larger float -> larger key),
// with -0.0 folded onto +0.0 so the two tie as floats do.
__device__ __forceinline__ uint32_t score_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// E8M0 exponent byte of a power-of-two fp32 scale (its biased exponent field).
__device__ __forceinline__ int e8m0_of(float s) {
    return (int)((__float_as_uint(s) >> 23) & 0xffu);
}

__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, kWave); }

}  // namespace gsa
