// Per-block FP8 E4M3 quantisation of indexer q/k rows on gfx950.
//
// "GLM-5.2 总览" sub-document index (row 02): the lightning indexer quantises
// q and k to FP8 per block, with a Hadamard rotation; glossary: the FP8 format
// is E4M3. The rotated variant multiplies each block by the orthonormal
// Hadamard matrix first (dot products are unchanged in exact arithmetic).
// Block = one 128-element row. Scale = 2^e, e the smallest integer with
// max|x| <= 448 * 2^e (clamped to [-126, 127]; e = 0 for a zero row). Codes are
// x / scale rounded to nearest even in E4M3FN (bias 7, max 448, no inf),
// saturating at +-448. With power-of-two scales the division is exact.
#include "device_common.h"
#include "launch.h"

namespace gsa {
namespace {

constexpr int kThreads = 256;   // 16 rows per work-group, 16 threads x 8 elements per row

__device__ __forceinline__ uint32_t encode_e4m3(float v) {
    const uint32_t u = __float_as_uint(v);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t mag = u & 0x7fffffffu;
    if (mag > 0x7f800000u) return 0x7fu;                 // NaN
    const float a = __uint_as_float(mag);
    if (a >= 448.f) return sign | 0x7eu;                 // saturate
    if (a < 0.015625f) {                                 // below 2^-6: steps of 2^-9
        return sign | (uint32_t)rintf(a * 512.f);        // 8 lands on the smallest normal code
    }
    const int ex = (int)(mag >> 23) - 127;               // a in [2^ex, 2^(ex+1)), ex in [-6, 8]
    const uint32_t frac = mag & 0x7fffffu;
    uint32_t keep = frac >> 20;                           // top 3 fraction bits
    const uint32_t rest = frac & 0xfffffu;
    const uint32_t half = 0x80000u;
    if (rest > half || (rest == half && (keep & 1u))) ++keep;   // nearest, ties to even
    uint32_t code = ((uint32_t)(ex + 7) << 3) + keep;     // a carry out of `keep` bumps the exponent
    if (code > 0x7eu) code = 0x7eu;
    return sign | code;
}

// y = H x / sqrt(128) over one 128-element block held by 16 lanes (8
// consecutive elements each), H the Sylvester-ordered Hadamard matrix
// (H[i][j] = (-1)^popcount(i & j)): the in-place butterflies (a, b) -> (a + b,
// a - b) at distances 1, 2, 4 inside a lane and 8 .. 64 across lanes give the
// exact +-1 sums (integer inputs stay exact in fp32), then one multiply by the
// fp32 value of 1/sqrt(128).
__device__ __forceinline__ void hadamard128(float (&v)[8], int part) {
#pragma unroll
    for (int h = 1; h < 8; h <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if ((e & h) == 0) {
                const float a = v[e], b = v[e + h];
                v[e] = a + b;
                v[e + h] = a - b;
            }
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) {
        const bool upper = (part & m) != 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float o = __shfl_xor(v[e], m, 64);
            v[e] = upper ? o - v[e] : v[e] + o;
        }
    }
    constexpr float kInvSqrt128 = 0.08838834764831844055f;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] *= kInvSqrt128;
}

template <bool kRotate>
__global__ __launch_bounds__(kThreads) void quantize_e4m3_kernel(const uint16_t* __restrict__ x,
                                                                 int64_t n_rows,
                                                                 uint8_t* __restrict__ codes,
                                                                 float* __restrict__ scales) {
    const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    const int part = threadIdx.x & 15;
    const bool ok = row < n_rows;
    float v[8];
    float amax = 0.f;
    {
        const i32x4 raw = ok ? *(const i32x4*)(x + row * 128 + part * 8) : i32x4{0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t w = (uint32_t)raw[e];
            v[2 * e] = __uint_as_float(w << 16);             // bf16 -> fp32 is exact
            v[2 * e + 1] = __uint_as_float(w & 0xffff0000u);
        }
        if constexpr (kRotate) hadamard128(v, part);       // every lane takes part in the shuffles
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
    }
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
    if (!ok) return;
    int e = 0;
    if (amax > 0.f) {
        const uint32_t b = __float_as_uint(amax);
        const int ea = (int)(b >> 23) - 127;              // amax = 1.m * 2^ea
        if ((b >> 23) == 0) e = -126;                    // fp32-subnormal amax: clamp
        else e = ((b & 0x7fffffu) <= 0x600000u) ? ea - 8 : ea - 7;   // 448 = 1.75 * 2^8
        e = e < -126 ? -126 : (e > 127 ? 127 : e);
    }
    const float inv = __uint_as_float((uint32_t)(127 - e) << 23);   // 2^-e, e in [-126, 120] for finite rows
    uint32_t packed[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) packed[i >> 2] |= encode_e4m3(v[i] * inv) << (8 * (i & 3));
    *(uint2*)(codes + row * 128 + part * 8) = make_uint2(packed[0], packed[1]);
    if (part == 0) scales[row] = __uint_as_float((uint32_t)(e + 127) << 23);
}

// The FP8 latent cache row: [512 E4M3 codes | 4 fp32 scales | 64 bf16 RoPE]
// (656 bytes). The latent is quantised in four 128-dim groups with the block
// rule above; the RoPE key is kept in bf16. One wave per row: 16 lanes per
// group, lanes 0-7 also move the RoPE bytes.
__global__ __launch_bounds__(kThreads) void quantize_latent_kernel(const uint16_t* __restrict__ x,
                                                                   int64_t n_rows,
                                                                   uint8_t* __restrict__ out) {
    const int64_t row = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int grp = lane >> 4, part = lane & 15;
    if (row >= n_rows) return;                            // uniform per wave
    const uint16_t* xr = x + row * 576;
    uint8_t* o = out + row * 656;
    float v[8];
    float amax = 0.f;
    const i32x4 raw = *(const i32x4*)(xr + grp * 128 + part * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t w = (uint32_t)raw[e];
        v[2 * e] = __uint_as_float(w << 16);
        v[2 * e + 1] = __uint_as_float(w & 0xffff0000u);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
    int e = 0;
    if (amax > 0.f) {
        const uint32_t b = __float_as_uint(amax);
        const int ea = (int)(b >> 23) - 127;
        if ((b >> 23) == 0) e = -126;
        else e = ((b & 0x7fffffu) <= 0x600000u) ? ea - 8 : ea - 7;
        e = e < -126 ? -126 : (e > 127 ? 127 : e);
    }
    const float inv = __uint_as_float((uint32_t)(127 - e) << 23);
    uint32_t packed[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) packed[i >> 2] |= encode_e4m3(v[i] * inv) << (8 * (i & 3));
    *(uint2*)(o + grp * 128 + part * 8) = make_uint2(packed[0], packed[1]);
    if (part == 0) *(float*)(o + 512 + 4 * grp) = __uint_as_float((uint32_t)(e + 127) << 23);
    if (lane < 8) *(i32x4*)(o + 528 + 16 * lane) = *(const i32x4*)(xr + 512 + 8 * lane);
}

}  // namespace

hipError_t launch_quantize_latent(const void* rows, int64_t n_rows, uint8_t* out, hipStream_t st) {
    if (n_rows == 0) return hipSuccess;
    hipLaunchKernelGGL(quantize_latent_kernel, dim3((unsigned)((n_rows + 3) / 4)), dim3(kThreads), 0, st,
                       (const uint16_t*)rows, n_rows, out);
    return hipGetLastError();
}

hipError_t launch_quantize_e4m3(const void* x, int64_t n_rows, uint8_t* codes, float* scales,
                                bool rotate, hipStream_t st) {
    if (n_rows == 0) return hipSuccess;
    if (rotate)
        hipLaunchKernelGGL(quantize_e4m3_kernel<true>, dim3((unsigned)((n_rows + 15) / 16)), dim3(kThreads),
                           0, st, (const uint16_t*)x, n_rows, codes, scales);
    else
        hipLaunchKernelGGL(quantize_e4m3_kernel<false>, dim3((unsigned)((n_rows + 15) / 16)), dim3(kThreads),
                           0, st, (const uint16_t*)x, n_rows, codes, scales);
    return hipGetLastError();
}

}  // namespace gsa
