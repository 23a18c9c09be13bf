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

// The fp32 value of an order-preserving key (inverse of score_key; +0 for the
// folded zero).
__device__ __forceinline__ float key_value(uint32_t key) {
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

// The largest key over the 32 lanes of each half-wave, in every lane: two
// quad permutations, the half-row and row mirrors (DPP) and a permlane16 swap
// between the two rows of the half-wave. VALU only.
__device__ __forceinline__ uint32_t max_x32(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xb1, 0xf, 0xf, false));   // lane ^ 1
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4e, 0xf, 0xf, false));   // lane ^ 2
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xf, 0xf, false));  // 7 - lane in 8
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xf, 0xf, false));  // 15 - lane in 16
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);                   // other row
    return max((uint32_t)r[0], (uint32_t)r[1]);
}

// The same over fp32 values (v_max_f32 with DPP operands): the result is one of
// the 32 values (a NaN counts as missing), and a zero maximum may be -0.0.
__device__ __forceinline__ float max_x32f(float v) {
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xb1, 0xf, 0xf, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4e, 0xf, 0xf, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xf, 0xf, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xf, 0xf, false)));
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// E8M0 exponent byte of a power-of-two fp32 scale (its biased exponent field).
__device__ __forceinline__ int e8m0_of(float s) {
    return (int)((__float_as_uint(s) >> 23) & 0xffu);
}

__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, kWave); }

// v(l) + v(l ^ 32) with the gfx950 permlane32 swap (VALU only, no LDS).
__device__ __forceinline__ float sum_x32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---- LDS-DMA rings ---------------------------------------------------------
// One 16-byte LDS-DMA load per lane: lane l's 16 bytes from `src` land at LDS
// address lds_base + 16*l (one wait state between the M0 write and the load,
// as the M0 -> LDS-DMA hazard requires). Issued through asm so that the
// compiler's wait insertion does not treat later LDS reads as depending on it
// (it would wait for every DMA in flight); each ring's own vmcnt waits and
// barriers order these loads against the reads of the slot they fill, so the
// asm carries no memory clobber and the index reads feeding it can be batched.
__device__ __forceinline__ void lds_dma16(const void* src, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_base))
                 : "m0");
}
// The same with 4 bytes per lane (64 lanes fill 256 contiguous LDS bytes).
__device__ __forceinline__ void lds_dma4(const void* src, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                 :
                 : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_base))
                 : "m0");
}
// Non-temporal forms (the nt cache-policy bit) for data read once: a stream of
// such loads reaches about 7.2 TB/s on MI355X against about 6.3 TB/s without
// the hint (1 GiB+ streams, LDS-DMA rings of 32-64 KiB tiles).
template <bool NT>
__device__ __forceinline__ void lds_dma16_t(const void* src, uint32_t lds_base) {
    if constexpr (NT)
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
                     :
                     : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_base))
                     : "m0");
    else
        lds_dma16(src, lds_base);
}
template <bool NT>
__device__ __forceinline__ void lds_dma4_t(const void* src, uint32_t lds_base) {
    if constexpr (NT)
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off nt"
                     :
                     : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_base))
                     : "m0");
    else
        lds_dma4(src, lds_base);
}

// Work-group barrier without the memory fence of __syncthreads(): that fence
// would wait for every outstanding LDS-DMA load, including those meant to stay
// in flight. Each wave first waits (vmcnt) for its own part of the slot it is
// about to read; the empty asm statements keep the compiler from moving
// memory accesses across the barrier.
__device__ __forceinline__ void ring_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Scalar-base forms: lane l's source is base + off (base wave-uniform, in an
// SGPR pair; off a 32-bit lane offset), which saves the 64-bit address
// arithmetic of every load when the lane offsets are computed once per ring.
template <bool NT>
__device__ __forceinline__ void lds_dma16_so(const void* base, uint32_t off, uint32_t lds_base) {
    const uint64_t b = (uint64_t)(uintptr_t)base;
    const uint64_t sb = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
    if constexpr (NT)
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                     :
                     : "v"(off), "s"(sb), "s"(__builtin_amdgcn_readfirstlane(lds_base))
                     : "m0");
    else
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                     :
                     : "v"(off), "s"(sb), "s"(__builtin_amdgcn_readfirstlane(lds_base))
                     : "m0");
}
template <bool NT>
__device__ __forceinline__ void lds_dma4_so(const void* base, uint32_t off, uint32_t lds_base) {
    const uint64_t b = (uint64_t)(uintptr_t)base;
    const uint64_t sb = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
    if constexpr (NT)
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1 nt"
                     :
                     : "v"(off), "s"(sb), "s"(__builtin_amdgcn_readfirstlane(lds_base))
                     : "m0");
    else
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
                     :
                     : "v"(off), "s"(sb), "s"(__builtin_amdgcn_readfirstlane(lds_base))
                     : "m0");
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Run-time count: waits until at most n (clamped to [0, 63]) vector-memory
// operations of this wave are outstanding. A smaller n only waits longer. The
// count is an immediate of s_waitcnt, so n (wave-uniform: pass it through
// readfirstlane, or the branches become exec-masked vector compares) selects
// one of 64 instructions by a binary dispatch of six scalar branches (a
// linear chain cost ~560 cycles per call at the counts the streaming rings use).
template <int LO = 0, int HI = 63>
__device__ __forceinline__ void wait_vmcnt_le(int n) {
    if constexpr (LO == HI) {
        wait_vmcnt<LO>();
    } else {
        constexpr int MID = (LO + HI + 1) / 2;
        if (n >= MID) wait_vmcnt_le<MID, HI>(n);
        else wait_vmcnt_le<LO, MID - 1>(n);
    }
}

}  // namespace gsa
