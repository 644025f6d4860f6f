// Device-side helpers for the gfx950 (CDNA4) kernels of libpagedkv.
// Wave64 cross-lane reductions use DPP row rotations inside each 16-lane row and
// the gfx950 permlane16/permlane32 swaps across rows, so no LDS round trip is
// needed for a wave-wide max or sum.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));
// Native vector types (first-class LLVM values, kept in registers even when loop-carried).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// A finite stand-in for "no score seen yet": exp2(x - kNoMax) never overflows for
// real scores, and exp2(-inf - m) is 0 for every finite running max m.
constexpr float kNoMax = -1.0e30f;

__device__ __forceinline__ uint32_t f2u(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ float u2f(uint32_t x) { return __builtin_bit_cast(float, x); }

// DPP row rotate right by N (1..15) inside each 16-lane row.
template <int N>
__device__ __forceinline__ float row_ror(float x) {
    static_assert(N >= 1 && N <= 15, "row_ror range");
    return u2f(__builtin_amdgcn_update_dpp(0u, f2u(x), 0x120 + N, 0xF, 0xF, false));
}

// Combine a value across the two 32-lane halves: every lane gets op(x_lo, x_hi)
// of its own half-position. permlane32_swap returns (lanes 0-31 duplicated,
// lanes 32-63 duplicated) when both operands are x.
__device__ __forceinline__ float swap32_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(f2u(x), f2u(x), false, false);
    return fmaxf(u2f(r[0]), u2f(r[1]));
}
__device__ __forceinline__ float swap32_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(f2u(x), f2u(x), false, false);
    return u2f(r[0]) + u2f(r[1]);
}
// Same across neighbouring 16-lane rows (0<->1, 2<->3).
__device__ __forceinline__ float swap16_max(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(f2u(x), f2u(x), false, false);
    return fmaxf(u2f(r[0]), u2f(r[1]));
}
__device__ __forceinline__ float swap16_sum(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(f2u(x), f2u(x), false, false);
    return u2f(r[0]) + u2f(r[1]);
}

__device__ __forceinline__ float row16_max(float x) {
    x = fmaxf(x, row_ror<8>(x));
    x = fmaxf(x, row_ror<4>(x));
    x = fmaxf(x, row_ror<2>(x));
    x = fmaxf(x, row_ror<1>(x));
    return x;
}
__device__ __forceinline__ float row16_sum(float x) {
    x += row_ror<8>(x);
    x += row_ror<4>(x);
    x += row_ror<2>(x);
    x += row_ror<1>(x);
    return x;
}

// All-reduce over the 64 lanes of a wave; every lane receives the result.
__device__ __forceinline__ float wave_max(float x) { return swap32_max(swap16_max(row16_max(x))); }
__device__ __forceinline__ float wave_sum(float x) { return swap32_sum(swap16_sum(row16_sum(x))); }

// Sum over lanes that differ only in the "row group" bits of a wave laid out as
// lane = group * (64 / R) + chunk, for R groups of 64/R lanes (R in {2, 4, 8}).
template <int R>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(R == 2 || R == 4 || R == 8, "row groups");
    if constexpr (R == 8) x += row_ror<8>(x);
    if constexpr (R >= 4) x = swap16_sum(x);
    return swap32_sum(x);
}

// Reads through the constant address space: the compiler then uses scalar
// (SMEM) loads for wave-uniform addresses such as block-table entries and q.
template <typename T>
using const_ptr = const __attribute__((address_space(4))) T*;
template <typename T>
__device__ __forceinline__ const_ptr<T> as_const(const T* p) {
    return (const_ptr<T>)p;
}

// A wave-uniform global pointer pinned to scalar registers.  Loads of
// (pinned + 32-bit per-lane offset) then use the scalar-base addressing form
// instead of a 64-bit per-lane address that the compiler would otherwise build by
// re-associating the sum.
template <typename T>
using global_ptr = const __attribute__((address_space(1))) T*;
__device__ __forceinline__ global_ptr<char> pin_uniform(const char* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (global_ptr<char>)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// dot of two bf16 pairs plus an fp32 addend (v_dot2 on gfx950).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return u2f(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return u2f(w & 0xFFFF0000u); }

// Round-to-nearest-even float -> bf16 bits (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}
// Two floats -> packed bf16 pair (lo in bits 0-15), one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((float2_t){lo, hi}, bf16x2_t));
}

// Byte permutes pairing the same half of two dwords: (a.lo, b.lo) and (a.hi, b.hi).
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) {
    return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) {
    return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

}  // namespace pkv
