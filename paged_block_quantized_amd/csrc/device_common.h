// Device helpers shared by the HIP kernels of libpbq (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pbq {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Pool codes and fp16 rows that a call reads exactly once are loaded with
// the non-temporal cache policy (a plain 2 KiB-tile read reaches about 84 %
// of the HBM peak that way against 75 % with the default policy on
// MI355X); data that several work groups reread (the multi-query and
// shared-prefix passes) keeps the default.
#ifndef PBQ_NT_CODES
#define PBQ_NT_CODES 1
#endif

template <bool NT, class T>
__device__ __forceinline__ T load_once(const T* p) {
    if constexpr (NT && PBQ_NT_CODES) return __builtin_nontemporal_load(p);
    else return *p;
}

template <bool NT, class T>
__device__ __forceinline__ void store_once(T x, T* p) {
    if constexpr (NT && PBQ_NT_CODES) __builtin_nontemporal_store(x, p);
    else *p = x;
}

__device__ __forceinline__ float bits_to_f16f(uint16_t b) {
    return (float)__builtin_bit_cast(_Float16, b);
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
    // fptrunc rounds to nearest-even in the default mode
    return __builtin_bit_cast(uint16_t, (_Float16)x);
}

// max |x| over eight fp16 values, as the bit pattern of |x| (for finite
// values the order of |x| and of its bit pattern agree).  The vector is
// reinterpreted whole: element-wise bit casts of vector subscripts are not
// used because clang lowers __builtin_bit_cast(T, v[e]) to element 0.
__device__ __forceinline__ uint32_t absmax_bits_f16x8(f16x8 x) {
    const u32x4 w = __builtin_bit_cast(u32x4, x);
    uint32_t m = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t lo = w[k] & 0x7FFFu, hi = (w[k] >> 16) & 0x7FFFu;
        m = m > lo ? m : lo;
        m = m > hi ? m : hi;
    }
    return m;
}

// ---- cross-lane moves (DPP within rows of 16 lanes) -----------------------
// DPP control words for gfx9: quad_perm(p0,p1,p2,p3) = p0 | p1<<2 | p2<<4 |
// p3<<6; row_half_mirror = 0x141; row_ror:n = 0x120 + n.
enum : int {
    kDppQuadXor1 = 0xB1,  // quad_perm [1,0,3,2]
    kDppQuadXor2 = 0x4E,  // quad_perm [2,3,0,1]
    kDppHalfMirror = 0x141,
    kDppRowRor8 = 0x128,
};

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float shfl_xor_f(float x, int m) {
    return __shfl_xor(x, m, 64);
}

// Sum over the 2^k lanes of an aligned group (k = 1..6) with result in every
// lane of the group.
template <int GROUP>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(GROUP == 2 || GROUP == 4 || GROUP == 8 || GROUP == 16 || GROUP == 32 || GROUP == 64, "group");
    x += dpp<kDppQuadXor1>(x);
    if constexpr (GROUP >= 4) x += dpp<kDppQuadXor2>(x);
    if constexpr (GROUP >= 8) x += dpp<kDppHalfMirror>(x);
    if constexpr (GROUP >= 16) x += dpp<kDppRowRor8>(x);
    if constexpr (GROUP >= 32) x += shfl_xor_f(x, 16);
    if constexpr (GROUP >= 64) x += shfl_xor_f(x, 32);
    return x;
}

// Sum over lanes that share (lane % STRIDE), STRIDE a power of two < 64.
template <int STRIDE>
__device__ __forceinline__ float strided_sum(float x) {
#pragma unroll
    for (int m = STRIDE; m < 64; m <<= 1) {
        if (m == 8) x += dpp<kDppRowRor8>(x);
        else x += shfl_xor_f(x, m);
    }
    return x;
}

template <int STRIDE>
__device__ __forceinline__ float strided_max(float x) {
#pragma unroll
    for (int m = STRIDE; m < 64; m <<= 1) {
        if (m == 8) x = fmaxf(x, dpp<kDppRowRor8>(x));
        else x = fmaxf(x, shfl_xor_f(x, m));
    }
    return x;
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}

// Wave-wide reductions with a wave-uniform (scalar) result: DPP within each
// row of 16 lanes, then the four row results read with readlane.
__device__ __forceinline__ uint32_t wave_max_u32_uniform(uint32_t x) {
    x = max(x, dpp_u<kDppQuadXor1>(x));
    x = max(x, dpp_u<kDppQuadXor2>(x));
    x = max(x, dpp_u<kDppHalfMirror>(x));
    x = max(x, dpp_u<kDppRowRor8>(x));
    const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)x, 0);
    const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)x, 16);
    const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)x, 32);
    const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)x, 48);
    return max(max(a, b), max(c, d));
}

__device__ __forceinline__ float wave_max_uniform(float x) {
    x = fmaxf(x, dpp<kDppQuadXor1>(x));
    x = fmaxf(x, dpp<kDppQuadXor2>(x));
    x = fmaxf(x, dpp<kDppHalfMirror>(x));
    x = fmaxf(x, dpp<kDppRowRor8>(x));
    const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 0));
    const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 16));
    const float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 32));
    const float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 48));
    return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

__device__ __forceinline__ float wave_min_uniform(float x) {
    x = fminf(x, dpp<kDppQuadXor1>(x));
    x = fminf(x, dpp<kDppQuadXor2>(x));
    x = fminf(x, dpp<kDppHalfMirror>(x));
    x = fminf(x, dpp<kDppRowRor8>(x));
    const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 0));
    const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 16));
    const float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 32));
    const float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 48));
    return fminf(fminf(a, b), fminf(c, d));
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
    return x;
}

__device__ __forceinline__ float wave_min(float x) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) x = fminf(x, __shfl_xor(x, m, 64));
    return x;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
        uint32_t y = (uint32_t)__shfl_xor((int)x, m, 64);
        x = x > y ? x : y;
    }
    return x;
}

__device__ __forceinline__ int readlane(int x, int lane) {
    return __builtin_amdgcn_readlane(x, lane);
}

__device__ __forceinline__ float readlane(float x, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

}  // namespace pbq
