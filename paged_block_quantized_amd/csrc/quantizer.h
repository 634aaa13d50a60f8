// Integer codes of one tile's elements under a nonzero fp16 scale, exact
// round-half-even without a per-element division.  Host and device: the
// store kernels use it on the GPU, and a CPU sweep checks it against the
// codec's definition for every fp16 scale.
//
// The codec (web pages cited by site and section): yunthe.com "KV-cache
// quantization and PagedAttention", "quantization principle" -- Q(x) =
// clamp(round(x / scale + zero_point), 0, 2^bits - 1); tbr8.org
// "PagedAttention + block-wise quantization against mobile OOM", §4
// store_kv -- INT8 codes of x / scale.  Reading: round half to even on the
// exact quotient by the stored fp16 scale.
#pragma once

#include <hip/hip_runtime.h>

namespace pbq {

// Codes of one tile with scale s (an fp16 value; s == 0 for an all-zero
// tile).  exact(): round-half-even of x / s + zp for fp16 x, without a
// division: n = rint(x * (1/s)) is within one of the answer, the remainder
// x - n*s is exact in one FMA, and comparing |rem| with s/2 (also exact)
// decides the nearest integer and the tie.  fast(): rint(x * (1/s) + off),
// clamped, as a float.  For fp16 x and s the quotient x / s is either exactly
// halfway between two integers or at least 2^-12 away from every halfway
// point (x / s - k - 1/2 is a multiple of 2^min(a+1, b) over 2 S 2^b, for
// x = X 2^a, s = S 2^b, S < 2^11), while the fused x * (1/s) + off is within
// 2^-15 of x / s + off for results up to 256 (1/s and the FMA each round
// once), so fast() agrees with exact() everywhere except on exact ties,
// which it flags (remainder of exactly s/2) for the caller to redo with
// exact().
struct Quantizer {
    float s, rcp, half_s;
    __host__ __device__ __forceinline__ explicit Quantizer(float sc)
        : s(sc), rcp(sc > 0.f ? 1.0f / sc : 0.f), half_s(sc > 0.f ? 0.5f * sc : -1.f) {}
    __host__ __device__ __forceinline__ int exact(float x, int zp) const {
        const float n = __builtin_rintf(x * rcp);
        const float rem = __builtin_fmaf(-n, s, x);
        const float arem = __builtin_fabsf(rem);
        const int dir = rem > 0.f ? 1 : -1;
        int q = (int)n + zp;
        q += arem > half_s ? dir : 0;                     // n was one off
        q += (arem == half_s && (q & 1)) ? dir : 0;       // exact tie -> even
        return q;
    }
    __host__ __device__ __forceinline__ float fast(float x, float off, float lo, float hi, bool& tie) const {
        const float u = __builtin_fminf(__builtin_fmaxf(__builtin_rintf(__builtin_fmaf(x, rcp, off)), lo), hi);
        const float rem = __builtin_fmaf(-(u - off), s, x);   // exact
        tie |= __builtin_fabsf(rem) == half_s;
        return u;
    }
};

}  // namespace pbq
