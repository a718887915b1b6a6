// quotient.hpp -- the element quotient x / s of the FP8 quantizers.
//
// Every element of a group is encoded from the correctly rounded fp32
// quotient x / s, where s = amax / 448 is the group's fp32 scale.  A full IEEE
// division costs about eleven vector instructions; a group shares one s, so
// the kernels compute the correctly rounded reciprocal r = 1 / s once per group
// and then, per element, one product and one residual correction (Markstein's
// reciprocal-based division, using an exact FMA residual).
//
// This is only used when s >= 2^-64; groups with a smaller (or zero) scale take
// a plain IEEE division.  Below that bound an element whose quotient matters
// (|x / s| >= 2^-11) can itself be an fp32 subnormal, and the FMA residual is
// then no longer exact.  That the corrected quotient equals
// the IEEE quotient bit for bit on the whole input domain (every bf16 x with
// |x| <= amax, for every positive bf16 amax, with s = amax / 448) is checked
// exhaustively on the host; the functions here are plain C++ so the same code
// compiles for that check and for the GPU.
#pragma once

#include <math.h>

#if defined(__HIPCC__)
#define FP8_HD __host__ __device__
#else
#define FP8_HD
#endif

namespace fp8q {

// Scales at or above 2^-64 use the reciprocal path.
constexpr float kFastMinScale = 5.42101086242752217004e-20f;  // 2^-64

FP8_HD inline bool scale_has_fast_path(float s) { return s >= kFastMinScale; }

// x / s correctly rounded, given r = RN(1 / s) and s >= 2^-64.
FP8_HD inline float quotient(float x, float s, float r) {
    float q0 = x * r;
    float e = fmaf(-q0, s, x);  // exact residual x - q0 * s
    // s > 0, so the quotient has the sign of x; this keeps -0 / s == -0
    // (the FMA alone would return +0 there).
    return copysignf(fmaf(e, r, q0), x);
}

}  // namespace fp8q
