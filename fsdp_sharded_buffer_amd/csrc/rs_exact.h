// Correctly rounded fp32 operations cheaper than the compiled IEEE
// sequences in the 8-bit AdamW step: division by a per-call constant and
// the square root.  Shared by the kernels and the test-only probe that
// checks each on every fp32 input.
#pragma once

#include <hip/hip_runtime.h>

namespace rs {

// The constants c this division accepts (checked on the host): normal and
// within [2^-16, 2^16].  Then for every x = sqrtf(y) of an fp32 y the
// quotient x / c is zero, infinite, NaN or a normal number, and so is every
// intermediate below.
inline bool div_by_const_ok(float c) { return c >= 0x1p-16f && c <= 0x1p16f; }

// x / c rounded to nearest even, given r = RN(1/c) (the host's IEEE fp32
// division).  q0 = fl(x * r) lies within one ulp of x / c; the residual
// e = x - q0 * c is exact in one FMA; and fl(q0 + e * r) is then the
// correctly rounded quotient (Markstein's theorem for FMA division with a
// correctly rounded reciprocal).  Where e is zero or NaN (x = +-0, +-Inf or
// NaN, or q0 already exact) q0 is the IEEE quotient itself, sign of zero
// included.  Three floating-point operations and a select, against about ten
// for the general IEEE division.
__device__ __forceinline__ float div_by_const(float x, float c, float r) {
  const float q0 = x * r;
  const float e = __builtin_fmaf(-q0, c, x);
  const float q1 = __builtin_fmaf(e, r, q0);
  return __builtin_fabsf(e) > 0.0f ? q1 : q0;
}

// sqrt(v) rounded to nearest even.  On [2^-96, +Inf) the hardware square
// root s is within one ulp of sqrt(v), so the result is s or a neighbour
// d = s - ulp, u = s + ulp.  The exact residuals v - d*s and v - u*s (one
// FMA each, exact there) decide: sqrt(v) lies below the midpoint of d and s
// exactly when v <= d*s, and above the midpoint of s and u exactly when
// v > u*s, because the squared midpoints exceed d*s and u*s by a quarter of
// a squared ulp, finer than the spacing of v near s*s.  Any other v (zero,
// subnormal, tiny, negative, Inf, NaN) takes the compiled IEEE square root,
// on a branch the wave skips when none of its lanes needs it.
__device__ __forceinline__ float sqrt_rn(float v) {
  const float s = __builtin_amdgcn_sqrtf(v);
  const float d = __uint_as_float(__float_as_uint(s) - 1u);
  const float u = __uint_as_float(__float_as_uint(s) + 1u);
  float r = __builtin_fmaf(-d, s, v) <= 0.0f ? d : s;
  r = __builtin_fmaf(-u, s, v) > 0.0f ? u : r;
  if (__builtin_expect(__float_as_uint(v) - 0x0f800000u >= 0x7f800000u - 0x0f800000u, 0))
    r = __builtin_sqrtf(v);
  return r;
}

}  // namespace rs
