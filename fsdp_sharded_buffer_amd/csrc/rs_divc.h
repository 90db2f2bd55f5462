// Correctly rounded division by a per-call constant, shared by the kernels
// and the test-only probe that checks it on every input it can receive.
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

}  // namespace rs
