// Test-only probes of device arithmetic the kernels rely on; not part of
// librs.so.
//  * gfx950's packed fp32 -> OCP E4M3 conversion (the block quantisation
//    fast path), applied to consecutive fp32 bit patterns four at a time
//    exactly as the kernel packs a word, so a test can compare every input
//    of the fast path's domain with the CPU oracle;
//  * fp32 division and square root as the kernels compile them (the exact
//    quantisation path and the AdamW steps rely on both being correctly
//    rounded);
//  * the division by a per-call constant and the square root of the 8-bit
//    AdamW step (rs_exact.h), on every fp32 input, against the IEEE results.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "rs_exact.h"

namespace {

__global__ void probe_kernel(uint32_t first, int64_t n, uint32_t sign, uint8_t* out) {
  const int64_t i = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) * 4;
  if (i >= n) return;
  float q[4];
  for (int j = 0; j < 4; ++j) {
    const int64_t k = i + j < n ? i + j : n - 1;
    q[j] = __uint_as_float((first + uint32_t(k)) | sign);
  }
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], w, true);
  for (int j = 0; j < 4; ++j)
    if (i + j < n) out[i + j] = uint8_t(uint32_t(w) >> (8 * j));
}

__global__ void divsqrt_kernel(const float* x, const float* y, int64_t n, float* q, float* r) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  q[i] = x[i] / y[i];
  r[i] = sqrtf(x[i]);
}

// For every fp32 y with bits first + i, i < n: rs::div_by_const(sqrtf(y),
// c, r) against the IEEE quotient sqrtf(y) / c.  Results whose bits differ
// (NaN results compare by class) are counted in *bad and the smallest such
// y pattern is kept in *first_bad.
__global__ void divc_kernel(uint32_t first, int64_t n, float c, float r, unsigned long long* bad,
                            uint32_t* first_bad) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
    const uint32_t bits = first + uint32_t(i);
    const float x = sqrtf(__uint_as_float(bits));
    const float a = rs::div_by_const(x, c, r);
    const float q = x / c;
    const bool same = (a != a && q != q) || __float_as_uint(a) == __float_as_uint(q);
    if (!same) {
      atomicAdd(bad, 1ull);
      atomicMin(first_bad, bits);
    }
  }
}

// For every fp32 v with bits first + i, i < n: rs::sqrt_rn(v) against the
// IEEE sqrtf(v), counted and located as above.
__global__ void sqrt_kernel(uint32_t first, int64_t n, unsigned long long* bad,
                            uint32_t* first_bad) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
    const uint32_t bits = first + uint32_t(i);
    const float v = __uint_as_float(bits);
    const float a = rs::sqrt_rn(v);
    const float q = sqrtf(v);
    const bool same = (a != a && q != q) || __float_as_uint(a) == __float_as_uint(q);
    if (!same) {
      atomicAdd(bad, 1ull);
      atomicMin(first_bad, bits);
    }
  }
}

}  // namespace

// The same count for rs::sqrt_rn against sqrtf over [first, first + n).
extern "C" int probe_sqrt(uint32_t first, int64_t n, unsigned long long* bad, uint32_t* first_bad,
                          void* stream) {
  if (n <= 0 || n > (int64_t(1) << 32) || !bad || !first_bad) return -1;
  hipLaunchKernelGGL(sqrt_kernel, dim3(8192), dim3(256), 0, static_cast<hipStream_t>(stream), first,
                     n, bad, first_bad);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

// Counts, over the fp32 patterns [first, first + n) (n <= 2^32), the y
// where the constant-divisor quotient of sqrtf(y) by c differs from IEEE's;
// bad and first_bad are device words the caller set to 0 and 0xffffffff.
extern "C" int probe_divc(uint32_t first, int64_t n, float c, float r, unsigned long long* bad,
                          uint32_t* first_bad, void* stream) {
  if (n <= 0 || n > (int64_t(1) << 32) || !bad || !first_bad) return -1;
  hipLaunchKernelGGL(divc_kernel, dim3(8192), dim3(256), 0, static_cast<hipStream_t>(stream), first,
                     n, c, r, bad, first_bad);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

// q[i] = x[i] / y[i] and r[i] = sqrtf(x[i]) for i < n (device arrays).
extern "C" int probe_div_sqrt(const float* x, const float* y, int64_t n, float* q, float* r,
                              void* stream) {
  if (n <= 0 || !x || !y || !q || !r) return -1;
  const unsigned grid = unsigned((n + 255) / 256);
  hipLaunchKernelGGL(divsqrt_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream), x,
                     y, n, q, r);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

// out[k] = E4M3 code of the fp32 with bits (first + k) | sign, k < n.
extern "C" int probe_e4m3_hw(uint32_t first, int64_t n, uint32_t sign, uint8_t* out, void* stream) {
  if (n <= 0 || !out) return -1;
  const int64_t threads = (n + 3) / 4;
  const unsigned grid = unsigned((threads + 255) / 256);
  hipLaunchKernelGGL(probe_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream), first,
                     n, sign, out);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}
