// Plain 128-bit streaming kernels: the practical HBM ceiling of each
// read:write mix the grouped operations use (include/hbm_ceiling.h).
// Measurement support only; nothing here is part of the hot path.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "hbm_ceiling.h"

#pragma clang fp contract(off)

namespace {

constexpr int kThreads = 256;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ u32x4 ld(const u32x4* p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(p);
  else
    return *p;
}

template <bool NT>
__device__ __forceinline__ void st(u32x4* p, u32x4 v) {
  if constexpr (NT)
    __builtin_nontemporal_store(v, p);
  else
    *p = v;
}

__device__ __forceinline__ uint32_t axpby(uint32_t y, uint32_t x) {
  const float u = 0.5f * __uint_as_float(y);
  const float w = 2.0f * __uint_as_float(x);
  return __float_as_uint(u + w);
}

__device__ __forceinline__ u32x4 axpby4(u32x4 y, u32x4 x) {
  return u32x4{axpby(y.x, x.x), axpby(y.y, x.y), axpby(y.z, x.z), axpby(y.w, x.w)};
}

// The block of units workgroup b covers.  The hardware hands workgroup b to
// XCD b % 8; order 1 gives XCD x block x of every round of 8 runs of 128
// blocks (a last partial round keeps the hardware order), order 2 one
// contiguous run of about G/8 blocks per XCD, order 0 the hardware order.
__device__ __forceinline__ int64_t block_of(int order) {
  const int64_t b = blockIdx.x, G = gridDim.x;
  if (order == 2) {
    const int64_t q = G >> 3, r = G & 7, x = b & 7, k = b >> 3;
    return x * q + (x < r ? x : r) + k;
  }
  if (order == 1) {
    const int64_t round = b >> 10;
    if ((round + 1) << 10 <= G) {
      const int64_t within = b & 1023;
      return (round << 10) + ((within & 7) << 7) + (within >> 3);
    }
  }
  return b;
}

// Workgroup b covers the units of block block_of(order): [B*256*VEC,
// (B+1)*256*VEC); lane i takes units i, i+256, ...  A unit is one 16-byte
// vector of the widest stream.  All loads of a lane are issued before its
// stores.
template <int KIND, int VEC, bool NT>
__global__ __launch_bounds__(kThreads) void stream_kernel(const u32x4* __restrict__ x,
                                                          u32x4* __restrict__ y,
                                                          u32x4* __restrict__ z, int order) {
  const int64_t u0 = block_of(order) * kThreads * VEC + threadIdx.x;
  if constexpr (KIND == HC_READ) {
    u32x4 r[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) r[v] = ld<NT>(x + u0 + v * kThreads);
    uint32_t acc = 0;
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc ^= r[v].x ^ r[v].y ^ r[v].z ^ r[v].w;
    for (int o = 32; o >= 1; o >>= 1) acc ^= __shfl_xor(acc, o);
    __shared__ uint32_t w[kThreads / 64];
    if (threadIdx.x % 64 == 0) w[threadIdx.x / 64] = acc;
    __syncthreads();
    if (threadIdx.x == 0)
      reinterpret_cast<uint32_t*>(y)[blockIdx.x] = w[0] ^ w[1] ^ w[2] ^ w[3];
  } else if constexpr (KIND == HC_WRITE) {
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int v = 0; v < VEC; ++v) st<NT>(y + u0 + v * kThreads, zero);
  } else if constexpr (KIND == HC_COPY) {
    u32x4 r[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) r[v] = ld<NT>(x + u0 + v * kThreads);
#pragma unroll
    for (int v = 0; v < VEC; ++v) st<NT>(y + u0 + v * kThreads, r[v]);
  } else if constexpr (KIND == HC_AXPBY_INPLACE || KIND == HC_AXPBY) {
    u32x4 ry[VEC], rx[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      ry[v] = ld<NT>(y + u0 + v * kThreads);
      rx[v] = ld<NT>(x + u0 + v * kThreads);
    }
    u32x4* out = KIND == HC_AXPBY ? z : y;
#pragma unroll
    for (int v = 0; v < VEC; ++v) st<NT>(out + u0 + v * kThreads, axpby4(ry[v], rx[v]));
  } else if constexpr (KIND == HC_F32_TO_BF16 + 16) {
    // narrow: unit = 4 fp32 in (one vector), 4 bf16 out (8 bytes)
    u32x4 r[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) r[v] = ld<NT>(x + u0 + v * kThreads);
    uint2* out = reinterpret_cast<uint2*>(y);
#pragma unroll
    for (int v = 0; v < VEC; ++v)
      out[u0 + v * kThreads] = uint2{(r[v].x >> 16) | (r[v].y & 0xffff0000u),
                                     (r[v].z >> 16) | (r[v].w & 0xffff0000u)};
  } else if constexpr (KIND == HC_F32_TO_U8 + 16) {
    // narrow: unit = 4 fp32 in (one vector), 4 bytes out
    u32x4 r[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) r[v] = ld<NT>(x + u0 + v * kThreads);
    uint32_t* out = reinterpret_cast<uint32_t*>(y);
#pragma unroll
    for (int v = 0; v < VEC; ++v)
      out[u0 + v * kThreads] = (r[v].x & 0xffu) | ((r[v].y & 0xffu) << 8) |
                               ((r[v].z & 0xffu) << 16) | (r[v].w << 24);
  } else if constexpr (KIND == HC_U8_TO_F32 + 16) {
    // narrow: unit = 4 bytes in, 4 fp32 out (one vector)
    uint32_t r[VEC];
    const uint32_t* in = reinterpret_cast<const uint32_t*>(x);
#pragma unroll
    for (int v = 0; v < VEC; ++v) r[v] = in[u0 + v * kThreads];
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      const uint32_t w = r[v];
      st<NT>(y + u0 + v * kThreads, u32x4{w & 0xffu, (w >> 8) & 0xffu, (w >> 16) & 0xffu, w >> 24});
    }
  } else if constexpr (KIND == HC_F32_TO_BF16) {
    // unit = 8 fp32 in (two vectors), 8 bf16 out (one vector)
    u32x4 a[VEC], b[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      a[v] = ld<NT>(x + 2 * (u0 + v * kThreads));
      b[v] = ld<NT>(x + 2 * (u0 + v * kThreads) + 1);
    }
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      const u32x4 o = {(a[v].x >> 16) | (a[v].y & 0xffff0000u), (a[v].z >> 16) | (a[v].w & 0xffff0000u),
                       (b[v].x >> 16) | (b[v].y & 0xffff0000u), (b[v].z >> 16) | (b[v].w & 0xffff0000u)};
      st<NT>(y + u0 + v * kThreads, o);
    }
  } else if constexpr (KIND == HC_F32_TO_U8) {
    // unit = 16 fp32 in (four vectors), 16 bytes out
    u32x4 r[VEC][4];
#pragma unroll
    for (int v = 0; v < VEC; ++v)
#pragma unroll
      for (int j = 0; j < 4; ++j) r[v][j] = ld<NT>(x + 4 * (u0 + v * kThreads) + j);
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      u32x4 o;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        o[j] = (r[v][j].x & 0xffu) | ((r[v][j].y & 0xffu) << 8) | ((r[v][j].z & 0xffu) << 16) |
               (r[v][j].w << 24);
      st<NT>(y + u0 + v * kThreads, o);
    }
  } else if constexpr (KIND == HC_U8_TO_F32) {  // unit = 16 bytes in, 16 fp32 out (four vectors)
    u32x4 r[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) r[v] = ld<NT>(x + u0 + v * kThreads);
#pragma unroll
    for (int v = 0; v < VEC; ++v)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w = r[v][j];
        st<NT>(y + 4 * (u0 + v * kThreads) + j,
               u32x4{w & 0xffu, (w >> 8) & 0xffu, (w >> 16) & 0xffu, w >> 24});
      }
  }
}

// fp32 (or u8) elements per unit of each kind (narrow variants: kind + 16)
constexpr int elems_per_unit(int kind) {
  return kind == HC_F32_TO_BF16 ? 8 : (kind == HC_F32_TO_U8 || kind == HC_U8_TO_F32) ? 16 : 4;
}

template <int KIND, int VEC>
hipError_t run(const void* x, void* y, void* z, int64_t n, int nt, int order, hipStream_t s) {
  const int64_t units = n / elems_per_unit(KIND);
  const dim3 grid(static_cast<unsigned>(units / (int64_t(kThreads) * VEC)));
  const u32x4* xx = static_cast<const u32x4*>(x);
  u32x4* yy = static_cast<u32x4*>(y);
  u32x4* zz = static_cast<u32x4*>(z);
  void* args[] = {&xx, &yy, &zz, &order};
  const void* k = nt ? reinterpret_cast<const void*>(&stream_kernel<KIND, VEC, true>)
                     : reinterpret_cast<const void*>(&stream_kernel<KIND, VEC, false>);
  return hipLaunchKernel(k, grid, dim3(kThreads), args, 0, s);  // this launch's own status
}

template <int KIND>
hipError_t run_vec(const void* x, void* y, void* z, int64_t n, int vec, int nt, int order,
                   hipStream_t s) {
  switch (vec) {
    case 1: return run<KIND, 1>(x, y, z, n, nt, order, s);
    case 2: return run<KIND, 2>(x, y, z, n, nt, order, s);
    case 4: return run<KIND, 4>(x, y, z, n, nt, order, s);
    default: return run<KIND, 8>(x, y, z, n, nt, order, s);
  }
}

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" int hc_stream(int kind, const void* x, void* y, void* z, int64_t n, int vec, int nt,
                         void* stream) {
  const int order = (kind & HC_XCD_ONE) ? 2 : (kind & HC_XCD_RUNS) ? 1 : 0;
  if ((kind & HC_XCD_ONE) && (kind & HC_XCD_RUNS)) return -1;
  kind &= ~(HC_XCD_RUNS | HC_XCD_ONE);
  const bool narrow = kind >= HC_NARROW;
  if (narrow) kind -= HC_NARROW;
  if (kind < HC_READ || kind > HC_U8_TO_F32 || n <= 0 || (vec != 1 && vec != 2 && vec != 4 && vec != 8) ||
      (narrow && kind < HC_F32_TO_BF16))
    return -1;
  if (n % (int64_t(4096) * vec) || n / (int64_t(4096) * vec) > (int64_t(1) << 31) / kThreads) return -1;
  const bool needs_x = kind != HC_WRITE, needs_z = kind == HC_AXPBY;
  if (!y || !al16(y) || (needs_x && (!x || !al16(x))) || (needs_z && (!z || !al16(z)))) return -1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (kind) {
    case HC_READ: e = run_vec<HC_READ>(x, y, z, n, vec, nt, order, s); break;
    case HC_WRITE: e = run_vec<HC_WRITE>(x, y, z, n, vec, nt, order, s); break;
    case HC_COPY: e = run_vec<HC_COPY>(x, y, z, n, vec, nt, order, s); break;
    case HC_AXPBY_INPLACE: e = run_vec<HC_AXPBY_INPLACE>(x, y, z, n, vec, nt, order, s); break;
    case HC_AXPBY: e = run_vec<HC_AXPBY>(x, y, z, n, vec, nt, order, s); break;
    case HC_F32_TO_BF16:
      e = narrow ? run_vec<HC_F32_TO_BF16 + 16>(x, y, z, n, vec, nt, order, s)
                 : run_vec<HC_F32_TO_BF16>(x, y, z, n, vec, nt, order, s);
      break;
    case HC_F32_TO_U8:
      e = narrow ? run_vec<HC_F32_TO_U8 + 16>(x, y, z, n, vec, nt, order, s)
                 : run_vec<HC_F32_TO_U8>(x, y, z, n, vec, nt, order, s);
      break;
    default:
      e = narrow ? run_vec<HC_U8_TO_F32 + 16>(x, y, z, n, vec, nt, order, s)
                 : run_vec<HC_U8_TO_F32>(x, y, z, n, vec, nt, order, s);
      break;
  }
  return e == hipSuccess ? 0 : -6;
}
