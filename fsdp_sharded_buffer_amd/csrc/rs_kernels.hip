// Grouped, memory-bound kernels over a RaggedShard flat buffer, for gfx950.
//
// Every kernel is driven by the layout's device tables: one launch covers
// all fragments of a rank range, whatever tensors they belong to
// (veScale-FSDP: Flexible and High-Performance FSDP at Scale, "DBuffer":
// group-level add/scale/zero/copy instead of one kernel per tensor).  The
// work unit is a chunk of at most chunk_elems positions that never crosses
// a tensor, padding or rank boundary, so work per workgroup stays even when
// fragments are ragged.  Nothing here is a contraction: the kernels are HBM
// bound and use 128-bit global accesses (global_load/store_dwordx4) wherever
// both sides of a run are 16-byte aligned, element accesses otherwise.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>

#include "rs_internal.h"

#pragma clang fp contract(off)

namespace rs {
namespace {

constexpr int kThreads = 256;
constexpr int kWave = 64;

// ------------------------------------------------------------------ casts

// fp32 -> bf16 bits, round to nearest even; NaN -> quiet NaN, same sign.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// FP8 E4M3FN (OCP): saturating round to nearest even; NaN -> 0x7F.
__device__ __forceinline__ uint32_t e4m3_encode(float q) {
  const uint32_t u = __float_as_uint(q);
  const uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu;
  if (a > 0x43e00000u) a = 0x43e00000u;  // |q| > 448 (or Inf) -> 448
  uint32_t code;
  if (a < 0x3c800000u) {                 // |q| < 2^-6: multiples of 2^-9
    code = uint32_t(__builtin_rintf(__uint_as_float(a) * 512.0f));
  } else {                               // keep 3 mantissa bits, RNE, rebias 127 -> 7
    a += 0x7ffffu + ((a >> 20) & 1u);
    code = (a >> 20) - (120u << 3);
  }
  return code | sign;
}

// INT8: round half to even, clip to [-127, 127]; NaN -> 0.
__device__ __forceinline__ uint32_t int8_encode(float q) {
  if (q != q) return 0u;
  float r = __builtin_rintf(q);
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return uint32_t(int32_t(r)) & 0xffu;
}

// ------------------------------------------------------- 8-element vectors

// Element kinds: 0 = fp32, 1 = bf16.
template <int K> struct Pack8;
template <> struct Pack8<0> { float4 a, b; };
template <> struct Pack8<1> { uint4 a; };

template <int K> constexpr int esize() { return K == 0 ? 4 : 2; }

template <int K> __device__ __forceinline__ Pack8<K> ld8(const void* p, int64_t i);
template <> __device__ __forceinline__ Pack8<0> ld8<0>(const void* p, int64_t i) {
  const float4* q = reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
  return Pack8<0>{q[0], q[1]};
}
template <> __device__ __forceinline__ Pack8<1> ld8<1>(const void* p, int64_t i) {
  return Pack8<1>{*reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p) + i)};
}

template <int K> __device__ __forceinline__ void st8(void* p, int64_t i, const Pack8<K>& v);
template <> __device__ __forceinline__ void st8<0>(void* p, int64_t i, const Pack8<0>& v) {
  float4* q = reinterpret_cast<float4*>(static_cast<float*>(p) + i);
  q[0] = v.a;
  q[1] = v.b;
}
template <> __device__ __forceinline__ void st8<1>(void* p, int64_t i, const Pack8<1>& v) {
  *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p) + i) = v.a;
}

__device__ __forceinline__ uint32_t pk2(float lo, float hi) {
  return bf16_rne(lo) | (bf16_rne(hi) << 16);
}

template <int SK, int DK> struct Conv;
template <int K> struct Conv<K, K> {
  static __device__ __forceinline__ Pack8<K> run(const Pack8<K>& v) { return v; }
};
template <> struct Conv<0, 1> {
  static __device__ __forceinline__ Pack8<1> run(const Pack8<0>& v) {
    return Pack8<1>{make_uint4(pk2(v.a.x, v.a.y), pk2(v.a.z, v.a.w), pk2(v.b.x, v.b.y),
                               pk2(v.b.z, v.b.w))};
  }
};
template <> struct Conv<1, 0> {
  static __device__ __forceinline__ Pack8<0> run(const Pack8<1>& v) {
    const uint4 u = v.a;
    return Pack8<0>{make_float4(bf16_to_f32(u.x & 0xffffu), bf16_to_f32(u.x >> 16),
                                bf16_to_f32(u.y & 0xffffu), bf16_to_f32(u.y >> 16)),
                    make_float4(bf16_to_f32(u.z & 0xffffu), bf16_to_f32(u.z >> 16),
                                bf16_to_f32(u.w & 0xffffu), bf16_to_f32(u.w >> 16))};
  }
};

// one element through fp32 (or raw bits when the kinds match)
template <int SK, int DK>
__device__ __forceinline__ void copy1(const void* s, void* d, int64_t i) {
  if constexpr (SK == DK) {
    if constexpr (SK == 0)
      static_cast<float*>(d)[i] = static_cast<const float*>(s)[i];
    else
      static_cast<uint16_t*>(d)[i] = static_cast<const uint16_t*>(s)[i];
  } else if constexpr (SK == 0) {
    static_cast<uint16_t*>(d)[i] = uint16_t(bf16_rne(static_cast<const float*>(s)[i]));
  } else {
    static_cast<float*>(d)[i] = bf16_to_f32(static_cast<const uint16_t*>(s)[i]);
  }
}

__device__ __forceinline__ bool aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

constexpr int kUnroll = 4;

// Convert-copy n elements; the workgroup's lanes stride over 8-element
// vectors, kUnroll vectors in flight per lane.
template <int SK, int DK>
__device__ __forceinline__ void copy_run(const void* src, void* dst, int n) {
  const int nv = (aligned16(src) && aligned16(dst)) ? n / 8 : 0;
  int v = threadIdx.x;
  for (; v + (kUnroll - 1) * kThreads < nv; v += kUnroll * kThreads) {
    Pack8<SK> r[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) r[u] = ld8<SK>(src, int64_t(v + u * kThreads) * 8);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      st8<DK>(dst, int64_t(v + u * kThreads) * 8, Conv<SK, DK>::run(r[u]));
  }
  for (; v < nv; v += kThreads) st8<DK>(dst, int64_t(v) * 8, Conv<SK, DK>::run(ld8<SK>(src, int64_t(v) * 8)));
  for (int i = nv * 8 + threadIdx.x; i < n; i += kThreads) copy1<SK, DK>(src, dst, i);
}

template <int K>
__device__ __forceinline__ void zero_run(void* dst, int n) {
  const int nv = aligned16(dst) ? n * esize<K>() / 16 : 0;
  uint4* d = static_cast<uint4*>(dst);
  for (int v = threadIdx.x; v < nv; v += kThreads) d[v] = make_uint4(0, 0, 0, 0);
  const int done = nv * 16 / esize<K>();
  for (int i = done + threadIdx.x; i < n; i += kThreads) {
    if constexpr (K == 0)
      static_cast<float*>(dst)[i] = 0.0f;
    else
      static_cast<uint16_t*>(dst)[i] = 0;
  }
}

// ------------------------------------------------------------ pack/unpack

template <int SK, int DK>
__global__ __launch_bounds__(kThreads) void pack_kernel(const ChunkDesc* __restrict__ chunks,
                                                        int64_t c0,
                                                        const void* const* __restrict__ src,
                                                        void* __restrict__ buf) {
  const ChunkDesc c = chunks[c0 + blockIdx.x];
  char* d = static_cast<char*>(buf) + c.buf_off * esize<DK>();
  if (c.tensor < 0) {
    zero_run<DK>(d, c.len);
    return;
  }
  const char* s = static_cast<const char*>(src[c.tensor]) + c.ten_off * esize<SK>();
  copy_run<SK, DK>(s, d, c.len);
}

template <int SK, int DK>
__global__ __launch_bounds__(kThreads) void unpack_kernel(const ChunkDesc* __restrict__ chunks,
                                                          int64_t c0,
                                                          const void* __restrict__ buf,
                                                          void* const* __restrict__ dst) {
  const ChunkDesc c = chunks[c0 + blockIdx.x];
  if (c.tensor < 0) return;
  const char* s = static_cast<const char*>(buf) + c.buf_off * esize<SK>();
  char* d = static_cast<char*>(dst[c.tensor]) + c.ten_off * esize<DK>();
  copy_run<SK, DK>(s, d, c.len);
}

// -------------------------------------------------------------- scale/add

__device__ __forceinline__ float axpby(float a, float y, float b, float x) {
  // separate roundings: fl(fl(a*y) + fl(b*x)); contraction is off in this file
  const float u = a * y;
  const float w = b * x;
  return u + w;
}

__device__ __forceinline__ bool finite(float v) {
  return (__float_as_uint(v) & 0x7f800000u) != 0x7f800000u;
}

// Marks found_inf[rank] from lane 0 of every wave that saw a bad value.
__device__ __forceinline__ void flag_rank(bool bad, uint32_t* found_inf, int rank) {
  if (found_inf && __any(bad) && (threadIdx.x % kWave) == 0) found_inf[rank] = 1u;
}

template <int XK>
__global__ __launch_bounds__(kThreads) void scale_add_kernel(
    const ChunkDesc* __restrict__ chunks, int64_t c0, float* __restrict__ y,
    const void* __restrict__ x, float alpha, float beta, const uint8_t* __restrict__ mask,
    uint32_t* __restrict__ found_inf) {
  const ChunkDesc c = chunks[c0 + blockIdx.x];
  if (c.tensor < 0) return;
  if (mask && !mask[c.tensor]) return;
  float* yp = y + c.buf_off;
  const char* xp = static_cast<const char*>(x) + c.buf_off * esize<XK>();
  const int n = c.len;
  bool bad = false;
  const int nv = (aligned16(yp) && aligned16(xp)) ? n / 8 : 0;
  int v = threadIdx.x;
  for (; v + (kUnroll - 1) * kThreads < nv; v += kUnroll * kThreads) {
    Pack8<0> ry[kUnroll];
    Pack8<0> rx[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = int64_t(v + u * kThreads) * 8;
      ry[u] = ld8<0>(yp, i);
      rx[u] = Conv<XK, 0>::run(ld8<XK>(xp, i));
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      Pack8<0> o;
      o.a.x = axpby(alpha, ry[u].a.x, beta, rx[u].a.x);
      o.a.y = axpby(alpha, ry[u].a.y, beta, rx[u].a.y);
      o.a.z = axpby(alpha, ry[u].a.z, beta, rx[u].a.z);
      o.a.w = axpby(alpha, ry[u].a.w, beta, rx[u].a.w);
      o.b.x = axpby(alpha, ry[u].b.x, beta, rx[u].b.x);
      o.b.y = axpby(alpha, ry[u].b.y, beta, rx[u].b.y);
      o.b.z = axpby(alpha, ry[u].b.z, beta, rx[u].b.z);
      o.b.w = axpby(alpha, ry[u].b.w, beta, rx[u].b.w);
      bad |= !(finite(o.a.x) && finite(o.a.y) && finite(o.a.z) && finite(o.a.w) &&
               finite(o.b.x) && finite(o.b.y) && finite(o.b.z) && finite(o.b.w));
      st8<0>(yp, int64_t(v + u * kThreads) * 8, o);
    }
  }
  for (; v < nv; v += kThreads) {
    const int64_t i = int64_t(v) * 8;
    const Pack8<0> ry = ld8<0>(yp, i);
    const Pack8<0> rx = Conv<XK, 0>::run(ld8<XK>(xp, i));
    Pack8<0> o;
    o.a.x = axpby(alpha, ry.a.x, beta, rx.a.x);
    o.a.y = axpby(alpha, ry.a.y, beta, rx.a.y);
    o.a.z = axpby(alpha, ry.a.z, beta, rx.a.z);
    o.a.w = axpby(alpha, ry.a.w, beta, rx.a.w);
    o.b.x = axpby(alpha, ry.b.x, beta, rx.b.x);
    o.b.y = axpby(alpha, ry.b.y, beta, rx.b.y);
    o.b.z = axpby(alpha, ry.b.z, beta, rx.b.z);
    o.b.w = axpby(alpha, ry.b.w, beta, rx.b.w);
    bad |= !(finite(o.a.x) && finite(o.a.y) && finite(o.a.z) && finite(o.a.w) &&
             finite(o.b.x) && finite(o.b.y) && finite(o.b.z) && finite(o.b.w));
    st8<0>(yp, i, o);
  }
  for (int i = nv * 8 + threadIdx.x; i < n; i += kThreads) {
    float xv;
    if constexpr (XK == 0)
      xv = reinterpret_cast<const float*>(xp)[i];
    else
      xv = bf16_to_f32(reinterpret_cast<const uint16_t*>(xp)[i]);
    const float o = axpby(alpha, yp[i], beta, xv);
    bad |= !finite(o);
    yp[i] = o;
  }
  flag_rank(bad, found_inf, c.rank);
}

// ------------------------------------------------------------------- zero

template <int K>
__global__ __launch_bounds__(kThreads) void zero_kernel(const ChunkDesc* __restrict__ chunks,
                                                        int64_t c0, void* __restrict__ y,
                                                        const uint8_t* __restrict__ mask) {
  const ChunkDesc c = chunks[c0 + blockIdx.x];
  if (mask && (c.tensor < 0 || !mask[c.tensor])) return;
  zero_run<K>(static_cast<char*>(y) + c.buf_off * esize<K>(), c.len);
}

// ----------------------------------------------------------------- sqnorm

// Fixed-order sum over the workgroup: butterfly inside each wave, then the
// four wave sums in wave order.  Result valid in thread 0.
__device__ __forceinline__ double block_sum(double v, double* lds) {
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  const int w = threadIdx.x / kWave;
  if (threadIdx.x % kWave == 0) lds[w] = v;
  __syncthreads();
  double s = 0.0;
  if (threadIdx.x == 0) {
    s = lds[0];
    for (int i = 1; i < kThreads / kWave; ++i) s += lds[i];
  }
  __syncthreads();
  return s;
}

__device__ __forceinline__ double sq(float v) {
  const double d = double(v);
  return d * d;
}

// Per chunk: fp64 sum of squares into part[chunk].
__global__ __launch_bounds__(kThreads) void sqnorm_partial_kernel(
    const ChunkDesc* __restrict__ chunks, int64_t c0, const float* __restrict__ x,
    double* __restrict__ part, uint32_t* __restrict__ found_inf) {
  __shared__ double lds[kThreads / kWave];
  const int64_t ci = c0 + blockIdx.x;
  const ChunkDesc c = chunks[ci];
  if (c.tensor < 0) return;
  const float* xp = x + c.buf_off;
  const int n = c.len;
  double acc = 0.0;
  bool bad = false;
  const int nv = aligned16(xp) ? n / 4 : 0;
  const float4* x4 = reinterpret_cast<const float4*>(xp);
  int v = threadIdx.x;
  constexpr int U = 8;
  for (; v + (U - 1) * kThreads < nv; v += U * kThreads) {
    float4 r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) r[u] = x4[v + u * kThreads];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      acc += sq(r[u].x);
      acc += sq(r[u].y);
      acc += sq(r[u].z);
      acc += sq(r[u].w);
      bad |= !(finite(r[u].x) && finite(r[u].y) && finite(r[u].z) && finite(r[u].w));
    }
  }
  for (; v < nv; v += kThreads) {
    const float4 r = x4[v];
    acc += sq(r.x);
    acc += sq(r.y);
    acc += sq(r.z);
    acc += sq(r.w);
    bad |= !(finite(r.x) && finite(r.y) && finite(r.z) && finite(r.w));
  }
  for (int i = nv * 4 + threadIdx.x; i < n; i += kThreads) {
    acc += sq(xp[i]);
    bad |= !finite(xp[i]);
  }
  flag_rank(bad, found_inf, c.rank);
  const double s = block_sum(acc, lds);
  if (threadIdx.x == 0) part[ci] = s;
}

// Per tensor: fragment sums in rank order, each the fixed-order sum of its
// chunk partials; writes partial[k*n + t] for every k of the range.
__global__ __launch_bounds__(kThreads) void sqnorm_combine_kernel(
    const TensorDesc* __restrict__ tensors, const FragDesc* __restrict__ frags,
    const double* __restrict__ part, int32_t n, int32_t k0, int32_t k1, double* __restrict__ sq_out,
    double* __restrict__ partial) {
  __shared__ double lds[kThreads / kWave];
  const int t = blockIdx.x;
  const TensorDesc td = tensors[t];
  double total = 0.0;
  for (int k = k0; k < k1; ++k) {
    const bool has = td.frag_begin >= 0 && k >= td.rank_lo && k < td.rank_hi;
    double s = 0.0;
    if (has) {  // uniform across the workgroup
      const FragDesc fd = frags[td.frag_begin + (k - td.rank_lo)];
      double a = 0.0;
      for (int i = fd.chunk_begin + threadIdx.x; i < fd.chunk_end; i += kThreads) a += part[i];
      s = block_sum(a, lds);
      if (threadIdx.x == 0) total += s;
    }
    if (partial && threadIdx.x == 0) partial[int64_t(k) * n + t] = s;
  }
  if (threadIdx.x == 0) sq_out[t] = total;
}

// ------------------------------------------------------------------ quant

// Each workgroup takes `count` consecutive tiles; tile j of the item is
// handled by lanes [j*team, (j+1)*team).  A lane keeps its (at most 64)
// elements in registers between the absmax and the encode pass, so x is
// read once.
template <int FMT>
__global__ __launch_bounds__(kThreads) void quant_kernel(const QuantWork* __restrict__ work,
                                                         int64_t w0,
                                                         const TileDesc* __restrict__ tiles,
                                                         const float* __restrict__ x,
                                                         uint8_t* __restrict__ codes,
                                                         float* __restrict__ scales,
                                                         int vec_ok) {
  __shared__ uint32_t lds[kThreads / kWave];
  const QuantWork w = work[w0 + blockIdx.x];
  const bool vec = w.vec && vec_ok;
  const int team = w.team;
  const int slot = threadIdx.x / team;
  const int lane = threadIdx.x % team;
  const bool active = slot < w.count;
  const TileDesc td = tiles[w.tile_begin + (active ? slot : 0)];
  float v[64];
  uint32_t amax = 0;
  const float* base = x + td.buf_off;
  if (vec) {
    const int c4 = td.cols >> 2;
    const int nf = active ? td.rows * c4 : 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int f = lane + i * team;
      float4 q = make_float4(0.f, 0.f, 0.f, 0.f);
      if (f < nf) {
        const int r = f / c4;
        const int cc = f - r * c4;
        q = *reinterpret_cast<const float4*>(base + int64_t(r) * td.ld + cc * 4);
      }
      v[4 * i + 0] = q.x;
      v[4 * i + 1] = q.y;
      v[4 * i + 2] = q.z;
      v[4 * i + 3] = q.w;
      amax = max(amax, __float_as_uint(q.x) & 0x7fffffffu);
      amax = max(amax, __float_as_uint(q.y) & 0x7fffffffu);
      amax = max(amax, __float_as_uint(q.z) & 0x7fffffffu);
      amax = max(amax, __float_as_uint(q.w) & 0x7fffffffu);
    }
  } else {
    const int ne = active ? td.rows * td.cols : 0;
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      const int e = lane + i * team;
      float q = 0.f;
      if (e < ne) {
        const int r = e / td.cols;
        const int cc = e - r * td.cols;
        q = base[int64_t(r) * td.ld + cc];
      }
      v[i] = q;
      amax = max(amax, __float_as_uint(q) & 0x7fffffffu);
    }
  }
  // absmax of the tile as the max of |x| bit patterns: NaN patterns sort
  // above +Inf, so a NaN anywhere yields a NaN amax
  const int red = team < kWave ? team : kWave;
  for (int o = red / 2; o >= 1; o >>= 1) amax = max(amax, uint32_t(__shfl_xor(int(amax), o)));
  if (team > kWave) {  // uniform
    if (threadIdx.x % kWave == 0) lds[threadIdx.x / kWave] = amax;
    __syncthreads();
    const int first = (threadIdx.x / team) * (team / kWave);
    uint32_t a = lds[first];
    for (int i = 1; i < team / kWave; ++i) a = max(a, lds[first + i]);
    amax = a;
  }
  if (!active) return;
  constexpr float Q = FMT == RS_Q_FP8_E4M3 ? 448.0f : 127.0f;
  const float famax = __uint_as_float(amax);
  float scale = famax / Q;
  const bool nan_tile = amax > 0x7f800000u;
  if (nan_tile) scale = __uint_as_float(0x7fc00000u);
  if (lane == 0) scales[td.scale_idx] = scale;
  const bool zero_tile = scale == 0.0f;
  uint8_t* cbase = codes + td.buf_off;
  auto enc = [&](float val) -> uint32_t {
    if (zero_tile) return 0u;
    if (nan_tile) return FMT == RS_Q_FP8_E4M3 ? 0x7fu : 0u;
    const float q = val / scale;
    return FMT == RS_Q_FP8_E4M3 ? e4m3_encode(q) : int8_encode(q);
  };
  if (vec) {
    const int c4 = td.cols >> 2;
    const int nf = td.rows * c4;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int f = lane + i * team;
      if (f < nf) {
        const int r = f / c4;
        const int cc = f - r * c4;
        const uint32_t word = enc(v[4 * i]) | (enc(v[4 * i + 1]) << 8) |
                              (enc(v[4 * i + 2]) << 16) | (enc(v[4 * i + 3]) << 24);
        *reinterpret_cast<uint32_t*>(cbase + int64_t(r) * td.ld + cc * 4) = word;
      }
    }
  } else {
    const int ne = td.rows * td.cols;
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      const int e = lane + i * team;
      if (e < ne) {
        const int r = e / td.cols;
        const int cc = e - r * td.cols;
        cbase[int64_t(r) * td.ld + cc] = uint8_t(enc(v[i]));
      }
    }
  }
}

// ------------------------------------------------------------- host glue

template <typename T>
const T* table(const rs_layout* L, size_t off) {
  return reinterpret_cast<const T*>(static_cast<const char*>(L->dev) + off);
}

rs_status check_common(const rs_layout* L, int32_t k0, int32_t k1, const char* fn) {
  if (!L) return fail(RS_ERR_INVALID_ARG, std::string(fn) + ": null layout");
  if (!L->dev) return fail(RS_ERR_STATE, std::string(fn) + ": layout not uploaded");
  if (k0 < 0 || k1 > L->m || k0 >= k1)
    return fail(RS_ERR_RANGE, std::string(fn) + ": rank range [" + std::to_string(k0) + ", " +
                                  std::to_string(k1) + ") outside [0, " + std::to_string(L->m) + ")");
  return RS_OK;
}

rs_status check_ptr(const void* p, size_t align, const char* fn, const char* what) {
  if (!p) return fail(RS_ERR_INVALID_ARG, std::string(fn) + ": null " + what);
  if (reinterpret_cast<uintptr_t>(p) % align)
    return fail(RS_ERR_ALIGN, std::string(fn) + ": " + what + " not aligned to its element size");
  return RS_OK;
}

rs_status after_launch(const char* fn) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(RS_ERR_HIP, std::string(fn) + ": " + hipGetErrorString(e));
  clear_error();
  return RS_OK;
}

bool float_kind(rs_dtype d) { return d == RS_F32 || d == RS_BF16; }

#define RS_TRY(x)                 \
  do {                            \
    const rs_status _st = (x);    \
    if (_st != RS_OK) return _st; \
  } while (0)

}  // namespace
}  // namespace rs

using namespace rs;

extern "C" rs_status rs_pack(const rs_layout* L, const void* const* src, rs_dtype src_dt, void* buf,
                             rs_dtype buf_dt, int32_t k0, int32_t k1, void* stream) {
  const char* fn = "rs_pack";
  RS_TRY(check_common(L, k0, k1, fn));
  if (!float_kind(src_dt) || !float_kind(buf_dt))
    return fail(RS_ERR_DTYPE, "rs_pack: dtypes must be RS_F32 or RS_BF16");
  RS_TRY(check_ptr(src, 8, fn, "src table"));
  RS_TRY(check_ptr(buf, buf_dt == RS_F32 ? 4 : 2, fn, "buf"));
  const int64_t c0 = L->rank_chunk[k0], nc = L->rank_chunk[k1] - c0;
  if (nc == 0) return RS_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const ChunkDesc* ch = table<ChunkDesc>(L, L->off_chunks);
  const dim3 g(static_cast<unsigned>(nc)), b(kThreads);
  if (src_dt == RS_F32 && buf_dt == RS_BF16)
    hipLaunchKernelGGL((pack_kernel<0, 1>), g, b, 0, s, ch, c0, src, buf);
  else if (src_dt == RS_F32 && buf_dt == RS_F32)
    hipLaunchKernelGGL((pack_kernel<0, 0>), g, b, 0, s, ch, c0, src, buf);
  else if (src_dt == RS_BF16 && buf_dt == RS_BF16)
    hipLaunchKernelGGL((pack_kernel<1, 1>), g, b, 0, s, ch, c0, src, buf);
  else
    hipLaunchKernelGGL((pack_kernel<1, 0>), g, b, 0, s, ch, c0, src, buf);
  return after_launch(fn);
}

extern "C" rs_status rs_unpack(const rs_layout* L, const void* buf, rs_dtype buf_dt,
                               void* const* dst, rs_dtype dst_dt, int32_t k0, int32_t k1,
                               void* stream) {
  const char* fn = "rs_unpack";
  RS_TRY(check_common(L, k0, k1, fn));
  if (!float_kind(dst_dt) || !float_kind(buf_dt))
    return fail(RS_ERR_DTYPE, "rs_unpack: dtypes must be RS_F32 or RS_BF16");
  RS_TRY(check_ptr(dst, 8, fn, "dst table"));
  RS_TRY(check_ptr(buf, buf_dt == RS_F32 ? 4 : 2, fn, "buf"));
  const int64_t c0 = L->rank_chunk[k0], nc = L->rank_chunk[k1] - c0;
  if (nc == 0) return RS_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const ChunkDesc* ch = table<ChunkDesc>(L, L->off_chunks);
  const dim3 g(static_cast<unsigned>(nc)), b(kThreads);
  if (buf_dt == RS_BF16 && dst_dt == RS_BF16)
    hipLaunchKernelGGL((unpack_kernel<1, 1>), g, b, 0, s, ch, c0, buf, dst);
  else if (buf_dt == RS_BF16 && dst_dt == RS_F32)
    hipLaunchKernelGGL((unpack_kernel<1, 0>), g, b, 0, s, ch, c0, buf, dst);
  else if (buf_dt == RS_F32 && dst_dt == RS_F32)
    hipLaunchKernelGGL((unpack_kernel<0, 0>), g, b, 0, s, ch, c0, buf, dst);
  else
    hipLaunchKernelGGL((unpack_kernel<0, 1>), g, b, 0, s, ch, c0, buf, dst);
  return after_launch(fn);
}

extern "C" rs_status rs_group_scale_add(const rs_layout* L, float* y, const void* x,
                                        rs_dtype x_dt, float alpha, float beta,
                                        const uint8_t* tensor_mask, uint32_t* found_inf,
                                        int32_t k0, int32_t k1, void* stream) {
  const char* fn = "rs_group_scale_add";
  RS_TRY(check_common(L, k0, k1, fn));
  if (!float_kind(x_dt)) return fail(RS_ERR_DTYPE, "rs_group_scale_add: x must be RS_F32 or RS_BF16");
  RS_TRY(check_ptr(y, 4, fn, "y"));
  RS_TRY(check_ptr(x, x_dt == RS_F32 ? 4 : 2, fn, "x"));
  if (found_inf) RS_TRY(check_ptr(found_inf, 4, fn, "found_inf"));
  const int64_t c0 = L->rank_chunk[k0], nc = L->rank_chunk[k1] - c0;
  if (nc == 0) return RS_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const ChunkDesc* ch = table<ChunkDesc>(L, L->off_chunks);
  const dim3 g(static_cast<unsigned>(nc)), b(kThreads);
  if (x_dt == RS_F32)
    hipLaunchKernelGGL((scale_add_kernel<0>), g, b, 0, s, ch, c0, y, x, alpha, beta, tensor_mask,
                       found_inf);
  else
    hipLaunchKernelGGL((scale_add_kernel<1>), g, b, 0, s, ch, c0, y, x, alpha, beta, tensor_mask,
                       found_inf);
  return after_launch(fn);
}

extern "C" rs_status rs_group_zero(const rs_layout* L, void* y, rs_dtype dt,
                                   const uint8_t* tensor_mask, int32_t k0, int32_t k1,
                                   void* stream) {
  const char* fn = "rs_group_zero";
  RS_TRY(check_common(L, k0, k1, fn));
  if (!float_kind(dt)) return fail(RS_ERR_DTYPE, "rs_group_zero: dt must be RS_F32 or RS_BF16");
  RS_TRY(check_ptr(y, dt == RS_F32 ? 4 : 2, fn, "y"));
  const int64_t c0 = L->rank_chunk[k0], nc = L->rank_chunk[k1] - c0;
  if (nc == 0) return RS_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const ChunkDesc* ch = table<ChunkDesc>(L, L->off_chunks);
  const dim3 g(static_cast<unsigned>(nc)), b(kThreads);
  if (dt == RS_F32)
    hipLaunchKernelGGL((zero_kernel<0>), g, b, 0, s, ch, c0, y, tensor_mask);
  else
    hipLaunchKernelGGL((zero_kernel<1>), g, b, 0, s, ch, c0, y, tensor_mask);
  return after_launch(fn);
}

extern "C" rs_status rs_ragged_sqnorm(const rs_layout* L, const float* x, double* sq_out,
                                      double* partial, uint32_t* found_inf, void* ws, int32_t k0,
                                      int32_t k1, void* stream) {
  const char* fn = "rs_ragged_sqnorm";
  RS_TRY(check_common(L, k0, k1, fn));
  RS_TRY(check_ptr(x, 4, fn, "x"));
  RS_TRY(check_ptr(sq_out, 8, fn, "sq"));
  RS_TRY(check_ptr(ws, 8, fn, "ws"));
  if (partial) RS_TRY(check_ptr(partial, 8, fn, "partial"));
  if (found_inf) RS_TRY(check_ptr(found_inf, 4, fn, "found_inf"));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t c0 = L->rank_chunk[k0], nc = L->rank_chunk[k1] - c0;
  double* part = static_cast<double*>(ws);
  if (nc > 0)
    hipLaunchKernelGGL(sqnorm_partial_kernel, dim3(unsigned(nc)), dim3(kThreads), 0, s,
                       table<ChunkDesc>(L, L->off_chunks), c0, x, part, found_inf);
  hipLaunchKernelGGL(sqnorm_combine_kernel, dim3(unsigned(L->n)), dim3(kThreads), 0, s,
                     table<TensorDesc>(L, L->off_tensors), table<FragDesc>(L, L->off_frags), part,
                     L->n, k0, k1, sq_out, partial);
  return after_launch(fn);
}

extern "C" rs_status rs_block_quant(const rs_layout* L, const float* x, rs_qfmt fmt,
                                    uint8_t* codes, float* scales, int32_t k0, int32_t k1,
                                    void* stream) {
  const char* fn = "rs_block_quant";
  RS_TRY(check_common(L, k0, k1, fn));
  if (fmt != RS_Q_FP8_E4M3 && fmt != RS_Q_INT8)
    return fail(RS_ERR_DTYPE, "rs_block_quant: fmt must be RS_Q_FP8_E4M3 or RS_Q_INT8");
  RS_TRY(check_ptr(x, 4, fn, "x"));
  RS_TRY(check_ptr(codes, 1, fn, "codes"));
  RS_TRY(check_ptr(scales, 4, fn, "scales"));
  // the 16-byte path needs x 16-byte aligned and codes 4-byte aligned
  const int vec_ok = (reinterpret_cast<uintptr_t>(x) % 16 == 0 &&
                      reinterpret_cast<uintptr_t>(codes) % 4 == 0) ? 1 : 0;
  const int64_t w0 = L->rank_work[k0], nw = L->rank_work[k1] - w0;
  if (nw == 0) return RS_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 g(static_cast<unsigned>(nw)), b(kThreads);
  if (fmt == RS_Q_FP8_E4M3)
    hipLaunchKernelGGL((quant_kernel<RS_Q_FP8_E4M3>), g, b, 0, s,
                       table<QuantWork>(L, L->off_work), w0, table<TileDesc>(L, L->off_tiles), x,
                       codes, scales, vec_ok);
  else
    hipLaunchKernelGGL((quant_kernel<RS_Q_INT8>), g, b, 0, s, table<QuantWork>(L, L->off_work),
                       w0, table<TileDesc>(L, L->off_tiles), x, codes, scales, vec_ok);
  return after_launch(fn);
}
