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

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <mutex>
#include <string>
#include <tuple>
#include <utility>

#include "rs_internal.h"
#include "rs_exact.h"

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

// Tuning knobs (compile-time; the defaults are the measured best on MI355X).
//   RS_UNROLL        8-element vectors in flight per lane (copies, scale/add)
//   RS_*_NT          per operation: nontemporal hint on streaming accesses;
//                    it helps the pure streams (copies, the norm read,
//                    quantisation input) and the in-place ones (scale/add,
//                    the fp32 optimizers), whose lanes take one 16-byte
//                    vector each; it hurts the zero
//   RS_SCALE_SPLIT   workgroups per chunk of scale/add (1024 elements each
//                    at the default chunk size)
//   RS_XCD_REMAP_MIN pack, unpack, scale/add and unmasked-zero ranges of at
//                    least this many elements group their chunks by XCD (0:
//                    never)
//   RS_XCD_RUN       chunks per XCD run for pack, unpack and scale/add, a
//                    power of two (the unmasked zero takes one run per XCD)
//   RS_QUANT_F,      256-lane sub-blocks per quantisation work item of wide
//   RS_QUANT_F_SMALL tiles, for launches of at least / fewer than
//                    RS_QUANT_SMALL_ITEMS work items (narrow tiles: one)
//   RS_SQNORM_FINE_BELOW  the norm reads fine chunks when the range has
//                    fewer coarse chunks than this (too few workgroups)
//   RS_UNPACK_SHORT_LANES  lanes per unpack workgroup on launches shorter
//                    than RS_XCD_REMAP_MIN elements (one rank's share):
//                    128 is 2-4% faster there; pack keeps 256 (128: 3% slower)
//   RS_SQNORM_FINE_LANES  lanes per norm workgroup over fine chunks (128:
//                    all of a 70B-layer rank's 3584 chunks resident at once)
//   RS_FILL_BYTES    bytes per workgroup of the unmasked zero: one 16-byte
//                    store per lane, as many short workgroups write fastest
//   RS_OPT_NT        nontemporal loads and stores of the streams the AdamW
//                    / SGD steps read and write in place (p, m, v, momentum)
//   RS_OPT_G_NT      nontemporal loads of the gradient (read once) in the
//                    AdamW / SGD steps, beside their read-modify-write streams
//   RS_ADAMW_SPLIT,  workgroups per chunk of the AdamW / SGD steps
//   RS_SGD_SPLIT
//   RS_DEQ_SPLIT     row bands (workgroups) per dequantised tile, where every
//                    tile of the class and range has that many rows
//   RS_DEQ_LDS       stage a tile's codes in LDS before decoding
//   RS_DEQ_XCD_RUN,  dequantisation takes runs of RS_DEQ_XCD_RUN workgroups
//   RS_DEQ_XCD_MIN_COLS  per XCD on long ranges whose tiles mostly belong
//                    to tensors of at least RS_DEQ_XCD_MIN_COLS columns
//                    (a 70B-layer group: 12% faster; narrower groups lose)
//   RS_ADAM8_F       256-lane sub-blocks per 8-bit Adam work item of wide tiles
//   RS_ADAM8_DIVC    8-bit Adam divides by sqrt(bc2) with div_by_const when
//                    the constant allows it
//   RS_ADAM8_SQRT    8-bit Adam takes sqrt(v') with sqrt_rn
//   RS_NT_STORE_BELOW  launches of quantisation, dequantisation and the
//                    unmasked zero that write fewer bytes than this (one
//                    rank's share, say) use nontemporal stores: a short
//                    launch then leaves less to write back from L2 at its
//                    end; long launches store faster without the hint
//   RS_QUANT_NT_WIDE_FROM  ... except quantisation of wide tiles over ranges
//                    of at least this many positions (codes written), which
//                    is 4-10% faster with the hint at 4 GiB of fp32 and
//                    3-7% slower at 1 GiB
#ifndef RS_UNROLL
#define RS_UNROLL 2
#endif
#ifndef RS_PACK_NT
#define RS_PACK_NT 1
#endif
#ifndef RS_SCALE_NT
#define RS_SCALE_NT 1
#endif
#ifndef RS_SCALE_SPLIT
#define RS_SCALE_SPLIT 2
#endif
#ifndef RS_SQNORM_NT
#define RS_SQNORM_NT 1
#endif
#ifndef RS_ZERO_NT
#define RS_ZERO_NT 0
#endif
#ifndef RS_QUANT_NT
#define RS_QUANT_NT 1
#endif
#ifndef RS_QUANT_F
#define RS_QUANT_F 2
#endif
#ifndef RS_QUANT_F_SMALL
#define RS_QUANT_F_SMALL 4
#endif
#ifndef RS_QUANT_SMALL_ITEMS
#define RS_QUANT_SMALL_ITEMS 1024
#endif
#ifndef RS_XCD_REMAP_MIN
#define RS_XCD_REMAP_MIN (int64_t(1) << 26)
#endif
#ifndef RS_XCD_RUN
#define RS_XCD_RUN 128
#endif
#ifndef RS_ADAM8_DIVC
#define RS_ADAM8_DIVC 1
#endif
#ifndef RS_ADAM8_SQRT
#define RS_ADAM8_SQRT 1
#endif
#ifndef RS_SQNORM_FINE_BELOW
#define RS_SQNORM_FINE_BELOW 256
#endif
#ifndef RS_FILL_BYTES
#define RS_FILL_BYTES 4096
#endif
#ifndef RS_OPT_G_NT
#define RS_OPT_G_NT 1
#endif
#ifndef RS_OPT_NT
#define RS_OPT_NT 1
#endif
#ifndef RS_ADAMW_SPLIT
#define RS_ADAMW_SPLIT 8
#endif
#ifndef RS_SGD_SPLIT
#define RS_SGD_SPLIT 4
#endif
#ifndef RS_DEQ_SPLIT
#define RS_DEQ_SPLIT 4
#endif
#ifndef RS_DEQ_LDS
#define RS_DEQ_LDS 1
#endif
#ifndef RS_ADAM8_F
#define RS_ADAM8_F 2
#endif
#ifndef RS_ADAM8_NT
#define RS_ADAM8_NT 1
#endif
#ifndef RS_NT_STORE_BELOW
#define RS_NT_STORE_BELOW (192ll << 20)
#endif
#ifndef RS_SQNORM_FINE_LANES
#define RS_SQNORM_FINE_LANES 128
#endif
#ifndef RS_UNPACK_SHORT_LANES
#define RS_UNPACK_SHORT_LANES 128
#endif
#ifndef RS_DEQ_XCD_RUN
#define RS_DEQ_XCD_RUN 16
#endif
#ifndef RS_QUANT_NT_WIDE_FROM
#define RS_QUANT_NT_WIDE_FROM (512ll << 20)
#endif
#ifndef RS_DEQ_XCD_MIN_COLS
#define RS_DEQ_XCD_MIN_COLS 8192
#endif


typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// one 128-bit global load / store (global_load_dwordx4 / global_store_dwordx4)
template <bool NT>
__device__ __forceinline__ u32x4 ld16(const void* p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(static_cast<const u32x4*>(p));
  else
    return *static_cast<const u32x4*>(p);
}

template <bool NT>
__device__ __forceinline__ void st16(void* p, u32x4 v) {
  if constexpr (NT)
    __builtin_nontemporal_store(v, static_cast<u32x4*>(p));
  else
    *static_cast<u32x4*>(p) = v;
}

__device__ __forceinline__ float f32(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t u32(float f) { return __float_as_uint(f); }

// Element kinds: 0 = fp32, 1 = bf16.  Eight elements as raw bits.
template <int K> struct Pack8;
template <> struct Pack8<0> { u32x4 a, b; };
template <> struct Pack8<1> { u32x4 a; };

template <int K> constexpr int esize() { return K == 0 ? 4 : 2; }

template <int K, bool NT>
__device__ __forceinline__ Pack8<K> ld8(const void* p, int64_t i) {
  if constexpr (K == 0) {
    const float* q = static_cast<const float*>(p) + i;
    return Pack8<0>{ld16<NT>(q), ld16<NT>(q + 4)};
  } else {
    return Pack8<1>{ld16<NT>(static_cast<const uint16_t*>(p) + i)};
  }
}

template <int K, bool NT>
__device__ __forceinline__ void st8(void* p, int64_t i, const Pack8<K>& v) {
  if constexpr (K == 0) {
    float* q = static_cast<float*>(p) + i;
    st16<NT>(q, v.a);
    st16<NT>(q + 4, v.b);
  } else {
    st16<NT>(static_cast<uint16_t*>(p) + i, v.a);
  }
}

__device__ __forceinline__ uint32_t pk2(uint32_t lo, uint32_t hi) {
  return bf16_rne(f32(lo)) | (bf16_rne(f32(hi)) << 16);
}

template <int SK, int DK> struct Conv;
template <int K> struct Conv<K, K> {
  static __device__ __forceinline__ Pack8<K> run(const Pack8<K>& v) { return v; }
};
template <> struct Conv<0, 1> {
  static __device__ __forceinline__ Pack8<1> run(const Pack8<0>& v) {
    u32x4 o;
    o.x = pk2(v.a.x, v.a.y);
    o.y = pk2(v.a.z, v.a.w);
    o.z = pk2(v.b.x, v.b.y);
    o.w = pk2(v.b.z, v.b.w);
    return Pack8<1>{o};
  }
};
template <> struct Conv<1, 0> {
  static __device__ __forceinline__ Pack8<0> run(const Pack8<1>& v) {
    const u32x4 u = v.a;
    u32x4 a, b;
    a.x = u.x << 16;
    a.y = u.x & 0xffff0000u;
    a.z = u.y << 16;
    a.w = u.y & 0xffff0000u;
    b.x = u.z << 16;
    b.y = u.z & 0xffff0000u;
    b.z = u.w << 16;
    b.w = u.w & 0xffff0000u;
    return Pack8<0>{a, b};
  }
};

// one element through fp32 (or raw bits when the kinds match)
template <int SK, int DK>
__device__ __forceinline__ void copy1(const void* s, void* d, int64_t i) {
  if constexpr (SK == DK) {
    if constexpr (SK == 0)
      static_cast<uint32_t*>(d)[i] = static_cast<const uint32_t*>(s)[i];
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

constexpr int kUnroll = RS_UNROLL;

// Convert-copy n elements; the workgroup's lanes stride over 8-element
// vectors.  Each pass issues the loads of kUnroll vectors per lane (the
// last pass predicated) before any of their stores.
template <int SK, int DK, bool NT, int LANES = kThreads>
__device__ __forceinline__ void copy_run(const void* src, void* dst, int n) {
  const int nv = (aligned16(src) && aligned16(dst)) ? n / 8 : 0;
  for (int b = threadIdx.x; b < nv; b += kUnroll * LANES) {
    Pack8<SK> r[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (b + u * LANES < nv) r[u] = ld8<SK, NT>(src, int64_t(b + u * LANES) * 8);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (b + u * LANES < nv)
        st8<DK, NT>(dst, int64_t(b + u * LANES) * 8, Conv<SK, DK>::run(r[u]));
  }
  for (int i = nv * 8 + threadIdx.x; i < n; i += LANES) copy1<SK, DK>(src, dst, i);
}

template <int K, bool NT, int LANES = kThreads>
__device__ __forceinline__ void zero_run(void* dst, int64_t n) {
  const int64_t nv = aligned16(dst) ? n * esize<K>() / 16 : 0;
  char* d = static_cast<char*>(dst);
  const u32x4 z = {0u, 0u, 0u, 0u};
  for (int64_t v = threadIdx.x; v < nv; v += LANES) st16<NT>(d + v * 16, z);
  const int64_t done = nv * 16 / esize<K>();
  for (int64_t i = done + threadIdx.x; i < n; i += LANES) {
    if constexpr (K == 0)
      static_cast<float*>(dst)[i] = 0.0f;
    else
      static_cast<uint16_t*>(dst)[i] = 0;
  }
}

// ------------------------------------------------------------ pack/unpack
//
// Chunk kernels take the chunk range [c0, c0 + nc); workgroup b handles
// chunk b (one workgroup per chunk measured fastest on MI355X: fewer,
// longer-lived workgroups or consecutive chunk runs per workgroup were
// slower), striding by the grid if the grid is ever smaller than nc.

// How a launch's workgroups map onto its items.  The hardware hands
// workgroup b to XCD b % 8.  kXcdRuns: in rounds of 8 runs of 2^shift
// consecutive items, XCD x takes run x of each round (a last partial round
// keeps the hardware order); kXcdOneRun: each XCD takes one contiguous run of
// about G/8 items; kXcdNone: the hardware order.  Shifts and masks only: the
// mapping runs once at the start of every (short-lived) workgroup.
enum { kXcdNone = 0, kXcdRuns = 1, kXcdOneRun = 2 };
struct XcdOrder {
  int32_t mode, shift;
};

// The first item of workgroup b of G under order o: a bijection on [0, G)
// in every mode (the identity when G < 8).
__device__ __forceinline__ int64_t first_item(int64_t b, int64_t G, XcdOrder o) {
  if (o.mode == kXcdNone) return b;
  if (o.mode == kXcdOneRun) {
    const int64_t q = G >> 3, r = G & 7, x = b & 7, k = b >> 3;
    return x * q + (x < r ? x : r) + k;
  }
  const int sr = o.shift + 3;  // items per round: 8 << shift
  const int64_t round = b >> sr;
  if ((round + 1) << sr > G) return b;
  const int64_t within = b & ((int64_t(1) << sr) - 1);
  return (round << sr) + ((within & 7) << o.shift) + (within >> 3);
}

template <int SK, int DK, int LANES = kThreads>
__global__ __launch_bounds__(LANES) void pack_kernel(const ChunkDesc* __restrict__ chunks,
                                                        int64_t c0, int64_t nc,
                                                        const void* const* __restrict__ src,
                                                        void* __restrict__ buf, XcdOrder run) {
  for (int64_t i = first_item(blockIdx.x, gridDim.x, run); i < nc; i += gridDim.x) {
    const ChunkDesc c = chunks[c0 + i];
    char* d = static_cast<char*>(buf) + c.buf_off * esize<DK>();
    if (c.tensor < 0) {
      zero_run<DK, RS_PACK_NT, LANES>(d, c.len);
    } else {
      const char* s = static_cast<const char*>(src[c.tensor]) + c.ten_off * esize<SK>();
      copy_run<SK, DK, RS_PACK_NT, LANES>(s, d, c.len);
    }
  }
}

template <int SK, int DK, int LANES = kThreads>
__global__ __launch_bounds__(LANES) void unpack_kernel(const ChunkDesc* __restrict__ chunks,
                                                          int64_t c0, int64_t nc,
                                                          const void* __restrict__ buf,
                                                          void* const* __restrict__ dst,
                                                          XcdOrder run) {
  for (int64_t i = first_item(blockIdx.x, gridDim.x, run); i < nc; i += gridDim.x) {
    const ChunkDesc c = chunks[c0 + i];
    if (c.tensor < 0) continue;
    const char* s = static_cast<const char*>(buf) + c.buf_off * esize<SK>();
    char* d = static_cast<char*>(dst[c.tensor]) + c.ten_off * esize<DK>();
    copy_run<SK, DK, RS_PACK_NT, LANES>(s, d, c.len);
  }
}

// -------------------------------------------------------------- scale/add

// With SPLIT > 1 workgroup ii takes piece ii % SPLIT of chunk ii / SPLIT:
// more, shorter workgroups (scale/add, the optimizer kernels).  Pieces
// are whole multiples of 64 elements, so 16-byte alignment is kept.
template <int SPLIT>
__device__ __forceinline__ bool piece_of(const ChunkDesc& c, int q, int64_t& off, int& n) {
  if (SPLIT == 1) {
    off = c.buf_off;
    n = c.len;
    return true;
  }
  const int per = ((c.len + SPLIT - 1) / SPLIT + 63) & ~63;
  const int lo = q * per;
  if (lo >= c.len) return false;
  off = c.buf_off + lo;
  n = c.len - lo < per ? c.len - lo : per;
  return true;
}


__device__ __forceinline__ float axpby(float a, float y, float b, float x) {
  // separate roundings: fl(fl(a*y) + fl(b*x)); contraction is off in this file
  const float u = a * y;
  const float w = b * x;
  return u + w;
}

__device__ __forceinline__ bool finite_bits(uint32_t u) {
  return (u & 0x7f800000u) != 0x7f800000u;
}

__device__ __forceinline__ bool finite(float v) { return finite_bits(__float_as_uint(v)); }

__device__ __forceinline__ u32x4 axpby4(float a, u32x4 y, float b, u32x4 x, bool& bad) {
  u32x4 o;
  o.x = u32(axpby(a, f32(y.x), b, f32(x.x)));
  o.y = u32(axpby(a, f32(y.y), b, f32(x.y)));
  o.z = u32(axpby(a, f32(y.z), b, f32(x.z)));
  o.w = u32(axpby(a, f32(y.w), b, f32(x.w)));
  bad |= !(finite_bits(o.x) && finite_bits(o.y) && finite_bits(o.z) && finite_bits(o.w));
  return o;
}

// Marks found_inf[rank] from lane 0 of every wave that saw a bad value.
__device__ __forceinline__ void flag_rank(bool bad, uint32_t* found_inf, int rank) {
  if (found_inf && __any(bad) && (threadIdx.x % kWave) == 0) found_inf[rank] = 1u;
}

// y <- fl(fl(alpha*y) + fl(beta*x)) over n elements: one 16-byte vector of y
// (and the matching 16 or 8 bytes of x) per lane per step, consecutive lanes
// on consecutive vectors, so each load and store instruction of a wave covers
// one contiguous 1 KB span.  x may be y: every element is loaded before it is
// stored, by the same lane.
template <int XK, bool NT>
__device__ __forceinline__ void scale_add_run(float* yp, const char* xp, int n, float alpha,
                                              float beta, bool& bad) {
  const bool vec = aligned16(yp) && (reinterpret_cast<uintptr_t>(xp) & (XK == 0 ? 15u : 7u)) == 0;
  const int nv = vec ? n / 4 : 0;
  for (int q0 = threadIdx.x; q0 < nv; q0 += kUnroll * kThreads) {
    u32x4 Y[kUnroll], X[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int q = q0 + u * kThreads;
      if (q < nv) {
        Y[u] = ld16<NT>(yp + 4 * q);
        if constexpr (XK == 0) {
          X[u] = ld16<NT>(xp + 16 * int64_t(q));
        } else {
          const u32x2* px = reinterpret_cast<const u32x2*>(xp) + q;
          const u32x2 w = NT ? __builtin_nontemporal_load(px) : *px;
          X[u] = u32x4{w.x << 16, w.x & 0xffff0000u, w.y << 16, w.y & 0xffff0000u};
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int q = q0 + u * kThreads;
      if (q < nv) st16<NT>(yp + 4 * q, axpby4(alpha, Y[u], beta, X[u], bad));
    }
  }
  for (int i = nv * 4 + threadIdx.x; i < n; i += kThreads) {
    float xv;
    if constexpr (XK == 0)
      xv = reinterpret_cast<const float*>(xp)[i];
    else
      xv = bf16_to_f32(reinterpret_cast<const uint16_t*>(xp)[i]);
    const float o = axpby(alpha, yp[i], beta, xv);
    bad |= !finite(o);
    yp[i] = o;
  }
}

template <int XK>
__global__ __launch_bounds__(kThreads) void scale_add_kernel(
    const ChunkDesc* __restrict__ chunks, int64_t c0, int64_t nc, float* y, const void* x,
    float alpha, float beta, const uint8_t* __restrict__ mask, uint32_t* __restrict__ found_inf,
    XcdOrder run) {
  for (int64_t ii = first_item(blockIdx.x, gridDim.x, run); ii < nc * RS_SCALE_SPLIT;
       ii += gridDim.x) {
    const ChunkDesc c = chunks[c0 + ii / RS_SCALE_SPLIT];
    if (c.tensor < 0) continue;
    if (mask && !mask[c.tensor]) continue;
    int64_t off;
    int n;
    if (!piece_of<RS_SCALE_SPLIT>(c, int(ii % RS_SCALE_SPLIT), off, n)) continue;
    bool bad = false;
    scale_add_run<XK, RS_SCALE_NT>(y + off, static_cast<const char*>(x) + off * esize<XK>(), n,
                                   alpha, beta, bad);
    flag_rank(bad, found_inf, c.rank);
  }
}

// ------------------------------------------------------------------- zero

// Masked zero over chunks (padding skipped).
template <int K>
__global__ __launch_bounds__(kThreads) void zero_kernel(const ChunkDesc* __restrict__ chunks,
                                                        int64_t c0, int64_t nc,
                                                        void* __restrict__ y,
                                                        const uint8_t* __restrict__ mask) {
  for (int64_t i = blockIdx.x; i < nc; i += gridDim.x) {
    const ChunkDesc c = chunks[c0 + i];
    if (mask && (c.tensor < 0 || !mask[c.tensor])) continue;
    zero_run<K, RS_ZERO_NT>(static_cast<char*>(y) + c.buf_off * esize<K>(), c.len);
  }
}

// Unmasked zero of a contiguous, 16-byte aligned byte range: RS_FILL_BYTES
// per workgroup.
template <bool NT>
__global__ __launch_bounds__(kThreads) void fill_zero_kernel(char* __restrict__ base,
                                                             int64_t nbytes, XcdOrder run) {
  const int64_t lo = first_item(blockIdx.x, gridDim.x, run) * RS_FILL_BYTES;
  const int64_t n16 = (nbytes - lo < RS_FILL_BYTES ? nbytes - lo : RS_FILL_BYTES) / 16;
  const u32x4 z = {0u, 0u, 0u, 0u};
  char* d = base + lo;
  for (int64_t v = threadIdx.x; v < n16; v += kThreads) st16<NT || RS_ZERO_NT>(d + v * 16, z);
}

// ----------------------------------------------------------------- sqnorm

// Fixed-order sum over a workgroup of NT lanes: butterfly inside each wave,
// then the wave sums in wave order.  Result valid in thread 0.
template <int NT = kThreads>
__device__ __forceinline__ double block_sum(double v, double* lds) {
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  const int w = threadIdx.x / kWave;
  if (threadIdx.x % kWave == 0) lds[w] = v;
  __syncthreads();
  double s = 0.0;
  if (threadIdx.x == 0) {
    s = lds[0];
    for (int i = 1; i < NT / kWave; ++i) s += lds[i];
  }
  __syncthreads();
  return s;
}

__device__ __forceinline__ double sq(uint32_t u) {
  const double d = double(f32(u));
  return d * d;
}

__device__ __forceinline__ void sq4(u32x4 r, double& acc, bool& bad) {
  acc += sq(r.x);
  acc += sq(r.y);
  acc += sq(r.z);
  acc += sq(r.w);
  bad |= !(finite_bits(r.x) && finite_bits(r.y) && finite_bits(r.z) && finite_bits(r.w));
}

// Per (fine or coarse) chunk ci of the range [c0, c0 + nc): fp64 sum of
// squares into part[ci - c0], so the scratch holds one partial per chunk of
// the range.  NT lanes per workgroup: fine chunks (few-rank ranges) take
// RS_SQNORM_FINE_LANES, so that more of their short workgroups are resident
// at once; each lane still adds its vectors in increasing order.
template <int NT>
__global__ __launch_bounds__(NT) void sqnorm_partial_kernel(
    const ChunkDesc* __restrict__ chunks, int64_t c0, int64_t nc, const float* __restrict__ x,
    double* __restrict__ part, uint32_t* __restrict__ found_inf) {
  __shared__ double lds[NT / kWave];
  for (int64_t ii = blockIdx.x; ii < nc; ii += gridDim.x) {
    const int64_t ci = c0 + ii;
    const ChunkDesc c = chunks[ci];
    if (c.tensor < 0) continue;
    const float* xp = x + c.buf_off;
    const int n = c.len;
    double acc = 0.0;
    bool bad = false;
    const int nv = aligned16(xp) ? n / 4 : 0;
    constexpr int U = 2 * kUnroll;
    int v = threadIdx.x;
    for (; v + (U - 1) * NT < nv; v += U * NT) {
      u32x4 r[U];
#pragma unroll
      for (int u = 0; u < U; ++u) r[u] = ld16<RS_SQNORM_NT>(xp + int64_t(v + u * NT) * 4);
#pragma unroll
      for (int u = 0; u < U; ++u) sq4(r[u], acc, bad);
    }
    {
      // the last (at most U - 1) vectors of the lane, loaded together before
      // any is used: a short chunk's few loads per lane are in flight at once
      u32x4 r[U - 1];
#pragma unroll
      for (int u = 0; u < U - 1; ++u)
        if (v + u * NT < nv) r[u] = ld16<RS_SQNORM_NT>(xp + int64_t(v + u * NT) * 4);
#pragma unroll
      for (int u = 0; u < U - 1; ++u)
        if (v + u * NT < nv) sq4(r[u], acc, bad);
    }
    for (int i = nv * 4 + threadIdx.x; i < n; i += NT) {
      const uint32_t u = __float_as_uint(xp[i]);
      acc += sq(u);
      bad |= !finite_bits(u);
    }
    flag_rank(bad, found_inf, c.rank);
    const double s = block_sum<NT>(acc, lds);
    if (threadIdx.x == 0) part[ii] = s;
  }
}

// Per tensor: the squared norm as the sum of its fragment sums in rank
// order.  Each fragment's chunk partials are summed in a fixed order that
// depends only on the fragment and the chunk table read, never on the rank
// range of the call: lanes stride over them with four accumulators, then a
// butterfly per wave.
//  * Fine chunks (ranges of few ranks, each fragment holding many chunks):
//    the whole workgroup sums one fragment at a time, the wave sums added
//    in wave order.
//  * Coarse chunks (ranges of many ranks): one wave per fragment, the
//    workgroup's kCombineWaves waves taking the range's fragments in turn
//    (sums staged in LDS, kCombineBatch ranks per pass), so a range of many
//    ranks costs about as much as one of kCombineWaves.
// Writes partial[k*n + t] for every k of the range.
constexpr int kCombineWaves = 16;
constexpr int kCombineBatch = 2048;

// One wave's fixed-order share of a fragment's chunk partials: lane `first`
// of the lanes that stride by `stride` over [cb, ce) takes its n partials
// j = 0, 1, ... in order; partial j goes to accumulator j % 4 while j is
// below 4 floor(n / 4), the rest to accumulator 0; then (a0 + a1) + (a2 +
// a3) and the sum over the wave (every lane of the wave gets it).  The
// partials are loaded kFragBatch at a time, all loads of a batch issued
// before the first addition, so a lane's few partials cost one round trip
// to memory instead of one each.  Every partial goes to its accumulator and
// +0.0 to the others; partials are sums of squares, never -0.0, so adding
// +0.0 changes no bits.
constexpr int kFragBatch = 8;
__device__ __forceinline__ double frag_lane_sum(const double* __restrict__ part, int cb, int ce,
                                                int first, int stride) {
  double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
  const int i0 = cb + first;
  const int n = i0 < ce ? (ce - i0 + stride - 1) / stride : 0;
  const int n4 = n & ~3;
  for (int j0 = 0; j0 < n; j0 += kFragBatch) {
    double v[kFragBatch];
#pragma unroll
    for (int b = 0; b < kFragBatch; ++b)
      v[b] = j0 + b < n ? part[i0 + (j0 + b) * stride] : 0.0;
#pragma unroll
    for (int b = 0; b < kFragBatch; ++b) {
      const bool grouped = j0 + b < n4;  // else the tail, all into a0
      switch (b % 4) {
        case 0: a0 += v[b]; break;
        case 1: a1 += grouped ? v[b] : 0.0; a0 += grouped ? 0.0 : v[b]; break;
        case 2: a2 += grouped ? v[b] : 0.0; a0 += grouped ? 0.0 : v[b]; break;
        default: a3 += grouped ? v[b] : 0.0; a0 += grouped ? 0.0 : v[b]; break;
      }
    }
  }
  double s = (a0 + a1) + (a2 + a3);
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) s += __shfl_xor(s, o);
  return s;
}

// A range of one rank holding at most kDirectFrags fragments: the partial
// index range of each (relative to c0), passed by value so the combine reads
// no descriptor; fragment i belongs to tensor t_lo + i.
constexpr int kDirectFrags = 32;
struct DirectFrags {
  int32_t nf;  // 0: read the descriptor tables instead
  int32_t cb[kDirectFrags], ce[kDirectFrags];
};

// One workgroup per tensor present in the range (tensors [t_lo, t_hi) in
// buffer order), plus, when some tensor is absent, one last workgroup that
// writes the zeros of the absent tensors' sq and partial entries.  part[i]
// is the partial of chunk c0 + i of the table read.
__global__ __launch_bounds__(kCombineWaves* kWave) void sqnorm_combine_kernel(
    const TensorDesc* __restrict__ tensors, const FragDesc* __restrict__ frags,
    const double* __restrict__ part, int64_t c0, int32_t n, int32_t k0, int32_t k1, int32_t t_lo,
    int32_t t_hi, double* __restrict__ sq_out, double* __restrict__ partial, int fine,
    DirectFrags direct) {
  __shared__ double fs[kCombineBatch];
  if (int(blockIdx.x) == t_hi - t_lo) {
    for (int t = threadIdx.x; t < n; t += blockDim.x)
      if (t < t_lo || t >= t_hi) sq_out[t] = 0.0;
    if (partial) {
      const int absent = n - (t_hi - t_lo);
      for (int64_t i = threadIdx.x; i < int64_t(k1 - k0) * absent; i += blockDim.x) {
        const int64_t k = k0 + i / absent;
        const int j = int(i % absent);
        partial[k * n + (j < t_lo ? j : j + (t_hi - t_lo))] = 0.0;
      }
    }
    return;
  }
  const int t = t_lo + int(blockIdx.x);
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (direct.nf > 0) {
    // one rank, one fragment per tensor, the same fixed order as below
    const int cb = direct.cb[blockIdx.x], ce = direct.ce[blockIdx.x];
    double s = 0.0;
    if (fine) {
      const double w = frag_lane_sum(part, cb, ce, threadIdx.x, kCombineWaves * kWave);
      if (lane == 0) fs[wave] = w;
      __syncthreads();
      if (threadIdx.x == 0) {
        s = fs[0];
        for (int i = 1; i < kCombineWaves; ++i) s += fs[i];
      }
    } else if (wave == 0) {
      s = frag_lane_sum(part, cb, ce, lane, kWave);
    }
    if (threadIdx.x == 0) {
      const double total = 0.0 + s;
      sq_out[t] = total;
      if (partial) partial[int64_t(k0) * n + t] = s;
    }
    return;
  }
  const TensorDesc td = tensors[t];
  double total = 0.0;
  if (fine) {
    for (int k = k0; k < k1; ++k) {
      const bool has = td.frag_begin >= 0 && k >= td.rank_lo && k < td.rank_hi;  // uniform
      double s = 0.0;
      if (has) {
        const FragDesc fd = frags[td.frag_begin + (k - td.rank_lo)];
        const double w = frag_lane_sum(part, int(fd.chunk_begin - c0), int(fd.chunk_end - c0),
                                       threadIdx.x, kCombineWaves * kWave);
        if (lane == 0) fs[wave] = w;
        __syncthreads();
        if (threadIdx.x == 0) {
          s = fs[0];
          for (int i = 1; i < kCombineWaves; ++i) s += fs[i];
          total += s;
        }
        __syncthreads();
      }
      if (partial && threadIdx.x == 0) partial[int64_t(k) * n + t] = s;
    }
    if (threadIdx.x == 0) sq_out[t] = total;
    return;
  }
  for (int kb = k0; kb < k1; kb += kCombineBatch) {
    const int ke = min(k1, kb + kCombineBatch);
    for (int k = kb + wave; k < ke; k += kCombineWaves) {
      const bool has = td.frag_begin >= 0 && k >= td.rank_lo && k < td.rank_hi;  // wave-uniform
      double s = 0.0;
      if (has) {
        const FragDesc fd = frags[td.frag_begin + (k - td.rank_lo)];
        s = frag_lane_sum(part, int(fd.cchunk_begin - c0), int(fd.cchunk_end - c0), lane, kWave);
      }
      if (lane == 0) {
        fs[k - kb] = s;
        if (partial) partial[int64_t(k) * n + t] = s;
      }
    }
    __syncthreads();
    if (threadIdx.x == 0)
      for (int k = kb; k < ke; ++k) total += fs[k - kb];
    __syncthreads();
  }
  if (threadIdx.x == 0) sq_out[t] = total;
}

// ------------------------------------------------------------------ quant
//
// Codes are encode(fl(x / scale)) with IEEE division.  Dividing every
// element makes the kernel ALU bound on gfx950 (the correctly rounded fp32
// division is a ~10-instruction sequence), so each element first takes
// q' = fl(x * fl(1/scale)), which is within 3 ulp of fl(x / scale) when the
// scale is a normal number.  The code can only differ when a rounding
// midpoint of the code grid lies within that distance; the elements near
// a midpoint (a window of at least 3.5 ulp), and every element of a tile
// whose scale is zero, subnormal, infinite or NaN, are encoded from the
// true quotient.

// Four values -> four E4M3 codes, little-endian in one word, with gfx950's
// conversion instruction (OCP E4M3, round to nearest even).  For finite
// inputs with |q| < 464 (464 is the first midpoint past 448) it equals the
// saturating encoder above, subnormal codes included; a test checks that
// on every such fp32 input.
__device__ __forceinline__ uint32_t e4m3_pack4(float q0, float q1, float q2, float q3) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(q2, q3, w, true);
  return uint32_t(w);
}

// Four fast-path E4M3 codes.  The encoder is monotone in |q| and keeps the
// sign, so when q'(1 - 2^-21) and q'(1 + 2^-21) have the same code, so has
// every value between them, and that interval holds the true quotient: it
// is within 2 ulp of q' (one rounding of x * rcp, one of x / scale, and the
// reciprocal's half ulp), while 2^-21 of a normal |q'| is at least 4 ulp,
// at least 3.5 after the product's own rounding.  A subnormal q' makes the
// interval a point, but then q' and the quotient both lie far below 2^-10,
// the half-way point to the smallest code, and both encode to a signed
// zero.  With a normal, finite scale, |q'| stays below 449, inside the
// instruction's checked domain.  safe turns false when the two codes
// differ: that value needs the exact quotient.
__device__ __forceinline__ uint32_t e4m3_fast4(const float* q, bool& safe) {
  constexpr float lo = 1.0f - 0x1p-21f, hi = 1.0f + 0x1p-21f;
  const uint32_t a = e4m3_pack4(q[0] * lo, q[1] * lo, q[2] * lo, q[3] * lo);
  const uint32_t b = e4m3_pack4(q[0] * hi, q[1] * hi, q[2] * hi, q[3] * hi);
  safe = safe && a == b;
  return a;
}

// INT8: q' is safe when its distance to the nearest integer is below
// 0.5 - |q'| * 2^-20, i.e. more than |q'| * 2^-20 (>= 8 ulp) from a
// half-integer; r = rint(q') is then also the rounded true quotient.
__device__ __forceinline__ bool int8_safe(float q, float r) {
  return fabsf(q - r) < 0.5f - fabsf(q) * 0x1p-20f;
}

__device__ __forceinline__ uint32_t int8_from_rint(float r) {
  return uint32_t(int32_t(fminf(fmaxf(r, -127.0f), 127.0f))) & 0xffu;
}

template <int FMT>
__device__ __forceinline__ uint32_t encode(float q) {
  return FMT == RS_Q_FP8_E4M3 ? e4m3_encode(q) : int8_encode(q);
}

// Exact code of one element, any tile.
template <int FMT>
__device__ __forceinline__ uint32_t encode_exact(float x, float scale, bool zero_tile,
                                                 bool nan_tile) {
  if (zero_tile) return 0u;
  if (nan_tile) return FMT == RS_Q_FP8_E4M3 ? 0x7fu : 0u;
  return encode<FMT>(x / scale);
}

// Walks the float4 slots f = lane, lane + team, ... of a tile with c4
// slots per row, as element offsets from the tile's first element (tiles
// span less than 2^31 elements; the layout checks it).
struct SlotWalk {
  int off, c, dr, c4, step, wrap;
  __device__ __forceinline__ SlotWalk(int lane, int team, int c4_, int ld) {
    c4 = c4_;
    const int r = lane / c4;
    c = lane - r * c4;
    const int dq = team / c4;
    dr = team - dq * c4;
    off = r * ld + c * 4;
    step = dq * ld + dr * 4;      // advance by team slots
    wrap = ld - c4 * 4;           // extra when the column wraps to the next row
  }
  __device__ __forceinline__ void next() {
    off += step;
    c += dr;
    if (c >= c4) {
      c -= c4;
      off += wrap;
    }
  }
};

// Place and shape of tile j of a work item (a run of consecutive tiles of
// one tensor; edge tiles clipped).
struct Tile {
  int64_t buf_off, ld;
  int rows, cols, scale_idx;
};

__device__ __forceinline__ Tile tile_of(const QuantWork& w, int j) {
  const int idx = w.t0 + j;
  const int tr = idx / w.ntc, tc = idx - tr * w.ntc;
  const int r0 = tr * w.q_rows, c0 = tc * w.q_cols;
  Tile t;
  t.buf_off = w.base + int64_t(r0) * w.cols + c0;
  t.ld = w.cols;
  t.rows = min(w.q_rows, w.rows - r0);
  t.cols = min(w.q_cols, w.cols - c0);
  t.scale_idx = w.scale0 + j;
  return t;
}

// Each workgroup takes `count` consecutive tiles; tile j of the item is
// handled by lanes [j*team, (j+1)*team) of each of F sub-blocks of kThreads
// lanes, sub-block f taking slots [f*NS, (f+1)*NS) of the lane's F*NS
// four-element slots (narrow tiles: F = 1, NS = 4; wide tiles: F*NS = 16).
// On the 16-byte path a lane keeps its 4*NS elements in registers between
// the absmax and the encode pass, so x is read once; the other path reads x
// twice.  F > 1 finishes each wide tile sooner, for launches with few tiles.
template <int FMT, int F, int NS, bool NTS>
__global__ __launch_bounds__(kThreads* F) void quant_kernel(const QuantWork* __restrict__ work,
                                                            int64_t w0,
                                                            const float* __restrict__ x,
                                                            uint8_t* __restrict__ codes,
                                                            float* __restrict__ scales,
                                                            uint32_t* __restrict__ found_inf,
                                                            int vec_ok) {
  __shared__ uint32_t lds[kThreads * F / kWave];
  __shared__ uint32_t ldt[F][kThreads];
  const QuantWork w = work[w0 + blockIdx.x];
  const bool vec = w.vec && vec_ok;
  const int team = w.team;
  const int sub = threadIdx.x / kThreads;
  const int tt = threadIdx.x % kThreads;
  const int slot = tt / team;
  const int lane = tt % team;
  const bool active = slot < w.count;
  const Tile td = tile_of(w, active ? slot : 0);
  const float* base = x + td.buf_off;
  uint8_t* cbase = codes + td.buf_off;
  const int s0 = sub * NS;
  float v[4 * NS];
  uint32_t amax = 0;
  const int c4 = td.cols >> 2;
  const int nf = active ? td.rows * c4 : 0;
  const int ne = active ? td.rows * td.cols : 0;
  if (vec) {
    SlotWalk sw(lane + s0 * team, team, c4, int(td.ld));
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      u32x4 q = {0u, 0u, 0u, 0u};
      if (lane + (s0 + i) * team < nf) q = ld16<RS_QUANT_NT>(base + sw.off);
      sw.next();
      v[4 * i + 0] = f32(q.x);
      v[4 * i + 1] = f32(q.y);
      v[4 * i + 2] = f32(q.z);
      v[4 * i + 3] = f32(q.w);
      amax = max(amax, max(max(q.x & 0x7fffffffu, q.y & 0x7fffffffu),
                           max(q.z & 0x7fffffffu, q.w & 0x7fffffffu)));
    }
  } else {
    for (int e = lane + sub * team; e < ne; e += team * F) {
      const int r = e / td.cols;
      amax = max(amax, __float_as_uint(base[int64_t(r) * td.ld + (e - r * td.cols)]) & 0x7fffffffu);
    }
  }
  // absmax of the tile as the max of |x| bit patterns: NaN patterns sort
  // above +Inf, so a NaN anywhere yields a NaN amax
  const int red = team < kWave ? team : kWave;
  for (int o = red / 2; o >= 1; o >>= 1) amax = max(amax, uint32_t(__shfl_xor(int(amax), o)));
  if (team > kWave) {  // uniform: the waves of a tile within a sub-block
    if (threadIdx.x % kWave == 0) lds[threadIdx.x / kWave] = amax;
    __syncthreads();
    const int first = sub * (kThreads / kWave) + (tt / team) * (team / kWave);
    uint32_t a = lds[first];
    for (int i = 1; i < team / kWave; ++i) a = max(a, lds[first + i]);
    amax = a;
  }
  if constexpr (F > 1) {  // the sub-blocks of a tile
    ldt[sub][tt] = amax;
    __syncthreads();
    amax = ldt[0][tt];
#pragma unroll
    for (int j = 1; j < F; ++j) amax = max(amax, ldt[j][tt]);
  }
  if (!active) return;
  constexpr float Q = FMT == RS_Q_FP8_E4M3 ? 448.0f : 127.0f;
  const float famax = __uint_as_float(amax);
  float scale = famax / Q;
  const bool nan_tile = amax > 0x7f800000u;
  if (nan_tile) scale = __uint_as_float(0x7fc00000u);
  if (lane == 0 && sub == 0) {
    scales[td.scale_idx] = scale;
    // an Inf or NaN |x| pattern is >= the +Inf pattern
    if (found_inf && amax >= 0x7f800000u) found_inf[w.rank] = 1u;
  }
  const bool zero_tile = scale == 0.0f;
  const float rcp = 1.0f / scale;
  // the reciprocal path needs a normal, finite scale (and so a finite rcp)
  const uint32_t sb = __float_as_uint(scale);
  const bool fast = sb >= 0x00800000u && sb < 0x7f800000u;
  // an Inf scale (an Inf but no NaN in the tile): rcp = 0 and x * 0 is
  // exactly x / Inf for every x of the tile (+-0, or NaN for +-Inf)
  const bool inf_scale = sb == 0x7f800000u;
  if (!vec) {
    for (int e = lane + sub * team; e < ne; e += team * F) {
      const int r = e / td.cols;
      const int64_t o = int64_t(r) * td.ld + (e - r * td.cols);
      cbase[o] = uint8_t(encode_exact<FMT>(base[o], scale, zero_tile, nan_tile));
    }
    return;
  }
  uint32_t slow = 0;  // bit i: slot s0 + i needs the exact path
  {
    SlotWalk sw(lane + s0 * team, team, c4, int(td.ld));
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if (lane + (s0 + i) * team < nf) {
        float q[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) q[j] = v[4 * i + j] * rcp;
        bool safe = fast;
        uint32_t word;
        if (!fast) {  // tile-uniform: codes that need no division, else exact
          safe = zero_tile || nan_tile || inf_scale;
          if (zero_tile)
            word = 0u;
          else if (nan_tile)
            word = FMT == RS_Q_FP8_E4M3 ? 0x7f7f7f7fu : 0u;
          else
            word = encode<FMT>(q[0]) | (encode<FMT>(q[1]) << 8) | (encode<FMT>(q[2]) << 16) |
                   (encode<FMT>(q[3]) << 24);
        } else if constexpr (FMT == RS_Q_FP8_E4M3) {
          word = e4m3_fast4(q, safe);
        } else {
          float r[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            r[j] = __builtin_rintf(q[j]);
            safe = safe && int8_safe(q[j], r[j]);
          }
          word = int8_from_rint(r[0]) | (int8_from_rint(r[1]) << 8) | (int8_from_rint(r[2]) << 16) |
                 (int8_from_rint(r[3]) << 24);
        }
        if (safe) {
          if constexpr (NTS)
            __builtin_nontemporal_store(word, reinterpret_cast<uint32_t*>(cbase + sw.off));
          else
            *reinterpret_cast<uint32_t*>(cbase + sw.off) = word;
        } else {
          slow |= 1u << i;
        }
      }
      sw.next();
    }
  }
  if (slow) {  // rare: divide the slot's values, still in registers
    SlotWalk sw(lane + s0 * team, team, c4, int(td.ld));
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if (slow & (1u << i)) {
        const uint32_t word = encode_exact<FMT>(v[4 * i + 0], scale, zero_tile, nan_tile) |
                              (encode_exact<FMT>(v[4 * i + 1], scale, zero_tile, nan_tile) << 8) |
                              (encode_exact<FMT>(v[4 * i + 2], scale, zero_tile, nan_tile) << 16) |
                              (encode_exact<FMT>(v[4 * i + 3], scale, zero_tile, nan_tile) << 24);
        *reinterpret_cast<uint32_t*>(cbase + sw.off) = word;
      }
      sw.next();
    }
  }
}

// ---------------------------------------------------------------- dequant
//
// y = fl(decode(code) * scale) per element of every tile in the range; the
// decode is exact (E4M3 with gfx950's widening conversion, INT8 as an
// integer), so the product is the only rounding (plus the bf16 cast).

template <int FMT>
__device__ __forceinline__ void decode4(uint32_t word, float d[4]) {
  if constexpr (FMT == RS_Q_FP8_E4M3) {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(int(word), false);
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(int(word), true);
    d[0] = lo[0];
    d[1] = lo[1];
    d[2] = hi[0];
    d[3] = hi[1];
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) d[j] = float(int8_t(uint8_t(word >> (8 * j))));
  }
}

template <int YK, bool NTS>
__device__ __forceinline__ void store4(char* yb, int64_t elem, const float d[4], float scale) {
  if constexpr (YK == 0) {
    u32x4 o;
    o.x = u32(d[0] * scale);
    o.y = u32(d[1] * scale);
    o.z = u32(d[2] * scale);
    o.w = u32(d[3] * scale);
    st16<NTS>(yb + elem * 4, o);
  } else {
    u32x2 o;
    o.x = bf16_rne(d[0] * scale) | (bf16_rne(d[1] * scale) << 16);
    o.y = bf16_rne(d[2] * scale) | (bf16_rne(d[3] * scale) << 16);
    if constexpr (NTS)
      __builtin_nontemporal_store(o, reinterpret_cast<u32x2*>(yb + elem * 2));
    else
      *reinterpret_cast<u32x2*>(yb + elem * 2) = o;
  }
}

// Lanes take 4 codes (one 32-bit load, one 16-byte fp32 store) per slot,
// all loads of a lane issued before its stores; unaligned tiles one code
// per lane.  (16 codes per lane - 16-byte loads, lane-strided stores - was
// several times slower.)
// With F > 1, F workgroups share a work item, each taking one band of
// about rows/F rows of every tile (more, shorter workgroups); the host uses
// F = 1 when some tile of the launch (one tile class of the range) has
// fewer than F rows.
template <int FMT, int YK, int F, bool NTS>
__global__ __launch_bounds__(kThreads) void dequant_kernel(const QuantWork* __restrict__ work,
                                                           int64_t w0,
                                                           const uint8_t* __restrict__ codes,
                                                           const float* __restrict__ scales,
                                                           void* __restrict__ y, int vec_ok,
                                                           XcdOrder run) {
  const int64_t item = first_item(blockIdx.x, gridDim.x, run);
  const QuantWork w = work[w0 + item / F];
  const int band = int(item % F);
  const int team = w.team;
  const int slot = threadIdx.x / team;
  const int lane = threadIdx.x % team;
  const bool active = slot < w.count;
  Tile td = tile_of(w, active ? slot : 0);
  const float scale = scales[td.scale_idx];
  if (F > 1) {
    const int rp = (td.rows + F - 1) / F;
    const int r0 = min(td.rows, band * rp);
    td.buf_off += int64_t(r0) * td.ld;
    td.rows = min(td.rows - r0, rp);
  }
  const uint8_t* cb = codes + td.buf_off;
  char* yb = static_cast<char*>(y) + td.buf_off * esize<YK>();
#if RS_DEQ_LDS
  // stage each team's tile codes in LDS with coalesced 16-byte loads, then
  // decode 4 codes per lane with lane-contiguous 16-byte stores
  __shared__ uint32_t stage[kThreads * 16];  // 16 KB: team * 64 codes per tile
  const bool g16 = vec_ok == 2 && td.cols % 16 == 0 && td.ld % 16 == 0 && td.buf_off % 16 == 0;
  if (__syncthreads_and(g16 || !active)) {  // uniform: every active tile qualifies
    uint32_t* tl = stage + slot * team * 16;
    const int c16 = td.cols >> 4;
    const int n16 = active ? td.rows * c16 : 0;
    for (int f = lane; f < n16; f += team) {
      const int r = f / c16;
      const int c = f - r * c16;
      const u32x4 q = ld16<RS_PACK_NT>(cb + int64_t(r) * td.ld + c * 16);
      uint32_t* dst = tl + (r * td.cols + c * 16) / 4;
      dst[0] = q.x;
      dst[1] = q.y;
      dst[2] = q.z;
      dst[3] = q.w;
    }
    __syncthreads();
    const int c4 = td.cols >> 2;
    const int nf = active ? td.rows * c4 : 0;
    for (int f = lane; f < nf; f += team) {
      const int r = f / c4;
      const int c = f - r * c4;
      float d[4];
      decode4<FMT>(tl[(r * td.cols) / 4 + c], d);
      store4<YK, NTS>(yb, int64_t(r) * td.ld + c * 4, d, scale);
    }
    return;
  }
#endif
  if (!active) return;
  if (w.vec && vec_ok) {
    const int c4 = td.cols >> 2;
    const int nf = td.rows * c4;
    SlotWalk sw(lane, team, c4, int(td.ld));
    uint32_t q[16];
    int off[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      off[i] = sw.off;
      if (lane + i * team < nf) q[i] = *reinterpret_cast<const uint32_t*>(cb + off[i]);
      sw.next();
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (lane + i * team < nf) {
        float d[4];
        decode4<FMT>(q[i], d);
        store4<YK, NTS>(yb, off[i], d, scale);
      }
    }
  } else {
    const int ne = td.rows * td.cols;
    for (int e = lane; e < ne; e += team) {
      const int r = e / td.cols;
      const int64_t o = int64_t(r) * td.ld + (e - r * td.cols);
      float d[4];
      decode4<FMT>(cb[o], d);
      const float v = d[0] * scale;
      if constexpr (YK == 0)
        reinterpret_cast<float*>(yb)[o] = v;
      else
        reinterpret_cast<uint16_t*>(yb)[o] = uint16_t(bf16_rne(v));
    }
  }
}

// -------------------------------------------------------------- optimizers
//
// Fused optimizer steps over the fragments of a rank range, one launch for
// the whole group, fp32 with every operation rounded once (contraction is
// off in this file; sqrt and division are IEEE, or in 8-bit AdamW the
// shorter forms of rs_exact.h, which give the same bits).

struct AdamConst {
  float beta1, beta2, omb1, omb2, eps, decay, step, bc2s, inv;
  float rbc2s;  // RN(1/bc2s), for div_by_const
};

// True (uniformly) when any of the m found-inf flags is set: the step is
// skipped, as the sharded gradient scaler does.
__device__ __forceinline__ bool skip_step(const uint32_t* found_inf, int m) {
  int hit = 0;
  if (found_inf)
    for (int i = threadIdx.x; i < m; i += blockDim.x) hit |= found_inf[i] != 0u;
  return __syncthreads_or(hit) != 0;
}

__device__ __forceinline__ void adamw1(float& p, float g, float& m, float& v, const AdamConst& k) {
  const float gg = g * k.inv;
  const float m2 = k.beta1 * m + k.omb1 * gg;
  const float v2 = k.beta2 * v + k.omb2 * (gg * gg);
  const float den = sqrtf(v2) / k.bc2s + k.eps;
  const float upd = m2 / den;
  p = p * k.decay - k.step * upd;
  m = m2;
  v = v2;
}

template <int SPLIT>
__global__ __launch_bounds__(kThreads) void adamw_kernel(
    const ChunkDesc* __restrict__ chunks, int64_t c0, int64_t nc, float* __restrict__ p,
    const float* __restrict__ g, float* __restrict__ m, float* __restrict__ v, AdamConst k,
    const uint8_t* __restrict__ mask, const uint32_t* __restrict__ found_inf, int m_ranks) {
  if (skip_step(found_inf, m_ranks)) return;
  for (int64_t ii = blockIdx.x; ii < nc * SPLIT; ii += gridDim.x) {
    const ChunkDesc c = chunks[c0 + ii / SPLIT];
    if (c.tensor < 0 || (mask && !mask[c.tensor])) continue;
    int64_t off;
    int n;
    if (!piece_of<SPLIT>(c, int(ii % SPLIT), off, n)) continue;
    float* pp = p + off;
    const float* gp = g + off;
    float* mp = m + off;
    float* vp = v + off;
    const bool vec = aligned16(pp) && aligned16(gp) && aligned16(mp) && aligned16(vp);
    const int nv = vec ? n / 4 : 0;
    for (int q0 = threadIdx.x; q0 < nv; q0 += kUnroll * kThreads) {
      u32x4 P[kUnroll], G[kUnroll], M[kUnroll], V[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int q = q0 + u * kThreads;
        if (q < nv) {
          P[u] = ld16<RS_OPT_NT>(pp + 4 * q);
          G[u] = ld16<RS_OPT_G_NT>(gp + 4 * q);
          M[u] = ld16<RS_OPT_NT>(mp + 4 * q);
          V[u] = ld16<RS_OPT_NT>(vp + 4 * q);
        }
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int q = q0 + u * kThreads;
        if (q < nv) {
          float a[4] = {f32(P[u].x), f32(P[u].y), f32(P[u].z), f32(P[u].w)};
          float b[4] = {f32(M[u].x), f32(M[u].y), f32(M[u].z), f32(M[u].w)};
          float d[4] = {f32(V[u].x), f32(V[u].y), f32(V[u].z), f32(V[u].w)};
          const float e[4] = {f32(G[u].x), f32(G[u].y), f32(G[u].z), f32(G[u].w)};
#pragma unroll
          for (int j = 0; j < 4; ++j) adamw1(a[j], e[j], b[j], d[j], k);
          st16<RS_OPT_NT>(pp + 4 * q, u32x4{u32(a[0]), u32(a[1]), u32(a[2]), u32(a[3])});
          st16<RS_OPT_NT>(mp + 4 * q, u32x4{u32(b[0]), u32(b[1]), u32(b[2]), u32(b[3])});
          st16<RS_OPT_NT>(vp + 4 * q, u32x4{u32(d[0]), u32(d[1]), u32(d[2]), u32(d[3])});
        }
      }
    }
    for (int e = nv * 4 + threadIdx.x; e < n; e += kThreads) {
      float a = pp[e], b = mp[e], d = vp[e];
      adamw1(a, gp[e], b, d, k);
      pp[e] = a;
      mp[e] = b;
      vp[e] = d;
    }
  }
}

struct SgdConst {
  float lr, mu, wd, inv;
  int nesterov;
};

__device__ __forceinline__ void sgd1(float& p, float g, float& b, const SgdConst& k) {
  const float gg = g * k.inv + k.wd * p;
  const float b2 = k.mu * b + gg;
  const float d = k.nesterov ? gg + k.mu * b2 : b2;
  p = p - k.lr * d;
  b = b2;
}

template <int SPLIT>
__global__ __launch_bounds__(kThreads) void sgd_kernel(
    const ChunkDesc* __restrict__ chunks, int64_t c0, int64_t nc, float* __restrict__ p,
    const float* __restrict__ g, float* __restrict__ buf, SgdConst k,
    const uint8_t* __restrict__ mask, const uint32_t* __restrict__ found_inf, int m_ranks) {
  if (skip_step(found_inf, m_ranks)) return;
  for (int64_t ii = blockIdx.x; ii < nc * SPLIT; ii += gridDim.x) {
    const ChunkDesc c = chunks[c0 + ii / SPLIT];
    if (c.tensor < 0 || (mask && !mask[c.tensor])) continue;
    int64_t off;
    int n;
    if (!piece_of<SPLIT>(c, int(ii % SPLIT), off, n)) continue;
    float* pp = p + off;
    const float* gp = g + off;
    float* bp = buf + off;
    const bool vec = aligned16(pp) && aligned16(gp) && aligned16(bp);
    const int nv = vec ? n / 4 : 0;
    for (int q0 = threadIdx.x; q0 < nv; q0 += kUnroll * kThreads) {
      u32x4 P[kUnroll], G[kUnroll], B[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int q = q0 + u * kThreads;
        if (q < nv) {
          P[u] = ld16<RS_OPT_NT>(pp + 4 * q);
          G[u] = ld16<RS_OPT_G_NT>(gp + 4 * q);
          B[u] = ld16<RS_OPT_NT>(bp + 4 * q);
        }
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int q = q0 + u * kThreads;
        if (q < nv) {
          float a[4] = {f32(P[u].x), f32(P[u].y), f32(P[u].z), f32(P[u].w)};
          float b[4] = {f32(B[u].x), f32(B[u].y), f32(B[u].z), f32(B[u].w)};
          const float e[4] = {f32(G[u].x), f32(G[u].y), f32(G[u].z), f32(G[u].w)};
#pragma unroll
          for (int j = 0; j < 4; ++j) sgd1(a[j], e[j], b[j], k);
          st16<RS_OPT_NT>(pp + 4 * q, u32x4{u32(a[0]), u32(a[1]), u32(a[2]), u32(a[3])});
          st16<RS_OPT_NT>(bp + 4 * q, u32x4{u32(b[0]), u32(b[1]), u32(b[2]), u32(b[3])});
        }
      }
    }
    for (int e = nv * 4 + threadIdx.x; e < n; e += kThreads) {
      float a = pp[e], b = bp[e];
      sgd1(a, gp[e], b, k);
      pp[e] = a;
      bp[e] = b;
    }
  }
}

// 8-bit AdamW: the moments of every quantised tensor are block-quantised
// (codes + one fp32 scale per tile, the layout's tile table).  Per tile:
// dequantise m and v, the AdamW update in fp32, requantise m' and v' with
// their new absmax scales.  A work item (the quantisation kernel's: `count`
// tiles of `team` lanes) is spread over F sub-blocks of kThreads threads,
// each taking NS of the lane's four-element slots (narrow tiles: F = 1,
// NS = 4; wide tiles: F*NS = 16), so a
// lane keeps its m' and v' in registers between the absmax pass and the
// encode pass (every input is read once) at a modest register count.  The
// first pass also writes p', which does not depend on the new scales, so
// the pass after the absmax reduction only encodes and stores codes.  Slots
// whose encode needs the exact quotient are redone from the same registers.

template <int FMT>
__device__ __forceinline__ void moments4(u32x4 G, uint32_t cm, uint32_t cv, float sm, float sv,
                                         const AdamConst& k, float* M, float* V) {
  float dm[4], dv[4];
  decode4<FMT>(cm, dm);
  decode4<FMT>(cv, dv);
  const float gs[4] = {f32(G.x), f32(G.y), f32(G.z), f32(G.w)};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float mo = dm[j] * sm;
    const float vo = dv[j] * sv;
    const float gg = gs[j] * k.inv;
    M[j] = k.beta1 * mo + k.omb1 * gg;
    V[j] = k.beta2 * vo + k.omb2 * (gg * gg);
  }
}

__device__ __forceinline__ uint32_t absmax4(const float* a, uint32_t acc) {
  return max(acc, max(max(u32(a[0]) & 0x7fffffffu, u32(a[1]) & 0x7fffffffu),
                      max(u32(a[2]) & 0x7fffffffu, u32(a[3]) & 0x7fffffffu)));
}

// Fast encode of four values with a normal, finite scale; safe = false when
// any of them needs the exact quotient.
template <int FMT>
__device__ __forceinline__ uint32_t fast_encode4(const float* a, float rcp, bool& safe) {
  float q[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) q[j] = a[j] * rcp;
  if constexpr (FMT == RS_Q_FP8_E4M3) {
    return e4m3_fast4(q, safe);
  } else {
    float r[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      r[j] = __builtin_rintf(q[j]);
      safe = safe && int8_safe(q[j], r[j]);
    }
    return int8_from_rint(r[0]) | (int8_from_rint(r[1]) << 8) | (int8_from_rint(r[2]) << 16) |
           (int8_from_rint(r[3]) << 24);
  }
}

template <int FMT>
__device__ __forceinline__ uint32_t exact_encode4(const float* a, float scale, bool zero_tile,
                                                  bool nan_tile) {
  return encode_exact<FMT>(a[0], scale, zero_tile, nan_tile) |
         (encode_exact<FMT>(a[1], scale, zero_tile, nan_tile) << 8) |
         (encode_exact<FMT>(a[2], scale, zero_tile, nan_tile) << 16) |
         (encode_exact<FMT>(a[3], scale, zero_tile, nan_tile) << 24);
}

struct TileScale {
  float scale, rcp;
  bool fast, zero_tile, nan_tile;
  __device__ __forceinline__ TileScale(uint32_t amax, float Q) {
    scale = __uint_as_float(amax) / Q;
    nan_tile = amax > 0x7f800000u;
    if (nan_tile) scale = __uint_as_float(0x7fc00000u);
    zero_tile = scale == 0.0f;
    rcp = 1.0f / scale;
    const uint32_t sb = __float_as_uint(scale);
    fast = sb >= 0x00800000u && sb < 0x7f800000u;
  }
};

// The AdamW parameter update from m' and v'.  DIVC: sqrt(v') / bc2s through
// div_by_const (the host checked bc2s), the same correctly rounded quotient
// in three operations instead of the IEEE division sequence; the square
// root through sqrt_rn.
template <bool DIVC>
__device__ __forceinline__ float adam_p(float p, float m2, float v2, const AdamConst& k) {
  const float sq = RS_ADAM8_SQRT ? sqrt_rn(v2) : sqrtf(v2);
  const float den = (DIVC ? div_by_const(sq, k.bc2s, k.rbc2s) : sq / k.bc2s) + k.eps;
  return p * k.decay - k.step * (m2 / den);
}

template <int FMT, int F, int NS, bool DIVC>
__global__ __launch_bounds__(kThreads* F) void adamw8_kernel(
    const QuantWork* __restrict__ work, int64_t w0, float* __restrict__ p, const float* __restrict__ g, uint8_t* __restrict__ mc,
    float* __restrict__ ms, uint8_t* __restrict__ vc, float* __restrict__ vs, AdamConst k,
    const uint32_t* __restrict__ found_inf, int m_ranks, int vec_ok) {
  // NS slots per lane and sub-block (narrow tiles: F = 1, NS = 4)
  __shared__ uint32_t ldw[2][kThreads * F / kWave];
  __shared__ uint32_t ldt[2][F][kThreads];
  if (skip_step(found_inf, m_ranks)) return;
  const QuantWork w = work[w0 + blockIdx.x];
  const bool vec = w.vec && vec_ok;
  const int team = w.team;
  const int sub = threadIdx.x / kThreads;
  const int tt = threadIdx.x % kThreads;
  const int slot = tt / team;
  const int lane = tt % team;
  const bool active = slot < w.count;
  const Tile td = tile_of(w, active ? slot : 0);
  const int64_t o0 = td.buf_off;
  const float sm_old = ms[td.scale_idx], sv_old = vs[td.scale_idx];
  const int c4 = td.cols >> 2;
  const int nf = active ? td.rows * c4 : 0;
  const int ne = active ? td.rows * td.cols : 0;
  const int s0 = sub * NS;  // first slot of this sub-block
  uint32_t am = 0, av = 0;
  float M[NS][4], V[NS][4];
  if (vec) {
    // p' needs m' and v' only, not the new scales: it is written here, so
    // the encode pass after the absmax reduction touches no input
    // One slot ahead: slot i + 1's loads are issued before slot i's
    // arithmetic, so their latency hides behind it.  The arithmetic runs on
    // every slot (zeros past the tile) and only the absmax and the store
    // are predicated: M and V are then never merged across branches, which
    // would copy the whole arrays once per slot.
    SlotWalk sw(lane + s0 * team, team, c4, int(td.ld));
    u32x4 Pc, Gc;
    uint32_t CMc, CVc;
    int oc;
    auto load_slot = [&](int i, u32x4& P_, u32x4& G_, uint32_t& CM_, uint32_t& CV_, int& o_) {
      o_ = sw.off;
      G_ = P_ = u32x4{0u, 0u, 0u, 0u};
      CM_ = CV_ = 0u;
      if (lane + (s0 + i) * team < nf) {
        const int64_t q = o0 + o_;
        G_ = ld16<RS_ADAM8_NT>(g + q);
        P_ = ld16<RS_ADAM8_NT>(p + q);
        CM_ = *reinterpret_cast<const uint32_t*>(mc + q);
        CV_ = *reinterpret_cast<const uint32_t*>(vc + q);
      }
      sw.next();
    };
    load_slot(0, Pc, Gc, CMc, CVc, oc);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      u32x4 Pn, Gn;
      uint32_t CMn = 0u, CVn = 0u;
      int on = 0;
      if (i + 1 < NS) load_slot(i + 1, Pn, Gn, CMn, CVn, on);
      const bool in = lane + (s0 + i) * team < nf;
      moments4<FMT>(Gc, CMc, CVc, sm_old, sv_old, k, M[i], V[i]);
      const uint32_t am2 = absmax4(M[i], am), av2 = absmax4(V[i], av);
      am = in ? am2 : am;
      av = in ? av2 : av;
      u32x4 out;
      out.x = u32(adam_p<DIVC>(f32(Pc.x), M[i][0], V[i][0], k));
      out.y = u32(adam_p<DIVC>(f32(Pc.y), M[i][1], V[i][1], k));
      out.z = u32(adam_p<DIVC>(f32(Pc.z), M[i][2], V[i][2], k));
      out.w = u32(adam_p<DIVC>(f32(Pc.w), M[i][3], V[i][3], k));
      if (in) st16<RS_ADAM8_NT>(p + o0 + oc, out);
      if (i + 1 < NS) {
        Pc = Pn;
        Gc = Gn;
        CMc = CMn;
        CVc = CVn;
        oc = on;
      }
    }
  } else {
    for (int e = lane + sub * team; e < ne; e += team * F) {
      const int r = e / td.cols;
      const int64_t o = o0 + int64_t(r) * td.ld + (e - r * td.cols);
      float m1[4], v1[4];
      moments4<FMT>(u32x4{u32(g[o]), 0u, 0u, 0u}, mc[o], vc[o], sm_old, sv_old, k, m1, v1);
      am = max(am, u32(m1[0]) & 0x7fffffffu);
      av = max(av, u32(v1[0]) & 0x7fffffffu);
      p[o] = adam_p<DIVC>(p[o], m1[0], v1[0], k);
    }
  }
  const int red = team < kWave ? team : kWave;
  for (int o = red / 2; o >= 1; o >>= 1) {
    am = max(am, uint32_t(__shfl_xor(int(am), o)));
    av = max(av, uint32_t(__shfl_xor(int(av), o)));
  }
  if (team > kWave) {  // uniform: combine the waves of a tile within a sub-block
    if (threadIdx.x % kWave == 0) {
      ldw[0][threadIdx.x / kWave] = am;
      ldw[1][threadIdx.x / kWave] = av;
    }
    __syncthreads();
    const int first = sub * (kThreads / kWave) + (tt / team) * (team / kWave);
    uint32_t a = ldw[0][first], b = ldw[1][first];
    for (int i = 1; i < team / kWave; ++i) {
      a = max(a, ldw[0][first + i]);
      b = max(b, ldw[1][first + i]);
    }
    am = a;
    av = b;
  }
  if constexpr (F > 1) {  // combine the sub-blocks
    ldt[0][sub][tt] = am;
    ldt[1][sub][tt] = av;
    __syncthreads();
    am = ldt[0][0][tt];
    av = ldt[1][0][tt];
#pragma unroll
    for (int j = 1; j < F; ++j) {
      am = max(am, ldt[0][j][tt]);
      av = max(av, ldt[1][j][tt]);
    }
  }
  if (!active) return;
  constexpr float Q = FMT == RS_Q_FP8_E4M3 ? 448.0f : 127.0f;
  const TileScale tm(am, Q), tv(av, Q);
  if (lane == 0 && sub == 0) {
    ms[td.scale_idx] = tm.scale;
    vs[td.scale_idx] = tv.scale;
  }
  if (!vec) {
    // every element's old codes are read and rewritten by one thread only
    for (int e = lane + sub * team; e < ne; e += team * F) {
      const int r = e / td.cols;
      const int64_t o = o0 + int64_t(r) * td.ld + (e - r * td.cols);
      float m1[4], v1[4];
      moments4<FMT>(u32x4{u32(g[o]), 0u, 0u, 0u}, mc[o], vc[o], sm_old, sv_old, k, m1, v1);
      mc[o] = uint8_t(encode_exact<FMT>(m1[0], tm.scale, tm.zero_tile, tm.nan_tile));
      vc[o] = uint8_t(encode_exact<FMT>(v1[0], tv.scale, tv.zero_tile, tv.nan_tile));
    }
    return;
  }
  uint32_t slow = 0;
  {
    SlotWalk sw(lane + s0 * team, team, c4, int(td.ld));
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if (lane + (s0 + i) * team < nf) {
        const int64_t q = o0 + sw.off;
        bool safe = tm.fast && tv.fast;
        const uint32_t wm = fast_encode4<FMT>(M[i], tm.rcp, safe);
        const uint32_t wv = fast_encode4<FMT>(V[i], tv.rcp, safe);
        if (safe) {
          *reinterpret_cast<uint32_t*>(mc + q) = wm;
          *reinterpret_cast<uint32_t*>(vc + q) = wv;
        } else {
          slow |= 1u << i;
        }
      }
      sw.next();
    }
  }
  if (slow) {  // rare: exact division for the slots that need it
    SlotWalk sw(lane + s0 * team, team, c4, int(td.ld));
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if (slow & (1u << i)) {
        const int64_t o = o0 + sw.off;
        *reinterpret_cast<uint32_t*>(mc + o) = exact_encode4<FMT>(M[i], tm.scale, tm.zero_tile, tm.nan_tile);
        *reinterpret_cast<uint32_t*>(vc + o) = exact_encode4<FMT>(V[i], tv.scale, tv.zero_tile, tv.nan_tile);
      }
      sw.next();
    }
  }
}

// ------------------------------------------------------------- host glue

// The status of each launch is its own hipLaunchKernel return code, never
// hipGetLastError(), which could report an error left by unrelated earlier
// work.  launch() keeps the first failure of the current call; check_common
// clears it when a call starts and after_launch reports and clears it.
thread_local hipError_t t_launch_err = hipSuccess;

template <typename... P, typename... A>
void launch(void (*kernel)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t s, A&&... a) {
  std::tuple<P...> args(std::forward<A>(a)...);
  const hipError_t e = std::apply(
      [&](auto&... v) {
        void* ptrs[] = {static_cast<void*>(&v)...};
        return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, lds, s);
      },
      args);
  if (e != hipSuccess && t_launch_err == hipSuccess) t_launch_err = e;
}


template <typename T>
const T* table(const rs_layout* L, size_t off) {
  return reinterpret_cast<const T*>(static_cast<const char*>(L->dev) + off);
}

rs_status check_common(const rs_layout* L, int32_t k0, int32_t k1, const char* fn) {
  t_launch_err = hipSuccess;
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

// Largest grid of one launch, in workgroups of `threads` lanes.  HIP takes
// fewer than 2^32 lanes per grid dimension; launches stay within 2^31.  The
// environment variable RS_MAX_GRID, read once, lowers the cap (tests use it
// to run the batched launch paths on small groups).
int64_t max_groups(int threads) {
  static const int64_t env_cap = [] {
    const char* e = std::getenv("RS_MAX_GRID");
    return e ? std::max<int64_t>(0, std::atoll(e)) : int64_t(0);
  }();
  const int64_t hw = (int64_t(1) << 31) / threads;
  return env_cap > 0 ? std::min(env_cap, hw) : hw;
}

// The workgroup order of pack, unpack and scale/add (runs of RS_XCD_RUN
// chunks per XCD, a power of two) and of the unmasked zero (one run per
// XCD) over ranges of at least RS_XCD_REMAP_MIN elements (0: never); the
// hardware order below that.  Environment variables of the same names, read
// once per process, override both (tests force short runs on small groups).
int64_t env_or(const char* name, int64_t dflt) {
  const char* e = std::getenv(name);
  return e ? std::atoll(e) : dflt;
}
XcdOrder xcd_run(const rs_layout* L, int32_t k0, int32_t k1, bool one_run) {
  static const int64_t min_elems = std::max<int64_t>(0, env_or("RS_XCD_REMAP_MIN", RS_XCD_REMAP_MIN));
  static const int shift = [] {  // log2 of the run, rounded down, in [0, 20]
    const int64_t run = std::max<int64_t>(1, std::min<int64_t>(env_or("RS_XCD_RUN", RS_XCD_RUN), 1 << 20));
    int sh = 0;
    while ((int64_t(2) << sh) <= run) ++sh;
    return sh;
  }();
  if (min_elems == 0 || int64_t(k1 - k0) * L->S < min_elems) return XcdOrder{kXcdNone, 0};
  return one_run ? XcdOrder{kXcdOneRun, 0} : XcdOrder{kXcdRuns, shift};
}

// The workgroup order of dequantisation: runs of RS_DEQ_XCD_RUN workgroups
// per XCD on long ranges (as xcd_run decides for the chunk kernels) when
// the class's tiles mostly belong to tensors of at least
// RS_DEQ_XCD_MIN_COLS columns, the hardware order otherwise.  Environment
// variables of the same names, read once per process, override both (tests
// force short runs on small groups).
XcdOrder deq_order(const rs_layout* L, int32_t k0, int32_t k1, int c) {
  static const int64_t min_cols = env_or("RS_DEQ_XCD_MIN_COLS", RS_DEQ_XCD_MIN_COLS);
  static const int shift = [] {  // log2 of the run, rounded down, in [0, 20]
    const int64_t run =
        std::max<int64_t>(1, std::min<int64_t>(env_or("RS_DEQ_XCD_RUN", RS_DEQ_XCD_RUN), 1 << 20));
    int sh = 0;
    while ((int64_t(2) << sh) <= run) ++sh;
    return sh;
  }();
  if (min_cols <= 0 || L->median_tile_tensor_cols[c] < min_cols ||
      xcd_run(L, k0, k1, false).mode == kXcdNone)
    return XcdOrder{kXcdNone, 0};
  return XcdOrder{kXcdRuns, shift};
}

// Workgroups for n chunk-kernel items: one per item, up to the launch cap;
// the chunk kernels stride by the grid beyond it.
dim3 chunk_grid(int64_t n) {
  return dim3(static_cast<unsigned>(std::min(n, max_groups(kThreads))));
}

rs_status after_launch(const char* fn) {
  const hipError_t e = t_launch_err;
  t_launch_err = hipSuccess;
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
                             rs_dtype buf_dt, int32_t k0, int32_t k1, void* stream) try {
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
  const dim3 g = chunk_grid(nc), b(kThreads);
  const XcdOrder run = xcd_run(L, k0, k1, false);
  if (src_dt == RS_F32 && buf_dt == RS_BF16)
    launch((pack_kernel<0, 1>), g, b, 0, s, ch, c0, nc, src, buf, run);
  else if (src_dt == RS_F32 && buf_dt == RS_F32)
    launch((pack_kernel<0, 0>), g, b, 0, s, ch, c0, nc, src, buf, run);
  else if (src_dt == RS_BF16 && buf_dt == RS_BF16)
    launch((pack_kernel<1, 1>), g, b, 0, s, ch, c0, nc, src, buf, run);
  else
    launch((pack_kernel<1, 0>), g, b, 0, s, ch, c0, nc, src, buf, run);
  return after_launch(fn);
} catch (...) {
  return rs::on_exception("rs_pack");
}

extern "C" rs_status rs_unpack(const rs_layout* L, const void* buf, rs_dtype buf_dt,
                               void* const* dst, rs_dtype dst_dt, int32_t k0, int32_t k1,
                               void* stream) try {
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
  // short launches (those xcd_run leaves in the hardware order, one rank's
  // share say) take RS_UNPACK_SHORT_LANES lanes per workgroup
  const XcdOrder run = xcd_run(L, k0, k1, false);
  constexpr int kShort = RS_UNPACK_SHORT_LANES;
  const bool narrow = run.mode == kXcdNone;
  const dim3 g(unsigned(std::min(nc, max_groups(narrow ? kShort : kThreads)))),
      b(narrow ? kShort : kThreads);
#define RS_UNPACK_LAUNCH(SK, DK)                                                        \
  (narrow ? launch((unpack_kernel<SK, DK, kShort>), g, b, 0, s, ch, c0, nc, buf, dst, run) \
          : launch((unpack_kernel<SK, DK>), g, b, 0, s, ch, c0, nc, buf, dst, run))
  if (buf_dt == RS_BF16 && dst_dt == RS_BF16)
    RS_UNPACK_LAUNCH(1, 1);
  else if (buf_dt == RS_BF16 && dst_dt == RS_F32)
    RS_UNPACK_LAUNCH(1, 0);
  else if (buf_dt == RS_F32 && dst_dt == RS_F32)
    RS_UNPACK_LAUNCH(0, 0);
  else
    RS_UNPACK_LAUNCH(0, 1);
#undef RS_UNPACK_LAUNCH
  return after_launch(fn);
} catch (...) {
  return rs::on_exception("rs_unpack");
}

extern "C" rs_status rs_group_scale_add(const rs_layout* L, float* y, const void* x,
                                        rs_dtype x_dt, float alpha, float beta,
                                        const uint8_t* tensor_mask, uint32_t* found_inf,
                                        int32_t k0, int32_t k1, void* stream) try {
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
  const dim3 g = chunk_grid(nc * RS_SCALE_SPLIT), b(kThreads);
  const XcdOrder run = xcd_run(L, k0, k1, false);
  if (x_dt == RS_F32)
    launch((scale_add_kernel<0>), g, b, 0, s, ch, c0, nc, y, x, alpha, beta, tensor_mask,
           found_inf, run);
  else
    launch((scale_add_kernel<1>), g, b, 0, s, ch, c0, nc, y, x, alpha, beta, tensor_mask,
           found_inf, run);
  return after_launch(fn);
} catch (...) {
  return rs::on_exception("rs_group_scale_add");
}

extern "C" rs_status rs_group_zero(const rs_layout* L, void* y, rs_dtype dt,
                                   const uint8_t* tensor_mask, int32_t k0, int32_t k1,
                                   void* stream) try {
  const char* fn = "rs_group_zero";
  RS_TRY(check_common(L, k0, k1, fn));
  if (!float_kind(dt)) return fail(RS_ERR_DTYPE, "rs_group_zero: dt must be RS_F32 or RS_BF16");
  RS_TRY(check_ptr(y, dt == RS_F32 ? 4 : 2, fn, "y"));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t es = dt == RS_F32 ? 4 : 2;
  char* lo = static_cast<char*>(y) + int64_t(k0) * L->S * es;
  const int64_t nbytes = int64_t(k1 - k0) * L->S * es;
  if (!tensor_mask && reinterpret_cast<uintptr_t>(lo) % 16 == 0 && nbytes % 16 == 0) {
    // the whole rank range, padding included: one contiguous fill, in
    // launches of at most the grid cap
    const int64_t per = max_groups(kThreads) * RS_FILL_BYTES;
    const XcdOrder run = xcd_run(L, k0, k1, true);
    for (int64_t o = 0; o < nbytes; o += per) {
      const int64_t nb = std::min(per, nbytes - o);
      const int64_t g = (nb + RS_FILL_BYTES - 1) / RS_FILL_BYTES;
      if (nbytes < RS_NT_STORE_BELOW)
        launch(fill_zero_kernel<true>, dim3(static_cast<unsigned>(g)), dim3(kThreads), 0,
                           s, lo + o, nb, run);
      else
        launch(fill_zero_kernel<false>, dim3(static_cast<unsigned>(g)), dim3(kThreads), 0,
                           s, lo + o, nb, run);
      RS_TRY(after_launch(fn));
    }
    return RS_OK;
  }
  const int64_t c0 = L->rank_cchunk[k0], nc = L->rank_cchunk[k1] - c0;
  if (nc == 0) return RS_OK;
  const ChunkDesc* ch = table<ChunkDesc>(L, L->off_cchunks);
  const dim3 g = chunk_grid(nc), b(kThreads);
  if (dt == RS_F32)
    launch((zero_kernel<0>), g, b, 0, s, ch, c0, nc, y, tensor_mask);
  else
    launch((zero_kernel<1>), g, b, 0, s, ch, c0, nc, y, tensor_mask);
  return after_launch(fn);
} catch (...) {
  return rs::on_exception("rs_group_zero");
}

namespace rs {
namespace {

// The norms of ranks [k0, k1) with chunk partials in `part` (at least
// sqnorm_partials() doubles): the partial kernel over the range's chunks,
// then the combine over the tensors present in the range.
int64_t sqnorm_partials(const rs_layout* L, int32_t k0, int32_t k1, int* fine) {
  // coarse chunks, unless the range has too few of them to fill the chip
  *fine = (L->rank_cchunk[k1] - L->rank_cchunk[k0]) < RS_SQNORM_FINE_BELOW ? 1 : 0;
  const std::vector<int64_t>& rb = *fine ? L->rank_chunk : L->rank_cchunk;
  return rb[k1] - rb[k0];
}

rs_status sqnorm_launch(const rs_layout* L, const float* x, double* sq_out, double* partial,
                        uint32_t* found_inf, double* part, int32_t k0, int32_t k1,
                        hipStream_t s, const char* fn) {
  int fine = 0;
  const int64_t nc = sqnorm_partials(L, k0, k1, &fine);
  const int64_t c0 = (fine ? L->rank_chunk : L->rank_cchunk)[k0];
  if (nc > 0) {
    const ChunkDesc* ct = table<ChunkDesc>(L, fine ? L->off_chunks : L->off_cchunks);
    if (fine && RS_SQNORM_FINE_LANES == 128)
      launch(sqnorm_partial_kernel<128>, dim3(unsigned(std::min(nc, max_groups(128)))), dim3(128), 0,
             s, ct, c0, nc, x, part, found_inf);
    else
      launch(sqnorm_partial_kernel<kThreads>, chunk_grid(nc), dim3(kThreads), 0, s, ct, c0, nc, x,
             part, found_inf);
  }
  // tensors with a fragment in the range: a contiguous run in buffer order
  const int64_t f0 = L->rank_frag[k0], f1 = L->rank_frag[k1];
  const int32_t t_lo = f1 > f0 ? L->frags[f0].tensor : 0;
  const int32_t t_hi = f1 > f0 ? L->frags[f1 - 1].tensor + 1 : 0;
  const unsigned groups = unsigned(t_hi - t_lo) + (t_hi - t_lo < L->n ? 1u : 0u);
  DirectFrags direct{};
  if (k1 - k0 == 1 && f1 - f0 <= kDirectFrags) {
    direct.nf = int32_t(f1 - f0);
    for (int64_t f = f0; f < f1; ++f) {
      const FragDesc& fd = L->frags[f];
      direct.cb[f - f0] = int32_t((fine ? fd.chunk_begin : fd.cchunk_begin) - c0);
      direct.ce[f - f0] = int32_t((fine ? fd.chunk_end : fd.cchunk_end) - c0);
    }
  }
  launch(sqnorm_combine_kernel, dim3(groups), dim3(kCombineWaves * kWave), 0, s,
         table<TensorDesc>(L, L->off_tensors), table<FragDesc>(L, L->off_frags), part, c0, L->n,
         k0, k1, t_lo, t_hi, sq_out, partial, fine, direct);
  return after_launch(fn);
}

}  // namespace
}  // namespace rs

extern "C" rs_status rs_ragged_sqnorm(const rs_layout* L, const float* x, double* sq_out,
                                      double* partial, uint32_t* found_inf, void* ws, int32_t k0,
                                      int32_t k1, void* stream) try {
  const char* fn = "rs_ragged_sqnorm";
  RS_TRY(check_common(L, k0, k1, fn));
  RS_TRY(check_ptr(x, 4, fn, "x"));
  RS_TRY(check_ptr(sq_out, 8, fn, "sq"));
  RS_TRY(check_ptr(ws, 8, fn, "ws"));
  if (partial) RS_TRY(check_ptr(partial, 8, fn, "partial"));
  if (found_inf) RS_TRY(check_ptr(found_inf, 4, fn, "found_inf"));
  return sqnorm_launch(L, x, sq_out, partial, found_inf, static_cast<double*>(ws), k0, k1,
                       static_cast<hipStream_t>(stream), fn);
} catch (...) {
  return rs::on_exception("rs_ragged_sqnorm");
}

extern "C" rs_status rs_block_quant(const rs_layout* L, const float* x, rs_qfmt fmt,
                                    uint8_t* codes, float* scales, uint32_t* found_inf, int32_t k0,
                                    int32_t k1, void* stream) try {
  const char* fn = "rs_block_quant";
  RS_TRY(check_common(L, k0, k1, fn));
  if (fmt != RS_Q_FP8_E4M3 && fmt != RS_Q_INT8)
    return fail(RS_ERR_DTYPE, "rs_block_quant: fmt must be RS_Q_FP8_E4M3 or RS_Q_INT8");
  RS_TRY(check_ptr(x, 4, fn, "x"));
  RS_TRY(check_ptr(codes, 1, fn, "codes"));
  if (L->num_tiles > 0) RS_TRY(check_ptr(scales, 4, fn, "scales"));  // no tiles: may be null
  if (found_inf) RS_TRY(check_ptr(found_inf, 4, fn, "found_inf"));
  // the 16-byte path needs x 16-byte aligned and codes 4-byte aligned
  const int vec_ok = (reinterpret_cast<uintptr_t>(x) % 16 == 0 &&
                      reinterpret_cast<uintptr_t>(codes) % 4 == 0) ? 1 : 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const QuantWork* wk = table<QuantWork>(L, L->off_work);
  // One launch per tile class present in the range.  Narrow tiles: one
  // sub-block, 4 slots per lane.  Wide tiles: 256-lane tiles spread over F
  // sub-blocks, more of them in launches with few work items.
  // nontemporal code stores for launches that write little (see
  // RS_NT_STORE_BELOW), and for wide tiles over ranges of at least
  // RS_QUANT_NT_WIDE_FROM buffer positions
  const int64_t span = int64_t(k1 - k0) * L->S;
  for (int c = 0; c < 2; ++c) {
    const int64_t w0 = L->rank_work[c][k0], nw = L->rank_work[c][k1] - w0;
    if (nw == 0) continue;
    const bool nts = span < RS_NT_STORE_BELOW || (c == 1 && span >= RS_QUANT_NT_WIDE_FROM);
    const int F = c == 0 ? 1 : nw < RS_QUANT_SMALL_ITEMS ? RS_QUANT_F_SMALL : RS_QUANT_F;
    const dim3 b(kThreads * F);
    const int64_t per = max_groups(kThreads * F);
    for (int64_t w1 = w0; w1 < w0 + nw; w1 += per) {  // one work item per workgroup
      const dim3 g(static_cast<unsigned>(std::min(per, w0 + nw - w1)));
#define RS_QUANT_LAUNCH(FM, NT)                                                                 \
  do {                                                                                          \
    if (c == 0)                                                                                 \
      launch((quant_kernel<FM, 1, kNarrowSlots, NT>), g, b, 0, s, wk, w1, x, codes, \
                         scales, found_inf, vec_ok);                                            \
    else if (F == RS_QUANT_F_SMALL)                                                             \
      launch((quant_kernel<FM, RS_QUANT_F_SMALL, kWideSlots / RS_QUANT_F_SMALL, NT>), \
                         g, b, 0, s, wk, w1, x, codes, scales, found_inf, vec_ok);              \
    else                                                                                        \
      launch((quant_kernel<FM, RS_QUANT_F, kWideSlots / RS_QUANT_F, NT>), g, b, 0,  \
                         s, wk, w1, x, codes, scales, found_inf, vec_ok);                       \
  } while (0)
      if (fmt == RS_Q_FP8_E4M3 && nts)
        RS_QUANT_LAUNCH(RS_Q_FP8_E4M3, true);
      else if (fmt == RS_Q_FP8_E4M3)
        RS_QUANT_LAUNCH(RS_Q_FP8_E4M3, false);
      else if (nts)
        RS_QUANT_LAUNCH(RS_Q_INT8, true);
      else
        RS_QUANT_LAUNCH(RS_Q_INT8, false);
#undef RS_QUANT_LAUNCH
      RS_TRY(after_launch(fn));
    }
  }
  return RS_OK;
} catch (...) {
  return rs::on_exception("rs_block_quant");
}

extern "C" rs_status rs_block_dequant(const rs_layout* L, const uint8_t* codes, rs_qfmt fmt,
                                      const float* scales, void* y, rs_dtype y_dt, int32_t k0,
                                      int32_t k1, void* stream) try {
  const char* fn = "rs_block_dequant";
  RS_TRY(check_common(L, k0, k1, fn));
  if (fmt != RS_Q_FP8_E4M3 && fmt != RS_Q_INT8)
    return fail(RS_ERR_DTYPE, "rs_block_dequant: fmt must be RS_Q_FP8_E4M3 or RS_Q_INT8");
  if (!float_kind(y_dt)) return fail(RS_ERR_DTYPE, "rs_block_dequant: y must be RS_F32 or RS_BF16");
  RS_TRY(check_ptr(codes, 1, fn, "codes"));
  if (L->num_tiles > 0) RS_TRY(check_ptr(scales, 4, fn, "scales"));  // no tiles: may be null
  RS_TRY(check_ptr(y, y_dt == RS_F32 ? 4 : 2, fn, "y"));
  const uintptr_t ca = reinterpret_cast<uintptr_t>(codes), ya = reinterpret_cast<uintptr_t>(y);
  int vec_ok = (ca % 4 == 0 && ya % (y_dt == RS_F32 ? 16 : 8) == 0) ? 1 : 0;
  if (vec_ok && ca % 16 == 0) vec_ok = 2;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const QuantWork* wk = table<QuantWork>(L, L->off_work);
  // nontemporal stores for launches that write little (see RS_NT_STORE_BELOW)
  const bool nts = int64_t(k1 - k0) * L->S * (y_dt == RS_F32 ? 4 : 2) < RS_NT_STORE_BELOW;
  for (int c = 0; c < 2; ++c) {  // one launch per tile class present in the range
    const int64_t w0 = L->rank_work[c][k0], nw = L->rank_work[c][k1] - w0;
    if (nw == 0) continue;
    // row bands per work item when every tile of the class and range has
    // that many rows
    int32_t min_rows = INT32_MAX;
    for (int32_t k = k0; k < k1; ++k) min_rows = std::min(min_rows, L->rank_min_tile_rows[c][k]);
    const bool split = RS_DEQ_SPLIT > 1 && min_rows >= RS_DEQ_SPLIT;
    const XcdOrder ord = deq_order(L, k0, k1, c);
    const int64_t bands = split ? RS_DEQ_SPLIT : 1;
    const dim3 b(kThreads);
    const int64_t per = std::max<int64_t>(1, max_groups(kThreads) / bands);  // items per launch
    for (int64_t w1 = w0; w1 < w0 + nw; w1 += per) {  // one workgroup per band of a work item
      const dim3 g(static_cast<unsigned>(std::min(per, w0 + nw - w1) * bands));
#define RS_DEQ_LAUNCH2(FM, YK, NT)                                                             \
  do {                                                                                         \
    if (split)                                                                                 \
      launch((dequant_kernel<FM, YK, RS_DEQ_SPLIT, NT>), g, b, 0, s, wk, w1, codes,  \
                         scales, y, vec_ok, ord);                                              \
    else                                                                                       \
      launch((dequant_kernel<FM, YK, 1, NT>), g, b, 0, s, wk, w1, codes, scales, y,  \
                         vec_ok, ord);                                                         \
  } while (0)
#define RS_DEQ_LAUNCH(FM, YK)          \
  do {                                 \
    if (nts)                           \
      RS_DEQ_LAUNCH2(FM, YK, true);    \
    else                               \
      RS_DEQ_LAUNCH2(FM, YK, false);   \
  } while (0)
      if (fmt == RS_Q_FP8_E4M3 && y_dt == RS_F32)
        RS_DEQ_LAUNCH(RS_Q_FP8_E4M3, 0);
      else if (fmt == RS_Q_FP8_E4M3)
        RS_DEQ_LAUNCH(RS_Q_FP8_E4M3, 1);
      else if (y_dt == RS_F32)
        RS_DEQ_LAUNCH(RS_Q_INT8, 0);
      else
        RS_DEQ_LAUNCH(RS_Q_INT8, 1);
#undef RS_DEQ_LAUNCH
#undef RS_DEQ_LAUNCH2
      RS_TRY(after_launch(fn));
    }
  }
  return RS_OK;
} catch (...) {
  return rs::on_exception("rs_block_dequant");
}

extern "C" rs_status rs_adamw_step(const rs_layout* L, float* p, const float* g, float* m, float* v,
                                   const rs_adamw_params* hp, const uint8_t* tensor_mask,
                                   const uint32_t* found_inf, int32_t k0, int32_t k1,
                                   void* stream) try {
  const char* fn = "rs_adamw_step";
  RS_TRY(check_common(L, k0, k1, fn));
  if (!hp) return fail(RS_ERR_INVALID_ARG, "rs_adamw_step: null hyperparameters");
  RS_TRY(check_ptr(p, 4, fn, "p"));
  RS_TRY(check_ptr(g, 4, fn, "g"));
  RS_TRY(check_ptr(m, 4, fn, "m"));
  RS_TRY(check_ptr(v, 4, fn, "v"));
  if (found_inf) RS_TRY(check_ptr(found_inf, 4, fn, "found_inf"));
  if (!(hp->bias_correction1 > 0.0f) || !(hp->bias_correction2 > 0.0f) || !(hp->grad_scale != 0.0f))
    return fail(RS_ERR_INVALID_ARG, "rs_adamw_step: bias corrections must be > 0, grad_scale != 0");
  AdamConst k;
  k.beta1 = hp->beta1;
  k.beta2 = hp->beta2;
  k.omb1 = 1.0f - hp->beta1;
  k.omb2 = 1.0f - hp->beta2;
  k.eps = hp->eps;
  const float lrwd = hp->lr * hp->weight_decay;
  k.decay = 1.0f - lrwd;
  k.step = hp->lr / hp->bias_correction1;
  k.bc2s = std::sqrt(hp->bias_correction2);
  k.inv = 1.0f / hp->grad_scale;
  const int64_t c0 = L->rank_chunk[k0], nc = L->rank_chunk[k1] - c0;
  if (nc == 0) return RS_OK;
  launch(adamw_kernel<RS_ADAMW_SPLIT>, chunk_grid(nc * RS_ADAMW_SPLIT), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), table<ChunkDesc>(L, L->off_chunks), c0, nc,
                     p, g, m, v, k, tensor_mask, found_inf, L->m);
  return after_launch(fn);
} catch (...) {
  return rs::on_exception("rs_adamw_step");
}

extern "C" rs_status rs_sgd_step(const rs_layout* L, float* p, const float* g, float* buf,
                                 const rs_sgd_params* hp, const uint8_t* tensor_mask,
                                 const uint32_t* found_inf, int32_t k0, int32_t k1, void* stream) try {
  const char* fn = "rs_sgd_step";
  RS_TRY(check_common(L, k0, k1, fn));
  if (!hp) return fail(RS_ERR_INVALID_ARG, "rs_sgd_step: null hyperparameters");
  RS_TRY(check_ptr(p, 4, fn, "p"));
  RS_TRY(check_ptr(g, 4, fn, "g"));
  RS_TRY(check_ptr(buf, 4, fn, "buf"));
  if (found_inf) RS_TRY(check_ptr(found_inf, 4, fn, "found_inf"));
  if (!(hp->grad_scale != 0.0f)) return fail(RS_ERR_INVALID_ARG, "rs_sgd_step: grad_scale == 0");
  SgdConst k;
  k.lr = hp->lr;
  k.mu = hp->momentum;
  k.wd = hp->weight_decay;
  k.inv = 1.0f / hp->grad_scale;
  k.nesterov = hp->nesterov ? 1 : 0;
  const int64_t c0 = L->rank_chunk[k0], nc = L->rank_chunk[k1] - c0;
  if (nc == 0) return RS_OK;
  launch(sgd_kernel<RS_SGD_SPLIT>, chunk_grid(nc * RS_SGD_SPLIT), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), table<ChunkDesc>(L, L->off_chunks), c0, nc,
                     p, g, buf, k, tensor_mask, found_inf, L->m);
  return after_launch(fn);
} catch (...) {
  return rs::on_exception("rs_sgd_step");
}

extern "C" rs_status rs_adamw8_step(const rs_layout* L, float* p, const float* g, uint8_t* m_codes,
                                    float* m_scales, uint8_t* v_codes, float* v_scales,
                                    rs_qfmt fmt, const rs_adamw_params* hp,
                                    const uint32_t* found_inf, int32_t k0, int32_t k1,
                                    void* stream) try {
  const char* fn = "rs_adamw8_step";
  RS_TRY(check_common(L, k0, k1, fn));
  if (!hp) return fail(RS_ERR_INVALID_ARG, "rs_adamw8_step: null hyperparameters");
  if (fmt != RS_Q_FP8_E4M3 && fmt != RS_Q_INT8)
    return fail(RS_ERR_DTYPE, "rs_adamw8_step: fmt must be RS_Q_FP8_E4M3 or RS_Q_INT8");
  RS_TRY(check_ptr(p, 4, fn, "p"));
  RS_TRY(check_ptr(g, 4, fn, "g"));
  RS_TRY(check_ptr(m_codes, 1, fn, "m_codes"));
  RS_TRY(check_ptr(v_codes, 1, fn, "v_codes"));
  if (L->num_tiles > 0) {  // no tiles: the scale arrays may be null
    RS_TRY(check_ptr(m_scales, 4, fn, "m_scales"));
    RS_TRY(check_ptr(v_scales, 4, fn, "v_scales"));
  }
  if (found_inf) RS_TRY(check_ptr(found_inf, 4, fn, "found_inf"));
  if (!(hp->bias_correction1 > 0.0f) || !(hp->bias_correction2 > 0.0f) || !(hp->grad_scale != 0.0f))
    return fail(RS_ERR_INVALID_ARG, "rs_adamw8_step: bias corrections must be > 0, grad_scale != 0");
  AdamConst k;
  k.beta1 = hp->beta1;
  k.beta2 = hp->beta2;
  k.omb1 = 1.0f - hp->beta1;
  k.omb2 = 1.0f - hp->beta2;
  k.eps = hp->eps;
  const float lrwd = hp->lr * hp->weight_decay;
  k.decay = 1.0f - lrwd;
  k.step = hp->lr / hp->bias_correction1;
  k.bc2s = std::sqrt(hp->bias_correction2);
  k.inv = 1.0f / hp->grad_scale;
  k.rbc2s = 1.0f / k.bc2s;
  const bool divc = RS_ADAM8_DIVC && div_by_const_ok(k.bc2s);
  const int vec_ok = (reinterpret_cast<uintptr_t>(p) % 16 == 0 &&
                      reinterpret_cast<uintptr_t>(g) % 16 == 0 &&
                      reinterpret_cast<uintptr_t>(m_codes) % 4 == 0 &&
                      reinterpret_cast<uintptr_t>(v_codes) % 4 == 0) ? 1 : 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const QuantWork* wk = table<QuantWork>(L, L->off_work);
  // one launch per tile class present in the range: narrow tiles with one
  // sub-block of 4 slots per lane, wide tiles over RS_ADAM8_F sub-blocks
  for (int c = 0; c < 2; ++c) {
    const int64_t w0 = L->rank_work[c][k0], nw = L->rank_work[c][k1] - w0;
    if (nw == 0) continue;
    const int F = c == 0 ? 1 : RS_ADAM8_F;
    const dim3 b(kThreads * F);
    const int64_t per = max_groups(kThreads * F);
    for (int64_t w1 = w0; w1 < w0 + nw; w1 += per) {  // one work item per workgroup
      const dim3 gr(static_cast<unsigned>(std::min(per, w0 + nw - w1)));
#define RS_ADAM8_LAUNCH(FM, DC)                                                                 \
  do {                                                                                          \
    if (c == 0)                                                                                 \
      launch((adamw8_kernel<FM, 1, kNarrowSlots, DC>), gr, b, 0, s, wk, w1, p, g,               \
             m_codes, m_scales, v_codes, v_scales, k, found_inf, L->m, vec_ok);                 \
    else                                                                                        \
      launch((adamw8_kernel<FM, RS_ADAM8_F, kWideSlots / RS_ADAM8_F, DC>), gr, b, 0, s, wk, w1, \
             p, g, m_codes, m_scales, v_codes, v_scales, k, found_inf, L->m, vec_ok);           \
  } while (0)
      if (fmt == RS_Q_FP8_E4M3 && divc)
        RS_ADAM8_LAUNCH(RS_Q_FP8_E4M3, true);
      else if (fmt == RS_Q_FP8_E4M3)
        RS_ADAM8_LAUNCH(RS_Q_FP8_E4M3, false);
      else if (divc)
        RS_ADAM8_LAUNCH(RS_Q_INT8, true);
      else
        RS_ADAM8_LAUNCH(RS_Q_INT8, false);
#undef RS_ADAM8_LAUNCH
      RS_TRY(after_launch(fn));
    }
  }
  return RS_OK;
} catch (...) {
  return rs::on_exception("rs_adamw8_step");
}

// ------------------------------------------------------ no-allocation norms
//
// rs_ragged_sqnorm_noalloc keeps the chunk partials in this file-scope device
// array instead of a caller workspace.  Each GPU the library runs on holds
// its own copy until the process ends.  Host code never passes the array's
// name to a kernel: its device address comes from hipGetSymbolAddress, taken
// once per device with that device current and kept in g_scratch_ptr.
constexpr int64_t kStaticPartials = 131072;  // 1 MiB of fp64 partials
static __device__ __align__(256) double scratch[kStaticPartials];

namespace {

constexpr int kMaxScratchDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// The current device's copy of `scratch` (looked up on the device's first call).
rs_status static_scratch(const char* fn, double** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(RS_ERR_HIP, std::string(fn) + ": " + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(RS_ERR_INVALID_ARG, std::string(fn) + ": device index beyond 255");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(RS_ERR_HIP, std::string(fn) + ": hipGetSymbolAddress: " + hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = static_cast<double*>(g_scratch_ptr[dev]);
  return RS_OK;
}

}  // namespace

extern "C" rs_status rs_ragged_sqnorm_noalloc(const rs_layout* L, const float* x, double* sq_out,
                                              double* partial, uint32_t* found_inf, int32_t k0,
                                              int32_t k1, void* stream) try {
  const char* fn = "rs_ragged_sqnorm_noalloc";
  RS_TRY(check_common(L, k0, k1, fn));
  RS_TRY(check_ptr(x, 4, fn, "x"));
  RS_TRY(check_ptr(sq_out, 8, fn, "sq"));
  if (partial) RS_TRY(check_ptr(partial, 8, fn, "partial"));
  if (found_inf) RS_TRY(check_ptr(found_inf, 4, fn, "found_inf"));
  int fine = 0;
  const int64_t need = sqnorm_partials(L, k0, k1, &fine);
  if (need > kStaticPartials)
    return fail(RS_ERR_INVALID_ARG,
                std::string(fn) + ": the rank range has " + std::to_string(need) +
                    " work chunks and the static scratch holds " + std::to_string(kStaticPartials) +
                    " partials; use rs_ragged_sqnorm with a workspace or a smaller range");
  double* part = nullptr;
  RS_TRY(static_scratch(fn, &part));
  return sqnorm_launch(L, x, sq_out, partial, found_inf, part, k0, k1,
                       static_cast<hipStream_t>(stream), fn);
} catch (...) {
  return rs::on_exception("rs_ragged_sqnorm_noalloc");
}
