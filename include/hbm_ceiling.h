/*
 * hbm_ceiling.h - plain streaming kernels that measure what MI355X's HBM
 * delivers for each read:write mix the grouped operations use: the practical
 * ceiling next to the 8 TB/s peak.  Measurement support for bench.py, not
 * part of the hot path: no layout, no descriptor table, one contiguous
 * buffer per stream, every access a 128-bit global load or store.
 *
 * Kinds and the operation whose byte mix each matches:
 *   HC_READ          x read (fp32), one word per workgroup written  - norms
 *   HC_WRITE         y = 0                                           - zero
 *   HC_COPY          y = x (same width)                              - unpack
 *   HC_AXPBY_INPLACE y = a*y + b*x, fp32, y read and written in place - scale/add
 *   HC_AXPBY         z = a*y + b*x, fp32, z a third buffer
 *   HC_F32_TO_BF16   y(bf16) = x(fp32) truncated: 2 bytes read per byte written - pack
 *   HC_F32_TO_U8     y(u8) = low byte of x(fp32): 4 read per 1 written - quantisation
 *   HC_U8_TO_F32     y(fp32) = x(u8) widened: 1 read per 4 written   - dequantisation
 *
 * hc_stream - one launch of kind `kind` over n fp32 elements (n u8 elements
 * for the u8 side of the conversions).
 *   x, y, z   device pointers, 16-byte aligned; unused ones may be NULL
 *             (HC_READ writes one word per workgroup to y: y holds n/1024
 *             words)
 *   n         elements, a multiple of 4096 * vec (the narrow forms convert
 *             4 elements per unit, the wide ones 8 or 16)
 *   vec       16-byte vectors per lane per workgroup: 1, 2, 4 or 8
 *   nt        1: nontemporal loads and stores
 *   stream    hipStream_t as void*
 * Returns 0, or -1 for a bad argument (nothing launched), or -6 when the
 * launch fails.  Each workgroup of 256 lanes covers 256*vec contiguous
 * 16-byte vectors of the widest stream (one block), lane-strided, as the
 * grouped kernels do; the blocks go to workgroups in the hardware order or
 * grouped by XCD (HC_XCD_RUNS, HC_XCD_ONE), as the grouped kernels may.
 */
#ifndef HBM_CEILING_H
#define HBM_CEILING_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  HC_READ = 0,
  HC_WRITE = 1,
  HC_COPY = 2,
  HC_AXPBY_INPLACE = 3,
  HC_AXPBY = 4,
  HC_F32_TO_BF16 = 5,
  HC_F32_TO_U8 = 6,
  HC_U8_TO_F32 = 7,
  /* added to a conversion kind: the narrow form, in which lane i converts
   * one 16-byte vector of the wider side and the narrower side is written or
   * read as consecutive 8- or 4-byte words, so every instruction of a wave
   * touches one contiguous span on both sides */
  HC_NARROW = 16,
  /* added to any kind: the workgroup order.  The hardware hands workgroup b
   * to XCD b % 8.  HC_XCD_RUNS: XCD x takes block x of every round of 8 runs
   * of 128 consecutive blocks; HC_XCD_ONE: each XCD takes one contiguous run
   * of about 1/8 of the blocks (not both) */
  HC_XCD_RUNS = 32,
  HC_XCD_ONE = 64
};

int hc_stream(int kind, const void* x, void* y, void* z, int64_t n, int vec, int nt, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HBM_CEILING_H */
