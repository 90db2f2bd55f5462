"""Oracle number conversions (test infrastructure; never used by the product).

Each conversion is written from its format definition, in float64 or integer
arithmetic that is exact for every fp32 input, so it can be checked by eye:

* bf16: IEEE-754 binary32 truncated to its top 16 bits with round to nearest,
  ties to even; overflow becomes +-Inf, NaN stays a quiet NaN with its sign.
  This is the fp32->bf16 cast of native mixed precision ("PyTorch FSDP:
  Experiences on Scaling Fully Sharded Data Parallel", native mixed precision
  section: the FlatParameter is cast once before forward).
* FP8 E4M3FN (OCP 8-bit floating point, "fn" variant): 1 sign, 4 exponent
  bits with bias 7, 3 mantissa bits, no infinities, NaN = S.1111.111, largest
  finite 448.  Saturating round-to-nearest-even: |q| > 448 (and +-Inf) give
  +-448; NaN gives 0x7F.
* INT8: round half to even, then clip to [-127, 127]; NaN gives 0.

These are the block-quantisation code formats of the 8-bit optimizer /
block-wise FP8 case (veScale-FSDP: Flexible and High-Performance FSDP at
Scale, problem statement and section 6.3).
"""
from __future__ import annotations

import numpy as np

F32 = np.float32


def f32_bits(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=F32).view(np.uint32)


def bits_f32(u: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(u, dtype=np.uint32).view(F32)


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even."""
    u = f32_bits(x).astype(np.uint64)
    hi = u >> 16
    lo = u & 0xFFFF
    # exact comparison of the dropped half against one half-ulp of bf16
    up = (lo > 0x8000) | ((lo == 0x8000) & ((hi & 1) == 1))
    out = hi + up.astype(np.uint64)
    x32 = np.asarray(x, dtype=F32)
    nan = np.isnan(x32)
    out = np.where(nan, hi | 0x40, out)
    return out.astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 (exact)."""
    return bits_f32(np.asarray(b, dtype=np.uint32) << 16)


E4M3_MAX = 448.0
INT8_MAX = 127.0


def e4m3fn_bits_from_f32(q: np.ndarray) -> np.ndarray:
    """fp32 -> FP8 E4M3FN codes (uint8), saturating RNE, NaN -> 0x7F."""
    with np.errstate(invalid="ignore"):
        q64 = np.asarray(q, dtype=F32).astype(np.float64)
    out = np.zeros(q64.shape, dtype=np.uint8)
    flat_q = q64.reshape(-1)
    flat = out.reshape(-1)
    nan = np.isnan(flat_q)
    sign = np.signbit(flat_q)
    a = np.minimum(np.abs(np.where(nan, 0.0, flat_q)), E4M3_MAX)
    # subnormal range: a < 2^-6 is a multiple of 2^-9 after rounding
    sub = a < 2.0 ** -6
    code = np.zeros(a.shape, dtype=np.int64)
    code[sub] = np.rint(a[sub] * 2.0 ** 9).astype(np.int64)  # 8 means 2^-6 = code 0x08
    # normal range: a = mant * 2^e with mant in [1, 2); keep 3 fraction bits
    nrm = ~sub
    mant, ex = np.frexp(a[nrm])          # a = mant * 2^ex, mant in [0.5, 1)
    e = ex.astype(np.int64) - 1          # a = (2*mant) * 2^e
    frac = np.rint((2.0 * mant - 1.0) * 8.0).astype(np.int64)
    carry = frac == 8
    e = e + carry
    frac = np.where(carry, 0, frac)
    code[nrm] = ((e + 7) << 3) | frac
    flat[:] = (code | (sign.astype(np.int64) << 7)).astype(np.uint8)
    flat[nan] = 0x7F
    return out


def e4m3fn_to_f64(codes: np.ndarray) -> np.ndarray:
    """Decode E4M3FN codes (uint8) to float64; 0x7F / 0xFF decode to NaN."""
    c = np.asarray(codes, dtype=np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    f = c & 7
    val = np.where(e == 0, f * 2.0 ** -9, (1.0 + f / 8.0) * np.exp2(e - 7.0))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return s * val


def int8_from_f32(q: np.ndarray) -> np.ndarray:
    """fp32 -> int8 codes (as int8): round half to even, clip to +-127."""
    q32 = np.asarray(q, dtype=F32)
    nan = np.isnan(q32)
    r = np.rint(np.where(nan, F32(0), q32).astype(np.float64))
    r = np.clip(r, -INT8_MAX, INT8_MAX)
    return r.astype(np.int8)
