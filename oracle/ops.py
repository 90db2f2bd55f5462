"""Oracle for the grouped flat-buffer operations (test infrastructure).

Only tests, the smoke check and the benchmark's CPU baseline may use this
module; the product path never imports it.

Everything here works on a planned layout (oracle.plan): tensor t lives at
buffer positions [l_t, l_t + E_t); rank k owns [k*S, (k+1)*S).  Every
operation takes a rank range [k0, k1) and touches only buffer positions in
[k0*S, k1*S): the part of the group one rank (or a few) holds, which is what
each device would run locally in a multi-GPU setting.

Sources (all from the pages):
* pack / unpack - the copy into and out of the communication buffer that
  FSDP2 does per parameter (Copy-In / Copy-Out, veScale-FSDP: Flexible and
  High-Performance FSDP at Scale, DBuffer section and Figure 2), with the
  fp32 -> bf16 cast of native mixed precision fused in ("PyTorch FSDP:
  Experiences on Scaling Fully Sharded Data Parallel", native mixed
  precision section); rebuilding a tensor from the flat buffer
  (veScale 深度技术分析, section 三 / RaggedShard Placement).
* group scale/add and zero - DBuffer's group-level add, scale and zero
  operators run over a whole tensor group at once (veScale-FSDP, DBuffer
  section, item 1); accumulation is gradient accumulation without
  communication ("PyTorch FSDP", communication optimisation 4); scaling with
  a non-finite check is the sharded gradient scaler's unscale
  ("PyTorch FSDP", native mixed precision section; veScale 深度技术分析,
  OpDispatcher: the found-inf handler).
* ragged squared norms - linalg_vector_norm over a tensor whose shard
  boundaries do not match its own (veScale 深度技术分析, OpDispatcher:
  the ragged norm handler); per-parameter norms are what element-wise
  sharding loses ("PyTorch FSDP", known limitations).
* block quantisation - absmax block INT8/FP8 quantisation that each device
  runs on its local shard without communication because block boundaries
  coincide with shard boundaries (veScale-FSDP, RaggedShard format section
  and section 6.3).

Arithmetic is fp32 where the operation is specified in fp32 (scale/add,
quantisation), fp64 for the norms.
"""
from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

import numpy as np

from . import casts
from .plan import Item, fragments

F32 = np.float32


def _range_of(l: int, n: int, S: int, k0: int, k1: int) -> Tuple[int, int]:
    """Element range [i0, i1) of a tensor at offset l that lies in ranks [k0, k1)."""
    lo = max(l, k0 * S)
    hi = min(l + n, k1 * S)
    if hi <= lo:
        return 0, 0
    return lo - l, hi - l


def pack(tensors: Sequence[np.ndarray], offsets: Sequence[int], S: int, m: int,
         buf: np.ndarray, buf_dtype: str, k0: int, k1: int, inplace: bool = False) -> np.ndarray:
    """buf[l_t + i] = cast(tensor_t.flat[i]) for positions in ranks [k0, k1);
    every other position of those ranks (the padding between tensors) = 0.

    buf holds fp32 values (buf_dtype "f32") or bf16 bit patterns ("bf16",
    uint16 array).  Sources are fp32 arrays or bf16 bit patterns (uint16).
    Returns a new array (buf itself when inplace); positions outside
    [k0*S, k1*S) are kept.
    """
    out = buf if inplace else buf.copy()
    out[k0 * S:k1 * S] = 0
    for t, l in zip(tensors, offsets):
        flat = np.asarray(t).reshape(-1)
        i0, i1 = _range_of(l, flat.size, S, k0, k1)
        if i1 <= i0:
            continue
        seg = flat[i0:i1]
        out[l + i0:l + i1] = _convert(seg, buf_dtype)
    return out


def _convert(seg: np.ndarray, to: str) -> np.ndarray:
    """Value conversion between fp32 arrays and bf16 bit patterns."""
    if seg.dtype == np.uint16:            # bf16 source
        return seg.copy() if to == "bf16" else casts.bf16_to_f32(seg)
    seg = np.asarray(seg, dtype=F32)
    return casts.bf16_bits_from_f32(seg) if to == "bf16" else seg.copy()


def unpack(buf: np.ndarray, shapes: Sequence[Tuple[int, int]], offsets: Sequence[int],
           S: int, m: int, dsts: Sequence[np.ndarray], dst_dtype: str,
           k0: int, k1: int, inplace: bool = False) -> List[np.ndarray]:
    """dst_t.flat[i] = cast(buf[l_t + i]) for positions in ranks [k0, k1);
    other destination elements are kept.  With inplace the destinations
    (contiguous arrays) are written and returned as views."""
    out = []
    for (r, c), l, d in zip(shapes, offsets, dsts):
        n = r * c
        dd = np.asarray(d).reshape(-1)
        if not inplace:
            dd = dd.copy()
        i0, i1 = _range_of(l, n, S, k0, k1)
        if i1 > i0:
            dd[i0:i1] = _convert(buf[l + i0:l + i1], dst_dtype)
        out.append(dd.reshape(r, c))
    return out


def scale_add(y: np.ndarray, x: np.ndarray, alpha: float, beta: float,
              items: Sequence[Item], offsets: Sequence[int], S: int, m: int,
              k0: int, k1: int, mask: Optional[Sequence[int]] = None, inplace: bool = False
              ) -> Tuple[np.ndarray, np.ndarray]:
    """y <- fl(fl(alpha*y) + fl(beta*x)) in fp32 over the tensor elements of
    ranks [k0, k1) (padding untouched; tensors with mask[t] == 0 skipped).

    x is fp32 or bf16 bit patterns (uint16).  found_inf[k] = 1 when any value
    written in rank k is not finite.  Returns (new y, found_inf[m] uint32);
    with inplace the new y is y itself.
    """
    out = y if inplace else y.copy()
    found = np.zeros(m, dtype=np.uint32)
    a, b = F32(alpha), F32(beta)
    for tid, k, lo, hi in fragments(items, offsets, S, m):
        if not (k0 <= k < k1) or (mask is not None and not mask[tid]):
            continue
        xs = x[lo:hi]
        xs = casts.bf16_to_f32(xs) if xs.dtype == np.uint16 else xs.astype(F32)
        with np.errstate(invalid="ignore", over="ignore"):   # Inf/NaN inputs are expected
            u = a * out[lo:hi]            # fp32 products and sum, each rounded
            v = b * xs
            w = (u + v).astype(F32)
        out[lo:hi] = w
        if not np.all(np.isfinite(w)):
            found[k] = 1
    return out, found


def zero(y: np.ndarray, items: Sequence[Item], offsets: Sequence[int], S: int, m: int,
         k0: int, k1: int, mask: Optional[Sequence[int]] = None, inplace: bool = False
         ) -> np.ndarray:
    """y <- +0 on the tensor elements of ranks [k0, k1) whose mask is set;
    with no mask, on every position of those ranks including padding.
    Returns a new array (y itself when inplace)."""
    out = y if inplace else y.copy()
    if mask is None:
        out[k0 * S:k1 * S] = 0
        return out
    for tid, k, lo, hi in fragments(items, offsets, S, m):
        if k0 <= k < k1 and mask[tid]:
            out[lo:hi] = 0
    return out


def sqnorm(x: np.ndarray, items: Sequence[Item], offsets: Sequence[int], S: int, m: int,
           k0: int, k1: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Per-tensor sum of squares over the elements that lie in ranks [k0, k1).

    Returns (sq[T] fp64, partial[m][T] fp64 where partial[k][t] is the sum
    over tensor t's fragment in rank k, found_inf[m] uint32 set when a value
    read in rank k is not finite).  Squares and sums are fp64; any NaN makes
    the sum NaN, otherwise any infinity makes it +Inf.
    """
    T = len(items)
    sq = np.zeros(T, dtype=np.float64)
    part = np.zeros((m, T), dtype=np.float64)
    found = np.zeros(m, dtype=np.uint32)
    for tid, k, lo, hi in fragments(items, offsets, S, m):
        if not (k0 <= k < k1):
            continue
        v = x[lo:hi].astype(np.float64)
        part[k, tid] = np.sum(v * v)
        if not np.all(np.isfinite(v)):
            found[k] = 1
    for t, (it, l) in enumerate(zip(items, offsets)):
        i0, i1 = _range_of(l, it.numel, S, k0, k1)
        v = x[l + i0:l + i1].astype(np.float64)
        sq[t] = np.sum(v * v)
    return sq, part, found


CANONICAL_NAN = np.uint32(0x7FC00000)


def tile_grid(rows: int, cols: int, q_rows: int, q_cols: int):
    """Tiles of a rows x cols tensor in row-major tile order: (r0, r1, c0, c1)."""
    out = []
    for r0 in range(0, rows, q_rows):
        for c0 in range(0, cols, q_cols):
            out.append((r0, min(rows, r0 + q_rows), c0, min(cols, c0 + q_cols)))
    return out


def quant_tile(tile: np.ndarray, fmt: str) -> Tuple[np.float32, np.ndarray]:
    """Absmax block quantisation of one tile.

    amax = max|x| (NaN if any element is NaN); scale = fp32(amax / Q) with
    Q = 448 (FP8 E4M3FN) or 127 (INT8); codes = encode(fp32(x / scale)).
    A zero scale gives all-zero codes; a NaN scale is stored as the quiet NaN
    0x7FC00000.  Returns (scale, codes as uint8 with the tile's shape).
    """
    x = np.asarray(tile, dtype=F32)
    Q = F32(casts.E4M3_MAX if fmt == "fp8_e4m3" else casts.INT8_MAX)
    if np.any(np.isnan(x)):
        amax = F32(np.nan)
    else:
        amax = F32(np.max(np.abs(x))) if x.size else F32(0)
    with np.errstate(all="ignore"):
        scale = F32(amax / Q)
    if scale == 0:
        return scale, np.zeros(x.shape, dtype=np.uint8)
    if np.isnan(scale):
        scale = CANONICAL_NAN.view(F32)
    with np.errstate(all="ignore"):
        q = (x / scale).astype(F32)
    if fmt == "fp8_e4m3":
        codes = casts.e4m3fn_bits_from_f32(q)
    else:
        codes = casts.int8_from_f32(q).view(np.uint8)
    return scale, codes


def tile_counts(spec) -> Tuple[int, int]:
    """(tile rows, tile cols) of a quantised tensor."""
    return -(-spec.rows // spec.q_rows), -(-spec.cols // spec.q_cols)


def tile_bounds(spec, local: int) -> Tuple[int, int, int, int]:
    """Tile number `local` of a tensor in row-major tile order -> (r0, r1, c0, c1)."""
    _, ntc = tile_counts(spec)
    ti, tj = divmod(local, ntc)
    r0, c0 = ti * spec.q_rows, tj * spec.q_cols
    return r0, min(spec.rows, r0 + spec.q_rows), c0, min(spec.cols, c0 + spec.q_cols)


def block_quant(x: np.ndarray, specs, offsets: Sequence[int], S: int, m: int, fmt: str,
                k0: int, k1: int, codes: np.ndarray, scales: np.ndarray,
                only_tiles=None, inplace: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """Quantise every tile of every quantised tensor that lies in ranks [k0, k1).

    codes: uint8 array parallel to the buffer (codes[p] encodes buffer
    position p); scales: fp32, one per tile, tiles numbered tensor by tensor
    (quantised tensors only, in group order), row-major inside a tensor.
    Positions and scales of other tiles are kept.  Every tile must lie inside
    one rank; an exception is raised otherwise.  only_tiles, when given, is a
    collection of global tile indices to compute (a sample of a large group).
    With inplace, codes and scales themselves are written and returned.
    """
    if not inplace:
        codes = codes.copy()
        scales = scales.copy()
    wanted = None if only_tiles is None else set(int(i) for i in only_tiles)
    base = 0
    for spec, l in zip(specs, offsets):
        if spec.q_rows <= 0:
            continue
        ntr, ntc = tile_counts(spec)
        count = ntr * ntc
        if wanted is None:
            locals_ = range(count)
        else:
            locals_ = sorted(i - base for i in wanted if base <= i < base + count)
        C = spec.cols
        for idx in locals_:
            r0, r1, c0, c1 = tile_bounds(spec, idx)
            first = l + r0 * C + c0
            last = l + (r1 - 1) * C + (c1 - 1)
            k = first // S
            if last // S != k:
                raise ValueError(f"tile {base + idx} of {spec.name} straddles a shard boundary")
            if not (k0 <= k < k1):
                continue
            pos = l + (np.arange(r0, r1)[:, None] * C + np.arange(c0, c1)[None, :])
            sc, cd = quant_tile(x[pos], fmt)
            scales[base + idx] = sc
            codes[pos] = cd
        base += count
    return codes, scales


def num_tiles(specs) -> int:
    return sum(tile_counts(s)[0] * tile_counts(s)[1] for s in specs if s.q_rows > 0)


def decode_codes(codes: np.ndarray, fmt: str) -> np.ndarray:
    """Code -> fp32 value (exact): E4M3FN per the OCP definition (0x7F/0xFF
    are NaN), INT8 as a signed integer."""
    c = np.asarray(codes, dtype=np.uint8)
    if fmt == "fp8_e4m3":
        return casts.e4m3fn_to_f64(c).astype(F32)
    return c.view(np.int8).astype(F32)


def block_dequant(codes: np.ndarray, scales: np.ndarray, specs, offsets: Sequence[int], S: int,
                  m: int, fmt: str, k0: int, k1: int, y: np.ndarray, y_dtype: str,
                  only_tiles=None, inplace: bool = False) -> np.ndarray:
    """Inverse of block_quant: y[p] = fl32(decode(codes[p]) * scale) for every
    element of every quantised tile in ranks [k0, k1); y holds fp32 values
    ("f32") or bf16 bit patterns ("bf16", the fp32 product rounded to
    nearest even).  Other positions of y are kept; with inplace, y itself is
    written and returned.

    This is the dequantisation step of an 8-bit optimizer's state
    (veScale-FSDP: Flexible and High-Performance FSDP at Scale, section 6.3).
    """
    if not inplace:
        y = y.copy()
    wanted = None if only_tiles is None else set(int(i) for i in only_tiles)
    base = 0
    for spec, l in zip(specs, offsets):
        if spec.q_rows <= 0:
            continue
        ntr, ntc = tile_counts(spec)
        count = ntr * ntc
        locals_ = range(count) if wanted is None else sorted(i - base for i in wanted
                                                                if base <= i < base + count)
        for idx in locals_:
            r0, r1, c0, c1 = tile_bounds(spec, idx)
            first = l + r0 * spec.cols + c0
            if not (k0 <= first // S < k1):
                continue
            pos = l + (np.arange(r0, r1)[:, None] * spec.cols + np.arange(c0, c1)[None, :])
            with np.errstate(all="ignore"):
                val = (decode_codes(codes[pos], fmt) * F32(scales[base + idx])).astype(F32)
            y[pos] = casts.bf16_bits_from_f32(val) if y_dtype == "bf16" else val
        base += count
    return y


def quant_found_inf(x: np.ndarray, specs, offsets: Sequence[int], S: int, m: int,
                    k0: int, k1: int) -> np.ndarray:
    """found_inf[k] = 1 when a quantised element read in rank k (k0 <= k < k1)
    is not finite - the non-finite check of the sharded gradient scaler
    applied to the values being quantised ("PyTorch FSDP", native mixed
    precision section)."""
    found = np.zeros(m, dtype=np.uint32)
    for spec, l in zip(specs, offsets):
        if spec.q_rows <= 0:
            continue
        for k in range(max(k0, l // S), min(k1, (l + spec.numel - 1) // S + 1)):
            lo, hi = max(l, k * S), min(l + spec.numel, (k + 1) * S)
            if lo < hi and not np.all(np.isfinite(x[lo:hi])):
                found[k] = 1
    return found
