"""Full-size cases of the tile operations (quantisation, dequantisation,
8-bit AdamW), shared by tests/test_gpu_fullsize.py and
tests/golden/make_fullsize_digests.py.

This module holds seeded inputs beyond workloads.make_inputs (the 8-bit AdamW
moment codes and scales, the step's hyperparameters), the list of fragments
(one quantised tensor's tiles inside one rank) that results are compared by,
and the digest of a fragment's outputs.  It holds none of the method's
arithmetic: the expected outputs come from oracle/, the observed ones from
the C-ABI.
"""
from __future__ import annotations

import hashlib
from typing import List, Tuple

import numpy as np

from oracle import ops as O

GROUPS = ("llama3_8b_layer", "moe_experts", "llama70b_layer", "ragged_mixed")
ALIGN = 16
# Tensors with more tiles than this (the mixed group's 128256 x 4096 embedding
# in one-row tiles: 4.1M of them) are compared on a sample of tiles instead.
SAMPLE_ABOVE = 1 << 20

ADAMW8_HP = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, wd=0.1, bc1=1 - 0.9 ** 5,
                 bc2=1 - 0.95 ** 5, grad_scale=1.0)
F32_NAN = np.uint32(0x7FC00000)


def flat(arrays, offsets, total: int) -> np.ndarray:
    """fp32 buffer image: each array at its offset, zeros elsewhere."""
    b = np.zeros(total, np.float32)
    for a, l in zip(arrays, offsets):
        b[l:l + a.size] = a.reshape(-1)
    return b


def random_codes(rng, n: int, fmt: str, signed: bool) -> np.ndarray:
    """Seeded valid codes: INT8 in [-127, 127] (or [0, 127]); E4M3FN without
    the NaN codes (and without the sign bit when unsigned)."""
    if fmt == "int8":
        lo = -127 if signed else 0
        return rng.integers(lo, 128, size=n, dtype=np.int16).astype(np.int8).view(np.uint8)
    c = rng.integers(0, 0x7F, size=n, dtype=np.uint8)          # 0x00..0x7E
    if signed:
        c |= (rng.integers(0, 2, size=n, dtype=np.uint8) << 7)
    return c


def adamw8_state(total: int, n_tiles: int, fmt: str):
    """(m codes, v codes, m scales, v scales) of the 8-bit AdamW case:
    seeded random codes and small positive scales."""
    rng = np.random.default_rng(31)
    qmax = 448.0 if fmt == "fp8_e4m3" else 127.0
    mc0 = random_codes(rng, total, fmt, True)
    vc0 = random_codes(rng, total, fmt, False)
    ms0 = (np.abs(rng.standard_normal(n_tiles)) * 1e-4 / qmax).astype(np.float32)
    vs0 = (np.abs(rng.standard_normal(n_tiles)) * 1e-6 / qmax).astype(np.float32)
    return mc0, vc0, ms0, vs0


def tile_ranks(spec, l: int, S: int) -> np.ndarray:
    """Rank of every tile of a quantised tensor, in row-major tile order
    (non-decreasing, since tile starts increase in that order)."""
    ntr, ntc = O.tile_counts(spec)
    r0 = np.arange(ntr, dtype=np.int64) * spec.q_rows
    c0 = np.arange(ntc, dtype=np.int64) * spec.q_cols
    return ((l + r0[:, None] * spec.cols + c0[None, :]) // S).reshape(-1)


def fragments(specs, offsets, S: int) -> List[Tuple[int, int, int, int, int, int]]:
    """(tensor, rank, lo, hi, first tile, end tile) for every quantised
    tensor with at most SAMPLE_ABOVE tiles and every rank it touches:
    buffer positions [lo, hi) and global tile indices [first, end)."""
    out, base = [], 0
    for t, (s, l) in enumerate(zip(specs, offsets)):
        if not s.q_rows:
            continue
        rk = tile_ranks(s, l, S)
        if rk.size <= SAMPLE_ABOVE:
            for k in np.unique(rk):
                on = np.flatnonzero(rk == k)
                lo, hi = max(l, int(k) * S), min(l + s.numel, (int(k) + 1) * S)
                out.append((t, int(k), lo, hi, base + int(on[0]), base + int(on[-1]) + 1))
        base += rk.size
    return out


def sampled_tensors(specs):
    """Indices of the quantised tensors compared on a tile sample."""
    return [t for t, s in enumerate(specs)
            if s.q_rows and np.prod(O.tile_counts(s)) > SAMPLE_ABOVE]


def digest(*arrays) -> str:
    """First 16 hex digits of SHA-256 over the arrays' bytes, fp32 NaNs
    replaced by one quiet NaN first (NaN payloads are not compared)."""
    h = hashlib.sha256()
    for a in arrays:
        a = np.ascontiguousarray(a)
        if a.dtype == np.float32:
            a = np.where(np.isnan(a), F32_NAN, a.view(np.uint32))
        h.update(a.tobytes())
    return h.hexdigest()[:16]
