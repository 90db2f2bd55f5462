"""Seeded synthetic workloads for the RaggedShard flat-buffer hot path.

This module only describes tensor groups and draws random numbers. It holds
none of the method's arithmetic (no planning, casting, scaling, norms or
quantisation), so both the CPU oracle and the HIP path may take their inputs
from it without sharing any of the computation under test.

Workload shapes follow the five parameter groups the build is measured on:
a toy two-layer unit, one Llama-3-8B-shaped decoder layer, a ragged mixed
group with a row-sharded embedding, a 64-expert MoE unit and one
Llama-70B-shaped layer. The pages evaluate on end-to-end training of
Llama-3-70B, GPT-OSS-120B, DeepSeek-V3 and internal MoE models
(veScale-FSDP: Flexible and High-Performance FSDP at Scale, experiment
setup); no dataset or weights are involved on this path, so random tensors
of these shapes stand in for those models' parameter groups.

Granularity reading (veScale-FSDP, RaggedShard format section, and the
6.3 case study: "32x32 blocks with 32-row granularity"): a tensor quantised
in b x b blocks may only be cut between row bands of b rows, so its granule
is b rows; a row-wise tensor has a granule of one row; vectors are
element-granular. Quantisation tiles are granule-rows x b columns.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Sequence, Tuple

import numpy as np


@dataclass(frozen=True)
class TensorSpec:
    """One row-major parameter tensor of a group.

    gran_rows: rows per indivisible granule (0 = element granularity).
    q_rows, q_cols: quantisation tile shape (0, 0 = not quantised).
    """

    name: str
    rows: int
    cols: int
    gran_rows: int
    q_rows: int = 0
    q_cols: int = 0

    @property
    def numel(self) -> int:
        return self.rows * self.cols


@dataclass(frozen=True)
class Workload:
    name: str
    tensors: Tuple[TensorSpec, ...]
    m: int                       # virtual ranks (slices of one buffer)
    qfmt: str                    # "fp8_e4m3" or "int8"
    block: int                   # block edge used for granules and tiles
    grad_dist: str = "normal"    # "normal" or "student_t3"
    nonfinite_frac: float = 0.0  # fraction of grad elements set to +-Inf/NaN
    seed: int = 0
    param_sigma: float = 0.02
    grad_sigma: float = 1e-3
    description: str = ""

    @property
    def numel(self) -> int:
        return sum(t.numel for t in self.tensors)


def _mat(name: str, rows: int, cols: int, b: int) -> TensorSpec:
    return TensorSpec(name, rows, cols, gran_rows=b, q_rows=b, q_cols=b)


def _vec(name: str, n: int) -> TensorSpec:
    return TensorSpec(name, 1, n, gran_rows=0)


def _llama_layer(prefix: str, d: int, d_kv: int, d_ff: int, b: int) -> List[TensorSpec]:
    return [
        _mat(prefix + "wq", d, d, b),
        _mat(prefix + "wk", d_kv, d, b),
        _mat(prefix + "wv", d_kv, d, b),
        _mat(prefix + "wo", d, d, b),
        _mat(prefix + "wgate", d_ff, d, b),
        _mat(prefix + "wup", d_ff, d, b),
        _mat(prefix + "wdown", d, d_ff, b),
        _vec(prefix + "norm1", d),
        _vec(prefix + "norm2", d),
    ]


def toy_unit() -> Workload:
    ts: List[TensorSpec] = []
    for layer in range(2):
        p = f"l{layer}."
        ts += [_mat(p + "wqkv", 384, 128, 32), _mat(p + "wo", 128, 128, 32),
               _mat(p + "w1", 512, 128, 32), _mat(p + "w2", 128, 512, 32)]
    return Workload("toy_unit", tuple(ts), m=4, qfmt="fp8_e4m3", block=32,
                    description="2 layers x {Wqkv 384x128, Wo 128x128, W1 512x128, "
                                "W2 128x512}, m=4, 32x32 blocks, FP8 e4m3")


def llama8b_layer() -> Workload:
    return Workload("llama3_8b_layer", tuple(_llama_layer("", 4096, 1024, 14336, 128)),
                    m=8, qfmt="fp8_e4m3", block=128,
                    description="one Llama-3-8B decoder layer (Wq, Wk, Wv, Wo, Wgate, Wup, "
                                "Wdown, 2 RMSNorm), m=8, 128x128 blocks, FP8 e4m3")


def ragged_mixed() -> Workload:
    emb = TensorSpec("embed", 128256, 4096, gran_rows=1, q_rows=1, q_cols=128)
    ts = [emb]
    for layer in range(4):
        ts += _llama_layer(f"l{layer}.", 4096, 1024, 14336, 128)
    return Workload("ragged_mixed", tuple(ts), m=32, qfmt="int8", block=128,
                    nonfinite_frac=1e-3,
                    description="embedding 128256x4096 (row granular) + 4 Llama-8B layers, "
                                "m=32, INT8, 0.1% +-Inf/NaN grads")


def moe_experts() -> Workload:
    ts: List[TensorSpec] = []
    for e in range(64):
        p = f"e{e}."
        ts += [_mat(p + "w1", 1408, 2048, 128), _mat(p + "w3", 1408, 2048, 128),
               _mat(p + "w2", 2048, 1408, 128)]
    ts.append(_mat("router", 64, 2048, 128))
    return Workload("moe_experts", tuple(ts), m=16, qfmt="fp8_e4m3", block=128,
                    grad_dist="student_t3",
                    description="64 experts x {W1 1408x2048, W3 1408x2048, W2 2048x1408} "
                                "+ router 64x2048, m=16, FP8 e4m3, Student-t(3) grads")


def llama70b_layer() -> Workload:
    return Workload("llama70b_layer", tuple(_llama_layer("", 8192, 1024, 28672, 128)),
                    m=128, qfmt="fp8_e4m3", block=128,
                    description="one Llama-70B decoder layer, m=128, FP8 e4m3")


WORKLOADS = {w.name: w for w in (toy_unit(), llama8b_layer(), ragged_mixed(),
                                  moe_experts(), llama70b_layer())}


def scaled_workload(w: Workload, row_div: int, col_div: int = 1, max_tensors: int = 0,
                    m: int = 0) -> Workload:
    """A smaller copy of a workload with every matrix dimension divided.

    Used for parity cases the oracle finishes in seconds while keeping the
    structure (tensor order, granules, ragged fragments) of the full group.
    """
    ts = []
    for t in w.tensors[: max_tensors or None]:
        rows = max(1, t.rows // row_div) if t.rows > 1 else 1
        cols = max(1, t.cols // col_div)
        ts.append(TensorSpec(t.name, rows, cols, t.gran_rows, t.q_rows, t.q_cols))
    return Workload(w.name + f"_div{row_div}x{col_div}", tuple(ts), m=m or w.m,
                    qfmt=w.qfmt, block=w.block, grad_dist=w.grad_dist,
                    nonfinite_frac=w.nonfinite_frac, seed=w.seed,
                    param_sigma=w.param_sigma, grad_sigma=w.grad_sigma)


@dataclass
class GroupInputs:
    """Per-tensor fp32 arrays (row-major, shape (rows, cols))."""

    params: List[np.ndarray]
    grads: List[np.ndarray]
    nonfinite_positions: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int64))


def make_inputs(w: Workload, seed: int | None = None, grads: bool = True) -> GroupInputs:
    """Draw params N(0, sigma_p) then grads (N(0, sigma_g) or Student-t(3)*sigma_g).

    One PCG64 generator per workload; params tensor by tensor in group order,
    then grads in the same order, then the non-finite injection positions.
    """
    rng = np.random.default_rng(w.seed if seed is None else seed)
    ps = [(rng.standard_normal(t.numel, dtype=np.float32) * np.float32(w.param_sigma))
          .reshape(t.rows, t.cols) for t in w.tensors]
    gs: List[np.ndarray] = []
    pos = np.zeros(0, np.int64)
    if grads:
        for t in w.tensors:
            if w.grad_dist == "student_t3":
                g = (rng.standard_t(3, size=t.numel) * w.grad_sigma).astype(np.float32)
            else:
                g = rng.standard_normal(t.numel, dtype=np.float32) * np.float32(w.grad_sigma)
            gs.append(g.reshape(t.rows, t.cols))
        if w.nonfinite_frac > 0:
            total = w.numel
            k = int(w.nonfinite_frac * total)
            pos = rng.choice(total, size=k, replace=False).astype(np.int64)
            specials = np.array([np.inf, -np.inf, np.nan], dtype=np.float32)
            starts = np.cumsum([0] + [t.numel for t in w.tensors])
            tid = np.searchsorted(starts, pos, side="right") - 1
            cyc = specials[np.arange(k) % 3]
            for t in np.unique(tid):
                sel = tid == t
                gs[t].reshape(-1)[pos[sel] - starts[t]] = cyc[sel]
    return GroupInputs(ps, gs, pos)


def random_tiny_specs(rng: np.random.Generator, max_t: int = 4, max_e: int = 24,
                      max_g: int = 8) -> List[Tuple[int, int]]:
    """Random (numel, granule) pairs for brute-force planner cases."""
    n = int(rng.integers(1, max_t + 1))
    out = []
    for _ in range(n):
        e = int(rng.integers(1, max_e + 1))
        g = int(rng.integers(1, max_g + 1))
        out.append((e, g))
    return out
