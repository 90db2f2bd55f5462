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

import os
from concurrent.futures import ThreadPoolExecutor
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


def ragged_small() -> Workload:
    """A small group for parity cases: element-, row- and block-granular
    tensors, non-square and partial edge tiles, odd sizes, five ranks."""
    ts = (TensorSpec("a", 40, 24, gran_rows=8, q_rows=8, q_cols=16),
          TensorSpec("v", 1, 37, gran_rows=0),
          TensorSpec("b", 30, 12, gran_rows=6, q_rows=6, q_cols=8),
          TensorSpec("e", 50, 10, gran_rows=1, q_rows=1, q_cols=4),
          TensorSpec("c", 7, 33, gran_rows=4, q_rows=4, q_cols=16))
    return Workload("ragged_small", ts, m=5, qfmt="fp8_e4m3", block=8)


WORKLOADS = {w.name: w for w in (toy_unit(), llama8b_layer(), ragged_mixed(),
                                  moe_experts(), llama70b_layer())}


def regranulated(specs: Sequence[TensorSpec], rows: int) -> Tuple[TensorSpec, ...]:
    """The same tensors with every matrix (more than one row) given a granule
    of `rows` rows and vectors left element-granular; quantisation tiles are
    dropped (the planner alone is studied).  The row-granularity sweep of
    the pages' padding study (veScale-FSDP, section 6.4) runs 1, 16 and 128
    rows."""
    return tuple(TensorSpec(s.name, s.rows, s.cols, rows if s.rows > 1 else 0)
                 for s in specs)


def fused_experts(w: Workload) -> Workload:
    """The expert unit with each expert matrix kind fused into one tensor
    (all experts' W1 stacked by rows, likewise W3 and W2), router kept.
    The pages trace their largest padding spikes to models that store all
    experts as one parameter tensor (veScale-FSDP, section 6.4); this is
    that storage applied to the expert unit's own shapes."""
    kinds: Dict[str, List[TensorSpec]] = {}
    rest: List[TensorSpec] = []
    for s in w.tensors:
        if s.name.startswith("e") and "." in s.name:
            kinds.setdefault(s.name.split(".", 1)[1], []).append(s)
        else:
            rest.append(s)
    fused = []
    for kind, ss in kinds.items():
        r0 = ss[0]
        assert all(x.cols == r0.cols and x.gran_rows == r0.gran_rows for x in ss)
        fused.append(TensorSpec("experts." + kind, sum(x.rows for x in ss), r0.cols, r0.gran_rows,
                                r0.q_rows, r0.q_cols))
    return Workload(w.name + "_fused", tuple(fused + rest), m=w.m, qfmt=w.qfmt, block=w.block,
                    grad_dist=w.grad_dist, description="expert unit with fused expert tensors")


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


PIECE = 1 << 22   # elements drawn from one generator


def _pieces(numel: int, ss: np.random.SeedSequence, kind: str, sigma: float, out: np.ndarray):
    """Jobs filling out[numel]: piece j of PIECE elements comes from its own
    PCG64 seeded by the j-th child of ss, so pieces can be drawn in parallel."""
    n_pieces = max(1, -(-numel // PIECE))
    kids = ss.spawn(n_pieces)

    def one(j):
        lo, hi = j * PIECE, min(numel, (j + 1) * PIECE)
        rng = np.random.default_rng(kids[j])
        if kind == "student_t3":
            out[lo:hi] = (rng.standard_t(3, size=hi - lo) * sigma).astype(np.float32)
        else:
            v = rng.standard_normal(hi - lo, dtype=np.float32)
            np.multiply(v, np.float32(sigma), out=out[lo:hi])

    return [lambda j=j: one(j) for j in range(n_pieces)]


def make_inputs(w: Workload, seed: int | None = None, grads: bool = True,
                threads: int | None = None) -> GroupInputs:
    """Seeded synthetic params and grads for a workload.

    Root SeedSequence(seed); its first T children draw the params of each
    tensor (N(0, param_sigma)), the next T the grads (N(0, grad_sigma), or
    Student-t(3) * grad_sigma), and one more child picks the non-finite
    positions: floor(frac * numel) distinct flat positions over the
    concatenated tensors, set in turn to +Inf, -Inf, NaN.
    """
    root = np.random.SeedSequence(w.seed if seed is None else seed)
    ss_p = root.spawn(len(w.tensors))
    ss_g = root.spawn(len(w.tensors))
    ss_i = root.spawn(1)[0]
    nthr = threads or min(16, os.cpu_count() or 1)
    ps = [np.empty(t.numel, np.float32) for t in w.tensors]
    gs = [np.empty(t.numel, np.float32) for t in w.tensors] if grads else []
    jobs = []
    for t, ss, out in zip(w.tensors, ss_p, ps):
        jobs += _pieces(t.numel, ss, "normal", w.param_sigma, out)
    for t, ss, out in zip(w.tensors, ss_g, gs):
        jobs += _pieces(t.numel, ss, w.grad_dist, w.grad_sigma, out)
    with ThreadPoolExecutor(max_workers=nthr) as pool:
        list(pool.map(lambda f: f(), jobs))
    ps = [a.reshape(t.rows, t.cols) for a, t in zip(ps, w.tensors)]
    gs = [a.reshape(t.rows, t.cols) for a, t in zip(gs, w.tensors)]
    pos = np.zeros(0, np.int64)
    if grads and w.nonfinite_frac > 0:
        total = w.numel
        k = int(w.nonfinite_frac * total)
        rng = np.random.default_rng(ss_i)
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
