"""Shared helpers for the GPU parity tests: run an operation through the
C-ABI on seeded inputs and run the oracle on the same bytes."""
from __future__ import annotations

import sys
from dataclasses import dataclass
from typing import List

import numpy as np

import workloads as W
from oracle import plan as P

GUARD = 64  # canary elements before and after every device output


def log(msg: str) -> None:
    """Progress line naming the case, flushed before each GPU step."""
    print(msg, flush=True)
    sys.stdout.flush()


def torch_mod():
    import torch
    return torch


_INT_VIEW = {4: "int32", 2: "int16", 1: "uint8", 8: "int64"}


def guarded(n: int, dtype, bits: int):
    """Device tensor of n elements with GUARD canaries on each side, every
    element preset to the bit pattern `bits`; returns (whole, view)."""
    torch = torch_mod()
    whole = torch.empty(n + 2 * GUARD, dtype=dtype, device="cuda")
    iv = getattr(torch, _INT_VIEW[whole.element_size()])
    width = 8 * whole.element_size()
    sval = bits - (1 << width) if (iv != torch.uint8 and bits >= 1 << (width - 1)) else bits
    whole.view(iv).fill_(sval)
    return whole, whole[GUARD:GUARD + n]


def check_guards(whole, bits: int, what: str) -> None:
    h = to_np(whole)
    u = h.view({4: np.uint32, 2: np.uint16, 1: np.uint8, 8: np.uint64}[h.itemsize])
    assert np.all(u[:GUARD] == bits), f"{what}: write before the buffer"
    assert np.all(u[-GUARD:] == bits), f"{what}: write past the buffer"


def to_np(t) -> np.ndarray:
    torch = torch_mod()
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def from_np(a: np.ndarray, dtype=None):
    torch = torch_mod()
    if a.dtype == np.uint16 and dtype is None:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@dataclass
class Case:
    """A workload planned by both sides, with its inputs on host and device."""

    w: W.Workload
    A: int
    chunk: int

    def __post_init__(self):
        import fsdp_sharded_buffer_amd as R
        self.R = R
        self.items = P.items_from_specs(self.w.tensors)
        offs, info = R.rs_plan(self.w.tensors, self.w.m, self.A)
        self.S = info["S"]
        self.offsets = offs
        # the oracle's own planner must agree (both are exact, same tie-break)
        if len(self.items) <= 40:
            p = P.plan(self.items, self.w.m, self.A)
            assert (p.S, p.offsets) == (self.S, offs)
        self.lay = R.Layout(self.w.tensors, self.w.m, self.S, offs, self.chunk)
        self.total = self.w.m * self.S
        self.inp = None

    @property
    def m(self) -> int:
        return self.w.m

    def inputs(self):
        if self.inp is None:
            self.inp = W.make_inputs(self.w)
        return self.inp

    def flat(self, arrays: List[np.ndarray], fill=0.0) -> np.ndarray:
        """Host fp32 buffer image: arrays at their offsets, fill elsewhere."""
        buf = np.full(self.total, fill, dtype=np.float32)
        for a, l in zip(arrays, self.offsets):
            buf[l:l + a.size] = a.reshape(-1)
        return buf

    def ranges(self):
        m = self.m
        rs = [(0, m), (0, 1), (m - 1, m)]
        if m > 2:
            rs.append((1, m - 1))
        return rs


def assert_bits_equal(got: np.ndarray, exp: np.ndarray, what: str) -> None:
    if got.dtype == np.float32:
        g, e = got.view(np.uint32), exp.astype(np.float32).view(np.uint32)
    elif got.dtype == np.float64:
        g, e = got.view(np.uint64), exp.astype(np.float64).view(np.uint64)
    else:
        g, e = got, exp
    if not np.array_equal(g, e):
        bad = np.flatnonzero(g.reshape(-1) != e.reshape(-1))
        i = bad[0]
        raise AssertionError(f"{what}: {bad.size} mismatches, first at {i}: got {got.reshape(-1)[i]!r} "
                             f"({g.reshape(-1)[i]:#x}) expected {exp.reshape(-1)[i]!r} ({e.reshape(-1)[i]:#x})")


def assert_f32_equal_nan_class(got: np.ndarray, exp: np.ndarray, what: str, max_ulp: int = 0) -> None:
    """Equal bits for non-NaN values (or within max_ulp), NaN where NaN."""
    gn, en = np.isnan(got), np.isnan(exp)
    assert np.array_equal(gn, en), f"{what}: NaN positions differ"
    if max_ulp == 0:
        ok = got.view(np.uint32) == exp.astype(np.float32).view(np.uint32)
        ok |= gn
        if not ok.all():
            i = int(np.flatnonzero(~ok)[0])
            raise AssertionError(f"{what}: {int((~ok).sum())} values differ; first at {i}: "
                                 f"got {got[i]!r} expected {exp[i]!r}")
        return
    g = got[~gn].view(np.int32).astype(np.int64)
    e = exp[~en].astype(np.float32).view(np.int32).astype(np.int64)
    # map sign-magnitude to a monotone integer line
    g = np.where(g < 0, -(g & 0x7FFFFFFF), g)
    e = np.where(e < 0, -(e & 0x7FFFFFFF), e)
    d = np.abs(g - e)
    if d.size and d.max() > max_ulp:
        i = int(np.argmax(d))
        raise AssertionError(f"{what}: {int((d > max_ulp).sum())} values off by more than {max_ulp} ulp; "
                             f"worst {int(d[i])} ulp")


# ------------------------------------------------------------ small cases

def _moe_small():
    w = W.moe_experts()
    ts = list(w.tensors[:12]) + [w.tensors[-1]]
    return W.scaled_workload(W.Workload("moe4", tuple(ts), m=16, qfmt="fp8_e4m3", block=128,
                                        grad_dist="student_t3"), 8, 8)


def _mixed_small():
    w = W.ragged_mixed()
    return W.scaled_workload(W.Workload("mixed2", w.tensors[:19], m=32, qfmt="int8", block=128,
                                        nonfinite_frac=1e-3), 32, 16)


def _bands():
    """Tiles of 30 and 7 rows (every tile at least 4 rows, heights not
    multiples of 4): dequantisation splits each tile into row bands here."""
    ts = (W.TensorSpec("a", 90, 64, 30, 30, 32), W.TensorSpec("v", 1, 100, 0),
          W.TensorSpec("b", 21, 48, 7, 7, 16), W.TensorSpec("c", 60, 40, 30, 30, 40))
    return W.Workload("bands", ts, m=3, qfmt="int8", block=32)


def _pad_ranks():
    """One 4x8 tensor whose granule is the whole tensor, on 4 ranks: rank 0
    holds it, ranks 1-3 are padding only."""
    return W.Workload("pad_ranks", (W.TensorSpec("a", 4, 8, 4, 4, 8),), m=4, qfmt="fp8_e4m3",
                      block=8)


def _tiny():
    """One-element tensors, a 3-element vector and a row-granular 3x5 tensor
    with 1x5 tiles, on 3 ranks."""
    ts = (W.TensorSpec("a", 1, 1, 0), W.TensorSpec("b", 1, 1, 0), W.TensorSpec("c", 3, 5, 1, 1, 5),
          W.TensorSpec("d", 1, 3, 0))
    return W.Workload("tiny", ts, m=3, qfmt="int8", block=5)


def _tall():
    """Tall, thin tiles: 4096x1 (narrow, one 256-lane team) and 16384x1
    (wide, the largest tile) on the element path, and 512x4 (narrow, one
    16-byte slot per row), on 2 ranks."""
    ts = (W.TensorSpec("a", 8192, 3, 4096, 4096, 1), W.TensorSpec("b", 16384, 2, 16384, 16384, 1),
          W.TensorSpec("c", 1024, 4, 512, 512, 4))
    return W.Workload("tall", ts, m=2, qfmt="fp8_e4m3", block=1)


def _no_quant():
    """Vectors only: no quantisation tiles at all."""
    ts = (W.TensorSpec("v1", 1, 1000, 0), W.TensorSpec("v2", 1, 77, 0))
    return W.Workload("no_quant", ts, m=2, qfmt="fp8_e4m3", block=1)


SMALL = {
    "toy": lambda: (W.toy_unit(), 16, 0),
    "toy_a1_c64": lambda: (W.toy_unit(), 1, 64),
    "ragged_a1_c64": lambda: (W.ragged_small(), 1, 64),
    "ragged_a16_c256": lambda: (W.ragged_small(), 16, 256),
    "llama8b_div16": lambda: (W.scaled_workload(W.llama8b_layer(), 16, 16), 16, 320),
    "llama8b_div16_a1": lambda: (W.scaled_workload(W.llama8b_layer(), 16, 16), 1, 1024),
    "mixed_div": lambda: (_mixed_small(), 16, 512),
    "moe_div8": lambda: (_moe_small(), 16, 2048),
    "llama70b_div32": lambda: (W.scaled_workload(W.llama70b_layer(), 32, 32), 16, 0),
    "bands": lambda: (_bands(), 16, 128),
    "single_rank": lambda: (W.Workload("toy_m1", W.toy_unit().tensors, m=1, qfmt="fp8_e4m3",
                                       block=32), 16, 0),
    "pad_ranks": lambda: (_pad_ranks(), 1, 64),
    "tiny": lambda: (_tiny(), 1, 64),
    "no_quant": lambda: (_no_quant(), 16, 128),
    "tall": lambda: (_tall(), 16, 0),
    "toy_chunk_max": lambda: (W.toy_unit(), 16, 1 << 22),   # largest chunk: one per fragment
}

_cases = {}


def case(name) -> Case:
    if name not in _cases:
        w, A, ch = SMALL[name]()
        _cases[name] = Case(w, A, ch)
    return _cases[name]


