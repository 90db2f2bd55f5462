"""GPU parity on seeded random groups: random tensor counts, shapes, row and
block granules, tile shapes (odd widths, narrow and wide tiles), rank
counts, alignments and chunk sizes.  A second generator draws wider groups:
up to 64 ranks, 1 x k tiles up to 1 x 16384, tall k x 1 tiles up to
16384 rows, square blocks of 8-128 with partial edges, alignment up to 64
and chunks up to 4096.  Every operation runs on the whole rank range and on
a random sub-range and is compared with the oracle (bit-exact; norms within
1e-5 relative of fp64), with canary guard bands around every output.
RS_RANDOM_SEED0 (default 0) shifts every seed, for a sweep over other
groups than the ones this file runs by default."""
import os

import numpy as np
import pytest

import workloads as W
from oracle import ops as O
from oracle import optim as OP

from harness import (Case, assert_bits_equal, assert_f32_equal_nan_class, check_guards, from_np,
                     guarded, log, to_np)

pytestmark = pytest.mark.gpu

F32_CANARY = 0x7FA5A5A5
BF16_CANARY = 0x7FA5
U8_CANARY = 0xAB
N_GROUPS = 120
N_WIDE = 40
SEED0 = int(os.environ.get("RS_RANDOM_SEED0", "0"))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def _random_workload(seed):
    rng = np.random.default_rng(1000 + seed)
    ts = []
    for i in range(int(rng.integers(1, 7))):
        kind = rng.integers(0, 3)
        if kind == 0:                                   # vector, element granular
            ts.append(W.TensorSpec(f"v{i}", 1, int(rng.integers(1, 3000)), 0))
        elif kind == 2 and rng.random() < 0.35:        # big tiles: narrow (128-256 lanes) and wide
            g = int(rng.choice([32, 64, 128]))
            cols = int(rng.choice([128, 256, 384]))
            qc = int(rng.choice([64, 128]))
            rows = int(rng.integers(1, 4)) * g + (int(rng.integers(0, g)) if rng.random() < 0.3 else 0)
            ts.append(W.TensorSpec(f"t{i}", rows, cols, g, g, qc))
        else:
            g = int(rng.choice([1, 2, 3, 4, 8, 16]))
            rows = int(rng.integers(1, 12)) * g + int(rng.integers(0, g)) if kind == 1 else \
                int(rng.integers(1, 6)) * g
            cols = int(rng.choice([3, 5, 8, 16, 40, 64, 100, 128, 130, 256]))
            qc = int(rng.choice([0, 4, 7, 8, 16, 32, 64]))
            qc = min(qc, cols) if qc else 0
            if qc and g * qc > 16384:
                qc = 0
            ts.append(W.TensorSpec(f"t{i}", rows, cols, g, g if qc else 0, qc))
    m = int(rng.integers(1, 7))
    fmt = "fp8_e4m3" if rng.random() < 0.5 else "int8"
    A = int(rng.choice([1, 4, 16]))
    chunk = int(rng.choice([64, 128, 192, 2048]))
    nf = 0.002 if rng.random() < 0.3 else 0.0
    return W.Workload(f"random{seed}", tuple(ts), m=m, qfmt=fmt, block=1, nonfinite_frac=nf,
                      seed=seed), A, chunk, rng


def _wide_workload(seed):
    rng = np.random.default_rng(99000 + seed)
    ts = []
    budget = 1_500_000
    for i in range(int(rng.integers(1, 10))):
        kind = int(rng.integers(0, 5))
        if kind == 0:                                   # vector, element granular
            ts.append(W.TensorSpec(f"v{i}", 1, int(rng.integers(1, 50000)), 0))
        elif kind == 1:                                 # 1 x k tiles, row granular
            cols = int(rng.choice([128, 256, 1000, 4096, 16384]))
            qc = min(cols, int(rng.choice([64, 128, 512, 4096, 16384])))
            rows = int(rng.integers(1, max(2, min(64, budget // cols))))
            ts.append(W.TensorSpec(f"e{i}", rows, cols, 1, 1, qc))
        elif kind == 2:                                 # tall k x 1 tiles
            cols = int(rng.choice([1, 2, 3, 5]))
            qr = int(rng.choice([256, 1024, 4096, 16384]))
            rows = qr * int(rng.integers(1, 3)) + (int(rng.integers(0, qr)) if rng.random() < 0.5 else 0)
            ts.append(W.TensorSpec(f"t{i}", rows, cols, qr, qr, 1))
        elif kind == 3:                                 # square blocks with partial edges
            b = int(rng.choice([8, 16, 32, 64, 128]))
            cols = int(rng.integers(b // 2, 5 * b))
            rows = int(rng.integers(1, 5)) * b + (int(rng.integers(0, b)) if rng.random() < 0.5 else 0)
            ts.append(W.TensorSpec(f"b{i}", rows, cols, b, b, b))
        else:                                           # row granular, not quantised
            g = int(rng.choice([1, 2, 7]))
            ts.append(W.TensorSpec(f"r{i}", g * int(rng.integers(1, 40)), int(rng.integers(1, 300)), g))
    m = int(rng.integers(1, 65))
    fmt = "fp8_e4m3" if rng.random() < 0.5 else "int8"
    A = int(rng.choice([1, 4, 16, 64]))
    chunk = int(rng.choice([64, 128, 2048, 4096]))
    nf = 0.002 if rng.random() < 0.3 else 0.0
    return W.Workload(f"wide{seed}", tuple(ts), m=m, qfmt=fmt, block=1, nonfinite_frac=nf,
                      seed=seed), A, chunk, rng


def _sync():
    import torch
    torch.cuda.synchronize()


@pytest.mark.parametrize("gen,seed", [("basic", SEED0 + s) for s in range(N_GROUPS)] +
                         [("wide", SEED0 + s) for s in range(N_WIDE)])
def test_random_group(gen, seed):
    import torch
    w, A, chunk, rng = (_random_workload if gen == "basic" else _wide_workload)(seed)
    c = Case(w, A, chunk)
    R = c.R
    h = c.lay.handle
    inp = c.inputs()
    ranges = [(0, c.m)]
    k0 = int(rng.integers(0, c.m))
    ranges.append((k0, int(rng.integers(k0 + 1, c.m + 1))))
    x_host = c.flat(inp.grads, fill=np.float32(np.nan))
    y_host = c.flat(inp.params, fill=np.float32(np.nan))
    nt = c.lay.info["num_tiles"]
    qf = R.RS_Q_FP8_E4M3 if w.qfmt == "fp8_e4m3" else R.RS_Q_INT8
    srcs = [torch.from_numpy(a).cuda() for a in inp.params]
    for k0, k1 in ranges:
        what = f"{w.name} (n={len(w.tensors)} m={c.m} A={A} chunk={chunk}) [{k0},{k1})"
        log(what)
        # pack fp32 -> bf16
        bw, buf = guarded(c.total, torch.bfloat16, BF16_CANARY)
        R.rs_pack(h, R.ptr_table(srcs), R.RS_F32, buf, R.RS_BF16, k0, k1)
        _sync()
        exp = O.pack(inp.params, c.offsets, c.S, c.m, np.full(c.total, BF16_CANARY, np.uint16), "bf16",
                     k0, k1)
        assert_bits_equal(to_np(buf), exp, what + " pack")
        check_guards(bw, BF16_CANARY, what + " pack")
        # unpack bf16 -> fp32
        outs = [guarded(s.numel, torch.float32, F32_CANARY) for s in w.tensors]
        R.rs_unpack(h, buf, R.RS_BF16, R.ptr_table([v for _, v in outs]), R.RS_F32, k0, k1)
        _sync()
        eo = O.unpack(exp, [(s.rows, s.cols) for s in w.tensors], c.offsets, c.S, c.m,
                      [np.full(s.numel, F32_CANARY, np.uint32).view(np.float32) for s in w.tensors],
                      "f32", k0, k1)
        for t, ((wh, v), e) in enumerate(zip(outs, eo)):
            assert_bits_equal(to_np(v), e.reshape(-1), f"{what} unpack t{t}")
            check_guards(wh, F32_CANARY, f"{what} unpack t{t}")
        # scale/add with found-inf, then norms of the result
        yw, y = guarded(c.total, torch.float32, F32_CANARY)
        y.copy_(torch.from_numpy(y_host))
        fi = torch.zeros(c.m, dtype=torch.int32, device="cuda")
        R.rs_group_scale_add(h, y, from_np(x_host), R.RS_F32, 0.75, -1.5, None, fi, k0, k1)
        _sync()
        ey, ef = O.scale_add(y_host, x_host, 0.75, -1.5, c.items, c.offsets, c.S, c.m, k0, k1)
        assert_f32_equal_nan_class(to_np(y), ey, what + " scale_add")
        assert np.array_equal(to_np(fi).astype(np.uint32), ef), what + " found_inf"
        check_guards(yw, F32_CANARY, what + " scale_add")
        sq = torch.empty(len(w.tensors), dtype=torch.float64, device="cuda")
        R.rs_ragged_sqnorm(h, y, sq, None, None, c.lay.ws, k0, k1)
        _sync()
        es = O.sqnorm(ey, c.items, c.offsets, c.S, c.m, k0, k1)[0]
        got = to_np(sq)
        fin = np.isfinite(es)
        assert np.array_equal(np.isnan(got), np.isnan(es)) and np.array_equal(np.isinf(got), np.isinf(es))
        np.testing.assert_allclose(got[fin], es[fin], rtol=1e-5, atol=0, err_msg=what + " sqnorm")
        # quantise and dequantise
        cw, codes = guarded(c.total, torch.uint8, U8_CANARY)
        sw, scales = guarded(max(nt, 1), torch.float32, F32_CANARY)
        R.rs_block_quant(h, from_np(x_host), qf, codes, scales, k0, k1)
        _sync()
        ec, es2 = O.block_quant(x_host, w.tensors, c.offsets, c.S, c.m, w.qfmt, k0, k1,
                                np.full(c.total, U8_CANARY, np.uint8),
                                np.full(max(nt, 1), F32_CANARY, np.uint32).view(np.float32))
        assert_bits_equal(to_np(codes), ec, what + " codes")
        assert_bits_equal(to_np(scales), es2, what + " scales")
        check_guards(cw, U8_CANARY, what + " codes")
        check_guards(sw, F32_CANARY, what + " scales")
        dw, dq = guarded(c.total, torch.float32, F32_CANARY)
        R.rs_block_dequant(h, codes, qf, scales, dq, R.RS_F32, k0, k1)
        _sync()
        ed = O.block_dequant(ec, es2, w.tensors, c.offsets, c.S, c.m, w.qfmt, k0, k1,
                             np.full(c.total, F32_CANARY, np.uint32).view(np.float32), "f32")
        assert_f32_equal_nan_class(to_np(dq), ed, what + " dequant")
        check_guards(dw, F32_CANARY, what + " dequant")
        # zero with a random mask
        mask = (rng.random(len(w.tensors)) < 0.6).astype(np.uint8)
        zw, z = guarded(c.total, torch.float32, F32_CANARY)
        z.copy_(torch.from_numpy(y_host))
        R.rs_group_zero(h, z, R.RS_F32, from_np(mask), k0, k1)
        _sync()
        ez = O.zero(y_host, c.items, c.offsets, c.S, c.m, k0, k1, mask=list(mask))
        assert_f32_equal_nan_class(to_np(z), ez, what + " zero")
        check_guards(zw, F32_CANARY, what + " zero")
        # optimizer steps (finite state)
        mom = (rng.standard_normal(c.total) * 1e-4).astype(np.float32)
        var = np.abs(rng.standard_normal(c.total) * 1e-6).astype(np.float32)
        hp = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, wd=0.1, bc1=0.3, bc2=0.2, grad_scale=2.0)
        p0 = np.nan_to_num(y_host, nan=0.5)
        g0 = np.nan_to_num(x_host, nan=0.0, posinf=1.0, neginf=-1.0)
        p, g, mm, vv = from_np(p0), from_np(g0), from_np(mom), from_np(var)
        R.rs_adamw_step(h, p, g, mm, vv, hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["wd"],
                        hp["bc1"], hp["bc2"], hp["grad_scale"], None, None, k0, k1)
        _sync()
        ep, em, ev = OP.adamw_step(p0, g0, mom, var, c.items, c.offsets, c.S, c.m, k0, k1, hp)
        for got_, exp_, nm in ((p, ep, "p"), (mm, em, "m"), (vv, ev, "v")):
            assert_f32_equal_nan_class(to_np(got_), exp_, f"{what} adamw {nm}")
        p, b = from_np(p0), from_np(mom)
        R.rs_sgd_step(h, p, g, b, 0.05, 0.9, 1e-4, bool(seed % 2), 1.0, None, None, k0, k1)
        _sync()
        ep, eb = OP.sgd_step(p0, g0, mom, c.items, c.offsets, c.S, c.m, k0, k1, 0.05, 0.9, 1e-4,
                             bool(seed % 2), 1.0)
        assert_f32_equal_nan_class(to_np(p), ep, what + " sgd p")
        assert_f32_equal_nan_class(to_np(b), eb, what + " sgd buf")
        if nt:
            mc0, ms0 = O.block_quant(mom, w.tensors, c.offsets, c.S, c.m, w.qfmt, 0, c.m,
                                     np.zeros(c.total, np.uint8), np.zeros(nt, np.float32))
            vc0, vs0 = O.block_quant(var, w.tensors, c.offsets, c.S, c.m, w.qfmt, 0, c.m,
                                     np.zeros(c.total, np.uint8), np.zeros(nt, np.float32))
            p = from_np(p0)
            mc, ms, vc, vs = from_np(mc0), from_np(ms0), from_np(vc0), from_np(vs0)
            R.rs_adamw8_step(h, p, g, mc, ms, vc, vs, qf, hp["lr"], hp["beta1"], hp["beta2"], hp["eps"],
                             hp["wd"], hp["bc1"], hp["bc2"], hp["grad_scale"], None, k0, k1)
            _sync()
            e = OP.adamw8_step(p0, g0, mc0, ms0, vc0, vs0, w.tensors, c.offsets, c.S, c.m, k0, k1,
                               w.qfmt, hp)
            assert_f32_equal_nan_class(to_np(p), e[0], what + " adamw8 p")
            assert np.array_equal(to_np(mc), e[1]) and np.array_equal(to_np(vc), e[3]), what + " adamw8 codes"
            assert np.array_equal(to_np(ms).view(np.uint32), e[2].view(np.uint32)), what + " adamw8 m scales"
            assert np.array_equal(to_np(vs).view(np.uint32), e[4].view(np.uint32)), what + " adamw8 v scales"
