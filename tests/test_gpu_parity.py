"""GPU parity: every entry point of include/rs.h, called through the C-ABI,
against the CPU oracle on the same seeded inputs.

Bar: bit-exact for copies, casts, zeros, block scales and FP8/INT8 codes;
scale/add bit-exact on non-NaN values (the kernel keeps the two products
and the sum as separate fp32 roundings; the 1-ulp allowance is checked
too) with NaN where the oracle has NaN; squared norms within 1e-5 relative
of the fp64 oracle with the same non-finite class.  Every device output is
surrounded by canary elements that must survive.
"""
import os

import numpy as np
import pytest

import workloads as W
from oracle import casts as OC
from oracle import ops as O

from harness import (SMALL, assert_bits_equal, assert_f32_equal_nan_class, case, check_guards,
                     from_np, guarded, log, to_np)

pytestmark = pytest.mark.gpu

F32_CANARY = 0x7FA5A5A5
BF16_CANARY = 0x7FA5
U8_CANARY = 0xAB
F64_CANARY = 0x7FF5A5A5A5A5A5A5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fsdp_sharded_buffer_amd  # noqa: F401  (fails loudly if librs.so is missing)
    yield


def _sync():
    import torch
    torch.cuda.synchronize()


def _dev_tensors(arrays, bf16=False):
    import torch
    ts = [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in arrays]
    if bf16:
        ts = [t.to(torch.bfloat16) for t in ts]
    return ts


# ------------------------------------------------------------------ pack


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("kinds", [("f32", "bf16"), ("f32", "f32"), ("bf16", "bf16"), ("bf16", "f32")])
def test_pack(name, kinds):
    import torch
    c = case(name)
    R = c.R
    src_k, buf_k = kinds
    ps = c.inputs().params
    src = _dev_tensors(ps, bf16=(src_k == "bf16"))
    src_host = [to_np(t) for t in src]          # bf16 bits or fp32
    table = R.ptr_table(src)
    bdt = torch.bfloat16 if buf_k == "bf16" else torch.float32
    canary = BF16_CANARY if buf_k == "bf16" else F32_CANARY
    for k0, k1 in c.ranges():
        log(f"pack {name} {kinds} ranks [{k0},{k1})")
        whole, buf = guarded(c.total, bdt, canary)
        R.rs_pack(c.lay.handle, table, R.RS_BF16 if src_k == "bf16" else R.RS_F32, buf,
                  R.RS_BF16 if buf_k == "bf16" else R.RS_F32, k0, k1)
        _sync()
        init = np.full(c.total, canary, dtype=np.uint16 if buf_k == "bf16" else np.uint32)
        if buf_k == "f32":
            init = init.view(np.float32)
        exp = O.pack(src_host, c.offsets, c.S, c.m, init, buf_k, k0, k1)
        assert_bits_equal(to_np(buf), exp, f"pack {name} {kinds} [{k0},{k1})")
        check_guards(whole, canary, "pack")


# ---------------------------------------------------------------- unpack


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("kinds", [("bf16", "bf16"), ("bf16", "f32"), ("f32", "f32"), ("f32", "bf16")])
def test_unpack(name, kinds):
    import torch
    c = case(name)
    R = c.R
    buf_k, dst_k = kinds
    ps = c.inputs().params
    host_buf = c.flat(ps, fill=np.float32(-7.0))
    if buf_k == "bf16":
        host_buf = OC.bf16_bits_from_f32(host_buf)
    dbuf = from_np(host_buf)
    ddt = torch.bfloat16 if dst_k == "bf16" else torch.float32
    canary = BF16_CANARY if dst_k == "bf16" else F32_CANARY
    for k0, k1 in c.ranges():
        log(f"unpack {name} {kinds} ranks [{k0},{k1})")
        outs = [guarded(s.numel, ddt, canary) for s in c.w.tensors]
        table = R.ptr_table([v for _, v in outs])
        R.rs_unpack(c.lay.handle, dbuf, R.RS_BF16 if buf_k == "bf16" else R.RS_F32, table,
                    R.RS_BF16 if dst_k == "bf16" else R.RS_F32, k0, k1)
        _sync()
        init_dt = np.uint16 if dst_k == "bf16" else np.uint32
        inits = [np.full(s.numel, canary, dtype=init_dt) for s in c.w.tensors]
        if dst_k == "f32":
            inits = [a.view(np.float32) for a in inits]
        exp = O.unpack(host_buf, [(s.rows, s.cols) for s in c.w.tensors], c.offsets, c.S, c.m,
                       inits, dst_k, k0, k1)
        for t, ((whole, v), e) in enumerate(zip(outs, exp)):
            assert_bits_equal(to_np(v), e.reshape(-1), f"unpack {name} {kinds} t{t} [{k0},{k1})")
            check_guards(whole, canary, f"unpack t{t}")


def test_pack_unpack_roundtrip_identity():
    import torch
    c = case("ragged_a1_c64")
    R = c.R
    src = _dev_tensors(c.inputs().params)
    buf = torch.empty(c.total, dtype=torch.float32, device="cuda")
    R.rs_pack(c.lay.handle, R.ptr_table(src), R.RS_F32, buf, R.RS_F32, 0, c.m)
    dst = [torch.empty_like(t) for t in src]
    R.rs_unpack(c.lay.handle, buf, R.RS_F32, R.ptr_table(dst), R.RS_F32, 0, c.m)
    _sync()
    for a, b in zip(src, dst):
        assert torch.equal(a, b)


# ------------------------------------------------------------- scale/add


def _mask(c, seed):
    rng = np.random.default_rng(seed)
    m = rng.integers(0, 2, size=len(c.w.tensors)).astype(np.uint8)
    m[0] = 1
    return m


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("xk", ["f32", "bf16"])
def test_scale_add(name, xk):
    import torch
    c = case(name)
    R = c.R
    inp = c.inputs()
    y0 = c.flat(inp.grads, fill=np.float32(12345.0))
    x0 = c.flat(inp.params, fill=np.float32(-3.0))
    if xk == "bf16":
        x0 = OC.bf16_bits_from_f32(x0)
    dx = from_np(x0)
    for (alpha, beta) in [(1.0, 1.0), (0.75, -1.5), (1.0, 0.0), (0.0, 2.0), (1.0 / 1024, 3.0e38)]:
        for use_mask in (False, True):
            for k0, k1 in c.ranges()[:3]:
                log(f"scale_add {name} x={xk} a={alpha} b={beta} mask={use_mask} [{k0},{k1})")
                whole, y = guarded(c.total, torch.float32, F32_CANARY)
                y.copy_(torch.from_numpy(y0))
                fi_whole, fi = guarded(c.m, torch.int32, 0)
                fi.zero_()
                mask = _mask(c, 3) if use_mask else None
                dmask = from_np(mask) if use_mask else None
                R.rs_group_scale_add(c.lay.handle, y, dx, R.RS_BF16 if xk == "bf16" else R.RS_F32,
                                     alpha, beta, dmask, fi, k0, k1)
                _sync()
                ey, ef = O.scale_add(y0, x0, alpha, beta, c.items, c.offsets, c.S, c.m, k0, k1,
                                     mask=None if mask is None else list(mask))
                got = to_np(y)
                what = f"scale_add {name} {xk} a={alpha} b={beta} [{k0},{k1})"
                assert_f32_equal_nan_class(got, ey, what, max_ulp=1)
                assert_f32_equal_nan_class(got, ey, what + " (exact)", max_ulp=0)
                assert np.array_equal(to_np(fi).astype(np.uint32), ef), what + " found_inf"
                check_guards(whole, F32_CANARY, "scale_add y")
                check_guards(fi_whole, 0, "found_inf")


def test_scale_add_found_inf_ors():
    import torch
    c = case("mixed_div")
    R = c.R
    inp = c.inputs()
    y0 = c.flat(inp.params)
    x0 = c.flat(inp.grads)        # holds +-Inf / NaN
    ey, ef = O.scale_add(y0, x0, 1.0, 1.0, c.items, c.offsets, c.S, c.m, 0, c.m)
    assert ef.any() and not ef.all()
    y = from_np(y0)
    fi = torch.zeros(c.m, dtype=torch.int32, device="cuda")
    clean = int(np.flatnonzero(ef == 0)[0])
    fi[clean] = 1                 # set before the call: must stay set
    R.rs_group_scale_add(c.lay.handle, y, from_np(x0), R.RS_F32, 1.0, 1.0, None, fi, 0, c.m)
    _sync()
    exp = ef.copy()
    exp[clean] = 1
    assert np.array_equal(to_np(fi).astype(np.uint32), exp)
    assert_f32_equal_nan_class(to_np(y), ey, "scale_add nonfinite")


@pytest.mark.parametrize("name", ["toy", "ragged_a1_c64", "mixed_div", "moe_div8", "tiny", "tall"])
def test_scale_add_in_place(name):
    """x is y itself, as in the sharded gradient scaler's in-place unscale:
    y' = fl(fl(alpha*y) + fl(beta*y)) per element, bit-exact against the
    oracle run on two separate copies of the same values."""
    import torch
    c = case(name)
    R = c.R
    inp = c.inputs()
    y0 = c.flat(inp.grads, fill=np.float32(12345.0))
    for (alpha, beta) in [(1.0 / 65536, 0.0), (1.0, 1.0), (0.75, -1.5), (0.0, 3.0e38)]:
        for k0, k1 in c.ranges()[:3]:
            log(f"scale_add in place {name} a={alpha} b={beta} [{k0},{k1})")
            whole, y = guarded(c.total, torch.float32, F32_CANARY)
            y.copy_(torch.from_numpy(y0))
            fi = torch.zeros(c.m, dtype=torch.int32, device="cuda")
            R.rs_group_scale_add(c.lay.handle, y, y, R.RS_F32, alpha, beta, None, fi, k0, k1)
            _sync()
            ey, ef = O.scale_add(y0, y0.copy(), alpha, beta, c.items, c.offsets, c.S, c.m, k0, k1)
            what = f"scale_add in place {name} a={alpha} b={beta} [{k0},{k1})"
            assert_f32_equal_nan_class(to_np(y), ey, what)
            assert np.array_equal(to_np(fi).astype(np.uint32), ef), what + " found_inf"
            check_guards(whole, F32_CANARY, "scale_add in place y")


# ------------------------------------------------------------------ zero


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("k", ["f32", "bf16"])
def test_zero(name, k):
    import torch
    c = case(name)
    R = c.R
    dt = torch.bfloat16 if k == "bf16" else torch.float32
    canary = BF16_CANARY if k == "bf16" else F32_CANARY
    for use_mask in (False, True):
        for k0, k1 in c.ranges():
            log(f"zero {name} {k} mask={use_mask} [{k0},{k1})")
            whole, y = guarded(c.total, dt, canary)
            mask = _mask(c, 5) if use_mask else None
            R.rs_group_zero(c.lay.handle, y, R.RS_BF16 if k == "bf16" else R.RS_F32,
                            from_np(mask) if use_mask else None, k0, k1)
            _sync()
            init = np.full(c.total, canary, dtype=np.uint16 if k == "bf16" else np.uint32)
            if k == "f32":
                init = init.view(np.float32)
            exp = O.zero(init, c.items, c.offsets, c.S, c.m, k0, k1,
                         mask=None if mask is None else list(mask))
            assert_bits_equal(to_np(y), exp, f"zero {name} {k} [{k0},{k1})")
            check_guards(whole, canary, "zero")


# ---------------------------------------------------------------- sqnorm


def _check_sq(got, exp, what):
    gn, en = np.isnan(got), np.isnan(exp)
    assert np.array_equal(gn, en), what + ": NaN class"
    gi, ei = np.isinf(got), np.isinf(exp)
    assert np.array_equal(gi, ei), what + ": Inf class"
    f = ~(gn | gi)
    rel = np.abs(got[f] - exp[f]) / np.maximum(np.abs(exp[f]), 1e-300)
    assert np.all((rel <= 1e-5) | (exp[f] == got[f])), f"{what}: rel err {rel.max()}"


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("src", ["params", "grads"])
def test_sqnorm(name, src):
    import torch
    c = case(name)
    R = c.R
    inp = c.inputs()
    x0 = c.flat(getattr(inp, src), fill=np.float32(1e30))   # padding must not count
    dx = from_np(x0)
    n = len(c.w.tensors)
    for k0, k1 in c.ranges():
        log(f"sqnorm {name} {src} [{k0},{k1})")
        sw, sq = guarded(n, torch.float64, F64_CANARY)
        pw, part = guarded(c.m * n, torch.float64, F64_CANARY)
        fw, fi = guarded(c.m, torch.int32, 0)
        R.rs_ragged_sqnorm(c.lay.handle, dx, sq, part, fi, c.lay.ws, k0, k1)
        _sync()
        esq, epart, ef = O.sqnorm(x0, c.items, c.offsets, c.S, c.m, k0, k1)
        what = f"sqnorm {name} {src} [{k0},{k1})"
        _check_sq(to_np(sq), esq, what)
        gp = to_np(part).reshape(c.m, n)
        _check_sq(gp[k0:k1], epart[k0:k1], what + " partial")
        # rows outside the range are not written
        assert np.all(gp[:k0].view(np.uint64) == F64_CANARY) and np.all(gp[k1:].view(np.uint64) == F64_CANARY)
        assert np.array_equal(to_np(fi).astype(np.uint32), ef), what + " found_inf"
        for wh, bits in ((sw, F64_CANARY), (pw, F64_CANARY), (fw, 0)):
            check_guards(wh, bits, what)
        # bit-identical on a second run (fixed-order combine)
        sq2 = torch.empty_like(sq)
        R.rs_ragged_sqnorm(c.lay.handle, dx, sq2, None, None, c.lay.ws, k0, k1)
        _sync()
        assert np.array_equal(to_np(sq2).view(np.uint64), to_np(sq).view(np.uint64)), what + " rerun"


@pytest.mark.parametrize("name", ["ragged_a1_c64", "mixed_div", "moe_div8", "llama70b_div32",
                                  "pad_ranks", "tiny"])
def test_sqnorm_one_rank_equals_wider_ranges(name):
    """A one-rank call (its fragments' chunk ranges passed to the combine by
    value) gives the same per-rank partials, bit for bit, as a call over all
    ranks that reads the same (fine) chunk table, and its per-tensor sums
    equal its partial row; padding-only ranks give zeros."""
    import torch
    c = case(name)
    R = c.R
    n = len(c.w.tensors)
    if c.lay.info["num_coarse_chunks"] >= 256:
        pytest.skip("the whole range would read coarse chunks")
    x = from_np(c.flat(c.inputs().grads, fill=np.float32(1e30)))
    pall = torch.full((c.m * n,), -1.0, dtype=torch.float64, device="cuda")
    sq = torch.empty(n, dtype=torch.float64, device="cuda")
    R.rs_ragged_sqnorm(c.lay.handle, x, sq, pall, None, c.lay.ws, 0, c.m)
    _sync()
    want = to_np(pall).reshape(c.m, n)
    for k in range(c.m):
        log(f"sqnorm one rank {name} [{k},{k + 1})")
        p1 = torch.full((c.m * n,), -1.0, dtype=torch.float64, device="cuda")
        sq1 = torch.full((n,), -1.0, dtype=torch.float64, device="cuda")
        R.rs_ragged_sqnorm(c.lay.handle, x, sq1, p1, None, c.lay.ws, k, k + 1)
        _sync()
        row = to_np(p1).reshape(c.m, n)[k]
        assert row.tobytes() == want[k].tobytes(), f"{name} rank {k} partial"
        assert to_np(sq1).tobytes() == row.tobytes(), f"{name} rank {k} sq"


def test_sqnorm_closed_forms():
    import torch
    c = case("ragged_a1_c64")
    R = c.R
    n = len(c.w.tensors)
    for fill, f in ((1.0, lambda E: float(E)), (3.0, lambda E: 9.0 * E)):
        x = torch.full((c.total,), fill, dtype=torch.float32, device="cuda")
        sq = torch.empty(n, dtype=torch.float64, device="cuda")
        R.rs_ragged_sqnorm(c.lay.handle, x, sq, None, None, c.lay.ws, 0, c.m)
        _sync()
        assert to_np(sq).tolist() == [f(s.numel) for s in c.w.tensors]


# ----------------------------------------------------------------- quant


def _quant_case(c, x0, fmt, k0, k1, what, only_tiles=None):
    import torch
    R = c.R
    nt = c.lay.info["num_tiles"]
    cw, codes = guarded(c.total, torch.uint8, U8_CANARY)
    sw, scales = guarded(max(nt, 1), torch.float32, F32_CANARY)
    R.rs_block_quant(c.lay.handle, from_np(x0), R.RS_Q_FP8_E4M3 if fmt == "fp8_e4m3" else R.RS_Q_INT8,
                     codes, scales, k0, k1)
    _sync()
    ecodes, escales = O.block_quant(x0, c.w.tensors, c.offsets, c.S, c.m, fmt, k0, k1,
                                    np.full(c.total, U8_CANARY, np.uint8),
                                    np.full(max(nt, 1), F32_CANARY, np.uint32).view(np.float32),
                                    only_tiles=only_tiles)
    gc, gs = to_np(codes), to_np(scales)
    if only_tiles is None:
        assert_bits_equal(gc, ecodes, what + " codes")
        assert_bits_equal(gs, escales, what + " scales")
    else:
        return gc, gs, ecodes, escales
    check_guards(cw, U8_CANARY, what + " codes")
    check_guards(sw, F32_CANARY, what + " scales")


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("fmt", ["fp8_e4m3", "int8"])
def test_block_quant(name, fmt):
    c = case(name)
    inp = c.inputs()
    for src in ("params", "grads"):
        x0 = c.flat(getattr(inp, src), fill=np.float32(np.nan))  # padding is never read
        for k0, k1 in c.ranges():
            log(f"quant {name} {fmt} {src} [{k0},{k1})")
            _quant_case(c, x0, fmt, k0, k1, f"quant {name} {fmt} {src} [{k0},{k1})")


def _tie_stress_values(rng, scale, fmt, n):
    """x such that x/scale lands on or next to a rounding midpoint of the
    code grid, where a wrongly rounded division changes the code."""
    if fmt == "fp8_e4m3":
        codes = np.arange(0, 0x7E)
        mids = (OC.e4m3fn_to_f64(codes) + OC.e4m3fn_to_f64(codes + 1)) / 2
    else:
        mids = np.arange(0, 127) + 0.5
    mids = rng.choice(mids, size=n)
    x = (mids * scale).astype(np.float32)
    bump = rng.integers(-2, 3, size=n).astype(np.int32)
    x = (x.view(np.int32) + bump).view(np.float32)
    sign = np.where(rng.random(n) < 0.5, -1, 1).astype(np.float32)
    return x * sign


@pytest.mark.parametrize("fmt", ["fp8_e4m3", "int8"])
def test_block_quant_special_values(fmt):
    """Zero tiles, underflowing scales, huge values, infinities, NaN,
    subnormals and division results next to code midpoints."""
    c = case("toy")
    rng = np.random.default_rng(17)
    x0 = c.flat(c.inputs().params, fill=np.float32(np.nan))
    tiles = []
    for s, l in zip(c.w.tensors, c.offsets):
        for (r0, r1, c0, c1) in O.tile_grid(s.rows, s.cols, s.q_rows, s.q_cols):
            pos = l + (np.arange(r0, r1)[:, None] * s.cols + np.arange(c0, c1)[None, :])
            tiles.append(pos.reshape(-1))
    Q = 448.0 if fmt == "fp8_e4m3" else 127.0
    for j, pos in enumerate(tiles):
        kind = j % 9
        n = pos.size
        if kind == 0:
            x0[pos] = 0.0
        elif kind == 1:
            x0[pos] = (rng.standard_normal(n) * 1e-42).astype(np.float32)   # subnormal, scale 0
        elif kind == 2:
            x0[pos] = (rng.standard_normal(n) * 1e37).astype(np.float32)
        elif kind == 3:
            x0[pos[rng.integers(0, n)]] = np.float32(np.inf) * (1 if j % 2 else -1)
        elif kind == 4:
            x0[pos[rng.integers(0, n)]] = np.nan
        elif kind in (5, 6, 7):
            amax = np.float32(Q * 10 ** rng.uniform(-3, 3))
            scale = np.float32(amax / np.float32(Q))
            v = _tie_stress_values(rng, float(scale), fmt, n - 1)
            v = np.clip(v, -amax, amax)
            x0[pos[0]] = amax
            x0[pos[1:]] = v
        else:
            x0[pos] = (rng.standard_normal(n) * 2.0 ** rng.integers(-140, -100)).astype(np.float32)
    for k0, k1 in c.ranges():
        _quant_case(c, x0, fmt, k0, k1, f"quant special {fmt} [{k0},{k1})")


def test_rank_range_errors():
    import torch
    c = case("toy")
    R = c.R
    x = torch.zeros(c.total, dtype=torch.float32, device="cuda")
    for k0, k1 in ((0, 0), (2, 1), (-1, 2), (0, c.m + 1)):
        with pytest.raises(R.RsError) as e:
            R.rs_group_zero(c.lay.handle, x, R.RS_F32, None, k0, k1)
        assert e.value.status == -5
    with pytest.raises(R.RsError) as e:
        R.rs_group_zero(c.lay.handle, x, R.RS_U8, None, 0, 1)
    assert e.value.status == -2
    with pytest.raises(R.RsError) as e:   # fp32 data at an odd byte address
        R.rs_group_zero(c.lay.handle, x.view(torch.uint8)[1:].data_ptr(), R.RS_F32, None, 0, 1)
    assert e.value.status == -3


# --------------------------------------------------------------- dequant


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("fmt", ["fp8_e4m3", "int8"])
def test_block_dequant(name, fmt):
    import torch
    c = case(name)
    R = c.R
    nt = c.lay.info["num_tiles"]
    x0 = c.flat(c.inputs().grads, fill=np.float32(np.nan))
    codes0, scales0 = O.block_quant(x0, c.w.tensors, c.offsets, c.S, c.m, fmt, 0, c.m,
                                    np.zeros(c.total, np.uint8), np.zeros(max(nt, 1), np.float32))
    dc, ds = from_np(codes0), from_np(scales0)
    qf = R.RS_Q_FP8_E4M3 if fmt == "fp8_e4m3" else R.RS_Q_INT8
    for yk in ("f32", "bf16"):
        ydt = torch.bfloat16 if yk == "bf16" else torch.float32
        canary = BF16_CANARY if yk == "bf16" else F32_CANARY
        for k0, k1 in c.ranges():
            log(f"dequant {name} {fmt} {yk} [{k0},{k1})")
            yw, y = guarded(c.total, ydt, canary)
            R.rs_block_dequant(c.lay.handle, dc, qf, ds, y, R.RS_BF16 if yk == "bf16" else R.RS_F32, k0, k1)
            _sync()
            init = np.full(c.total, canary, dtype=np.uint16 if yk == "bf16" else np.uint32)
            if yk == "f32":
                init = init.view(np.float32)
            exp = O.block_dequant(codes0, scales0, c.w.tensors, c.offsets, c.S, c.m, fmt, k0, k1,
                                  init, yk)
            got = to_np(y)
            what = f"dequant {name} {fmt} {yk} [{k0},{k1})"
            if yk == "f32":
                assert_f32_equal_nan_class(got, exp, what)
            else:
                gn = (got & 0x7FFF) > 0x7F80
                en = (exp & 0x7FFF) > 0x7F80
                assert np.array_equal(gn, en), what + " NaN"
                assert_bits_equal(np.where(gn, 0, got), np.where(en, 0, exp), what)
            check_guards(yw, canary, what)


@pytest.mark.parametrize("fmt", ["fp8_e4m3", "int8"])
def test_block_dequant_all_codes(fmt):
    import torch
    c = case("toy")
    R = c.R
    nt = c.lay.info["num_tiles"]
    rng = np.random.default_rng(41)
    codes = rng.integers(0, 256, size=c.total).astype(np.uint8)
    codes[c.offsets[0]:c.offsets[0] + 256] = np.arange(256, dtype=np.uint8)
    scales = (2.0 ** rng.uniform(-20, 20, size=nt)).astype(np.float32)
    scales[0] = 1.0
    y = torch.empty(c.total, dtype=torch.float32, device="cuda")
    R.rs_block_dequant(c.lay.handle, from_np(codes), R.RS_Q_FP8_E4M3 if fmt == "fp8_e4m3" else R.RS_Q_INT8,
                       from_np(scales), y, R.RS_F32, 0, c.m)
    _sync()
    exp = O.block_dequant(codes, scales, c.w.tensors, c.offsets, c.S, c.m, fmt, 0, c.m,
                          np.zeros(c.total, np.float32), "f32")
    assert_f32_equal_nan_class(to_np(y), exp, f"dequant all codes {fmt}")


def test_block_quant_found_inf():
    import torch
    c = case("mixed_div")
    R = c.R
    nt = c.lay.info["num_tiles"]
    x0 = c.flat(c.inputs().grads)
    ef = O.quant_found_inf(x0, c.w.tensors, c.offsets, c.S, c.m, 0, c.m)
    assert ef.any()
    fi = torch.zeros(c.m, dtype=torch.int32, device="cuda")
    codes = torch.empty(c.total, dtype=torch.uint8, device="cuda")
    scales = torch.empty(nt, dtype=torch.float32, device="cuda")
    R.rs_block_quant(c.lay.handle, from_np(x0), R.RS_Q_INT8, codes, scales, 0, c.m, found_inf=fi)
    _sync()
    assert np.array_equal(to_np(fi).astype(np.uint32), ef)


def test_no_tiles_accepts_null_scales():
    """A layout without quantisation tiles: quantise, dequantise and the
    8-bit step accept NULL scale arrays and write nothing."""
    import torch
    c = case("no_quant")
    R = c.R
    assert c.lay.info["num_tiles"] == 0
    x = from_np(c.flat(c.inputs().grads))
    codes = torch.full((c.total,), U8_CANARY, dtype=torch.uint8, device="cuda")
    y = torch.full((c.total,), 3.0, dtype=torch.float32, device="cuda")
    for fmt in (R.RS_Q_FP8_E4M3, R.RS_Q_INT8):
        R.rs_block_quant(c.lay.handle, x, fmt, codes, None, 0, c.m)
        R.rs_block_dequant(c.lay.handle, codes, fmt, None, y, R.RS_F32, 0, c.m)
        R.rs_adamw8_step(c.lay.handle, y, x, codes, None, codes, None, fmt, 1e-3, 0.9, 0.95, 1e-8, 0.0,
                         0.5, 0.5, 1.0, None, 0, c.m)
    _sync()
    assert bool((codes == U8_CANARY).all()) and bool((y == 3.0).all())


@pytest.mark.timeout(900)
def test_pack_bf16_cast_every_fp32_pattern():
    """rs_pack's fp32 -> bf16 cast on all 2^32 fp32 bit patterns (one vector
    tensor, one rank, 2^24 patterns per launch) against the oracle's RNE
    cast, NaN payloads included.  The oracle runs on host threads, a wave of
    chunks at a time."""
    from concurrent.futures import ThreadPoolExecutor

    import torch
    R = case("toy").R
    N = 1 << 24
    spec = [W.TensorSpec("v", 1, N, 0)]
    offs, info = R.rs_plan(spec, 1, 16)
    lay = R.Layout(spec, 1, info["S"], offs)
    src = torch.empty(N, dtype=torch.int32, device="cuda")
    table = R.ptr_table([src])
    buf = torch.empty(info["S"], dtype=torch.bfloat16, device="cuda")
    base = torch.arange(N, dtype=torch.int64, device="cuda")

    def expected(first):
        return OC.bf16_bits_from_f32(np.arange(first, first + N, dtype=np.uint64).astype(np.uint32)
                                     .view(np.float32))

    wave = 16
    with ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
        for w0 in range(0, 1 << 32, wave * N):
            firsts = list(range(w0, min(w0 + wave * N, 1 << 32), N))
            futs = [ex.submit(expected, f) for f in firsts]
            got = []
            for first in firsts:
                v = base + first
                src.copy_(torch.where(v >= (1 << 31), v - (1 << 32), v).to(torch.int32))
                R.rs_pack(lay.handle, table, R.RS_F32, buf, R.RS_BF16, 0, 1)
                got.append(to_np(buf)[:N].copy())
            log(f"bf16 cast: patterns up to {firsts[-1] + N:#011x}")
            for first, g, f in zip(firsts, got, futs):
                exp = f.result()
                if not np.array_equal(g, exp):
                    i = int(np.flatnonzero(g != exp)[0])
                    raise AssertionError(f"bf16 cast of {first + i:#010x}: got {g[i]:#06x} "
                                         f"expected {exp[i]:#06x}")
    lay.close()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("fmt,amax_value", [("fp8_e4m3", 1344.0), ("int8", 1344.0),
                                            ("fp8_e4m3", 1791.9998779296875),
                                            ("fp8_e4m3", 448.0), ("int8", 127.0)])
def test_quant_every_fp32_up_to_amax(fmt, amax_value):
    """Quantisation of every fp32 value x with |x| <= amax, both signs, in
    1 x 16384 tiles whose first element is amax.  With amax = 1344 the scale
    is fl(1344/Q) (3 for E4M3), an inexact reciprocal, so the codes come
    through the reciprocal fast path, its safety windows and the exact
    fallback over the whole code range.  amax = 1791.9998779296875 (the fp32
    below 1792) gives the scale just below 4 whose rounded reciprocal is off
    by almost half an ulp, the most rounding allows and the largest relative
    error for amax in [1024, 2048): there x times
    the reciprocal misses the rounded quotient for about 43% of x, so the
    window test decides many codes.  With amax = Q the scale is 1 and
    every code is the encoder applied to x itself: every fp32 input of the
    code range, each rounding midpoint included.  Against the oracle's cast
    of the fp32 quotient, with the oracle on host threads."""
    from concurrent.futures import ThreadPoolExecutor

    import torch
    R = case("toy").R
    T = 16384
    N = 1024 * T
    spec = [W.TensorSpec("v", 1, N, 1, 1, T)]
    offs, info = R.rs_plan(spec, 1, 16)
    lay = R.Layout(spec, 1, info["S"], offs)
    qf = R.RS_Q_FP8_E4M3 if fmt == "fp8_e4m3" else R.RS_Q_INT8
    Q = np.float32(448.0 if fmt == "fp8_e4m3" else 127.0)
    amax = np.float32(amax_value)
    scale = np.float32(amax / Q)
    top = int(amax.view(np.uint32))            # every magnitude pattern 0 .. top
    per = N - N // T                           # test values per launch (tile heads hold amax)
    x = torch.empty(N, dtype=torch.int32, device="cuda")
    codes = torch.empty(info["S"], dtype=torch.uint8, device="cuda")
    scales = torch.empty(N // T, dtype=torch.float32, device="cuda")
    body = torch.ones(N, dtype=torch.bool, device="cuda")
    body[::T] = False
    ar = torch.arange(per, dtype=torch.int64, device="cuda")

    def expected(first, sign):
        u = (np.arange(first, first + per, dtype=np.uint64).clip(max=top) | sign).astype(np.uint32)
        q = (u.view(np.float32) / scale).astype(np.float32)
        c = OC.e4m3fn_bits_from_f32(q) if fmt == "fp8_e4m3" else OC.int8_from_f32(q).view(np.uint8)
        return c

    hq = np.array([amax], np.float32) / scale
    head = int((OC.e4m3fn_bits_from_f32(hq) if fmt == "fp8_e4m3"
                else OC.int8_from_f32(hq).view(np.uint8))[0])
    body_np = to_np(body)
    jobs = [(first, sign) for sign in (0, 0x80000000) for first in range(0, top + 1, per)]
    with ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
        for j0 in range(0, len(jobs), 16):
            wave = jobs[j0:j0 + 16]
            futs = [ex.submit(expected, f, sg) for f, sg in wave]
            got = []
            for first, sign in wave:
                v = (ar + first).clamp(max=top) | sign
                v = torch.where(v >= (1 << 31), v - (1 << 32), v).to(torch.int32)
                x.fill_(int(amax.view(np.int32)))
                x[body] = v
                R.rs_block_quant(lay.handle, x.view(torch.float32), qf, codes, scales, 0, 1)
                c = to_np(codes)[:N]
                assert np.all(to_np(scales).view(np.uint32) == scale.view(np.uint32))
                assert np.all(c[::T] == head)
                got.append(c[body_np])
            log(f"quant {fmt}: {j0 + len(wave)} of {len(jobs)} launches")
            for (first, sign), g, f in zip(wave, got, futs):
                e = f.result()
                if not np.array_equal(g, e):
                    i = int(np.flatnonzero(g != e)[0])
                    raise AssertionError(f"{fmt} code of x = {(min(first + i, top) | sign):#010x} "
                                         f"/ {float(scale)}: got {g[i]:#04x} expected {e[i]:#04x}")
    lay.close()
