"""GPU parity of the fused optimizer steps (rs_adamw_step, rs_sgd_step)
through the C-ABI against the oracle: bit-exact fp32 (each operation rounded
once, IEEE sqrt and division on both sides), padding and masked tensors
untouched, guard bands intact, skipped when found_inf is set."""
import numpy as np
import pytest

from oracle import optim as OP

from harness import (SMALL, assert_f32_equal_nan_class, case, check_guards, from_np, guarded, log,
                     to_np)

pytestmark = pytest.mark.gpu

F32_CANARY = 0x7FA5A5A5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def _sync():
    import torch
    torch.cuda.synchronize()


def _state(c, seed):
    rng = np.random.default_rng(seed)
    inp = c.inputs()
    p = c.flat(inp.params, fill=np.float32(5.0))
    g = c.flat(inp.grads, fill=np.float32(-5.0))
    m = (rng.standard_normal(c.total) * 1e-4).astype(np.float32)
    v = np.abs(rng.standard_normal(c.total) * 1e-6).astype(np.float32)
    return p, g, m, v


def _dev(a):
    import torch
    whole, view = guarded(a.size, torch.float32, F32_CANARY)
    view.copy_(torch.from_numpy(a))
    return whole, view


HP = [
    dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, wd=0.1, bc1=1 - 0.9 ** 3, bc2=1 - 0.95 ** 3,
         grad_scale=1.0),
    dict(lr=3e-4, beta1=0.8, beta2=0.999, eps=1e-6, wd=0.0, bc1=0.2, bc2=0.001, grad_scale=65536.0),
]


@pytest.mark.parametrize("name", list(SMALL))
def test_adamw(name):
    import torch
    c = case(name)
    R = c.R
    p0, g0, m0, v0 = _state(c, 1)
    n = len(c.w.tensors)
    for hi, hp in enumerate(HP):
        for use_mask in (False, True):
            for k0, k1 in c.ranges()[:3]:
                log(f"adamw {name} hp{hi} mask={use_mask} [{k0},{k1})")
                (pw, p), (gw, g), (mw, m), (vw, v) = (_dev(a) for a in (p0, g0, m0, v0))
                mask = np.random.default_rng(2).integers(0, 2, size=n).astype(np.uint8) if use_mask else None
                R.rs_adamw_step(c.lay.handle, p, g, m, v, hp["lr"], hp["beta1"], hp["beta2"], hp["eps"],
                                hp["wd"], hp["bc1"], hp["bc2"], hp["grad_scale"],
                                from_np(mask) if use_mask else None, None, k0, k1)
                _sync()
                ep, em, ev = OP.adamw_step(p0, g0, m0, v0, c.items, c.offsets, c.S, c.m, k0, k1, hp,
                                           mask=None if mask is None else list(mask))
                what = f"adamw {name} hp{hi} [{k0},{k1})"
                for got, exp, nm in ((p, ep, "p"), (m, em, "m"), (v, ev, "v")):
                    assert_f32_equal_nan_class(to_np(got), exp, f"{what} {nm}")
                for wh in (pw, gw, mw, vw):
                    check_guards(wh, F32_CANARY, what)


def test_adamw_skipped_on_found_inf():
    import torch
    c = case("toy")
    R = c.R
    p0, g0, m0, v0 = _state(c, 3)
    p, g, m, v = (from_np(a) for a in (p0, g0, m0, v0))
    fi = torch.zeros(c.m, dtype=torch.int32, device="cuda")
    fi[c.m - 1] = 1
    hp = HP[0]
    R.rs_adamw_step(c.lay.handle, p, g, m, v, hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["wd"],
                    hp["bc1"], hp["bc2"], 1.0, None, fi, 0, c.m)
    _sync()
    assert np.array_equal(to_np(p), p0) and np.array_equal(to_np(m), m0) and np.array_equal(to_np(v), v0)
    fi.zero_()
    R.rs_adamw_step(c.lay.handle, p, g, m, v, hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["wd"],
                    hp["bc1"], hp["bc2"], 1.0, None, fi, 0, c.m)
    _sync()
    ep, _, _ = OP.adamw_step(p0, g0, m0, v0, c.items, c.offsets, c.S, c.m, 0, c.m, hp)
    assert_f32_equal_nan_class(to_np(p), ep, "adamw after clearing found_inf")


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("nesterov", [False, True])
def test_sgd(name, nesterov):
    import torch
    c = case(name)
    R = c.R
    p0, g0, b0, _ = _state(c, 4)
    for k0, k1 in c.ranges()[:3]:
        log(f"sgd {name} nesterov={nesterov} [{k0},{k1})")
        (pw, p), (gw, g), (bw, b) = (_dev(a) for a in (p0, g0, b0))
        R.rs_sgd_step(c.lay.handle, p, g, b, 0.05, 0.9, 1e-4, nesterov, 2.0, None, None, k0, k1)
        _sync()
        ep, eb = OP.sgd_step(p0, g0, b0, c.items, c.offsets, c.S, c.m, k0, k1, 0.05, 0.9, 1e-4,
                             nesterov, 2.0)
        what = f"sgd {name} [{k0},{k1})"
        assert_f32_equal_nan_class(to_np(p), ep, what + " p")
        assert_f32_equal_nan_class(to_np(b), eb, what + " buf")
        for wh in (pw, gw, bw):
            check_guards(wh, F32_CANARY, what)


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("fmt", ["int8", "fp8_e4m3"])
def test_adamw8(name, fmt):
    import torch
    from oracle import ops as O
    c = case(name)
    R = c.R
    nt = c.lay.info["num_tiles"]
    p0, g0, m0, v0 = _state(c, 6)
    mc0, ms0 = O.block_quant(m0, c.w.tensors, c.offsets, c.S, c.m, fmt, 0, c.m,
                             np.zeros(c.total, np.uint8), np.zeros(max(nt, 1), np.float32))
    vc0, vs0 = O.block_quant(v0, c.w.tensors, c.offsets, c.S, c.m, fmt, 0, c.m,
                             np.zeros(c.total, np.uint8), np.zeros(max(nt, 1), np.float32))
    hp = HP[0]
    qf = R.RS_Q_FP8_E4M3 if fmt == "fp8_e4m3" else R.RS_Q_INT8
    for step in range(2):          # two steps in a row: the second reads requantised states
        for k0, k1 in c.ranges()[:3]:
            if step == 1 and (k0, k1) != (0, c.m):
                continue
            log(f"adamw8 {name} {fmt} step{step} [{k0},{k1})")
            p, g = from_np(p0), from_np(g0)
            mc, ms, vc, vs = from_np(mc0), from_np(ms0), from_np(vc0), from_np(vs0)
            for _ in range(step + 1):
                R.rs_adamw8_step(c.lay.handle, p, g, mc, ms, vc, vs, qf, hp["lr"], hp["beta1"],
                                 hp["beta2"], hp["eps"], hp["wd"], hp["bc1"], hp["bc2"], hp["grad_scale"],
                                 None, k0, k1)
            _sync()
            e = (p0, mc0, ms0, vc0, vs0)
            for _ in range(step + 1):
                e = OP.adamw8_step(e[0], g0, e[1], e[2], e[3], e[4], c.w.tensors, c.offsets, c.S, c.m,
                                   k0, k1, fmt, hp)
            what = f"adamw8 {name} {fmt} step{step} [{k0},{k1})"
            assert_f32_equal_nan_class(to_np(p), e[0], what + " p")
            assert np.array_equal(to_np(mc), e[1]), what + " m codes"
            assert np.array_equal(to_np(ms).view(np.uint32), e[2].view(np.uint32)), what + " m scales"
            assert np.array_equal(to_np(vc), e[3]), what + " v codes"
            assert np.array_equal(to_np(vs).view(np.uint32), e[4].view(np.uint32)), what + " v scales"
