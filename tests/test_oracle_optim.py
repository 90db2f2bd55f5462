"""Pins for the optimizer oracle (CPU only): torch.optim's AdamW and SGD
(an independent implementation whose operation order differs, hence a
tolerance of a few ulp), closed forms of the first step, the skip on
found_inf, masks and rank ranges."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import optim as OP
from oracle import plan as P


def _group():
    return W.ragged_small()


def _setup():
    w = _group()
    items = P.items_from_specs(w.tensors)
    p = P.plan(items, w.m, 1)
    return w, items, p


def _bufs(total, seed=0):
    rng = np.random.default_rng(seed)
    p = (rng.standard_normal(total) * 0.02).astype(np.float32)
    g = (rng.standard_normal(total) * 1e-3).astype(np.float32)
    m = (rng.standard_normal(total) * 1e-4).astype(np.float32)
    v = np.abs(rng.standard_normal(total) * 1e-6).astype(np.float32)
    return p, g, m, v


@pytest.mark.parametrize("step", [1, 7, 1000])
def test_adamw_matches_torch(step):
    w, items, pl = _setup()
    p, g, m, v = _bufs(pl.total, step)
    lr, b1, b2, eps, wd = 1e-3, 0.9, 0.95, 1e-8, 0.1
    hp = dict(lr=lr, beta1=b1, beta2=b2, eps=eps, wd=wd, bc1=1 - b1 ** step, bc2=1 - b2 ** step,
              grad_scale=1.0)
    p2, m2, v2 = OP.adamw_step(p, g, m, v, items, pl.offsets, pl.S, w.m, 0, w.m, hp)
    for it, l in zip(items, pl.offsets):
        sl = slice(l, l + it.numel)
        tp = torch.nn.Parameter(torch.from_numpy(p[sl].copy()))
        opt = torch.optim.AdamW([tp], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd,
                                foreach=False, fused=False)
        opt.state[tp]["step"] = torch.tensor(float(step - 1))
        opt.state[tp]["exp_avg"] = torch.from_numpy(m[sl].copy())
        opt.state[tp]["exp_avg_sq"] = torch.from_numpy(v[sl].copy())
        tp.grad = torch.from_numpy(g[sl].copy())
        opt.step()
        # absolute tolerances of a few ulp of the operands (torch forms the
        # first moment with lerp, so cancellation shows up as absolute error)
        np.testing.assert_allclose(p2[sl], tp.detach().numpy(), rtol=2e-6, atol=1e-8)
        np.testing.assert_allclose(m2[sl], opt.state[tp]["exp_avg"].numpy(), rtol=2e-6,
                                   atol=1e-6 * float(np.abs(g[sl]).max()))
        np.testing.assert_allclose(v2[sl], opt.state[tp]["exp_avg_sq"].numpy(), rtol=2e-6,
                                   atol=1e-6 * float((g[sl].astype(np.float64) ** 2).max()))


def test_adamw_first_step_closed_form():
    # from zero moments, step 1: m' = (1-b1) g, v' = (1-b2) g^2, so the update
    # is g / (|g| + eps) in exact arithmetic: about sign(g) when |g| >> eps
    w, items, pl = _setup()
    p, g, _, _ = _bufs(pl.total, 3)
    g = np.where(np.abs(g) < 1e-4, np.float32(1e-3), g).astype(np.float32)
    z = np.zeros_like(p)
    lr, b1, b2 = 1e-2, 0.9, 0.999
    hp = dict(lr=lr, beta1=b1, beta2=b2, eps=1e-12, wd=0.0, bc1=1 - b1, bc2=1 - b2, grad_scale=1.0)
    p2, m2, v2 = OP.adamw_step(p, g, z, z, items, pl.offsets, pl.S, w.m, 0, w.m, hp)
    for it, l in zip(items, pl.offsets):
        sl = slice(l, l + it.numel)
        np.testing.assert_allclose(p2[sl], p[sl] - lr * np.sign(g[sl]), rtol=0, atol=lr * 1e-5)
        np.testing.assert_allclose(m2[sl], (1 - b1) * g[sl], rtol=1e-6)


def test_adamw_skip_mask_range_and_unscale():
    w, items, pl = _setup()
    p, g, m, v = _bufs(pl.total, 5)
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, wd=0.01, bc1=0.1, bc2=0.001, grad_scale=1.0)
    found = np.zeros(w.m, np.uint32)
    found[3] = 1
    out = OP.adamw_step(p, g, m, v, items, pl.offsets, pl.S, w.m, 0, w.m, hp, found_inf=found)
    assert np.array_equal(out[0], p) and np.array_equal(out[1], m) and np.array_equal(out[2], v)
    mask = [1, 0, 1, 0, 1]
    p2, m2, v2 = OP.adamw_step(p, g, m, v, items, pl.offsets, pl.S, w.m, 1, 3, hp, mask=mask)
    changed = p2 != p
    for t, (it, l) in enumerate(zip(items, pl.offsets)):
        seg = changed[l:l + it.numel]
        pos = np.arange(l, l + it.numel)
        inside = (pos >= pl.S) & (pos < 3 * pl.S)
        if not mask[t]:
            assert not seg.any()
        else:
            assert not seg[~inside].any()
    pads = np.ones(pl.total, bool)
    for it, l in zip(items, pl.offsets):
        pads[l:l + it.numel] = False
    assert not changed[pads].any()
    # grad_scale: scaling g by 1024 and passing grad_scale=1024 gives the same step
    g_scaled = (g * np.float32(1024)).astype(np.float32)
    hp2 = dict(hp, grad_scale=1024.0)
    a = OP.adamw_step(p, g, m, v, items, pl.offsets, pl.S, w.m, 0, w.m, hp)
    b = OP.adamw_step(p, g_scaled, m, v, items, pl.offsets, pl.S, w.m, 0, w.m, hp2)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)      # power-of-two scaling is exact


@pytest.mark.parametrize("nesterov", [False, True])
def test_sgd_matches_torch(nesterov):
    w, items, pl = _setup()
    p, g, b, _ = _bufs(pl.total, 9)
    lr, mu, wd = 0.05, 0.9, 1e-4
    p2, b2 = OP.sgd_step(p, g, b, items, pl.offsets, pl.S, w.m, 0, w.m, lr, mu, wd, nesterov, 1.0)
    for it, l in zip(items, pl.offsets):
        sl = slice(l, l + it.numel)
        tp = torch.nn.Parameter(torch.from_numpy(p[sl].copy()))
        opt = torch.optim.SGD([tp], lr=lr, momentum=mu, weight_decay=wd, nesterov=nesterov,
                              foreach=False)
        opt.state[tp]["momentum_buffer"] = torch.from_numpy(b[sl].copy())
        tp.grad = torch.from_numpy(g[sl].copy())
        opt.step()
        np.testing.assert_allclose(p2[sl], tp.detach().numpy(), rtol=1e-6, atol=1e-10)
        np.testing.assert_allclose(b2[sl], opt.state[tp]["momentum_buffer"].numpy(), rtol=1e-6, atol=1e-10)


@pytest.mark.parametrize("fmt", ["int8", "fp8_e4m3"])
def test_adamw8_composes_pinned_parts(fmt):
    """8-bit Adam = dequantise, the fp32 AdamW update, requantise: each part
    is pinned on its own; check the composition, the untouched vector and
    the found_inf skip."""
    from oracle import ops as O
    w, items, pl = _setup()
    p, g, m, v = _bufs(pl.total, 11)
    nt = O.num_tiles(w.tensors)
    mc, ms = O.block_quant(m, w.tensors, pl.offsets, pl.S, w.m, fmt, 0, w.m,
                           np.zeros(pl.total, np.uint8), np.zeros(nt, np.float32))
    vc, vs = O.block_quant(v, w.tensors, pl.offsets, pl.S, w.m, fmt, 0, w.m,
                           np.zeros(pl.total, np.uint8), np.zeros(nt, np.float32))
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, wd=0.1, bc1=0.5, bc2=0.2, grad_scale=1.0)
    p2, mc2, ms2, vc2, vs2 = OP.adamw8_step(p, g, mc, ms, vc, vs, w.tensors, pl.offsets, pl.S, w.m,
                                            0, w.m, fmt, hp)
    md = O.block_dequant(mc, ms, w.tensors, pl.offsets, pl.S, w.m, fmt, 0, w.m, m.copy(), "f32")
    vd = O.block_dequant(vc, vs, w.tensors, pl.offsets, pl.S, w.m, fmt, 0, w.m, v.copy(), "f32")
    ep, em, ev = OP.adamw_step(p, g, md, vd, items, pl.offsets, pl.S, w.m, 0, w.m, hp)
    quantised = np.zeros(pl.total, bool)
    for s, l in zip(w.tensors, pl.offsets):
        if s.q_rows:
            quantised[l:l + s.numel] = True
    assert np.array_equal(p2[quantised], ep[quantised])
    assert np.array_equal(p2[~quantised], p[~quantised])        # vector untouched
    emc, ems = O.block_quant(em, w.tensors, pl.offsets, pl.S, w.m, fmt, 0, w.m,
                             np.zeros(pl.total, np.uint8), np.zeros(nt, np.float32))
    assert np.array_equal(mc2[quantised], emc[quantised]) and np.array_equal(ms2, ems)
    evc, evs = O.block_quant(ev, w.tensors, pl.offsets, pl.S, w.m, fmt, 0, w.m,
                             np.zeros(pl.total, np.uint8), np.zeros(nt, np.float32))
    assert np.array_equal(vc2[quantised], evc[quantised]) and np.array_equal(vs2, evs)
    # found_inf skips everything
    out = OP.adamw8_step(p, g, mc, ms, vc, vs, w.tensors, pl.offsets, pl.S, w.m, 0, w.m, fmt, hp,
                         found_inf=np.ones(w.m, np.uint32))
    for a, b in zip(out, (p, mc, ms, vc, vs)):
        assert np.array_equal(a, b)
