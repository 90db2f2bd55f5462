"""GPU parity at the full sizes of the four large groups, in the launch
configuration bench.py times (align 16, default chunks, the whole rank
range).  Whole-buffer outputs are compared with the oracle run rank by rank.

The tile operations (quantisation, dequantisation, 8-bit AdamW) are compared
on every tile of every group, fragment by fragment (one quantised tensor's
tiles inside one rank), with digests of the oracle's outputs written by
tests/golden/make_fullsize_digests.py, which runs only the oracle; a
fragment whose digest differs is recomputed here by the oracle to name the
first differing element.  The one exception is the mixed group's embedding
(4.1M one-row tiles): it is compared with the oracle on a sample of tiles
(random ones, the first and last of every rank, and tiles holding injected
non-finite values).
"""
import gc
import json
import os

import numpy as np
import pytest

import workloads as W
from oracle import ops as O
from oracle import plan as P

import fullsize_cases as FC
from harness import assert_bits_equal, assert_f32_equal_nan_class, log, to_np

pytestmark = pytest.mark.gpu

FULL = list(FC.GROUPS)
DIGESTS = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "fullsize_digests.json")


class Full:
    def __init__(self, name):
        import torch

        import fsdp_sharded_buffer_amd as R
        self.R = R
        self.w = w = W.WORKLOADS[name]
        log(f"full {name}: plan")
        offs, info = R.rs_plan(w.tensors, w.m, 16)
        self.S, self.offsets, self.m = info["S"], offs, w.m
        self.items = P.items_from_specs(w.tensors)
        self.total = w.m * self.S
        self.lay = R.Layout(w.tensors, w.m, self.S, offs)
        log(f"full {name}: inputs ({w.numel} elements)")
        self.inp = W.make_inputs(w)
        self.params = [torch.from_numpy(a).cuda() for a in self.inp.params]
        self.grad_host = self._flat(self.inp.grads)
        self.param_host = self._flat(self.inp.params)
        log(f"full {name}: ready, S={self.S}")

    def _flat(self, arrays):
        b = np.zeros(self.total, np.float32)
        for a, l in zip(arrays, self.offsets):
            b[l:l + a.size] = a.reshape(-1)
        return b

    def free(self):
        import torch
        self.lay.close()
        for k in list(self.__dict__):
            if k not in ("w", "m", "S", "offsets"):
                setattr(self, k, None)
        gc.collect()
        torch.cuda.empty_cache()


@pytest.fixture(scope="module", params=FULL)
def fx(request):
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    f = Full(request.param)
    yield f
    f.free()


def _sync():
    import torch
    torch.cuda.synchronize()


@pytest.mark.timeout(600)
def test_full_pack_unpack(fx):
    import torch
    R = fx.R
    log(f"full pack {fx.w.name}")
    buf = torch.empty(fx.total, dtype=torch.bfloat16, device="cuda")
    buf.view(torch.int16).fill_(0x7FA5)
    R.rs_pack(fx.lay.handle, R.ptr_table(fx.params), R.RS_F32, buf, R.RS_BF16, 0, fx.m)
    _sync()
    got = to_np(buf)
    exp = np.full(fx.total, 0x7FA5, np.uint16)
    for k in range(fx.m):
        O.pack(fx.inp.params, fx.offsets, fx.S, fx.m, exp, "bf16", k, k + 1, inplace=True)
    assert_bits_equal(got, exp, f"full pack {fx.w.name}")
    log(f"full unpack {fx.w.name}")
    outs = [torch.empty(s.numel, dtype=torch.float32, device="cuda") for s in fx.w.tensors]
    R.rs_unpack(fx.lay.handle, buf, R.RS_BF16, R.ptr_table(outs), R.RS_F32, 0, fx.m)
    _sync()
    for t, (o, s) in enumerate(zip(outs, fx.w.tensors)):
        l = fx.offsets[t]
        ref = (exp[l:l + s.numel].astype(np.uint32) << 16).view(np.float32)
        assert_bits_equal(to_np(o), ref, f"full unpack {fx.w.name} t{t}")
    del outs, buf


@pytest.mark.timeout(600)
def test_full_scale_add_zero(fx):
    import torch
    R = fx.R
    log(f"full scale_add {fx.w.name}")
    y = torch.from_numpy(fx.param_host).cuda()
    x = torch.from_numpy(fx.grad_host).cuda()
    fi = torch.zeros(fx.m, dtype=torch.int32, device="cuda")
    R.rs_group_scale_add(fx.lay.handle, y, x, R.RS_F32, 0.5, -2.0, None, fi, 0, fx.m)
    _sync()
    ey = fx.param_host.copy()
    ef = np.zeros(fx.m, np.uint32)
    for k in range(fx.m):
        _, f = O.scale_add(ey, fx.grad_host, 0.5, -2.0, fx.items, fx.offsets, fx.S, fx.m, k, k + 1,
                           inplace=True)
        ef |= f
    assert_f32_equal_nan_class(to_np(y), ey, f"full scale_add {fx.w.name}")
    assert np.array_equal(to_np(fi).astype(np.uint32), ef)
    if fx.w.nonfinite_frac:
        assert ef.sum() >= fx.m - 1       # non-finite grads reach (nearly) every rank
    log(f"full zero {fx.w.name}")
    R.rs_group_zero(fx.lay.handle, x, R.RS_F32, None, 0, fx.m)
    _sync()
    assert not torch.any(x != 0).item()
    del y, x


@pytest.mark.timeout(600)
def test_full_sqnorm(fx):
    import torch
    R = fx.R
    log(f"full sqnorm {fx.w.name}")
    n = len(fx.w.tensors)
    for src, host in (("params", fx.param_host), ("grads", fx.grad_host)):
        x = torch.from_numpy(host).cuda()
        sq = torch.empty(n, dtype=torch.float64, device="cuda")
        part = torch.empty(fx.m * n, dtype=torch.float64, device="cuda")
        fi = torch.zeros(fx.m, dtype=torch.int32, device="cuda")
        R.rs_ragged_sqnorm(fx.lay.handle, x, sq, part, fi, fx.lay.ws, 0, fx.m)
        sq2 = torch.empty_like(sq)
        R.rs_ragged_sqnorm(fx.lay.handle, x, sq2, None, None, fx.lay.ws, 0, fx.m)
        _sync()
        esq, epart, ef = O.sqnorm(host, fx.items, fx.offsets, fx.S, fx.m, 0, fx.m)
        g, gp = to_np(sq), to_np(part).reshape(fx.m, n)
        for got, exp, what in ((g, esq, "sq"), (gp, epart, "partial")):
            assert np.array_equal(np.isnan(got), np.isnan(exp)), what
            assert np.array_equal(np.isinf(got), np.isinf(exp)), what
            f = np.isfinite(exp)
            rel = np.abs(got[f] - exp[f]) / np.maximum(np.abs(exp[f]), 1e-300)
            assert np.all(rel <= 1e-5), f"{fx.w.name} {src} {what}: {rel.max()}"
        assert np.array_equal(to_np(fi).astype(np.uint32), ef)
        assert np.array_equal(to_np(sq2).view(np.uint64), g.view(np.uint64))
        del x


@pytest.mark.timeout(600)
def test_full_adamw(fx):
    import torch
    from oracle import optim as OP
    R = fx.R
    log(f"full adamw {fx.w.name}")
    rng = np.random.default_rng(29)
    m0 = (rng.standard_normal(fx.total) * 1e-4).astype(np.float32)
    v0 = np.abs(rng.standard_normal(fx.total) * 1e-6).astype(np.float32)
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, wd=0.1, bc1=1 - 0.9 ** 5,
              bc2=1 - 0.95 ** 5, grad_scale=1.0)
    p = torch.from_numpy(fx.param_host).cuda()
    g = torch.from_numpy(fx.grad_host).cuda()
    m = torch.from_numpy(m0).cuda()
    v = torch.from_numpy(v0).cuda()
    R.rs_adamw_step(fx.lay.handle, p, g, m, v, hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["wd"],
                    hp["bc1"], hp["bc2"], 1.0, None, None, 0, fx.m)
    _sync()
    ep, em, ev = fx.param_host.copy(), m0, v0
    for k in range(fx.m):
        OP.adamw_step(ep, fx.grad_host, em, ev, fx.items, fx.offsets, fx.S, fx.m, k, k + 1, hp,
                      inplace=True)
    assert_f32_equal_nan_class(to_np(p), ep, f"full adamw {fx.w.name} p")
    assert_f32_equal_nan_class(to_np(m), em, f"full adamw {fx.w.name} m")
    assert_f32_equal_nan_class(to_np(v), ev, f"full adamw {fx.w.name} v")
    del p, g, m, v


@pytest.mark.timeout(600)
def test_full_sgd(fx):
    import torch
    from oracle import optim as OP
    R = fx.R
    log(f"full sgd {fx.w.name}")
    rng = np.random.default_rng(37)
    b0 = (rng.standard_normal(fx.total) * 1e-3).astype(np.float32)
    p = torch.from_numpy(fx.param_host).cuda()
    g = torch.from_numpy(fx.grad_host).cuda()
    b = torch.from_numpy(b0).cuda()
    R.rs_sgd_step(fx.lay.handle, p, g, b, 0.05, 0.9, 1e-4, True, 1.0, None, None, 0, fx.m)
    _sync()
    ep, eb = OP.sgd_step(fx.param_host, fx.grad_host, b0, fx.items, fx.offsets, fx.S, fx.m, 0, fx.m,
                         0.05, 0.9, 1e-4, True, 1.0)
    assert_f32_equal_nan_class(to_np(p), ep, f"full sgd {fx.w.name} p")
    assert_f32_equal_nan_class(to_np(b), eb, f"full sgd {fx.w.name} buf")
    del p, g, b


def _digests(fx):
    """The oracle's digests for this group; the layout must be the one they
    were computed on."""
    d = json.load(open(DIGESTS))[fx.w.name]
    assert d["S"] == fx.S and d["offsets"] == list(fx.offsets), "digests are for another layout"
    assert d["num_tiles"] == fx.lay.info["num_tiles"]
    return d


def _embedding_sample(fx, rng, n_random, ranks=None):
    """Global tile indices of a sample of each tensor with more than
    FC.SAMPLE_ABOVE tiles: n_random random tiles, the first and last tile of
    every rank, and up to 200 tiles holding injected non-finite values
    (restricted to `ranks` when given)."""
    out, base = [], 0
    flat_starts = np.cumsum([0] + [s.numel for s in fx.w.tensors])
    bad = fx.inp.nonfinite_positions
    for t, (s, l) in enumerate(zip(fx.w.tensors, fx.offsets)):
        if not s.q_rows:
            continue
        rk = FC.tile_ranks(s, l, fx.S)
        if rk.size > FC.SAMPLE_ABOVE:
            keep = np.ones(rk.size, bool) if ranks is None else np.isin(rk, ranks)
            idx = np.flatnonzero(keep)
            pick = set(int(i) for i in rng.choice(idx, size=min(n_random, idx.size), replace=False))
            for k in np.unique(rk[keep]):
                on = np.flatnonzero(rk == k)
                pick.update((int(on[0]), int(on[-1])))
            mine = bad[(bad >= flat_starts[t]) & (bad < flat_starts[t + 1])] - flat_starts[t]
            if mine.size:
                r, c = np.divmod(mine, s.cols)
                _, ntc = O.tile_counts(s)
                ti = (r // s.q_rows) * ntc + c // s.q_cols
                ti = ti[keep[ti]]
                pick.update(int(i) for i in rng.choice(ti, size=min(200, ti.size), replace=False))
            out.append(base + np.array(sorted(pick), np.int64))
        base += rk.size
    return np.concatenate(out) if out else np.zeros(0, np.int64)


def _compare_fragments(fx, frags, got, expected, oracle_frag, what):
    """Digest of each fragment's device outputs against the oracle's; on a
    difference, the oracle recomputes that fragment (oracle_frag(frag) ->
    list of (device array, expected array, name)) to report the element."""
    bad = [f for f, e in zip(frags, expected) if got(f) != e]
    if bad:
        t, k, lo, hi, a, b = bad[0]
        for dev, exp, name in oracle_frag(bad[0]):
            if exp.dtype == np.float32:
                assert_f32_equal_nan_class(dev, exp, f"{what}: tensor {t} rank {k} {name}")
            else:
                assert_bits_equal(dev, exp, f"{what}: tensor {t} rank {k} {name}")
        raise AssertionError(f"{what}: {len(bad)} fragments differ from the oracle's digests, "
                             f"first tensor {t} rank {k}, yet its outputs match on recomputation")


@pytest.mark.timeout(900)
def test_full_block_quant(fx):
    """Quantisation of the params and the grads buffers over the whole range
    and dequantisation of the device's codes, every fragment against the
    oracle's digests (the embedding against the oracle on a tile sample)."""
    import torch
    R = fx.R
    dig = _digests(fx)
    frags = [tuple(f) for f in dig["frags"]]
    rng = np.random.default_rng(23)
    fmt = fx.w.qfmt
    qf = R.RS_Q_FP8_E4M3 if fmt == "fp8_e4m3" else R.RS_Q_INT8
    nt = fx.lay.info["num_tiles"]
    sample = _embedding_sample(fx, rng, 3000)
    spos = _tile_positions(fx, list(sample)) if sample.size else np.zeros(0, np.int64)
    quantised = np.zeros(fx.total, bool)
    for s, l in zip(fx.w.tensors, fx.offsets):
        if s.q_rows:
            quantised[l:l + s.numel] = True
    for src, host in (("params", fx.param_host), ("grads", fx.grad_host)):
        log(f"full quant {fx.w.name} {src}: {len(frags)} fragments, {sample.size} sampled tiles")
        x = torch.from_numpy(host).cuda()
        codes = torch.full((fx.total,), 0xAB, dtype=torch.uint8, device="cuda")
        scales = torch.empty(nt, dtype=torch.float32, device="cuda")
        R.rs_block_quant(fx.lay.handle, x, qf, codes, scales, 0, fx.m)
        y = torch.full((fx.total,), float("nan"), dtype=torch.float32, device="cuda")
        R.rs_block_dequant(fx.lay.handle, codes, qf, scales, y, R.RS_F32, 0, fx.m)
        _sync()
        gc_, gs, gy = to_np(codes), to_np(scales), to_np(y)

        def oracle_frag(f, host=host):
            t, k, lo, hi, a, b = f
            ec, es = np.zeros(fx.total, np.uint8), np.zeros(nt, np.float32)
            O.block_quant(host, fx.w.tensors, fx.offsets, fx.S, fx.m, fmt, k, k + 1, ec, es,
                          only_tiles=range(a, b), inplace=True)
            ey = O.block_dequant(ec, es, fx.w.tensors, fx.offsets, fx.S, fx.m, fmt, k, k + 1,
                                 np.zeros(fx.total, np.float32), "f32", only_tiles=range(a, b))
            return [(gc_[lo:hi], ec[lo:hi], "codes"), (gs[a:b], es[a:b], "scales"),
                    (gy[lo:hi], ey[lo:hi], "dequant")]

        _compare_fragments(fx, frags, lambda f: FC.digest(gc_[f[2]:f[3]], gs[f[4]:f[5]], gy[f[2]:f[3]]),
                           dig["quant_" + src], oracle_frag, f"full quant {fx.w.name} {src}")
        if sample.size:
            ec, es = np.zeros(fx.total, np.uint8), np.zeros(nt, np.float32)
            O.block_quant(host, fx.w.tensors, fx.offsets, fx.S, fx.m, fmt, 0, fx.m, ec, es,
                          only_tiles=sample, inplace=True)
            assert_bits_equal(gs[sample], es[sample], f"full quant {fx.w.name} {src} sampled scales")
            assert_bits_equal(gc_[spos], ec[spos], f"full quant {fx.w.name} {src} sampled codes")
            ey = O.block_dequant(gc_, gs, fx.w.tensors, fx.offsets, fx.S, fx.m, fmt, 0, fx.m,
                                 np.zeros(fx.total, np.float32), "f32", only_tiles=sample)
            assert_f32_equal_nan_class(gy[spos], ey[spos], f"full dequant {fx.w.name} {src} sampled")
        # padding and non-quantised positions keep their canaries
        assert np.all(gc_[~quantised] == 0xAB)
        assert np.all(np.isnan(gy[~quantised]))
        del x, codes, y, gc_, gy


def _tile_positions(fx, tiles):
    pos = []
    base = 0
    for s, l in zip(fx.w.tensors, fx.offsets):
        if not s.q_rows:
            continue
        ntr, ntc = O.tile_counts(s)
        for i in [t - base for t in tiles if base <= t < base + ntr * ntc]:
            r0, r1, c0, c1 = O.tile_bounds(s, i)
            pos.append((l + np.arange(r0, r1)[:, None] * s.cols + np.arange(c0, c1)[None, :]).reshape(-1))
        base += ntr * ntc
    return np.concatenate(pos)


@pytest.mark.timeout(900)
def test_full_adamw8(fx):
    """8-bit AdamW over the whole buffer in one launch, from the seeded
    moment state of fullsize_cases; every fragment against the oracle's
    digests (the embedding on a tile sample), non-quantised elements
    untouched."""
    import torch
    from oracle import optim as OP
    R = fx.R
    dig = _digests(fx)
    frags = [tuple(f) for f in dig["frags"]]
    log(f"full adamw8 {fx.w.name}: {len(frags)} fragments")
    rng = np.random.default_rng(37)
    fmt = fx.w.qfmt
    nt = fx.lay.info["num_tiles"]
    hp = FC.ADAMW8_HP
    mc0, vc0, ms0, vs0 = FC.adamw8_state(fx.total, nt, fmt)
    p = torch.from_numpy(fx.param_host).cuda()
    g = torch.from_numpy(fx.grad_host).cuda()
    mc, vc = torch.from_numpy(mc0).cuda(), torch.from_numpy(vc0).cuda()
    ms, vs = torch.from_numpy(ms0).cuda(), torch.from_numpy(vs0).cuda()
    qf = R.RS_Q_FP8_E4M3 if fmt == "fp8_e4m3" else R.RS_Q_INT8
    R.rs_adamw8_step(fx.lay.handle, p, g, mc, ms, vc, vs, qf, hp["lr"], hp["beta1"], hp["beta2"],
                     hp["eps"], hp["wd"], hp["bc1"], hp["bc2"], hp["grad_scale"], None, 0, fx.m)
    _sync()
    gp, gmc, gvc, gms, gvs = to_np(p), to_np(mc), to_np(vc), to_np(ms), to_np(vs)

    def oracle_frag(f):
        t, k, lo, hi, a, b = f
        ep, emc, ems, evc, evs = OP.adamw8_step(fx.param_host, fx.grad_host, mc0, ms0, vc0, vs0,
                                                fx.w.tensors, fx.offsets, fx.S, fx.m, k, k + 1, fmt,
                                                hp, only_tiles=range(a, b))
        return [(gp[lo:hi], ep[lo:hi], "p"), (gmc[lo:hi], emc[lo:hi], "m codes"),
                (gvc[lo:hi], evc[lo:hi], "v codes"), (gms[a:b], ems[a:b], "m scales"),
                (gvs[a:b], evs[a:b], "v scales")]

    what = f"full adamw8 {fx.w.name}"
    _compare_fragments(fx, frags, lambda f: FC.digest(gp[f[2]:f[3]], gmc[f[2]:f[3]], gvc[f[2]:f[3]],
                                                      gms[f[4]:f[5]], gvs[f[4]:f[5]]),
                       dig["adamw8"], oracle_frag, what)
    sample = _embedding_sample(fx, rng, 2000)
    if sample.size:
        ep, emc, evc = fx.param_host.copy(), mc0.copy(), vc0.copy()
        ems, evs = ms0.copy(), vs0.copy()
        OP.adamw8_step(ep, fx.grad_host, emc, ems, evc, evs, fx.w.tensors, fx.offsets, fx.S, fx.m, 0,
                       fx.m, fmt, hp, only_tiles=sample, inplace=True)
        pos = _tile_positions(fx, list(sample))
        assert_f32_equal_nan_class(gp[pos], ep[pos], what + " sampled p")
        assert_bits_equal(gmc[pos], emc[pos], what + " sampled m codes")
        assert_bits_equal(gvc[pos], evc[pos], what + " sampled v codes")
        assert_bits_equal(gms[sample], ems[sample], what + " sampled m scales")
        assert_bits_equal(gvs[sample], evs[sample], what + " sampled v scales")
    quantised = np.zeros(fx.total, bool)
    for s, l in zip(fx.w.tensors, fx.offsets):
        if s.q_rows:
            quantised[l:l + s.numel] = True
    assert np.array_equal(gp[~quantised].view(np.uint32), fx.param_host[~quantised].view(np.uint32))
    assert np.array_equal(gmc[~quantised], mc0[~quantised])
    del p, g, mc, vc, ms, vs


@pytest.mark.timeout(900)
def test_full_rank_shares(fx):
    """One rank's share at full size, in the launch configuration of the
    bench's per-rank timing (range [k, k+1): fine chunks for the norms,
    four sub-blocks per wide quantisation tile where the rank has fewer than
    1024 work items): scale/add with found-inf, norms with partials,
    quantisation and dequantisation (every tile, against the oracle's
    digests) for the first, a middle and the last rank."""
    import torch
    R = fx.R
    rng = np.random.default_rng(29)
    fmt = fx.w.qfmt
    qf = R.RS_Q_FP8_E4M3 if fmt == "fp8_e4m3" else R.RS_Q_INT8
    nt = fx.lay.info["num_tiles"]
    n = len(fx.w.tensors)
    dig = _digests(fx)
    for k in sorted({0, fx.m // 2, fx.m - 1}):
        log(f"full rank share {fx.w.name} rank {k}")
        lo, hi = k * fx.S, (k + 1) * fx.S
        # scale/add and found-inf
        y = torch.from_numpy(fx.param_host).cuda()
        x = torch.from_numpy(fx.grad_host).cuda()
        fi = torch.zeros(fx.m, dtype=torch.int32, device="cuda")
        R.rs_group_scale_add(fx.lay.handle, y, x, R.RS_F32, 0.5, -2.0, None, fi, k, k + 1)
        _sync()
        ey, ef = O.scale_add(fx.param_host, fx.grad_host, 0.5, -2.0, fx.items, fx.offsets, fx.S,
                             fx.m, k, k + 1)
        gy = to_np(y)
        assert_f32_equal_nan_class(gy[lo:hi], ey[lo:hi], f"rank {k} scale_add")
        assert np.array_equal(gy[:lo].view(np.uint32), fx.param_host[:lo].view(np.uint32))
        assert np.array_equal(gy[hi:].view(np.uint32), fx.param_host[hi:].view(np.uint32))
        assert np.array_equal(to_np(fi).astype(np.uint32), ef)
        # norms over the rank: per-tensor sums and the partial row of rank k
        sq = torch.empty(n, dtype=torch.float64, device="cuda")
        part = torch.zeros(fx.m * n, dtype=torch.float64, device="cuda")
        R.rs_ragged_sqnorm(fx.lay.handle, x, sq, part, None, fx.lay.ws, k, k + 1)
        _sync()
        esq = O.sqnorm(fx.grad_host, fx.items, fx.offsets, fx.S, fx.m, k, k + 1)[0]
        got = to_np(sq)
        prow = to_np(part).reshape(fx.m, n)[k]
        for g_, what in ((got, "sq"), (prow, "partial")):
            assert np.array_equal(np.isnan(g_), np.isnan(esq)), what
            assert np.array_equal(np.isinf(g_), np.isinf(esq)), what
            f = np.isfinite(esq)
            rel = np.abs(g_[f] - esq[f]) / np.maximum(np.abs(esq[f]), 1e-300)
            assert np.all(rel <= 1e-5), f"rank {k} {what}: {rel.max()}"
        # quantisation and dequantisation of every tile of the rank: each
        # of its fragments against the oracle's digests of the grads'
        # quantisation, the embedding on a tile sample
        frags = [tuple(f) for f in dig["frags"] if f[1] == k]
        exp = [e for f, e in zip(dig["frags"], dig["quant_grads"]) if f[1] == k]
        sample = _embedding_sample(fx, rng, 3000, ranks=[k])
        codes = torch.full((fx.total,), 0xAB, dtype=torch.uint8, device="cuda")
        scales = torch.full((nt,), -1.0, dtype=torch.float32, device="cuda")
        R.rs_block_quant(fx.lay.handle, x, qf, codes, scales, k, k + 1)
        yq = torch.full((fx.total,), float("nan"), dtype=torch.float32, device="cuda")
        R.rs_block_dequant(fx.lay.handle, codes, qf, scales, yq, R.RS_F32, k, k + 1)
        _sync()
        gc_, gs, gyq = to_np(codes), to_np(scales), to_np(yq)

        def oracle_frag(f):
            t, kk, flo, fhi, a, b = f
            ec, es = np.zeros(fx.total, np.uint8), np.zeros(nt, np.float32)
            O.block_quant(fx.grad_host, fx.w.tensors, fx.offsets, fx.S, fx.m, fmt, kk, kk + 1, ec, es,
                          only_tiles=range(a, b), inplace=True)
            ey = O.block_dequant(ec, es, fx.w.tensors, fx.offsets, fx.S, fx.m, fmt, kk, kk + 1,
                                 np.zeros(fx.total, np.float32), "f32", only_tiles=range(a, b))
            return [(gc_[flo:fhi], ec[flo:fhi], "codes"), (gs[a:b], es[a:b], "scales"),
                    (gyq[flo:fhi], ey[flo:fhi], "dequant")]

        _compare_fragments(fx, frags, lambda f: FC.digest(gc_[f[2]:f[3]], gs[f[4]:f[5]],
                                                          gyq[f[2]:f[3]]),
                           exp, oracle_frag, f"rank {k} quant")
        if sample.size:
            ec, es = np.zeros(fx.total, np.uint8), np.zeros(nt, np.float32)
            O.block_quant(fx.grad_host, fx.w.tensors, fx.offsets, fx.S, fx.m, fmt, k, k + 1, ec, es,
                          only_tiles=sample, inplace=True)
            spos = _tile_positions(fx, list(sample))
            assert_bits_equal(gs[sample], es[sample], f"rank {k} sampled scales")
            assert_bits_equal(gc_[spos], ec[spos], f"rank {k} sampled codes")
            ey = O.block_dequant(gc_, gs, fx.w.tensors, fx.offsets, fx.S, fx.m, fmt, k, k + 1,
                                 np.zeros(fx.total, np.float32), "f32", only_tiles=sample)
            assert_f32_equal_nan_class(gyq[spos], ey[spos], f"rank {k} sampled dequant")
        assert np.all(gc_[:lo] == 0xAB) and np.all(gc_[hi:] == 0xAB)
        assert np.all(np.isnan(gyq[:lo])) and np.all(np.isnan(gyq[hi:]))
        del codes, scales, yq, gc_, gyq
        del y, x
