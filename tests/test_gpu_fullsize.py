"""GPU parity at the full sizes of the four large groups, in the launch
configuration bench.py times (align 16, default chunks, the whole rank
range).  Whole-buffer outputs are compared with the oracle run rank by rank;
quantisation is compared on a sample of tiles (every tile of the 8B layer)
that includes the first and last tile of each tensor and every tile holding
an injected non-finite value.
"""
import gc

import numpy as np
import pytest

import workloads as W
from oracle import ops as O
from oracle import plan as P

from harness import assert_bits_equal, assert_f32_equal_nan_class, log, to_np

pytestmark = pytest.mark.gpu

FULL = ["llama3_8b_layer", "moe_experts", "llama70b_layer", "ragged_mixed"]


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


def _tile_sample(fx, rng, n_random):
    specs = fx.w.tensors
    nt = O.num_tiles(specs)
    pick = set(int(i) for i in rng.choice(nt, size=min(n_random, nt), replace=False))
    base = 0
    starts = []
    for s, l in zip(specs, fx.offsets):
        if not s.q_rows:
            continue
        ntr, ntc = O.tile_counts(s)
        pick.update((base, base + ntr * ntc - 1))
        starts.append((base, s, l))
        base += ntr * ntc
    # tiles holding injected non-finite grads
    if fx.inp.nonfinite_positions.size:
        flat_starts = np.cumsum([0] + [s.numel for s in specs])
        tbase = {}
        b = 0
        for s in specs:
            if s.q_rows:
                tbase[s.name] = b
                ntr, ntc = O.tile_counts(s)
                b += ntr * ntc
        for p in rng.choice(fx.inp.nonfinite_positions, size=200, replace=False):
            t = int(np.searchsorted(flat_starts, p, side="right") - 1)
            s = specs[t]
            if not s.q_rows:
                continue
            e = int(p - flat_starts[t])
            r, c = divmod(e, s.cols)
            _, ntc = O.tile_counts(s)
            pick.add(tbase[s.name] + (r // s.q_rows) * ntc + c // s.q_cols)
    return sorted(pick)


@pytest.mark.timeout(600)
def test_full_block_quant(fx):
    import torch
    R = fx.R
    rng = np.random.default_rng(23)
    fmt = fx.w.qfmt
    nt = fx.lay.info["num_tiles"]
    for src, host in (("params", fx.param_host), ("grads", fx.grad_host)):
        log(f"full quant {fx.w.name} {src}")
        x = torch.from_numpy(host).cuda()
        codes = torch.full((fx.total,), 0xAB, dtype=torch.uint8, device="cuda")
        scales = torch.empty(nt, dtype=torch.float32, device="cuda")
        R.rs_block_quant(fx.lay.handle, x, R.RS_Q_FP8_E4M3 if fmt == "fp8_e4m3" else R.RS_Q_INT8,
                         codes, scales, 0, fx.m)
        _sync()
        tiles = list(range(nt)) if nt <= 20000 else _tile_sample(fx, rng, 3000)
        ecodes, escales = O.block_quant(host, fx.w.tensors, fx.offsets, fx.S, fx.m, fmt, 0, fx.m,
                                        np.zeros(fx.total, np.uint8), np.zeros(nt, np.float32),
                                        only_tiles=tiles)
        gc_, gs = to_np(codes), to_np(scales)
        assert_bits_equal(gs[tiles], escales[tiles], f"full quant {fx.w.name} {src} scales")
        pos = _tile_positions(fx, tiles)
        assert_bits_equal(gc_[pos], ecodes[pos], f"full quant {fx.w.name} {src} codes")
        # padding and non-quantised positions keep the canary
        quantised = np.zeros(fx.total, bool)
        for s, l in zip(fx.w.tensors, fx.offsets):
            if s.q_rows:
                quantised[l:l + s.numel] = True
        assert np.all(gc_[~quantised] == 0xAB)
        # dequantise the device codes back to fp32 and check the same tiles
        y = torch.full((fx.total,), float("nan"), dtype=torch.float32, device="cuda")
        R.rs_block_dequant(fx.lay.handle, codes, R.RS_Q_FP8_E4M3 if fmt == "fp8_e4m3" else R.RS_Q_INT8,
                           scales, y, R.RS_F32, 0, fx.m)
        _sync()
        ey = O.block_dequant(gc_, gs, fx.w.tensors, fx.offsets, fx.S, fx.m, fmt, 0, fx.m,
                             np.zeros(fx.total, np.float32), "f32", only_tiles=tiles)
        assert_f32_equal_nan_class(to_np(y)[pos], ey[pos], f"full dequant {fx.w.name} {src}")
        del x, codes, y


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


def _random_codes(rng, n, fmt, signed):
    """Seeded valid codes: INT8 in [-127, 127] (or [0, 127]); E4M3FN without
    the NaN codes (and without the sign bit when unsigned)."""
    if fmt == "int8":
        lo = -127 if signed else 0
        return rng.integers(lo, 128, size=n, dtype=np.int16).astype(np.int8).view(np.uint8)
    c = rng.integers(0, 0x7F, size=n, dtype=np.uint8)          # 0x00..0x7E
    if signed:
        c |= (rng.integers(0, 2, size=n, dtype=np.uint8) << 7)
    return c


@pytest.mark.timeout(900)
def test_full_adamw8(fx):
    """8-bit AdamW over the whole buffer in one launch; compared on sampled
    tiles (every tile of the 8B layer), non-quantised elements untouched."""
    import torch
    from oracle import optim as OP
    R = fx.R
    log(f"full adamw8 {fx.w.name}")
    rng = np.random.default_rng(31)
    fmt = fx.w.qfmt
    nt = fx.lay.info["num_tiles"]
    qmax = 448.0 if fmt == "fp8_e4m3" else 127.0
    mc0 = _random_codes(rng, fx.total, fmt, True)
    vc0 = _random_codes(rng, fx.total, fmt, False)
    ms0 = (np.abs(rng.standard_normal(nt)) * 1e-4 / qmax).astype(np.float32)
    vs0 = (np.abs(rng.standard_normal(nt)) * 1e-6 / qmax).astype(np.float32)
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, wd=0.1, bc1=1 - 0.9 ** 5,
              bc2=1 - 0.95 ** 5, grad_scale=1.0)
    p = torch.from_numpy(fx.param_host).cuda()
    g = torch.from_numpy(fx.grad_host).cuda()
    mc, vc = torch.from_numpy(mc0).cuda(), torch.from_numpy(vc0).cuda()
    ms, vs = torch.from_numpy(ms0).cuda(), torch.from_numpy(vs0).cuda()
    qf = R.RS_Q_FP8_E4M3 if fmt == "fp8_e4m3" else R.RS_Q_INT8
    R.rs_adamw8_step(fx.lay.handle, p, g, mc, ms, vc, vs, qf, hp["lr"], hp["beta1"], hp["beta2"],
                     hp["eps"], hp["wd"], hp["bc1"], hp["bc2"], hp["grad_scale"], None, 0, fx.m)
    _sync()
    tiles = list(range(nt)) if nt <= 20000 else _tile_sample(fx, rng, 2000)
    ep, emc, ems, evc, evs = OP.adamw8_step(fx.param_host, fx.grad_host, mc0, ms0, vc0, vs0,
                                            fx.w.tensors, fx.offsets, fx.S, fx.m, 0, fx.m, fmt, hp,
                                            only_tiles=tiles)
    pos = _tile_positions(fx, tiles)
    what = f"full adamw8 {fx.w.name}"
    gp = to_np(p)
    assert_f32_equal_nan_class(gp[pos], ep[pos], what + " p")
    assert_bits_equal(to_np(mc)[pos], emc[pos], what + " m codes")
    assert_bits_equal(to_np(vc)[pos], evc[pos], what + " v codes")
    assert_bits_equal(to_np(ms)[tiles], ems[tiles], what + " m scales")
    assert_bits_equal(to_np(vs)[tiles], evs[tiles], what + " v scales")
    quantised = np.zeros(fx.total, bool)
    for s, l in zip(fx.w.tensors, fx.offsets):
        if s.q_rows:
            quantised[l:l + s.numel] = True
    assert np.array_equal(gp[~quantised].view(np.uint32), fx.param_host[~quantised].view(np.uint32))
    assert np.array_equal(to_np(mc)[~quantised], mc0[~quantised])
    del p, g, mc, vc, ms, vs


def _tiles_of_rank(fx, k):
    """Global indices of the quantisation tiles whose elements lie in rank k."""
    out, base = [], 0
    for s, l in zip(fx.w.tensors, fx.offsets):
        if not s.q_rows:
            continue
        ntr, ntc = O.tile_counts(s)
        r0 = np.arange(ntr, dtype=np.int64) * s.q_rows
        c0 = np.arange(ntc, dtype=np.int64) * s.q_cols
        first = l + r0[:, None] * s.cols + c0[None, :]
        out.append(base + np.flatnonzero((first // fx.S).reshape(-1) == k))
        base += ntr * ntc
    return np.concatenate(out) if out else np.zeros(0, np.int64)


@pytest.mark.timeout(900)
def test_full_rank_shares(fx):
    """One rank's share at full size, in the launch configuration of the
    bench's per-rank timing (range [k, k+1): fine chunks for the norms,
    four sub-blocks per wide quantisation tile where the rank has fewer than
    1024 work items): scale/add with found-inf, norms with partials,
    quantisation and dequantisation for the first, a middle and the last
    rank, against the oracle over that rank."""
    import torch
    R = fx.R
    rng = np.random.default_rng(29)
    fmt = fx.w.qfmt
    qf = R.RS_Q_FP8_E4M3 if fmt == "fp8_e4m3" else R.RS_Q_INT8
    nt = fx.lay.info["num_tiles"]
    n = len(fx.w.tensors)
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
        # quantisation and dequantisation of the rank's tiles (a sample on big groups)
        tiles = _tiles_of_rank(fx, k)
        if tiles.size:
            if tiles.size > 3000:
                tiles = np.sort(rng.choice(tiles, size=3000, replace=False))
            codes = torch.full((fx.total,), 0xAB, dtype=torch.uint8, device="cuda")
            scales = torch.full((nt,), -1.0, dtype=torch.float32, device="cuda")
            R.rs_block_quant(fx.lay.handle, x, qf, codes, scales, k, k + 1)
            _sync()
            ec, es = O.block_quant(fx.grad_host, fx.w.tensors, fx.offsets, fx.S, fx.m, fmt, k, k + 1,
                                   np.zeros(fx.total, np.uint8), np.zeros(nt, np.float32),
                                   only_tiles=tiles)
            gc_, gs = to_np(codes), to_np(scales)
            assert_bits_equal(gs[tiles], es[tiles], f"rank {k} scales")
            pos = _tile_positions(fx, list(tiles))
            assert_bits_equal(gc_[pos], ec[pos], f"rank {k} codes")
            assert np.all(gc_[:lo] == 0xAB) and np.all(gc_[hi:] == 0xAB)
            yq = torch.full((fx.total,), float("nan"), dtype=torch.float32, device="cuda")
            R.rs_block_dequant(fx.lay.handle, codes, qf, scales, yq, R.RS_F32, k, k + 1)
            _sync()
            eq = O.block_dequant(gc_, gs, fx.w.tensors, fx.offsets, fx.S, fx.m, fmt, k, k + 1,
                                 np.zeros(fx.total, np.float32), "f32", only_tiles=list(tiles))
            assert_f32_equal_nan_class(to_np(yq)[pos], eq[pos], f"rank {k} dequant")
            assert np.all(np.isnan(to_np(yq)[:lo])) and np.all(np.isnan(to_np(yq)[hi:]))
            del codes, scales, yq
        del y, x
