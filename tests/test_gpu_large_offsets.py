"""Positions past 2^31 elements: a group whose flat buffer holds more than
2^31 elements (8.6 GB of fp32).  Its first tensor alone has 2^31 + 524288
elements, so its own indices pass 2^31, and the tensors after it lie wholly
beyond element 2^31 (fp32 byte offsets past 2^33, codes past 2^31 bytes).
Every operation runs over the last ranks of the buffer, which hold the end
of the first tensor and all the others, and matches the oracle there; a
guard just below the window must survive.  Nothing before the window is
read by either side, so host arrays are allocated lazily (untouched pages
cost nothing) and only the window is filled, with seeded normal values
(params N(0, 0.02), grads N(0, 1e-3) with a few +-Inf/NaN).

Tensors: the large matrix (128-row granules, 128x128 tiles), a 1000-row
matrix (clipped edge tiles), an element-granular vector, a row-granular
333x2048 matrix with 1x128 tiles, and a 384x384 matrix with 32x32 tiles.
The large tensor's 128-row granules force S to a multiple of 524288 (2S
is shorter than the tensor), so S = 2621440; m = 822 is the fewest ranks
that hold the group, leaving the last rank partly padding.
"""
import numpy as np
import pytest

import workloads as W
from oracle import ops as O
from oracle import plan as P

from harness import assert_bits_equal, assert_f32_equal_nan_class, log, to_np

pytestmark = pytest.mark.gpu

G = 4096                      # guard elements below the window
CANARY16 = 0x7FA5
CANARY8 = 0xAB
BIG_ROWS = (1 << 31) // 4096 + 128


def _group() -> W.Workload:
    return W.Workload("beyond_2g", (
        W.TensorSpec("big", BIG_ROWS, 4096, 128, 128, 128),
        W.TensorSpec("mat", 1000, 4096, 128, 128, 128),
        W.TensorSpec("vec", 1, 4096, 0),
        W.TensorSpec("rows", 333, 2048, 1, 1, 128),
        W.TensorSpec("small", 384, 384, 32, 32, 32),
    ), m=822, qfmt="fp8_e4m3", block=128)


class Big:
    """The planned group, its lazily allocated host images and the device
    buffers, filled over the window [W0, W1) only."""

    def __init__(self):
        import torch
        import fsdp_sharded_buffer_amd as R
        self.R = R
        self.w = _group()
        self.specs = self.w.tensors
        self.m = self.w.m
        self.items = P.items_from_specs(self.specs)
        offs, info = R.rs_plan(self.specs, self.m, 16)
        p = P.plan(self.items, self.m, 16)
        assert (p.S, p.offsets) == (info["S"], offs), "planner disagrees with the oracle"
        self.S, self.offsets = info["S"], offs
        self.total = self.m * self.S
        assert self.total > (1 << 31) + (1 << 19)
        self.lay = R.Layout(self.specs, self.m, self.S, offs)
        big_end = offs[0] + self.specs[0].numel
        # window: the ranks holding the large tensor's last 64K elements
        # before index 2^31, and everything after
        self.ka = (offs[0] + (1 << 31) - 65536) // self.S
        self.W0, self.W1 = self.ka * self.S, self.total
        assert offs[0] < self.W0 < offs[0] + (1 << 31) < big_end and offs[1] >= (1 << 31)
        assert offs[-1] + self.specs[-1].numel > self.total - self.S, "last rank is all padding"
        rng = np.random.default_rng(2031)
        n = self.W1 - self.W0
        self.y_win = rng.normal(0.0, 0.02, n).astype(np.float32)
        xw = rng.normal(0.0, 1e-3, n).astype(np.float32)
        # a few non-finite grads on tensor elements of the window
        for v, pos in zip((np.inf, -np.inf, np.nan, np.inf),
                          rng.integers(0, n, 4)):
            xw[pos] = v
        self.x_win = xw
        self.y_host = np.zeros(self.total, dtype=np.float32)   # lazily allocated
        self.x_host = np.zeros(self.total, dtype=np.float32)
        self.y_host[self.W0:] = self.y_win
        self.x_host[self.W0:] = self.x_win
        self.y = torch.empty(self.total, dtype=torch.float32, device="cuda")
        self.x = torch.empty(self.total, dtype=torch.float32, device="cuda")
        self.reset()
        self.x[self.W0:].copy_(torch.from_numpy(self.x_win))

    def reset(self):
        """Window of y (device and host) back to the seeded params."""
        import torch
        self.y_host[self.W0:] = self.y_win
        self.y[self.W0:].copy_(torch.from_numpy(self.y_win))

    def local_start(self, t: int) -> int:
        """First element of tensor t inside the window."""
        return max(0, self.W0 - self.offsets[t])


@pytest.fixture(scope="module")
def big():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    log("large offsets: planning and filling the window")
    b = Big()
    yield b
    b.lay.close()
    del b
    torch.cuda.empty_cache()


def _sync():
    import torch
    torch.cuda.synchronize()


def _win(t, a, b):
    return to_np(t[a:b])


def test_pack_unpack_beyond_2g(big):
    import torch
    R, b = big.R, big
    # sources: per-tensor views of the params image; the large tensor's
    # device copy holds only its part in the window (from G before it)
    src_host = [b.y_host[l:l + s.numel] for s, l in zip(b.specs, b.offsets)]
    src = []
    for t, s in enumerate(b.specs):
        d = torch.empty(s.numel, dtype=torch.float32, device="cuda")
        i0 = b.local_start(t)
        d[i0:].copy_(torch.from_numpy(np.ascontiguousarray(src_host[t][i0:])))
        src.append(d)
    log(f"large offsets: pack ranks [{b.ka},{b.m})")
    buf = torch.empty(b.total, dtype=torch.bfloat16, device="cuda")
    buf[b.W0 - G:].view(torch.int16).fill_(CANARY16)
    R.rs_pack(b.lay.handle, R.ptr_table(src), R.RS_F32, buf, R.RS_BF16, b.ka, b.m)
    _sync()
    init = np.zeros(b.total, dtype=np.uint16)
    init[b.W0 - G:] = CANARY16
    exp = O.pack(src_host, b.offsets, b.S, b.m, init, "bf16", b.ka, b.m, inplace=True)
    assert_bits_equal(_win(buf, b.W0 - G, b.W1), exp[b.W0 - G:], "pack beyond 2^31")
    log(f"large offsets: unpack ranks [{b.ka},{b.m})")
    dsts, inits = [], []
    for t, s in enumerate(b.specs):
        i0 = max(0, b.local_start(t) - G)
        d = torch.empty(s.numel, dtype=torch.float32, device="cuda")
        d[i0:].view(torch.int32).fill_(0x7FA5A5A5)
        h = np.zeros(s.numel, dtype=np.uint32)
        h[i0:] = 0x7FA5A5A5
        dsts.append(d)
        inits.append(h.view(np.float32))
    del src
    R.rs_unpack(b.lay.handle, buf, R.RS_BF16, R.ptr_table(dsts), R.RS_F32, b.ka, b.m)
    _sync()
    outs = O.unpack(exp, [(s.rows, s.cols) for s in b.specs], b.offsets, b.S, b.m, inits, "f32",
                    b.ka, b.m, inplace=True)
    for t, (d, e) in enumerate(zip(dsts, outs)):
        i0 = max(0, b.local_start(t) - G)
        assert_bits_equal(_win(d, i0, d.numel()), e.reshape(-1)[i0:], f"unpack beyond 2^31 t{t}")
    del dsts, buf


def test_scale_add_zero_beyond_2g(big):
    import torch
    R, b = big.R, big
    b.reset()
    b.y[b.W0 - G:b.W0].view(torch.int32).fill_(0x7FA5A5A5)
    log(f"large offsets: scale/add ranks [{b.ka},{b.m})")
    fi = torch.zeros(b.m, dtype=torch.int32, device="cuda")
    R.rs_group_scale_add(b.lay.handle, b.y, b.x, R.RS_F32, 0.5, -2.0, None, fi, b.ka, b.m)
    _sync()
    ey, ef = O.scale_add(b.y_host, b.x_host, 0.5, -2.0, b.items, b.offsets, b.S, b.m, b.ka, b.m,
                         inplace=True)
    assert_f32_equal_nan_class(_win(b.y, b.W0, b.W1), ey[b.W0:], "scale/add beyond 2^31")
    assert np.all(_win(b.y, b.W0 - G, b.W0).view(np.uint32) == 0x7FA5A5A5), "write below the range"
    assert np.array_equal(to_np(fi).astype(np.uint32), ef), "found_inf beyond 2^31"
    log(f"large offsets: masked zero ranks [{b.ka},{b.m})")
    mask_h = np.array([1, 0, 1, 1, 0], dtype=np.uint8)
    mask = torch.from_numpy(mask_h).cuda()
    R.rs_group_zero(b.lay.handle, b.y, R.RS_F32, mask, b.ka, b.m)
    _sync()
    ez = O.zero(ey, b.items, b.offsets, b.S, b.m, b.ka, b.m, mask_h, inplace=True)
    assert_f32_equal_nan_class(_win(b.y, b.W0, b.W1), ez[b.W0:], "masked zero beyond 2^31")
    log(f"large offsets: zero (no mask) ranks [{b.ka},{b.m})")
    R.rs_group_zero(b.lay.handle, b.y, R.RS_F32, None, b.ka, b.m)
    _sync()
    assert not np.any(_win(b.y, b.W0, b.W1).view(np.uint32)), "zero beyond 2^31"
    assert np.all(_win(b.y, b.W0 - G, b.W0).view(np.uint32) == 0x7FA5A5A5), "zero below the range"
    b.reset()


def _check_sq(got, exp, what):
    assert np.array_equal(np.isnan(got), np.isnan(exp)), what
    assert np.array_equal(np.isinf(got), np.isinf(exp)), what
    f = np.isfinite(exp)
    rel = np.abs(got[f] - exp[f]) / np.maximum(np.abs(exp[f]), 1e-300)
    assert np.all(rel <= 1e-5), f"{what}: {rel.max()}"


def test_sqnorm_beyond_2g(big):
    import torch
    R, b = big.R, big
    n = len(b.specs)
    ranges = [(b.ka, b.m)] + [(k, k + 1) for k in range(b.ka, b.m)]
    for k0, k1 in ranges:
        log(f"large offsets: sqnorm ranks [{k0},{k1})")
        sq = torch.empty(n, dtype=torch.float64, device="cuda")
        part = torch.zeros(b.m * n, dtype=torch.float64, device="cuda")
        fi = torch.zeros(b.m, dtype=torch.int32, device="cuda")
        R.rs_ragged_sqnorm(b.lay.handle, b.x, sq, part, fi, b.lay.ws, k0, k1)
        _sync()
        esq, epart, ef = O.sqnorm(b.x_host, b.items, b.offsets, b.S, b.m, k0, k1)
        what = f"sqnorm beyond 2^31 [{k0},{k1})"
        _check_sq(to_np(sq), esq, what)
        _check_sq(to_np(part).reshape(b.m, n)[k0:k1], epart[k0:k1], what + " partial")
        assert np.array_equal(to_np(fi).astype(np.uint32), ef), what + " found_inf"


@pytest.mark.parametrize("fmt", ["fp8_e4m3", "int8"])
def test_quant_dequant_beyond_2g(big, fmt):
    import torch
    R, b = big.R, big
    qf = R.RS_Q_FP8_E4M3 if fmt == "fp8_e4m3" else R.RS_Q_INT8
    nt = b.lay.info["num_tiles"]
    assert nt == O.num_tiles(b.specs)
    log(f"large offsets: {fmt} quantisation ranks [{b.ka},{b.m})")
    codes = torch.empty(b.total, dtype=torch.uint8, device="cuda")
    codes[b.W0 - G:].fill_(CANARY8)
    scales = torch.full((nt,), -1.0, dtype=torch.float32, device="cuda")
    fi = torch.zeros(b.m, dtype=torch.int32, device="cuda")
    R.rs_block_quant(b.lay.handle, b.x, qf, codes, scales, b.ka, b.m, found_inf=fi)
    _sync()
    ec = np.zeros(b.total, dtype=np.uint8)
    ec[b.W0 - G:] = CANARY8
    es = np.full(nt, -1.0, dtype=np.float32)
    O.block_quant(b.x_host, b.specs, b.offsets, b.S, b.m, fmt, b.ka, b.m, ec, es, inplace=True)
    assert_bits_equal(_win(codes, b.W0 - G, b.W1), ec[b.W0 - G:], f"{fmt} codes beyond 2^31")
    assert_bits_equal(to_np(scales), es, f"{fmt} scales beyond 2^31")
    assert np.array_equal(to_np(fi).astype(np.uint32),
                          O.quant_found_inf(b.x_host, b.specs, b.offsets, b.S, b.m, b.ka, b.m))
    log(f"large offsets: {fmt} dequantisation ranks [{b.ka},{b.m})")
    yq = torch.empty(b.total, dtype=torch.float32, device="cuda")
    yq[b.W0 - G:].view(torch.int32).fill_(0x7FA5A5A5)
    R.rs_block_dequant(b.lay.handle, codes, qf, scales, yq, R.RS_F32, b.ka, b.m)
    _sync()
    ey = np.zeros(b.total, dtype=np.uint32)
    ey[b.W0 - G:] = 0x7FA5A5A5
    ey = ey.view(np.float32)
    O.block_dequant(ec, es, b.specs, b.offsets, b.S, b.m, fmt, b.ka, b.m, ey, "f32", inplace=True)
    # NaN codes decode to NaN of either sign: compared by class, as in the
    # other dequantisation tests; the guard (a NaN pattern) by its bits
    got = _win(yq, b.W0 - G, b.W1)
    assert np.all(got[:G].view(np.uint32) == 0x7FA5A5A5), f"{fmt} dequant below the range"
    assert_f32_equal_nan_class(got[G:], ey[b.W0:], f"{fmt} dequant beyond 2^31")
    del codes, yq


def test_optimizers_beyond_2g(big):
    """AdamW, SGD (Nesterov) and 8-bit AdamW (both code formats) over the
    last ranks: params, moments, codes and scales against the oracle."""
    import torch
    from oracle import optim as OP
    R, b = big.R, big
    rng = np.random.default_rng(77)
    n = b.W1 - b.W0
    m_win = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v_win = np.abs(rng.standard_normal(n) * 1e-6).astype(np.float32)
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, wd=0.1, bc1=1 - 0.9 ** 3,
              bc2=1 - 0.95 ** 3, grad_scale=1.0)
    hpa = (hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["wd"], hp["bc1"], hp["bc2"],
           hp["grad_scale"])

    def dev(win):
        t = torch.empty(b.total, dtype=torch.float32, device="cuda")
        t[b.W0 - G:b.W0].view(torch.int32).fill_(0x7FA5A5A5)
        t[b.W0:].copy_(torch.from_numpy(win))
        return t

    def host(win):
        h = np.zeros(b.total, dtype=np.float32)
        h[b.W0:] = win
        return h

    def check(got, exp, what):
        w = _win(got, b.W0 - G, b.W1)
        assert np.all(w[:G].view(np.uint32) == 0x7FA5A5A5), what + ": write below the range"
        assert_f32_equal_nan_class(w[G:], exp[b.W0:], what)

    b.reset()
    b.y[b.W0 - G:b.W0].view(torch.int32).fill_(0x7FA5A5A5)
    log(f"large offsets: adamw ranks [{b.ka},{b.m})")
    md, vd = dev(m_win), dev(v_win)
    R.rs_adamw_step(b.lay.handle, b.y, b.x, md, vd, *hpa, None, None, b.ka, b.m)
    _sync()
    ep, em, ev = OP.adamw_step(b.y_host, b.x_host, host(m_win), host(v_win), b.items, b.offsets,
                               b.S, b.m, b.ka, b.m, hp, inplace=True)
    for got, exp, nm in ((b.y, ep, "p"), (md, em, "m"), (vd, ev, "v")):
        check(got, exp, f"adamw beyond 2^31 {nm}")
    del md, vd

    b.reset()
    log(f"large offsets: sgd ranks [{b.ka},{b.m})")
    bd = dev(m_win)
    R.rs_sgd_step(b.lay.handle, b.y, b.x, bd, 0.05, 0.9, 1e-4, True, 2.0, None, None, b.ka, b.m)
    _sync()
    ep, eb = OP.sgd_step(b.y_host, b.x_host, host(m_win), b.items, b.offsets, b.S, b.m, b.ka, b.m,
                         0.05, 0.9, 1e-4, True, 2.0, inplace=True)
    check(b.y, ep, "sgd beyond 2^31 p")
    check(bd, eb, "sgd beyond 2^31 buf")
    del bd

    nt = b.lay.info["num_tiles"]
    for fmt in ("fp8_e4m3", "int8"):
        b.reset()
        log(f"large offsets: adamw8 {fmt} ranks [{b.ka},{b.m})")
        qf = R.RS_Q_FP8_E4M3 if fmt == "fp8_e4m3" else R.RS_Q_INT8
        states = []
        for win in (m_win, v_win):
            c0 = np.zeros(b.total, dtype=np.uint8)
            c0[b.W0 - G:b.W0] = CANARY8
            s0 = np.zeros(nt, dtype=np.float32)
            O.block_quant(host(win), b.specs, b.offsets, b.S, b.m, fmt, b.ka, b.m, c0, s0,
                          inplace=True)
            cd = torch.empty(b.total, dtype=torch.uint8, device="cuda")
            cd[b.W0 - G:].copy_(torch.from_numpy(c0[b.W0 - G:]))
            states += [(c0, s0), (cd, torch.from_numpy(s0).cuda())]
        (mc0, ms0), (mcd, msd), (vc0, vs0), (vcd, vsd) = states
        R.rs_adamw8_step(b.lay.handle, b.y, b.x, mcd, msd, vcd, vsd, qf, *hpa, None, b.ka, b.m)
        _sync()
        e = OP.adamw8_step(b.y_host, b.x_host, mc0, ms0, vc0, vs0, b.specs, b.offsets, b.S, b.m,
                           b.ka, b.m, fmt, hp, inplace=True)
        what = f"adamw8 {fmt} beyond 2^31"
        assert_f32_equal_nan_class(_win(b.y, b.W0, b.W1), e[0][b.W0:], what + " p")
        for got, exp, nm in ((mcd, e[1], "m codes"), (vcd, e[3], "v codes")):
            assert_bits_equal(_win(got, b.W0 - G, b.W1), exp[b.W0 - G:], f"{what} {nm}")
        for got, exp, nm in ((msd, e[2], "m scales"), (vsd, e[4], "v scales")):
            assert_bits_equal(to_np(got), exp, f"{what} {nm}")
        del mcd, vcd
    b.reset()
