"""Layouts planned in another tensor order, run through the kernels.

The pages compare three tensor orders for the planner: the given one, one by
block size and one by shape (veScale-FSDP: Flexible and High-Performance FSDP
at Scale, "Planning Algorithm").  Here each order is planned through the
C-ABI (rs_plan_ordered, via Layout.plan(order=...)) on scaled-down mixed and
expert groups where the block order (and, on two of them, the shape order)
needs a smaller S than the given order.  The permutation and offsets must
equal the oracle's ordered plan, and pack, unpack, scale/add, norms and
quantisation over that layout must match the oracle.  The caller keeps its
tensors in the given order; the binding maps them through perm.
"""
import numpy as np
import pytest

import workloads as W
from oracle import casts as OC
from oracle import ops as O
from oracle import plan as P

from harness import assert_bits_equal, assert_f32_equal_nan_class, log, to_np

pytestmark = pytest.mark.gpu


def _regranule(ts, rows, q_cols):
    """Every matrix cut in bands of `rows` rows and quantised in rows x
    q_cols tiles; vectors stay element-granular and unquantised."""
    out = []
    for s in ts:
        if s.rows > 1:
            out.append(W.TensorSpec(s.name, s.rows, s.cols, rows, rows, min(q_cols, s.cols)))
        else:
            out.append(W.TensorSpec(s.name, 1, s.cols, 0))
    return tuple(out)


def _mixed(row_div, col_div, rows, m):
    w = W.ragged_mixed()
    sw = W.scaled_workload(W.Workload("mixed", w.tensors[:19], m=m, qfmt="int8", block=128,
                                      nonfinite_frac=1e-3), row_div, col_div)
    return W.Workload(f"mixed_div{row_div}x{col_div}_g{rows}_m{m}", _regranule(sw.tensors, rows, 32),
                      m=m, qfmt="int8", block=rows, nonfinite_frac=1e-3)


def _moe(row_div, col_div, rows, m):
    w = W.moe_experts()
    ts = list(w.tensors[:12]) + [w.tensors[-1]]
    sw = W.scaled_workload(W.Workload("moe", tuple(ts), m=m, qfmt="fp8_e4m3", block=128,
                                      grad_dist="student_t3"), row_div, col_div)
    return W.Workload(f"moe_div{row_div}x{col_div}_g{rows}_m{m}", _regranule(sw.tensors, rows, 16),
                      m=m, qfmt="fp8_e4m3", block=rows, grad_dist="student_t3")


# groups where the block order needs a smaller S than the given one
GROUPS = {
    "mixed_g16_m8": (lambda: _mixed(16, 16, 16, 8)),
    "mixed_g32_m4": (lambda: _mixed(64, 16, 32, 4)),
    "moe_g4_m8": (lambda: _moe(16, 8, 4, 8)),
    "moe_g1_m16": (lambda: _moe(32, 8, 1, 16)),
}
ALIGN = 16


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def _sync():
    import torch
    torch.cuda.synchronize()


@pytest.mark.parametrize("kind", ["block", "shape", "best"])
@pytest.mark.parametrize("group", list(GROUPS))
def test_ordered_layout_through_kernels(group, kind):
    import torch

    import fsdp_sharded_buffer_amd as R
    w = GROUPS[group]()
    specs, m = list(w.tensors), w.m
    log(f"orders {group} {kind}: plan")
    given = P.plan_ordered(specs, m, ALIGN, "given")
    exp = P.plan_ordered(specs, m, ALIGN, kind)
    lay = R.Layout.plan(specs, m, align=ALIGN, order=kind)
    try:
        perm, S = lay.perm, lay.S
        assert (perm, S) == (exp[0], exp[2]), f"{group} {kind}: plan differs from the oracle"
        assert [exp[1][t] for t in perm] == lay.offsets
        if kind != "shape":
            assert S < given[2], f"{group}: the {kind} order should beat the given one here"
        items = P.items_from_specs(lay.specs)          # buffer order
        inp = W.make_inputs(w)                         # caller (given) order
        params = [inp.params[t] for t in perm]
        grads = [inp.grads[t] for t in perm]
        total, n = m * S, len(specs)

        def flat(arrays, fill=0.0):
            b = np.full(total, fill, np.float32)
            for a, l in zip(arrays, lay.offsets):
                b[l:l + a.size] = a.reshape(-1)
            return b

        # pack: the caller's tensors through the permuted pointer table
        dparams = [torch.from_numpy(a).cuda() for a in inp.params]
        buf = torch.empty(total, dtype=torch.bfloat16, device="cuda")
        buf.view(torch.int16).fill_(0x7FA5)
        log(f"orders {group} {kind}: pack/unpack S={S}")
        R.rs_pack(lay.handle, R.ptr_table([dparams[t] for t in perm]), R.RS_F32, buf, R.RS_BF16,
                  0, m)
        _sync()
        ebuf = O.pack(params, lay.offsets, S, m, np.zeros(total, np.uint16), "bf16", 0, m)
        gbuf = to_np(buf)
        assert_bits_equal(gbuf, ebuf, f"{group} {kind} pack")
        # unpack back into tensors kept in the caller's order
        outs = [torch.zeros(s.numel, dtype=torch.float32, device="cuda") for s in specs]
        R.rs_unpack(lay.handle, buf, R.RS_BF16, R.ptr_table([outs[t] for t in perm]), R.RS_F32,
                    0, m)
        _sync()
        for t in range(n):
            ref = (OC.bf16_bits_from_f32(inp.params[t].reshape(-1)).astype(np.uint32) << 16)
            assert_bits_equal(to_np(outs[t]), ref.view(np.float32), f"{group} {kind} unpack t{t}")
        # scale/add with found-inf, then norms and quantisation of the result
        y0, x0 = flat(params), flat(grads)
        y = torch.from_numpy(y0).cuda()
        fi = torch.zeros(m, dtype=torch.int32, device="cuda")
        log(f"orders {group} {kind}: scale_add, norms, quant")
        R.rs_group_scale_add(lay.handle, y, torch.from_numpy(x0).cuda(), R.RS_F32, 0.5, -2.0, None,
                             fi, 0, m)
        sq = torch.empty(n, dtype=torch.float64, device="cuda")
        R.rs_ragged_sqnorm(lay.handle, y, sq, None, None, lay.ws, 0, m)
        codes = torch.full((total,), 0xAB, dtype=torch.uint8, device="cuda")
        scales = torch.zeros(max(lay.info["num_tiles"], 1), dtype=torch.float32, device="cuda")
        qf = R.RS_Q_FP8_E4M3 if w.qfmt == "fp8_e4m3" else R.RS_Q_INT8
        R.rs_block_quant(lay.handle, y, qf, codes, scales, 0, m)
        _sync()
        ey, ef = O.scale_add(y0, x0, 0.5, -2.0, items, lay.offsets, S, m, 0, m)
        gy = to_np(y)
        assert_f32_equal_nan_class(gy, ey, f"{group} {kind} scale_add")
        assert np.array_equal(to_np(fi).astype(np.uint32), ef)
        esq = O.sqnorm(ey, items, lay.offsets, S, m, 0, m)[0]
        got = to_np(sq)
        assert np.array_equal(np.isnan(got), np.isnan(esq)) and np.array_equal(np.isinf(got),
                                                                               np.isinf(esq))
        f = np.isfinite(esq)
        assert np.all(np.abs(got[f] - esq[f]) <= 1e-5 * np.abs(esq[f])), f"{group} {kind} sqnorm"
        nt = lay.info["num_tiles"]
        ec, es = O.block_quant(ey, lay.specs, lay.offsets, S, m, w.qfmt, 0, m,
                               np.full(total, 0xAB, np.uint8), np.zeros(nt, np.float32))
        assert_bits_equal(to_np(codes), ec, f"{group} {kind} codes")
        assert_bits_equal(to_np(scales)[:nt], es, f"{group} {kind} scales")
    finally:
        lay.close()
