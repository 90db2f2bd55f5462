"""The hot calls enqueue kernels only (no allocation, synchronisation or
memset), so a whole step can be captured into a HIP graph and replayed.
The step (pack, unpack, scale/add with found-inf, norms, quantisation,
zero) is captured once and replayed several times; between replays the
program does its own eager work and synchronises, and every replay must
reproduce the eager results bit for bit."""
import numpy as np
import pytest

from harness import case, from_np, log, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


@pytest.mark.parametrize("name", ["toy", "mixed_div"])
def test_step_replays_from_a_graph(name):
    import torch
    c = case(name)
    R = c.R
    h = c.lay.handle
    inp = c.inputs()
    params = [torch.from_numpy(a).cuda() for a in inp.params]
    outs = [torch.empty(s.numel, dtype=torch.bfloat16, device="cuda") for s in c.w.tensors]
    ptab, otab = R.ptr_table(params), R.ptr_table(outs)
    g0 = from_np(c.flat(inp.grads))
    buf = torch.empty(c.total, dtype=torch.bfloat16, device="cuda")
    acc = torch.empty(c.total, dtype=torch.float32, device="cuda")
    grad = torch.empty(c.total, dtype=torch.float32, device="cuda")
    found = torch.zeros(c.m, dtype=torch.int32, device="cuda")
    sq = torch.empty(len(c.w.tensors), dtype=torch.float64, device="cuda")
    part = torch.empty(c.m * len(c.w.tensors), dtype=torch.float64, device="cuda")
    codes = torch.empty(c.total, dtype=torch.uint8, device="cuda")
    scales = torch.empty(max(c.lay.info["num_tiles"], 1), dtype=torch.float32, device="cuda")
    qf = R.RS_Q_FP8_E4M3 if c.w.qfmt == "fp8_e4m3" else R.RS_Q_INT8

    def reset():                      # eager work between replays
        acc.copy_(g0)
        grad.copy_(g0)
        found.zero_()
        for t in (buf, codes, sq, part, scales):
            t.zero_()
        for t in outs:
            t.zero_()

    def step():
        R.rs_pack(h, ptab, R.RS_F32, buf, R.RS_BF16, 0, c.m)
        R.rs_unpack(h, buf, R.RS_BF16, otab, R.RS_BF16, 0, c.m)
        R.rs_group_scale_add(h, acc, grad, R.RS_F32, 0.5, 2.0, None, found, 0, c.m)
        R.rs_ragged_sqnorm(h, acc, sq, part, found, c.lay.ws, 0, c.m)
        R.rs_block_quant(h, acc, qf, codes, scales, 0, c.m, found_inf=found)
        R.rs_group_zero(h, grad, R.RS_F32, None, 0, c.m)

    def snapshot():
        torch.cuda.synchronize()
        return [to_np(t).copy() for t in (buf, acc, grad, found, sq, part, codes, scales)] + \
               [to_np(t).copy() for t in outs]

    reset()
    step()
    eager = snapshot()

    graph = torch.cuda.CUDAGraph()
    reset()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):      # warm-up on the capture stream, outside the graph
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    reset()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    for r in range(4):
        log(f"graph replay {name} #{r}")
        reset()
        torch.cuda.synchronize()
        graph.replay()
        got = snapshot()
        for i, (a, b) in enumerate(zip(got, eager)):
            assert a.dtype == b.dtype and np.array_equal(a.view(np.uint8), b.view(np.uint8)), \
                f"replay {r}: output {i} differs from the eager step"
