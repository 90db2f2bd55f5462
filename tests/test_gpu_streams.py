"""Calls on two streams at once.  Every call touches only its rank range, so
two calls over disjoint rank ranges may run concurrently on two streams (as
ranks' work would on their own devices).  Each operation is issued as two
half-range calls on two default-priority streams without waiting between
them, and the results must equal one whole-range call bit for bit.  The
norms use one workspace and one sq array per stream (rs_ragged_sqnorm
writes sq for every tensor); the per-rank partials must equal the
whole-range call's, and each stream's sq must equal the oracle's sums over
that stream's ranks and a later call over the same ranks on one stream."""
import numpy as np
import pytest

from oracle import ops as O

from harness import case, from_np, log, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


@pytest.mark.parametrize("name", ["llama8b_div16", "mixed_div", "bands"])
def test_disjoint_rank_ranges_on_two_streams(name):
    import torch
    c = case(name)
    R, h, m = c.R, c.lay.handle, c.m
    if m < 2:
        pytest.skip("one rank")
    half = m // 2
    inp = c.inputs()
    n = len(c.w.tensors)
    nt = max(c.lay.info["num_tiles"], 1)
    qf = R.RS_Q_FP8_E4M3 if c.w.qfmt == "fp8_e4m3" else R.RS_Q_INT8
    params = [torch.from_numpy(a).cuda() for a in inp.params]
    ptab = R.ptr_table(params)
    x0 = from_np(c.flat(inp.grads))
    y0 = from_np(c.flat(inp.params))
    ws2 = torch.zeros_like(c.lay.ws)

    def buffers():
        b = {
            "buf": torch.full((c.total,), 7, dtype=torch.int16, device="cuda").view(torch.bfloat16),
            "outs": [torch.zeros(s.numel, dtype=torch.float32, device="cuda") for s in c.w.tensors],
            "y": y0.clone(), "found": torch.zeros(m, dtype=torch.int32, device="cuda"),
            "sq": torch.zeros(n, dtype=torch.float64, device="cuda"),
            "sq2": torch.zeros(n, dtype=torch.float64, device="cuda"),
            "part": torch.zeros(m * n, dtype=torch.float64, device="cuda"),
            "codes": torch.full((c.total,), 0xAB, dtype=torch.uint8, device="cuda"),
            "scales": torch.zeros(nt, dtype=torch.float32, device="cuda"),
            "deq": torch.zeros(c.total, dtype=torch.float32, device="cuda"),
            "z": y0.clone(),
            "p": y0.clone(), "mom": torch.zeros(c.total, dtype=torch.float32, device="cuda"),
            "var": torch.zeros(c.total, dtype=torch.float32, device="cuda"),
        }
        b["otab"] = R.ptr_table(b["outs"])  # device pointer table, built before any stream work
        return b

    def run(b, k0, k1, stream, ws, sq="sq"):
        s = stream.cuda_stream
        R.rs_pack(h, ptab, R.RS_F32, b["buf"], R.RS_BF16, k0, k1, s)
        R.rs_unpack(h, b["buf"], R.RS_BF16, b["otab"], R.RS_F32, k0, k1, s)
        R.rs_group_scale_add(h, b["y"], x0, R.RS_F32, 0.5, 2.0, None, b["found"], k0, k1, s)
        R.rs_ragged_sqnorm(h, b["y"], b[sq], b["part"], None, ws, k0, k1, s)
        R.rs_block_quant(h, b["y"], qf, b["codes"], b["scales"], k0, k1, s)
        R.rs_block_dequant(h, b["codes"], qf, b["scales"], b["deq"], R.RS_F32, k0, k1, s)
        R.rs_group_zero(h, b["z"], R.RS_F32, None, k0, k1, s)
        R.rs_adamw_step(h, b["p"], x0, b["mom"], b["var"], 1e-3, 0.9, 0.95, 1e-8, 0.1, 0.3, 0.2,
                        1.0, None, None, k0, k1, s)

    torch.cuda.synchronize()
    whole = buffers()
    run(whole, 0, m, torch.cuda.current_stream(), c.lay.ws)
    torch.cuda.synchronize()

    split = buffers()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    for _ in range(3):  # several rounds, each pair issued without waiting between the streams
        run(split, 0, half, s1, c.lay.ws)
        run(split, half, m, s2, ws2, "sq2")
    torch.cuda.synchronize()
    # the repeated rounds are idempotent except the accumulating ones: redo
    # those once more from a fresh state, concurrently
    once = buffers()
    run(once, 0, half, s1, c.lay.ws)
    run(once, half, m, s2, ws2, "sq2")
    torch.cuda.synchronize()
    log(f"{name}: m={m}, ranges [0,{half}) and [{half},{m}) on two streams")

    def same(a, b):  # bit for bit (NaNs included)
        a, b = to_np(a), to_np(b)
        return a.shape == b.shape and a.tobytes() == b.tobytes()

    for key in ("buf", "codes", "scales", "deq", "z", "found", "y", "p", "mom", "var", "part"):
        assert same(once[key], whole[key]), f"{name} {key}"
    for t, (a, b) in enumerate(zip(once["outs"], whole["outs"])):
        assert same(a, b), f"{name} unpack t{t}"
    # the idempotent outputs of the repeated rounds also match
    for key in ("buf", "z"):
        assert same(split[key], whole[key]), f"{name} repeated {key}"
    for t, (a, b) in enumerate(zip(split["outs"], whole["outs"])):
        assert same(a, b), f"{name} repeated unpack t{t}"
    # each stream's own sq: the oracle's sums over its ranks (of the y both
    # streams produced), and bit-equal to a later single-stream call
    yh = to_np(once["y"])
    for key, (k0, k1) in (("sq", (0, half)), ("sq2", (half, m))):
        got = to_np(once[key])
        esq = O.sqnorm(yh, c.items, c.offsets, c.S, m, k0, k1)[0]
        assert np.array_equal(np.isnan(got), np.isnan(esq)), f"{name} {key}"
        f = np.isfinite(esq)
        assert np.all(np.abs(got[f] - esq[f]) <= 1e-5 * np.abs(esq[f])), f"{name} {key}"
        ref = torch.zeros(n, dtype=torch.float64, device="cuda")
        R.rs_ragged_sqnorm(h, once["y"], ref, None, None, c.lay.ws, k0, k1)
        torch.cuda.synchronize()
        assert same(once[key], ref), f"{name} {key} against one stream"
