"""rs_ragged_sqnorm_noalloc, the norm entry point that allocates nothing
(for callers that cannot allocate: graph capture, serving loops): called
through the C-ABI, it must give the workspace entry point's results bit for
bit, and the oracle's within 1e-5, on two calls in a row with the second on
a smaller input, in both the fine-chunk (few ranks) and coarse-chunk
(many ranks) configurations; and it must refuse a range whose partials do
not fit its static scratch before enqueueing anything."""
import numpy as np
import pytest

import workloads as W
from oracle import ops as O
from oracle import plan as P

from harness import case, log, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def _both(c, x, k0, k1, with_partial=True):
    """(sq, partial, found_inf) from the workspace call and from the
    no-allocation call, each into fresh canary-filled outputs."""
    import torch
    R, n, m = c.R, len(c.w.tensors), c.m
    outs = []
    for noalloc in (False, True):
        sq = torch.full((n,), -7.0, dtype=torch.float64, device="cuda")
        part = torch.full((m * n,), -7.0, dtype=torch.float64, device="cuda") if with_partial else None
        fi = torch.zeros(m, dtype=torch.int32, device="cuda")
        if noalloc:
            R.rs_ragged_sqnorm_noalloc(c.lay.handle, x, sq, part, fi, k0, k1)
        else:
            R.rs_ragged_sqnorm(c.lay.handle, x, sq, part, fi, c.lay.ws, k0, k1)
        torch.cuda.synchronize()
        outs.append((to_np(sq), None if part is None else to_np(part).reshape(m, n), to_np(fi)))
    return outs


def _check(c, host, k0, k1, what):
    import torch
    x = torch.from_numpy(host).cuda()
    (sq_w, part_w, fi_w), (sq_s, part_s, fi_s) = _both(c, x, k0, k1)
    assert sq_s.tobytes() == sq_w.tobytes(), what + ": sq differs from the workspace call"
    assert part_s.tobytes() == part_w.tobytes(), what + ": partial differs"
    assert np.array_equal(fi_s, fi_w), what + ": found_inf differs"
    esq, epart, ef = O.sqnorm(host, c.items, c.offsets, c.S, c.m, k0, k1)
    assert np.array_equal(np.isnan(sq_s), np.isnan(esq)) and np.array_equal(np.isinf(sq_s),
                                                                             np.isinf(esq))
    f = np.isfinite(esq)
    assert np.all(np.abs(sq_s[f] - esq[f]) <= 1e-5 * np.abs(esq[f])), what
    rows = part_s[k0:k1]
    er = epart[k0:k1]
    fr = np.isfinite(er)
    assert np.all(np.abs(rows[fr] - er[fr]) <= 1e-5 * np.abs(er[fr])), what + " partial"
    assert np.all(part_s[:k0] == -7.0) and np.all(part_s[k1:] == -7.0), what + ": rows outside"
    assert np.array_equal(fi_s.astype(np.uint32), ef), what + " found_inf"


def test_noalloc_matches_workspace_call_twice_in_a_row():
    """A larger group's whole range, then a smaller group's: each equals
    the workspace call's output and the oracle's sums.  The second call
    reads a scratch that still holds the first call's partials."""
    big = case("llama8b_div16")
    small = case("toy")
    log(f"noalloc: {big.w.name} whole range (m={big.m}), then {small.w.name} whole range")
    _check(big, big.flat(big.inputs().grads), 0, big.m, "big group, all ranks")
    _check(small, small.flat(small.inputs().grads), 0, small.m, "small group, all ranks")
    log("noalloc: one rank, then a smaller middle range of the mixed group (non-finite grads)")
    mixed = case("mixed_div")
    xm = mixed.flat(mixed.inputs().grads)
    _check(mixed, xm, 0, mixed.m, "mixed group, all ranks")
    _check(mixed, xm, mixed.m // 2, mixed.m // 2 + 1, "mixed group, one rank")


def test_noalloc_coarse_range_at_full_size():
    """The 8B layer at full size: the whole range reads coarse chunks (the
    configuration the bench times), then one rank reads fine chunks."""
    import torch
    w = W.WORKLOADS["llama3_8b_layer"]
    from harness import Case
    c = Case(w, 16, 0)
    rng = np.random.default_rng(5)
    host = np.zeros(c.total, np.float32)
    for s, l in zip(w.tensors, c.offsets):
        host[l:l + s.numel] = rng.standard_normal(s.numel, dtype=np.float32)
    assert c.lay.info["num_coarse_chunks"] >= 256
    log("noalloc: llama3_8b_layer whole range, then rank 3")
    _check(c, host, 0, c.m, "8B layer, all ranks")
    _check(c, host, 3, 4, "8B layer, rank 3")
    c.lay.close()
    del host
    torch.cuda.empty_cache()


def test_noalloc_refuses_a_range_beyond_its_scratch():
    """A range of more than 131072 coarse chunks is refused with
    RS_ERR_INVALID_ARG, nothing enqueued and the outputs untouched; the
    workspace entry point still takes it, and so does the no-allocation one
    over a smaller range of the same layout."""
    import torch
    import fsdp_sharded_buffer_amd as R
    n_el = (131072 * 2048) + 64                     # 131073 coarse chunks of 2048 elements
    specs = [W.TensorSpec("a", 1, n_el, 0), W.TensorSpec("b", 1, 64, 0)]
    offs, info = R.rs_plan(specs, 2, 64)
    lay = R.Layout(specs, 2, info["S"], offs, chunk_elems=64)
    try:
        x = torch.ones(lay.total, dtype=torch.float32, device="cuda")
        sq = torch.full((2,), -7.0, dtype=torch.float64, device="cuda")
        log(f"noalloc: refuse {lay.info['num_coarse_chunks']} coarse chunks")
        with pytest.raises(R.RsError) as e:
            R.rs_ragged_sqnorm_noalloc(lay.handle, x, sq, None, None, 0, 2)
        assert e.value.status == -1 and "static scratch" in R.rs_last_error()
        torch.cuda.synchronize()
        assert np.all(to_np(sq) == -7.0)
        # rank 1 alone holds fewer chunks: accepted, and all-ones sums are exact
        k1_el = [min(l + s.numel, 2 * info["S"]) - max(l, info["S"]) for s, l in zip(specs, offs)]
        R.rs_ragged_sqnorm_noalloc(lay.handle, x, sq, None, None, 1, 2)
        torch.cuda.synchronize()
        assert np.array_equal(to_np(sq), np.array([max(0, v) for v in k1_el], np.float64))
    finally:
        lay.close()
