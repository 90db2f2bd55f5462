"""Host-side checks of bench.py's byte accounting (CPU only): the per-rank
algorithmic bytes of every operation sum to the whole-buffer bytes on every
group, and the whole-buffer bytes follow their definitions."""
import pytest

import bench as Bn
import workloads as W
from oracle import ops as O
from oracle import plan as P


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_rank_bytes_sum_to_whole_buffer(name):
    w = W.WORKLOADS[name]
    pl = P.plan(P.items_from_specs(w.tensors), w.m, 16) if name != "moe_experts" else None
    if pl is None:      # the oracle scan is slow on 193 tensors; use the C-ABI planner
        import fsdp_sharded_buffer_amd as R
        offs, info = R.rs_plan(w.tensors, w.m, 16)
        S = info["S"]
    else:
        offs, S = pl.offsets, pl.S
    nt = O.num_tiles(w.tensors)
    whole = dict(Bn.op_bytes(w, S, nt), **Bn.extra_bytes(w, S, nt))
    ranks = Bn.rank_bytes(w, offs, S)
    assert len(ranks) == w.m
    assert set(ranks[0]) == set(whole)
    for op, b in whole.items():
        assert sum(r[op] for r in ranks) == b, op
    E = w.numel
    Eq = sum(t.numel for t in w.tensors if t.q_rows)
    assert whole["scale_add"] == 12 * E and whole["zero"] == 4 * w.m * S
    assert whole["block_quant"] == 5 * Eq + 4 * nt
