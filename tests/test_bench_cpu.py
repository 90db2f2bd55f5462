"""Host-side checks of bench.py (CPU only): the per-rank algorithmic bytes
of every operation sum to the whole-buffer bytes on every group, the
whole-buffer bytes follow their definitions, and the HBM counter passes run
only where they can."""
import argparse

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


def test_live_counters_only_where_they_can_run():
    def a(**kw):
        d = dict(per_rank_only=False, no_live_counters=False)
        d.update(kw)
        return argparse.Namespace(**d)

    assert Bn.want_live_counters(a(), [], {})
    assert Bn.want_live_counters(a(), ["pack", "scale_add"], {})
    assert not Bn.want_live_counters(a(), ["block_quant"], {})          # scale/add not timed
    assert not Bn.want_live_counters(a(per_rank_only=True), [], {})
    assert not Bn.want_live_counters(a(no_live_counters=True), [], {})
    assert not Bn.want_live_counters(a(), [], {"ROCPROF_OUTPUT_PATH": "out"})   # under rocprofv3
