"""Pins for the layout-planner oracle (CPU only).

Each test checks the oracle against something other than itself: the
hand-derived toy plan, closed forms, a non-monotone instance, exhaustive
search on tiny inputs and the layout constraints restated independently.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import workloads as W
from oracle import plan as P

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _items(pairs):
    return [P.Item(e, g) for e, g in pairs]


def _independent_check(items, offsets, S, m, A):
    """The constraints written once more without the oracle's helpers."""
    prev_end = 0
    for it, l in zip(items, offsets):
        assert l % A == 0 and l >= prev_end
        r = l + it.numel
        for k in range(1, m):
            b = k * S
            if l < b < r:
                assert (b - l) % it.granule == 0, (l, b, it)
        prev_end = r
    assert prev_end <= m * S and S % A == 0


def test_toy_plan_matches_hand_derivation():
    g = json.load(open(os.path.join(GOLD, "toy_plan.json")))
    items = P.items_from_specs(W.toy_unit().tensors)
    assert [it.granule for it in items] == g["granules"]
    assert [it.numel for it in items] == g["numels"]
    for A in g["alignments"]:
        p = P.plan(items, g["m"], A)
        assert p.S == g["S"]
        assert p.offsets == g["offsets"]
        assert p.total - sum(g["numels"]) == g["padding_elems"]
        assert P.peak_param_bytes(p.S, g["m"]) == g["peak_param_bytes"]


def test_peak_bytes_formula_no_padding():
    # psi/F + max psi sizing: with no padding, K_full*E/m + K_low*E exactly
    items = P.items_from_specs(W.toy_unit().tensors)
    p = P.plan(items, 4, 1)
    E = sum(it.numel for it in items)
    assert P.peak_param_bytes(p.S, 4, 4, 2) == 4 * E // 4 + 2 * E


def test_nonmonotone_feasibility():
    g = json.load(open(os.path.join(GOLD, "nonmonotone.json")))
    it = [P.Item(g["numel"], g["granule"])]
    for S in g["feasible"]:
        assert P.greedy_offsets(it, g["m"], S, 1) is not None, S
    for S in g["infeasible"]:
        assert P.greedy_offsets(it, g["m"], S, 1) is None, S
    assert P.plan(it, g["m"], 1).S == 4


@pytest.mark.parametrize("A", [1, 4, 16])
def test_element_granular_closed_form(A):
    # FlatParameter sizing: all granules 1 -> S* = ceil(E/m) rounded up to A
    rng = np.random.default_rng(1)
    for _ in range(40):
        n = int(rng.integers(1, 6))
        es = [int(x) for x in rng.integers(1, 200, size=n)]
        m = int(rng.integers(1, 9))
        items = _items([(e, 1) for e in es])
        p = P.plan(items, m, A)
        if A == 1:
            assert p.S == -(-sum(es) // m)
        else:
            # alignment may add padding between tensors; S* is still at
            # least the aligned lower bound and the layout is valid
            assert p.S >= P.round_up(-(-sum(es) // m), A)
        _independent_check(items, p.offsets, p.S, m, A)


def test_single_tensor_whole_blocks_closed_form():
    # one tensor of nb whole blocks: S* = ceil(nb/m) * g
    for g in (1, 3, 4, 7):
        for nb in range(1, 13):
            for m in range(1, 6):
                p = P.plan([P.Item(nb * g, g)], m, 1)
                assert p.S == -(-nb // m) * g, (g, nb, m, p.S)


def test_lower_bound_is_a_bound():
    items = _items([(10, 10), (3, 1)])
    assert P.lower_bound(items, 4, 1) == 10     # the unsplittable block
    assert P.plan(items, 4, 1).S == 10


def _brute_cases(seed, n):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        pairs = W.random_tiny_specs(rng, max_t=3, max_e=14, max_g=6)
        m = int(rng.integers(1, 5))
        A = int(rng.choice([1, 1, 2, 4]))
        cases.append((pairs, m, A))
    return cases


@pytest.mark.parametrize("case", _brute_cases(7, 120))
def test_scan_equals_bruteforce(case):
    pairs, m, A = case
    items = _items(pairs)
    bf = P.plan_bruteforce(items, m, A)
    p = P.plan(items, m, A)
    assert bf is not None and p is not None
    assert (p.S, p.offsets) == (bf[0], bf[1]), (pairs, m, A)
    _independent_check(items, p.offsets, p.S, m, A)


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_full_workload_layouts_valid(name):
    w = W.WORKLOADS[name]
    items = P.items_from_specs(w.tensors)
    A = 16
    p = P.plan(items, w.m, A)
    _independent_check(items, p.offsets, p.S, w.m, A)
    ends = [l + it.numel for l, it in zip(p.offsets, items)]
    assert P.check_layout(items, p.offsets, ends, [k * p.S for k in range(w.m + 1)], A) == []
    assert p.S >= P.lower_bound(items, w.m, A)
    # every quantisation tile lies inside one rank (no communication needed)
    for s, l in zip(w.tensors, p.offsets):
        if s.q_rows:
            for r0 in range(0, s.rows, s.q_rows):
                r1 = min(s.rows, r0 + s.q_rows)
                assert (l + r0 * s.cols) // p.S == (l + r1 * s.cols - 1) // p.S
    # S* is minimal: no smaller aligned S passes the greedy test
    lb = P.lower_bound(items, w.m, A)
    for S in range(lb, p.S, A):
        if P.shard_multiple_required(items, S):
            assert P.greedy_offsets(items, w.m, S, A) is None


def test_shard_multiple_condition_is_necessary():
    # a tensor longer than 2S forces S to be a multiple of its granule:
    # check by exhaustive placement on small numbers
    for g in range(1, 7):
        for S in range(1, 12):
            for E in range(2 * S + 1, 2 * S + 8):
                m = E // S + 3
                ok = any(P.offset_is_valid(l, P.Item(E, g), S, m, 1) for l in range(0, m * S))
                if S % g != 0:
                    assert not ok, (g, S, E)


def test_naive_concatenation_failures_detected():
    # Figure 6(a): the three failure modes of naive concatenation
    items = _items([(6, 3), (6, 3)])
    # 1) block split: plain concatenation cut at 5 (m=2 of 12 -> 6 each is fine,
    #    so use 3 ranks of 4)
    errs = P.check_layout(items, [0, 6], [6, 12], [0, 4, 8, 12])
    assert any("block split" in e for e in errs)
    # 2) padding inside a tensor to meet alignment -> non-contiguous memory
    errs = P.check_layout(items, [0, 8], [8, 14], [0, 7, 14])
    assert any("non-contiguous" in e for e in errs)
    # 3) unequal per-rank sizes
    errs = P.check_layout(items, [0, 6], [6, 12], [0, 6, 9, 12])
    assert any("imbalanced" in e for e in errs)
    # the planner's layout for the same group has none of them
    p = P.plan(items, 3, 1)
    ends = [l + it.numel for l, it in zip(p.offsets, items)]
    assert P.check_layout(items, p.offsets, ends, [k * p.S for k in range(4)]) == []


def test_fragments_cover_tensors():
    w = W.toy_unit()
    items = P.items_from_specs(w.tensors)
    p = P.plan(items, w.m, 1)
    fr = P.fragments(items, p.offsets, p.S, w.m)
    for t, it in enumerate(items):
        tot = sum(hi - lo for tid, k, lo, hi in fr if tid == t)
        assert tot == it.numel
    for tid, k, lo, hi in fr:
        assert k * p.S <= lo < hi <= (k + 1) * p.S


# ------------------------------------------------------------ tensor orders

def test_order_perm_hand_example():
    """The three orders worked by hand on four tensors:
    t0 4x8 gran 2 rows (g=16), t1 1x5 vector (g=1), t2 8x4 gran 4 rows
    (g=16), t3 4x8 gran 1 row (g=8).
    block (g descending, stable): t0, t2, t3, t1.
    shape ((rows, cols) descending, stable): t2 (8,4), t0 (4,8), t3 (4,8), t1 (1,5)."""
    specs = [W.TensorSpec("t0", 4, 8, 2), W.TensorSpec("t1", 1, 5, 0),
             W.TensorSpec("t2", 8, 4, 4), W.TensorSpec("t3", 4, 8, 1)]
    assert P.order_perm(specs, "given") == [0, 1, 2, 3]
    assert P.order_perm(specs, "block") == [0, 2, 3, 1]
    assert P.order_perm(specs, "shape") == [2, 0, 3, 1]


def _rand_specs(rng, max_t=5):
    """Random small row-major specs: vectors, row-granular and block-granular."""
    out = []
    for i in range(int(rng.integers(1, max_t + 1))):
        rows, cols = int(rng.integers(1, 7)), int(rng.integers(1, 6))
        gran = 0 if rows == 1 else int(rng.integers(0, rows + 1))
        out.append(W.TensorSpec(f"t{i}", rows, cols, gran))
    return out


def _layout_ok(specs, perm, offs, S, m, A):
    items = P.items_from_specs([specs[t] for t in perm])
    starts = [offs[t] for t in perm]
    ends = [l + it.numel for l, it in zip(starts, items)]
    return P.check_layout(items, starts, ends, [k * S for k in range(m + 1)], A) == []


def test_plan_ordered_valid_and_best_is_min():
    rng = np.random.default_rng(41)
    for _ in range(150):
        specs = _rand_specs(rng, 5)
        m = int(rng.integers(1, 5))
        A = int(rng.choice([1, 1, 2, 3]))
        got = {k: P.plan_ordered(specs, m, A, k) for k in ("given", "block", "shape", "best")}
        for k, (perm, offs, S) in got.items():
            assert sorted(perm) == list(range(len(specs)))
            assert _layout_ok(specs, perm, offs, S, m, A), (k, specs, m, A)
        Ss = [got[k][2] for k in ("given", "block", "shape")]
        assert got["best"][2] == min(Ss)
        # ties go to the earliest order in (given, block, shape)
        first = ("given", "block", "shape")[Ss.index(min(Ss))]
        assert got["best"][0] == got[first][0]
        # the given order is the plain planner
        p = P.plan(P.items_from_specs(specs), m, A)
        assert got["given"][2] == p.S and got["given"][1] == p.offsets


def test_orders_against_every_permutation():
    """Exhaustive over tensor orders on tiny groups: no order beats the
    minimum over all permutations, and that minimum is attained by some
    permutation (sanity of the order-free optimum the pages' NP-hardness
    refers to)."""
    rng = np.random.default_rng(43)
    for _ in range(60):
        specs = _rand_specs(rng, 4)
        m = int(rng.integers(1, 4))
        best_any = min(P.plan(P.items_from_specs([specs[t] for t in perm]), m, 1).S
                       for perm in itertools.permutations(range(len(specs))))
        assert P.plan_ordered(specs, m, 1, "best")[2] >= best_any


def test_coarser_granule_never_shrinks_S():
    """Row granules r | r': every layout valid with granule r' rows is valid
    with r rows, so S*(1 row) <= S*(2 rows) <= S*(4 rows) for the same order."""
    rng = np.random.default_rng(47)
    for _ in range(80):
        n = int(rng.integers(1, 5))
        specs = [W.TensorSpec(f"t{i}", int(rng.integers(1, 9)) * 4, int(rng.integers(1, 5)), 1)
                 for i in range(n)]
        m = int(rng.integers(1, 6))
        S = [P.plan(P.items_from_specs(W.regranulated(specs, r)), m, 1).S for r in (1, 2, 4)]
        assert S[0] <= S[1] <= S[2], (specs, m, S)


@pytest.mark.parametrize("name,A", [("llama3_8b_layer", 16), ("llama3_8b_layer", 1),
                                    ("llama70b_layer", 16)])
def test_s_star_closed_form_of_llama_layers(name, A):
    """S* of the Llama layer groups from a hand argument.  Every tensor at
    least twice as long as a candidate S holds two shard boundaries S apart,
    so S must be a multiple of its granule.  In the 8B layer, Wgate, Wup
    and Wdown (58,720,256 elements each, granules 128*4096 and 128*14336)
    are that long for every S below 29,360,128 = 8 * lcm(524288, 1835008),
    and 7 * 3,670,016 lies below ceil(E/8); in the 70B layer
    the same holds at 7,340,032 = lcm(128*8192, 128*28672).  So S* is the
    smallest lcm multiple at or above the lower bound, provided a layout
    exists there, which the oracle's plan shows."""
    w = W.WORKLOADS[name]
    items = P.items_from_specs(w.tensors)
    E = sum(it.numel for it in items)
    lb = -(-E // w.m)
    long_ = [it for it in items if it.granule > 1]
    L = 1
    for it in long_:
        L = math.lcm(L, it.granule)
    cand = -(-lb // L) * L
    # every S in [lb, cand) leaves the long tensors longer than 2S
    big = [it for it in long_ if 2 * (cand - 1) < it.numel]
    L_big = 1
    for it in big:
        L_big = math.lcm(L_big, it.granule)
    assert L_big == L and cand % A == 0
    expect = {"llama3_8b_layer": 29_360_128, "llama70b_layer": 7_340_032}[name]
    assert cand == expect
    p = P.plan(items, w.m, A)
    assert p.S == cand
    _independent_check(items, p.offsets, p.S, w.m, A)


def test_padding_fraction_hand_values():
    """padding_fraction = (m*S - E)/E on values worked by hand: the toy unit
    packs exactly (S = 98,304 = E/4, no padding), and the Llama-3-8B layer
    at S = 29,360,128 on 8 ranks holds E = 2*4096^2 + 2*1024*4096 +
    3*14336*4096 + 2*4096 = 218,112,000 elements in 234,881,024 positions,
    16,769,024 of them padding."""
    toy = P.items_from_specs(W.toy_unit().tensors)
    assert P.padding_fraction(toy, 98_304, 4) == 0.0
    c2 = P.items_from_specs(W.llama8b_layer().tensors)
    assert sum(it.numel for it in c2) == 218_112_000
    assert P.padding_fraction(c2, 29_360_128, 8) == 16_769_024 / 218_112_000
    # one 10-element tensor on 3 ranks of 4: 2 of 12 positions are padding
    assert P.padding_fraction([P.Item(10, 1)], 4, 3) == 0.2


# ------------------------------------------------- S* by a plain scan
#
# An independent check of S* for the groups whose S* has no closed form:
# offsets are found by testing the layout constraints on every aligned
# candidate offset in turn (no granule or lcm jumps), and every aligned S from
# ceil(E/m) up to the planner's S* is tried.  Greedy earliest placement is
# exact for a fixed S (pinned by exhaustive search on tiny groups).


def _plain_earliest(lo, E, g, S, m, A):
    """Smallest aligned l >= lo with l + E <= m*S such that every shard
    boundary strictly inside (l, l + E) is a whole number of granules after
    l, found by testing the candidates lo, lo + A, ... in order."""
    l0 = -(-lo // A) * A
    end = m * S
    W = 64
    while l0 + E <= end:
        cand = l0 + A * np.arange(W, dtype=np.int64)
        cand = cand[cand + E <= end]
        ok = np.ones(cand.size, bool)
        for k in range(int(cand[0]) // S + 1, min(m - 1, (int(cand[-1]) + E - 1) // S) + 1):
            b = k * S
            inside = (cand < b) & (b < cand + E)
            ok &= ~inside | ((b - cand) % g == 0)
        hit = np.flatnonzero(ok)
        if hit.size:
            return int(cand[hit[0]])
        l0 = int(cand[-1]) + A
        W = min(W * 4, 1 << 16)
    return None


def _plain_greedy(items, m, S, A):
    end, offs = 0, []
    for it in items:
        l = _plain_earliest(end, it.numel, it.granule, S, m, A)
        if l is None:
            return None
        offs.append(l)
        end = l + it.numel
    return offs


def _plain_scan_chunk(args):
    name, A, lo, hi, step = args
    items = P.items_from_specs(W.WORKLOADS[name].tensors)
    m = W.WORKLOADS[name].m
    return [S for S in range(lo, hi, step) if _plain_greedy(items, m, S, A) is not None]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["ragged_mixed", "moe_experts"])
def test_s_star_of_mixed_and_expert_groups_by_plain_scan(name):
    """S* of the ragged mixed group (44,040,192) and of the MoE expert unit
    (34,734,080) at align 16: no aligned S from ceil(E/m) up to S* admits a
    layout, and at S* the plain placement gives the planner's offsets.  For
    the mixed group only multiples of 4096 are tried below S*: its
    embedding (525,336,576 elements, granule 4096) is longer than 2S for
    every S there, so it holds two boundaries S apart, each a whole number
    of granules from its start, which forces S % 4096 == 0."""
    import multiprocessing as mp
    A = 16
    w = W.WORKLOADS[name]
    items = P.items_from_specs(w.tensors)
    E = sum(it.numel for it in items)
    lb = -(-(-(-E // w.m)) // A) * A
    p = P.plan(items, w.m, A)
    assert p.S == {"ragged_mixed": 44_040_192, "moe_experts": 34_734_080}[name]
    assert _plain_greedy(items, w.m, p.S, A) == p.offsets
    if name == "ragged_mixed":
        emb = items[0]
        assert emb.granule == 4096 and emb.numel > 2 * p.S
        lo, step = -(-lb // 4096) * 4096, 4096
    else:
        lo, step = lb, A
    bounds = list(range(lo, p.S, step * 256)) + [p.S]
    jobs = [(name, A, a, b, step) for a, b in zip(bounds[:-1], bounds[1:])]
    with mp.get_context("fork").Pool(min(8, os.cpu_count() or 1)) as pool:
        feasible = [S for part in pool.map(_plain_scan_chunk, jobs) for S in part]
    assert feasible == [], feasible[:5]
