"""C-ABI checks that need no GPU: the library loads and exports every entry
point of include/rs.h, the host planner agrees with the oracle, layouts are
validated, and hot calls reject bad arguments before touching a device."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import workloads as W
from oracle import plan as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rs.h")

R = pytest.importorskip("fsdp_sharded_buffer_amd")
from fsdp_sharded_buffer_amd import _lib  # noqa: E402


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(rs_[a-z_0-9]+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert len(names) >= 13
    lib = _lib.lib()
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (rs_\w+)", out))
    assert set(names) <= exported
    # the binding declares exactly the header's entry points
    assert set(_lib.SIGNATURES) == set(names)


def test_binding_has_same_names():
    for n in _declared():
        assert callable(getattr(R, n)), n


@pytest.mark.parametrize("name", list(W.WORKLOADS))
@pytest.mark.parametrize("A", [1, 16])
def test_planner_matches_oracle(name, A):
    w = W.WORKLOADS[name]      # the oracle's scan of the 193-tensor unit at A=1 takes ~50 s
    offs, info = R.rs_plan(w.tensors, w.m, A)
    p = P.plan(P.items_from_specs(w.tensors), w.m, A)
    assert info["S"] == p.S and offs == p.offsets
    assert info["total"] == w.m * p.S
    assert info["numel"] == w.numel
    assert info["pad_elems"] == w.m * p.S - w.numel
    assert info["lower_bound"] == P.lower_bound(P.items_from_specs(w.tensors), w.m, A)
    assert info["peak_param_bytes"] == P.peak_param_bytes(p.S, w.m)
    assert info["seconds"] < 0.3     # the pages' planner budget


def test_planner_matches_bruteforce_random():
    rng = np.random.default_rng(11)
    for _ in range(300):
        pairs = W.random_tiny_specs(rng, max_t=4, max_e=16, max_g=6)
        m = int(rng.integers(1, 5))
        A = int(rng.choice([1, 2, 4]))
        specs = [W.TensorSpec("t", 1, e, 0) if g == 1 else W.TensorSpec("t", e, 1, g)
                 for e, g in pairs]
        items = P.items_from_specs(specs)
        assert [(i.numel, i.granule) for i in items] == [(e, g) for e, g in pairs]
        bf = P.plan_bruteforce(items, m, A)
        offs, info = R.rs_plan(specs, m, A)
        assert (info["S"], offs) == (bf[0], bf[1]), (pairs, m, A)


def _rand_specs(rng, max_t=5):
    out = []
    for i in range(int(rng.integers(1, max_t + 1))):
        rows, cols = int(rng.integers(1, 7)), int(rng.integers(1, 6))
        gran = 0 if rows == 1 else int(rng.integers(0, rows + 1))
        out.append(W.TensorSpec(f"t{i}", rows, cols, gran))
    return out


def _study_groups():
    moe = W.WORKLOADS["moe_experts"]
    groups = {n: w.tensors for n, w in W.WORKLOADS.items()}
    groups["moe_experts_fused"] = W.fused_experts(moe).tensors
    for n in ("llama3_8b_layer", "ragged_mixed", "moe_experts_fused"):
        for r in (1, 16, 128):
            groups[f"{n}@{r}"] = W.regranulated(groups[n], r)
    return groups


def test_plan_order_matches_oracle():
    for name, specs in _study_groups().items():
        for k in ("given", "block", "shape"):
            assert R.rs_plan_order(specs, k) == P.order_perm(specs, k), (name, k)
    rng = np.random.default_rng(53)
    for _ in range(200):
        specs = _rand_specs(rng)
        for k in ("given", "block", "shape"):
            assert R.rs_plan_order(specs, k) == P.order_perm(specs, k)


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_plan_ordered_matches_oracle_on_configs(name):
    w = W.WORKLOADS[name]
    for k in ("given", "block", "shape", "best"):
        perm, offs, info = R.rs_plan_ordered(w.tensors, w.m, 16, k)
        o = P.plan_ordered(w.tensors, w.m, 16, k)
        assert (perm, offs, info["S"]) == (o[0], o[1], o[2]), k
        assert info["seconds"] < 0.3 * (3 if k == "best" else 1)


def test_plan_ordered_matches_oracle_random_and_study_cases():
    rng = np.random.default_rng(59)
    for _ in range(300):
        specs = _rand_specs(rng)
        m = int(rng.integers(1, 6))
        A = int(rng.choice([1, 2, 3, 4]))
        for k in ("given", "block", "shape", "best"):
            perm, offs, info = R.rs_plan_ordered(specs, m, A, k)
            o = P.plan_ordered(specs, m, A, k)
            assert (perm, offs, info["S"]) == (o[0], o[1], o[2]), (specs, m, A, k)
    # regranulated groups where long tensors force S to a multiple of their
    # granules (the planner skips the S values they reject), at A = 1
    g = _study_groups()
    for name, m in (("llama3_8b_layer@16", 64), ("llama70b_layer", 32), ("ragged_mixed@128", 16),
                    ("moe_experts_fused@16", 128), ("moe_experts_fused@128", 16)):
        specs = g[name] if "@" in name else W.regranulated(g[name], 16)
        for k in ("given", "best"):
            perm, offs, info = R.rs_plan_ordered(specs, m, 1, k)
            o = P.plan_ordered(specs, m, 1, k)
            assert (perm, offs, info["S"]) == (o[0], o[1], o[2]), (name, m, k)


def test_parallel_scan_equals_sequential(monkeypatch):
    """Long S scans (thousands of candidates past the lower bound) run in
    blocks on host threads; the plan must be the single-threaded one.  The
    separate-expert unit at 128-row granules and m = 128 scans about 130K
    candidates."""
    moe = W.WORKLOADS["moe_experts"]
    cases = [(W.regranulated(moe.tensors, 128), 128), (W.regranulated(moe.tensors, 16), 256)]
    got = {}
    for th in ("1", "7"):
        monkeypatch.setenv("RS_PLAN_THREADS", th)
        got[th] = [R.rs_plan_ordered(sp, m, 1, "best") for sp, m in cases]
    for a, b in zip(got["1"], got["7"]):
        assert a[0] == b[0] and a[1] == b[1] and a[2]["S"] == b[2]["S"]
        assert a[2]["S"] - a[2]["lower_bound"] > 4096      # the threaded path ran


def test_lcm_of_granules_sets_S():
    """Llama-8B layer, 16-row granules, 64 ranks: Wgate, Wup (14336x4096) and
    Wdown (4096x14336) are each longer than 2S, so S must be a multiple of
    both 16*4096 and 16*14336, i.e. of lcm = 2^16 * 7; the smallest such S
    above ceil(E/64) is 8 * 458752, and a layout exists there."""
    specs = W.regranulated(W.WORKLOADS["llama3_8b_layer"].tensors, 16)
    E = sum(s.numel for s in specs)
    L = 458752
    assert L == np.lcm(16 * 4096, 16 * 14336)
    expect = -(-(-(-E // 64)) // L) * L
    assert expect == 8 * L
    _, info = R.rs_plan(specs, 64, 1)
    assert info["S"] == expect
    assert abs(info["pad_frac"] - (64 * expect / E - 1)) < 1e-12


def test_layout_accepts_ordered_plan():
    w = W.WORKLOADS["ragged_mixed"]
    specs = W.regranulated(w.tensors, 128)
    perm, offs, info = R.rs_plan_ordered(specs, 16, 1, "best")
    assert perm != list(range(len(specs)))          # another order wins here
    ordered = [specs[t] for t in perm]
    h = R.rs_layout_create(ordered, 16, info["S"], [offs[t] for t in perm])
    li = R.rs_layout_get_info(h)
    R.rs_layout_destroy(h)
    assert li["total"] == 16 * info["S"] and li["n"] == len(specs)
    # in the given order the same offsets are rejected (tensors overlap or
    # are out of order)
    with pytest.raises(R.RsError):
        R.rs_layout_create(specs, 16, info["S"], offs)


def test_planner_infeasible_cap_and_bad_args():
    specs = [W.TensorSpec("a", 12, 1, 4)]
    with pytest.raises(R.RsError) as e:
        R.rs_plan(specs, 3, 1, S_cap=3)
    assert e.value.status == -4
    with pytest.raises(R.RsError) as e:
        R.rs_plan(specs, 0, 1)
    assert e.value.status == -1
    with pytest.raises(R.RsError):
        R.rs_plan([W.TensorSpec("a", 0, 4, 0)], 2, 1)
    assert "rs_plan" in R.rs_last_error()
    # an empty group is rejected, by the planner and by the layout builder
    with pytest.raises(R.RsError) as e:
        R.rs_plan([], 2, 1)
    assert e.value.status == -1
    with pytest.raises(R.RsError) as e:
        R.rs_layout_create([], 2, 16, [])
    assert e.value.status == -1


def test_size_limits_keep_int64_arithmetic_exact():
    """Sizes whose products or sums could overflow int64 are rejected:
    fewer than 2^40 elements per tensor, granule and group, at most 2^18
    ranks, an alignment of at most 2^20, S at most 2^41."""
    ok = [W.TensorSpec("a", 1 << 20, 1 << 19, 0)]          # 2^39 elements: accepted
    offs, info = R.rs_plan(ok, 1 << 18, 1 << 20)
    assert info["S"] >= (1 << 39) >> 18
    bad = [
        ([W.TensorSpec("a", 1 << 20, 1 << 20, 0)], 2, 1),            # 2^40 elements
        ([W.TensorSpec("a", 2, 3, 1 << 62)], 2, 1),                   # granule overflows
        ([W.TensorSpec("a", 1 << 62, 4, 0)], 2, 1),                   # rows * cols overflows
        ([W.TensorSpec("a", 1 << 20, 1 << 19, 0)] * 2, 2, 1),         # group of 2^40
        ([W.TensorSpec("a", 4, 4, 0)], (1 << 18) + 1, 1),             # ranks
        ([W.TensorSpec("a", 4, 4, 0)], 2, (1 << 20) + 1),             # alignment
    ]
    for specs, m, align in bad:
        with pytest.raises(R.RsError) as e:
            R.rs_plan(specs, m, align)
        assert e.value.status == -1
        with pytest.raises(R.RsError) as e:
            R.rs_plan_ordered(specs, m, align, "best")
        assert e.value.status == -1
    small = [W.TensorSpec("a", 4, 4, 0)]
    for specs, m, S, offs in [
        (small, (1 << 18) + 1, 16, [0]),                             # ranks
        (small, 2, (1 << 41) + 1, [0]),                              # S
        (small, 2, 16, [(1 << 62)]),                                 # offset: l + E overflows
        ([W.TensorSpec("a", 1 << 62, 4, 0)], 2, 16, [0]),            # rows * cols overflows
    ]:
        with pytest.raises(R.RsError) as e:
            R.rs_layout_create(specs, m, S, offs)
        assert e.value.status == -1, R.rs_last_error()


def test_plan_order_entry_points_reject_bad_args():
    specs = [W.TensorSpec("a", 12, 1, 4), W.TensorSpec("b", 4, 2, 1)]
    with pytest.raises(R.RsError) as e:
        R.rs_plan_order(specs, 3)             # BEST is not a single order
    assert e.value.status == -1 and "rs_plan_order" in R.rs_last_error()
    with pytest.raises(R.RsError) as e:
        R.rs_plan_ordered(specs, 2, 1, 7)
    assert e.value.status == -1
    with pytest.raises(R.RsError) as e:
        R.rs_plan_ordered(specs, 0, 1, "best")
    assert e.value.status == -1
    with pytest.raises(R.RsError) as e:
        R.rs_plan_ordered([W.TensorSpec("a", 0, 4, 0)], 2, 1, "given")
    assert e.value.status == -1
    # infeasible under the cap for every order
    with pytest.raises(R.RsError) as e:
        R.rs_plan_ordered(specs, 3, 1, "best", S_cap=3)
    assert e.value.status == -4
    # success clears the message
    R.rs_plan_ordered(specs, 2, 1, "best")
    assert R.rs_last_error() == ""


def test_layout_create_validates():
    w = W.toy_unit()
    offs, info = R.rs_plan(w.tensors, w.m, 16)
    h = R.rs_layout_create(w.tensors, w.m, info["S"], offs)
    li = R.rs_layout_get_info(h)
    assert li["num_tiles"] == 384 and li["total"] == w.m * info["S"]
    R.rs_layout_destroy(h)
    bad = list(offs)
    bad[2] = bad[1] + 100            # overlaps and misplaces W1
    with pytest.raises(R.RsError) as e:
        R.rs_layout_create(w.tensors, w.m, info["S"], bad)
    assert e.value.status == -1
    # a granule cut by a boundary
    specs = [W.TensorSpec("a", 8, 4, 4)]
    with pytest.raises(R.RsError):
        R.rs_layout_create(specs, 3, 12, [2])
    # a quantisation tile crossing a boundary (element granular tensor)
    specs = [W.TensorSpec("a", 8, 4, 0, 4, 4)]
    with pytest.raises(R.RsError) as e:
        R.rs_layout_create(specs, 3, 11, [0])
    assert "tile" in R.rs_last_error()
    # oversized tile
    with pytest.raises(R.RsError):
        R.rs_layout_create([W.TensorSpec("a", 256, 256, 256, 256, 256)], 1, 65536, [0])
    with pytest.raises(R.RsError):
        R.rs_layout_create(w.tensors, w.m, info["S"], offs, chunk_elems=100)


def test_layout_tables_partition_buffer():
    """Chunks cover the buffer exactly, never cross a rank or tensor edge."""
    w = W.scaled_workload(W.moe_experts(), 16, 8, max_tensors=13, m=5)
    offs, info = R.rs_plan(w.tensors, w.m, 1)
    h = R.rs_layout_create(w.tensors, w.m, info["S"], offs, chunk_elems=256)
    li = R.rs_layout_get_info(h)
    R.rs_layout_destroy(h)
    items = P.items_from_specs(w.tensors)
    fr = P.fragments(items, offs, info["S"], w.m)
    assert li["num_frags"] == len(fr)
    # every fragment splits into ceil(len/256) chunks; padding gaps likewise
    used = sum(-(-(hi - lo) // 256) for _, _, lo, hi in fr)
    assert li["num_chunks"] >= used


def test_hot_calls_reject_before_launch():
    """Calls on a layout that was never uploaded fail with RS_ERR_STATE and
    range errors are reported; no device is touched."""
    w = W.toy_unit()
    offs, info = R.rs_plan(w.tensors, w.m, 16)
    h = R.rs_layout_create(w.tensors, w.m, info["S"], offs)
    lib = _lib.lib()
    st = lib.rs_pack(h, 16, 0, 16, 1, 0, 1, None)
    assert st == -7 and "not uploaded" in R.rs_last_error()
    st = lib.rs_block_quant(None, 16, 0, 16, 16, None, 0, 1, None)
    assert st == -1
    R.rs_layout_destroy(h)
    assert R.rs_status_str(-5) == "rank range out of bounds"
    assert R.rs_status_str(0) == "ok"


def test_struct_layouts_match_header(tmp_path):
    """The binding's ctypes structs have the sizes and field offsets of the
    structs in include/rs.h, compiled as C by the host compiler."""
    import shutil
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    structs = [_lib.rs_tensor_spec, _lib.rs_plan_info, _lib.rs_layout_info, _lib.rs_adamw_params,
               _lib.rs_sgd_params]
    lines = ["#include <stddef.h>", "#include <stdio.h>", '#include "rs.h"', "int main(void) {"]
    for st in structs:
        name = st.__name__
        lines.append(f'  printf("{name} %zu\\n", sizeof({name}));')
        for f, _ in st._fields_:
            lines.append(f'  printf("{name}.{f} %zu\\n", offsetof({name}, {f}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layouts.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layouts"
    subprocess.run([cc, "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True, capture_output=True)
    got = dict(line.split() for line in subprocess.run([str(exe)], check=True, capture_output=True,
                                                       text=True).stdout.splitlines())
    for st in structs:
        name = st.__name__
        assert int(got[name]) == ctypes.sizeof(st), name
        for f, _ in st._fields_:
            assert int(got[f"{name}.{f}"]) == getattr(st, f).offset, f"{name}.{f}"


def test_signatures_match_header_parameter_counts():
    """Each ctypes signature has as many arguments as the declaration in
    include/rs.h, and returns a value exactly when the declaration does."""
    txt = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    decls = re.findall(r"\b([a-z_]+\s*\**)\s*\b(rs_[a-z_0-9]+)\s*\(([^;{]*?)\)\s*;", txt, flags=re.S)
    seen = set()
    for ret, name, params in decls:
        params = " ".join(params.split())
        n = 0 if params in ("", "void") else params.count(",") + 1
        restype, argtypes = _lib.SIGNATURES[name]
        assert len(argtypes) == n, f"{name}: {len(argtypes)} ctypes arguments, {n} in rs.h"
        assert (restype is None) == (ret.strip() == "void"), name
        seen.add(name)
    assert seen == set(_lib.SIGNATURES)


def test_layout_rejects_a_tile_across_a_shard_boundary():
    """Row granules with 4-row tiles: on 4 ranks S = 8 cuts the first 4x4
    tile of an 8x4 tensor in half, so the layout is refused (such a tile
    could not be quantised without communication); on 2 ranks the cut falls
    between tiles and the layout is accepted."""
    specs = [W.TensorSpec("a", 8, 4, 1, 4, 4)]
    offs, info = R.rs_plan(specs, 4, 1)
    assert info["S"] == 8
    with pytest.raises(R.RsError) as e:
        R.rs_layout_create(specs, 4, info["S"], offs)
    assert e.value.status == -1 and "crosses a shard boundary" in R.rs_last_error()
    offs, info = R.rs_plan(specs, 2, 1)
    h = R.rs_layout_create(specs, 2, info["S"], offs)
    assert R.rs_layout_get_info(h)["num_tiles"] == 2
    R.rs_layout_destroy(h)


def test_size_getters_match_layout_info():
    """rs_layout_device_bytes / rs_workspace_bytes give the sizes the caller
    allocates, equal to the layout info's, and 0 for a NULL layout."""
    w = W.llama8b_layer()
    offs, info = R.rs_plan(w.tensors, w.m, 16)
    h = R.rs_layout_create(w.tensors, w.m, info["S"], offs)
    li = R.rs_layout_get_info(h)
    assert R.rs_layout_device_bytes(h) == li["device_bytes"] > 0
    assert R.rs_workspace_bytes(h) == li["workspace_bytes"] >= 8 * li["num_chunks"]
    R.rs_layout_destroy(h)
    assert R.rs_layout_device_bytes(None) == 0 and R.rs_workspace_bytes(None) == 0


def test_layout_refuses_unindexable_chunk_tables_before_building():
    """A layout within the size limits whose fine chunk table would exceed
    int32 indices is refused with RS_ERR_INVALID_ARG, quickly and without
    building it; larger chunks make the same layout acceptable."""
    import time
    one = [W.TensorSpec("a", 1, 4, 0)]
    t0 = time.perf_counter()
    with pytest.raises(R.RsError) as e:
        R.rs_layout_create(one, 4, 1 << 40, [0])
    assert e.value.status == -1 and "chunks" in R.rs_last_error()
    assert time.perf_counter() - t0 < 1.0
    h = R.rs_layout_create(one, 4, 1 << 40, [0], chunk_elems=1 << 22)
    # the 4-element tensor splits the first chunk in two
    assert R.rs_layout_get_info(h)["num_chunks"] == ((4 << 40) >> 22) + 1
    R.rs_layout_destroy(h)
    assert R.rs_status_str(R.RS_ERR_NOMEM) == "out of host resources"
