"""Pins for the oracle's buffer operations (CPU only).

Checks round trips, special cases that reduce to a library routine (torch
CPU casts and fp32 arithmetic, math.fsum), closed forms (all-ones and
integer norms, the tile absmax element encoding to +-Q) and the tile
numbering on a non-square group where a transposed index would fail.
"""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import casts as C
from oracle import ops as O
from oracle import plan as P


def _setup(w, A=1):
    items = P.items_from_specs(w.tensors)
    p = P.plan(items, w.m, A)
    return items, p


def _ragged_group():
    """Small group with ragged fragments, element/row/block granules,
    non-square tiles and partial edge tiles."""
    ts = (W.TensorSpec("a", 40, 24, gran_rows=8, q_rows=8, q_cols=16),
          W.TensorSpec("v", 1, 37, gran_rows=0),
          W.TensorSpec("b", 30, 12, gran_rows=6, q_rows=6, q_cols=8),
          W.TensorSpec("e", 50, 10, gran_rows=1, q_rows=1, q_cols=4),
          W.TensorSpec("c", 7, 33, gran_rows=4, q_rows=4, q_cols=16))
    return W.Workload("ragged_small", ts, m=5, qfmt="fp8_e4m3", block=8)


@pytest.mark.parametrize("A", [1, 16])
def test_pack_unpack_roundtrip(A):
    w = _ragged_group()
    items, p = _setup(w, A)
    inp = W.make_inputs(w)
    buf = np.full(p.total, 7.0, dtype=np.float32)
    packed = O.pack(inp.params, p.offsets, p.S, w.m, buf, "f32", 0, w.m)
    dsts = [np.zeros_like(t) for t in inp.params]
    back = O.unpack(packed, [(s.rows, s.cols) for s in w.tensors], p.offsets, p.S, w.m,
                    dsts, "f32", 0, w.m)
    for a, b in zip(inp.params, back):
        assert np.array_equal(a, b)
    # padding positions are zero; tensor positions hold the tensor
    used = np.zeros(p.total, bool)
    for t, l in zip(inp.params, p.offsets):
        used[l:l + t.size] = True
        assert np.array_equal(packed[l:l + t.size], t.reshape(-1))
    assert np.all(packed[~used] == 0)
    # bf16 buffer: equals torch's cast of the concatenation
    bufh = np.zeros(p.total, dtype=np.uint16)
    ph = O.pack(inp.params, p.offsets, p.S, w.m, bufh, "bf16", 0, w.m)
    for t, l in zip(inp.params, p.offsets):
        ref = torch.from_numpy(t.reshape(-1).copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(ph[l:l + t.size], ref)
    back = O.unpack(ph, [(s.rows, s.cols) for s in w.tensors], p.offsets, p.S, w.m,
                    [np.zeros_like(t) for t in inp.params], "f32", 0, w.m)
    for t, b in zip(inp.params, back):
        ref = torch.from_numpy(t.copy()).to(torch.bfloat16).to(torch.float32).numpy()
        assert np.array_equal(b, ref)


def test_pack_rank_range_only():
    w = _ragged_group()
    items, p = _setup(w, 1)
    inp = W.make_inputs(w)
    buf = np.full(p.total, 7.0, dtype=np.float32)
    k0, k1 = 1, 3
    out = O.pack(inp.params, p.offsets, p.S, w.m, buf, "f32", k0, k1)
    assert np.all(out[:k0 * p.S] == 7.0) and np.all(out[k1 * p.S:] == 7.0)
    full = O.pack(inp.params, p.offsets, p.S, w.m, buf, "f32", 0, w.m)
    assert np.array_equal(out[k0 * p.S:k1 * p.S], full[k0 * p.S:k1 * p.S])


def test_scale_add_special_cases_and_torch():
    w = _ragged_group()
    items, p = _setup(w, 1)
    rng = np.random.default_rng(2)
    y = rng.standard_normal(p.total).astype(np.float32)
    x = rng.standard_normal(p.total).astype(np.float32)
    pads = np.ones(p.total, bool)
    for it, l in zip(items, p.offsets):
        pads[l:l + it.numel] = False
    out, f = O.scale_add(y, x, 1.0, 0.0, items, p.offsets, p.S, w.m, 0, w.m)
    assert np.array_equal(out, y) and not f.any()
    out, _ = O.scale_add(y, x, 0.0, 1.5, items, p.offsets, p.S, w.m, 0, w.m)
    assert np.array_equal(out[~pads], (np.float32(1.5) * x)[~pads])
    assert np.array_equal(out[pads], y[pads])
    out, _ = O.scale_add(y, x, 1.0, 1.0, items, p.offsets, p.S, w.m, 0, w.m)
    ref = (torch.from_numpy(y) + torch.from_numpy(x)).numpy()
    assert np.array_equal(out[~pads], ref[~pads])
    a, b = 0.37, -1.25
    out, _ = O.scale_add(y, x, a, b, items, p.offsets, p.S, w.m, 0, w.m)
    ty, tx = torch.from_numpy(y), torch.from_numpy(x)
    ref = torch.add(torch.mul(ty, a), torch.mul(tx, b)).numpy()
    assert np.array_equal(out[~pads], ref[~pads])
    # bf16 x is widened exactly
    xh = C.bf16_bits_from_f32(x)
    out, _ = O.scale_add(y, xh, 1.0, 1.0, items, p.offsets, p.S, w.m, 0, w.m)
    ref = (ty + torch.from_numpy(x).to(torch.bfloat16).to(torch.float32)).numpy()
    assert np.array_equal(out[~pads], ref[~pads])


def test_scale_add_mask_and_found_inf():
    w = _ragged_group()
    items, p = _setup(w, 1)
    y = np.ones(p.total, np.float32)
    x = np.ones(p.total, np.float32)
    fr = P.fragments(items, p.offsets, p.S, w.m)
    # one inf in the fragment of tensor 2 that lies in its last rank
    t2 = [f for f in fr if f[0] == 2]
    tid, k, lo, hi = t2[-1]
    x[lo] = np.inf
    out, found = O.scale_add(y, x, 1.0, 1.0, items, p.offsets, p.S, w.m, 0, w.m)
    assert found.tolist() == [1 if r == k else 0 for r in range(w.m)]
    mask = [1, 1, 0, 1, 1]
    out, found = O.scale_add(y, x, 1.0, 1.0, items, p.offsets, p.S, w.m, 0, w.m, mask=mask)
    assert not found.any()
    assert np.all(out[p.offsets[2]:p.offsets[2] + items[2].numel] == 1)
    # outside the rank range nothing changes and nothing is flagged
    out, found = O.scale_add(y, x, 1.0, 1.0, items, p.offsets, p.S, w.m, 0, k)
    assert not found.any() and np.all(out[k * p.S:] == 1)


def test_zero_mask_and_pads():
    w = _ragged_group()
    items, p = _setup(w, 16)
    y = np.full(p.total, 3.0, np.float32)
    out = O.zero(y, items, p.offsets, p.S, w.m, 1, 4)
    assert np.all(out[p.S:4 * p.S] == 0) and np.all(out[:p.S] == 3) and np.all(out[4 * p.S:] == 3)
    mask = [0, 1, 0, 0, 1]
    out = O.zero(y, items, p.offsets, p.S, w.m, 0, w.m, mask=mask)
    for t, (it, l) in enumerate(zip(items, p.offsets)):
        assert np.all(out[l:l + it.numel] == (0 if mask[t] else 3))
    pads = np.ones(p.total, bool)
    for it, l in zip(items, p.offsets):
        pads[l:l + it.numel] = False
    assert np.all(out[pads] == 3)


def test_sqnorm_closed_forms():
    w = _ragged_group()
    items, p = _setup(w, 1)
    ones = np.ones(p.total, np.float32)
    sq, part, found = O.sqnorm(ones, items, p.offsets, p.S, w.m, 0, w.m)
    assert sq.tolist() == [float(it.numel) for it in items]
    assert np.array_equal(part.sum(axis=0), sq)
    rng = np.random.default_rng(4)
    ints = rng.integers(-50, 51, size=p.total).astype(np.float32)
    sq, part, _ = O.sqnorm(ints, items, p.offsets, p.S, w.m, 0, w.m)
    for t, (it, l) in enumerate(zip(items, p.offsets)):
        exact = sum(int(v) ** 2 for v in ints[l:l + it.numel])
        assert sq[t] == exact
    x = rng.standard_normal(p.total).astype(np.float32)
    sq, part, _ = O.sqnorm(x, items, p.offsets, p.S, w.m, 0, w.m)
    for t, (it, l) in enumerate(zip(items, p.offsets)):
        ref = math.fsum(float(v) * float(v) for v in x[l:l + it.numel])
        assert abs(sq[t] - ref) <= 1e-13 * ref
        # partials are the fragment sums, in rank order
        for k in range(w.m):
            lo, hi = max(l, k * p.S), min(l + it.numel, (k + 1) * p.S)
            ref_k = math.fsum(float(v) * float(v) for v in x[lo:hi]) if hi > lo else 0.0
            assert abs(part[k, t] - ref_k) <= 1e-13 * max(ref_k, 1e-300)


def test_sqnorm_nonfinite_classes():
    w = _ragged_group()
    items, p = _setup(w, 1)
    x = np.ones(p.total, np.float32)
    l0, l2 = p.offsets[0], p.offsets[2]
    x[l0 + 3] = np.inf
    x[l2 + 5] = np.nan
    x[l2 + 6] = -np.inf
    sq, part, found = O.sqnorm(x, items, p.offsets, p.S, w.m, 0, w.m)
    assert sq[0] == np.inf and np.isnan(sq[2]) and np.isfinite(sq[1])
    assert found[(l0 + 3) // p.S] == 1 and found[(l2 + 5) // p.S] == 1


def test_quant_tile_amax_encodes_to_q():
    rng = np.random.default_rng(9)
    for fmt, top in (("fp8_e4m3", 0x7E), ("int8", 127)):
        for _ in range(200):
            t = (rng.standard_normal((8, 16)) * 10 ** rng.uniform(-30, 30)).astype(np.float32)
            sc, cd = O.quant_tile(t, fmt)
            i = np.unravel_index(np.argmax(np.abs(t)), t.shape)
            c = int(cd[i])
            if fmt == "fp8_e4m3":
                assert c & 0x7F == top and (c >> 7) == int(t[i] < 0)
            else:
                assert np.int8(np.uint8(c)) == (top if t[i] > 0 else -top)


def test_quant_dequant_error_bound_and_torch_fp8():
    rng = np.random.default_rng(10)
    t = (rng.standard_normal((32, 32)) * 0.02).astype(np.float32)
    sc, cd = O.quant_tile(t, "fp8_e4m3")
    q = (t / sc).astype(np.float32)
    ref = torch.from_numpy(np.clip(q, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(cd, ref)
    dq = C.e4m3fn_to_f64(cd) * np.float64(sc)
    # relative error of a normal E4M3 value is at most 2^-4; subnormals 2^-10 * scale
    err = np.abs(dq - t)
    bound = np.maximum(np.abs(t) * 2.0 ** -4, 2.0 ** -10 * sc) * 1.0001
    assert np.all(err <= bound)
    sc, cd = O.quant_tile(t, "int8")
    dq = cd.view(np.int8).astype(np.float64) * sc
    assert np.all(np.abs(dq - t) <= 0.5 * sc * 1.0001)


def test_quant_special_tiles():
    z = np.zeros((4, 4), np.float32)
    sc, cd = O.quant_tile(z, "fp8_e4m3")
    assert sc == 0 and not cd.any()
    n = np.ones((4, 4), np.float32)
    n[1, 2] = np.nan
    sc, cd = O.quant_tile(n, "fp8_e4m3")
    assert np.float32(sc).view(np.uint32) == 0x7FC00000 and np.all(cd == 0x7F)
    sc, cd = O.quant_tile(n, "int8")
    assert np.all(cd == 0)
    i = np.ones((4, 4), np.float32)
    i[0, 0] = -np.inf
    sc, cd = O.quant_tile(i, "fp8_e4m3")
    assert sc == np.inf and cd[0, 0] == 0x7F and np.all(cd.reshape(-1)[1:] == 0x00)
    i[0, 1] = -1.0
    sc, cd = O.quant_tile(i, "fp8_e4m3")
    assert cd[0, 1] == 0x80     # -1/inf = -0
    tiny = np.full((2, 2), 1e-44, np.float32)   # amax/448 underflows to 0
    sc, cd = O.quant_tile(tiny, "int8")
    assert sc == 0 and not cd.any()


def test_block_quant_tile_numbering_and_positions():
    w = _ragged_group()
    items, p = _setup(w, 1)
    x = np.zeros(p.total, np.float32)
    # give every tile a distinct amax at a known element
    tiles = []
    for s, l in zip(w.tensors, p.offsets):
        if s.q_rows:
            for (r0, r1, c0, c1) in O.tile_grid(s.rows, s.cols, s.q_rows, s.q_cols):
                tiles.append((l, s.cols, r0, r1, c0, c1))
    for j, (l, C_, r0, r1, c0, c1) in enumerate(tiles):
        rr, cc = r1 - 1, c1 - 1           # bottom-right element of the tile
        x[l + rr * C_ + cc] = np.float32(448.0 * (j + 1))
        x[l + r0 * C_ + c0] = np.float32(-1.0)
    assert len(tiles) == O.num_tiles(w.tensors)
    codes = np.full(p.total, 0xAB, np.uint8)
    scales = np.full(len(tiles), -1.0, np.float32)
    cd, sc = O.block_quant(x, w.tensors, p.offsets, p.S, w.m, "fp8_e4m3", 0, w.m, codes, scales)
    for j, (l, C_, r0, r1, c0, c1) in enumerate(tiles):
        assert sc[j] == np.float32(j + 1)
        assert cd[l + (r1 - 1) * C_ + (c1 - 1)] == 0x7E
        if (r1 - 1, c1 - 1) != (r0, c0):
            # -1/(j+1) encodes as a negative code
            assert cd[l + r0 * C_ + c0] & 0x80
    # non-quantised tensor and padding positions untouched
    v = p.offsets[1]
    assert np.all(cd[v:v + 37] == 0xAB)


def test_block_quant_straddle_rejected():
    ts = (W.TensorSpec("a", 8, 4, gran_rows=0, q_rows=4, q_cols=4),)
    items = P.items_from_specs(ts)
    p = P.plan(items, 3, 1)
    x = np.ones(p.total, np.float32)
    with pytest.raises(ValueError):
        O.block_quant(x, ts, p.offsets, p.S, 3, "int8", 0, 3,
                      np.zeros(p.total, np.uint8), np.zeros(2, np.float32))


def test_decode_codes_against_torch():
    codes = np.arange(256, dtype=np.uint8)
    dec = O.decode_codes(codes, "fp8_e4m3")
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(dec), nan)
    assert np.array_equal(dec[~nan], ref[~nan])
    dec = O.decode_codes(codes, "int8")
    assert np.array_equal(dec, codes.view(np.int8).astype(np.float32))


@pytest.mark.parametrize("fmt", ["fp8_e4m3", "int8"])
def test_dequant_roundtrip_error_bound(fmt):
    """|dequant(quant(x)) - x| <= scale * (half a code step at q + half an fp32
    ulp of q) + half an fp32 ulp of the result."""
    w = _ragged_group()
    items, p = _setup(w, 1)
    x = (np.random.default_rng(31).standard_normal(p.total) * 0.02).astype(np.float32)
    nt = O.num_tiles(w.tensors)
    codes, scales = O.block_quant(x, w.tensors, p.offsets, p.S, w.m, fmt, 0, w.m,
                                  np.zeros(p.total, np.uint8), np.zeros(nt, np.float32))
    y = O.block_dequant(codes, scales, w.tensors, p.offsets, p.S, w.m, fmt, 0, w.m,
                        np.full(p.total, np.nan, np.float32), "f32")
    base = 0
    for s, l in zip(w.tensors, p.offsets):
        if not s.q_rows:
            continue
        for (r0, r1, c0, c1) in O.tile_grid(s.rows, s.cols, s.q_rows, s.q_cols):
            pos = l + (np.arange(r0, r1)[:, None] * s.cols + np.arange(c0, c1)[None, :])
            sc = np.float64(scales[base])
            q = np.abs(x[pos].astype(np.float64)) / sc
            if fmt == "fp8_e4m3":
                step = np.where(q < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(q, 2.0 ** -6))) - 3))
            else:
                step = np.ones_like(q)
            ulp32 = np.spacing(np.abs(x[pos]).astype(np.float32)).astype(np.float64)
            bound = sc * (step / 2 + np.spacing(q.astype(np.float32)).astype(np.float64) / 2) + ulp32
            assert np.all(np.abs(y[pos].astype(np.float64) - x[pos]) <= bound * 1.000001)
            base += 1
    # positions outside quantised tiles untouched
    v = p.offsets[1]
    assert np.all(np.isnan(y[v:v + 37]))


def test_dequant_bf16_and_special_scales():
    codes = np.array([0x38, 0xB8, 0x7F, 0x00, 0x80, 0x01], np.uint8)  # 1, -1, NaN, 0, -0, 2^-9
    ts = (W.TensorSpec("a", 2, 3, 2, 2, 3),)
    items = P.items_from_specs(ts)
    p = P.plan(items, 1, 1)
    y = O.block_dequant(codes, np.array([3.0], np.float32), ts, p.offsets, p.S, 1, "fp8_e4m3",
                        0, 1, np.zeros(6, np.float32), "f32")
    assert y[0] == 3.0 and y[1] == -3.0 and np.isnan(y[2]) and y[3] == 0.0
    assert np.signbit(y[4]) and y[5] == np.float32(3.0 * 2.0 ** -9)
    yb = O.block_dequant(codes, np.array([1.0 / 3.0], np.float32), ts, p.offsets, p.S, 1,
                         "fp8_e4m3", 0, 1, np.zeros(6, np.uint16), "bf16")
    ref = torch.tensor([1 / 3, -1 / 3], dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(yb[:2], ref)


def test_quant_found_inf():
    w = _ragged_group()
    items, p = _setup(w, 1)
    x = np.ones(p.total, np.float32)
    l = p.offsets[3]        # row-granular tensor "e"
    x[l + 7] = np.inf
    v = p.offsets[1]        # the vector is not quantised: ignored
    x[v + 2] = np.nan
    f = O.quant_found_inf(x, w.tensors, p.offsets, p.S, w.m, 0, w.m)
    assert f.tolist() == [1 if k == (l + 7) // p.S else 0 for k in range(w.m)]


def test_quant_tiles_match_hand_worked_values():
    """tests/golden/quant_tiles.json: tiles quantised by hand from the OCP
    E4M3FN and INT8 definitions (scale, every code, ties to even, subnormals,
    a zero tile)."""
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "quant_tiles.json")))
    for t in g["tiles"]:
        scale, codes = O.quant_tile(np.array(t["x"], np.float32), t["fmt"])
        assert float(scale) == t["scale"], t["why"]
        assert [int(c) for c in codes.reshape(-1)] == [int(c, 16) for c in t["codes"]], t["why"]


def test_fullsize_digests_reproduce_from_the_oracle():
    """The stored digests of the full-size tile outputs are the oracle's:
    the fragment holding the whole of the Llama-3-8B layer's Wk (rank 0),
    quantised from the params and dequantised here by the oracle, matches
    tests/golden/fullsize_digests.json as written by
    tests/golden/make_fullsize_digests.py.  Only Wk's params are drawn: each
    tensor's params come from its own child of the root seed, in tensor
    order, so the group cut after Wk draws the same values for it."""
    import json
    import os
    import sys
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import fullsize_cases as FC
    from oracle import plan as P

    d = json.load(open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                                    "fullsize_digests.json")))["llama3_8b_layer"]
    w = W.WORKLOADS["llama3_8b_layer"]
    p = P.plan(P.items_from_specs(w.tensors), w.m, FC.ALIGN)
    assert (p.S, p.offsets) == (d["S"], d["offsets"])
    frags = [tuple(f) for f in d["frags"]]
    assert frags == FC.fragments(w.tensors, p.offsets, p.S)
    i = 1
    t, k, lo, hi, a, b = frags[i]
    assert (t, k, lo, hi) == (1, 0, p.offsets[1], p.offsets[1] + w.tensors[1].numel)
    cut = W.Workload(w.name, w.tensors[:2], m=w.m, qfmt=w.qfmt, block=w.block)
    wk = W.make_inputs(cut, grads=False).params[1]
    total, nt = w.m * p.S, O.num_tiles(w.tensors)
    # whole-buffer arrays whose untouched pages stay unallocated
    x = np.zeros(total, np.float32)
    x[lo:hi] = wk.reshape(-1)
    codes, scales = np.zeros(total, np.uint8), np.zeros(nt, np.float32)
    O.block_quant(x, w.tensors, p.offsets, p.S, w.m, w.qfmt, k, k + 1, codes, scales,
                  only_tiles=range(a, b), inplace=True)
    y = np.zeros(total, np.float32)
    O.block_dequant(codes, scales, w.tensors, p.offsets, p.S, w.m, w.qfmt, k, k + 1, y, "f32",
                    only_tiles=range(a, b), inplace=True)
    assert FC.digest(codes[lo:hi], scales[a:b], y[lo:hi]) == d["quant_params"][i]
