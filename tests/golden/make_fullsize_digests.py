"""Write tests/golden/fullsize_digests.json: digests of the oracle's outputs
for the tile operations at full size, fragment by fragment.

For each of the four large groups (planned by the oracle at align 16, inputs
from workloads.make_inputs) and each fragment of a quantised tensor (its
tiles inside one rank; the mixed group's embedding, 4.1M one-row tiles, is
left to a sampled check), three digests of the oracle's results:
  * quantisation of the params buffer: the fragment's codes, its tiles'
    scales, and the dequantisation of those codes to fp32;
  * the same for the grads buffer;
  * one 8-bit AdamW step from the seeded moment state of
    tests/fullsize_cases.py: the fragment's new params, m codes, v codes and
    its tiles' new m and v scales.
tests/test_gpu_fullsize.py hashes the library's outputs the same way.

Only oracle/ and workloads (inputs) compute anything here.  Run from the
repository root:  python tests/golden/make_fullsize_digests.py  (CPU only,
one worker process per core; about 10 minutes on 8 cores).
"""
from __future__ import annotations

import json
import multiprocessing as mp
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

import numpy as np  # noqa: E402

import fullsize_cases as FC  # noqa: E402
import workloads as W  # noqa: E402
from oracle import ops as O  # noqa: E402
from oracle import optim as OP  # noqa: E402
from oracle import plan as P  # noqa: E402

OUT = os.path.join(ROOT, "tests", "golden", "fullsize_digests.json")

# set in the parent before the workers fork; read-only in the workers
G = {}


def _one(i):
    w, specs, offsets, S, m = G["w"], G["w"].tensors, G["offsets"], G["S"], G["w"].m
    t, k, lo, hi, a, b = G["frags"][i]
    fmt, nt = w.qfmt, G["nt"]
    tiles = range(a, b)
    # Outputs are whole-buffer arrays from np.zeros, whose pages are only
    # materialised where the fragment's tiles write; the oracle reads and
    # writes nothing outside the requested tiles.
    out = []
    for src in ("params", "grads"):
        x = G[src]
        codes = np.zeros(G["total"], np.uint8)
        scales = np.zeros(nt, np.float32)
        O.block_quant(x, specs, offsets, S, m, fmt, k, k + 1, codes, scales, only_tiles=tiles,
                      inplace=True)
        y = np.zeros(G["total"], np.float32)
        O.block_dequant(codes, scales, specs, offsets, S, m, fmt, k, k + 1, y, "f32",
                        only_tiles=tiles, inplace=True)
        out.append(FC.digest(codes[lo:hi], scales[a:b], y[lo:hi]))
        del codes, y
    p = np.zeros(G["total"], np.float32)
    mc, vc = np.zeros(G["total"], np.uint8), np.zeros(G["total"], np.uint8)
    p[lo:hi], mc[lo:hi], vc[lo:hi] = G["params"][lo:hi], G["mc0"][lo:hi], G["vc0"][lo:hi]
    ms, vs = G["ms0"].copy(), G["vs0"].copy()
    OP.adamw8_step(p, G["grads"], mc, ms, vc, vs, specs, offsets, S, m, k, k + 1, fmt, FC.ADAMW8_HP,
                   only_tiles=tiles, inplace=True)
    out.append(FC.digest(p[lo:hi], mc[lo:hi], vc[lo:hi], ms[a:b], vs[a:b]))
    return i, out


def group_digests(name: str, workers: int) -> dict:
    w = W.WORKLOADS[name]
    p = P.plan(P.items_from_specs(w.tensors), w.m, FC.ALIGN)
    S, offsets, total = p.S, p.offsets, w.m * p.S
    inp = W.make_inputs(w)
    G.clear()
    G.update(w=w, S=S, offsets=offsets, total=total, nt=O.num_tiles(w.tensors),
             params=FC.flat(inp.params, offsets, total), grads=FC.flat(inp.grads, offsets, total),
             frags=FC.fragments(w.tensors, offsets, S))
    del inp
    G["mc0"], G["vc0"], G["ms0"], G["vs0"] = FC.adamw8_state(total, G["nt"], w.qfmt)
    res = [None] * len(G["frags"])
    t0 = time.time()
    with mp.get_context("fork").Pool(workers) as pool:
        for i, d in pool.imap_unordered(_one, range(len(G["frags"]))):
            res[i] = d
    print(f"{name}: {len(res)} fragments in {time.time() - t0:.0f} s", flush=True)
    return {"S": S, "offsets": offsets, "num_tiles": G["nt"], "qfmt": w.qfmt,
            "frags": [list(f) for f in G["frags"]],
            "quant_params": [r[0] for r in res], "quant_grads": [r[1] for r in res],
            "adamw8": [r[2] for r in res]}


def main():
    workers = int(os.environ.get("DIGEST_WORKERS", os.cpu_count() or 1))
    out = {"_about": "digests of the oracle's full-size tile outputs per fragment; written by "
                     "tests/golden/make_fullsize_digests.py"}
    names = sys.argv[1:] or list(FC.GROUPS)
    if os.path.exists(OUT) and sys.argv[1:]:
        out.update(json.load(open(OUT)))
    for name in names:
        out[name] = group_digests(name, workers)
        G.clear()
        with open(OUT, "w") as f:   # one line per key of each group
            f.write("{\n" + ",\n".join(
                f"{json.dumps(g)}: " + (json.dumps(v) if not isinstance(v, dict) else
                                        "{\n" + ",\n".join(f" {json.dumps(k)}: {json.dumps(x)}"
                                                            for k, x in v.items()) + "\n}")
                for g, v in out.items()) + "\n}\n")


if __name__ == "__main__":
    main()
