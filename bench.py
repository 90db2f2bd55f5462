"""Benchmark of the RaggedShard flat-buffer hot path on one MI355X.

One step = one pass of every grouped operation over one FSDP unit's planned
buffer, all ranks (the whole buffer):
  pack (fp32 params -> bf16 buffer), unpack (bf16 buffer -> bf16 tensors),
  group scale-add (fp32 grad accumulation with found-inf), ragged squared
  norms (fp64), block quantisation (FP8 E4M3 / INT8 codes + fp32 scales) and
  group zero (fp32 grad buffer, padding included).
Inputs are resident in HBM before timing.  Prints one JSON line.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import itertools
import json
import os
import ctypes
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

METRIC = "HBM GB/s and % of MI355X peak per DBuffer op on the Llama-8B-layer group"
HBM_PEAK_GBS = 8000.0
# the files the kernels are compiled from: counters taken on other sources
# are not reported as this build's traffic
KERNEL_SRCS = [os.path.join(ROOT, "fsdp_sharded_buffer_amd", "csrc", f)
               for f in ("rs_kernels.hip", "rs_exact.h", "rs_internal.h")]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_hash() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def op_bytes(w, S, n_tiles):
    """Algorithmic bytes per launch of each operation (whole buffer)."""
    E = w.numel
    mS = w.m * S
    Eq = sum(t.numel for t in w.tensors if t.q_rows)
    return {
        "pack": 4 * E + 2 * mS,          # fp32 tensors in, whole bf16 buffer out (pads zeroed)
        "unpack": 2 * E + 2 * E,         # bf16 buffer in, bf16 tensors out
        "scale_add": 12 * E,             # y in, x in, y out (fp32)
        "sqnorm": 4 * E,                 # fp32 in
        "block_quant": 5 * Eq + 4 * n_tiles,  # fp32 in, codes + scales out
        "zero": 4 * mS,                  # whole fp32 buffer out
    }


def rank_bytes(w, offs, S):
    """Algorithmic bytes of each operation (the step's and those measured
    beside it) over one rank's shard [kS, (k+1)S): the tensor elements and
    quantisation tiles that fall in it."""
    m = w.m
    E = np.zeros(m, np.int64)
    Eq = np.zeros(m, np.int64)
    tiles = np.zeros(m, np.int64)
    for t, l in zip(w.tensors, offs):
        for k in range(l // S, (l + t.numel - 1) // S + 1):
            n = min(l + t.numel, (k + 1) * S) - max(l, k * S)
            E[k] += n
            if t.q_rows:
                Eq[k] += n
        if t.q_rows:
            r0 = np.arange(0, t.rows, t.q_rows, dtype=np.int64)
            c0 = np.arange(0, t.cols, t.q_cols, dtype=np.int64)
            first = l + r0[:, None] * t.cols + c0[None, :]
            tiles += np.bincount((first // S).reshape(-1), minlength=m)
    return [{"pack": 4 * int(E[k]) + 2 * S, "unpack": 4 * int(E[k]), "scale_add": 12 * int(E[k]),
             "sqnorm": 4 * int(E[k]), "block_quant": 5 * int(Eq[k]) + 4 * int(tiles[k]),
             "zero": 4 * S, "block_dequant": 5 * int(Eq[k]) + 4 * int(tiles[k]),
             "adamw_step": 28 * int(E[k]), "sgd_step": 20 * int(E[k]),
             "adamw8_step": 16 * int(Eq[k]) + 16 * int(tiles[k])} for k in range(m)]


def extra_bytes(w, S, n_tiles):
    """Algorithmic bytes of the operations measured beside the step."""
    Eq = sum(t.numel for t in w.tensors if t.q_rows)
    E = w.numel
    return {
        "block_dequant": Eq + 4 * n_tiles + 4 * Eq,   # codes + scales in, fp32 out
        "adamw_step": 28 * E,    # p, g, m, v in; p, m, v out (fp32)
        "sgd_step": 20 * E,      # p, g, buf in; p, buf out (fp32)
        "adamw8_step": 8 * Eq + 2 * Eq + 4 * Eq + 2 * Eq + 16 * n_tiles,  # p,g in; 2 codes in;
                                                                          # p out; 2 codes out
    }


def read_counters(workload: str):
    """HBM traffic of the scale-add kernel from the committed rocprofv3
    counter summary, if it was taken on the current kernel source."""
    p = os.path.join(ROOT, "profiles", f"counters_scale_add_{workload}.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("source_sha256_16") != source_hash():
        return None
    return d.get("traffic_bytes_per_launch")


def live_counters(workload: str, align: int, chunk: int, timeout_s: float = 150.0):
    """HBM traffic of one whole-buffer scale-add launch, measured in this run:
    two rocprofv3 counter passes (FETCH_SIZE, then WRITE_SIZE) over a child
    run of this script in --counter-pass mode, each counter scaled by what it
    reads for a plain 1 GiB device copy in the same child.  None when
    rocprofv3 is missing or a pass gives no complete counter file."""
    import csv
    import shutil
    import signal
    import subprocess
    import tempfile

    exe = shutil.which("rocprofv3")
    if not exe:
        return None
    per = {}
    with tempfile.TemporaryDirectory(prefix="rs_pmc_") as tmp:
        for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
            out = os.path.join(tmp, ctr.lower())
            cmd = [exe, "--pmc", ctr, "-f", "csv", "-d", out, "-o", "c", "--", sys.executable,
                   os.path.abspath(__file__), "--counter-pass", "--workload", workload,
                   "--align", str(align), "--chunk", str(chunk)]
            log(f"live counters: {ctr}")
            p = subprocess.Popen(cmd, cwd=ROOT, stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL,
                                 env=dict(os.environ, TMPDIR="/tmp"), start_new_session=True)
            try:
                p.wait(timeout=timeout_s)
            except subprocess.TimeoutExpired:
                os.killpg(p.pid, signal.SIGKILL)
                p.wait()
                log(f"live counters: {ctr} pass timed out")
                return None
            # the profiler may exit non-zero after the program finished and
            # its files are whole: the file decides
            files = [os.path.join(dp, f) for dp, _, fs in os.walk(out) for f in fs
                     if f.endswith("counter_collection.csv")]
            if not files:
                log(f"live counters: no {ctr} file (rocprofv3 exit {p.returncode})")
                return None
            copy, kern = [], {}
            with open(files[0]) as f:
                for r in csv.DictReader(f):
                    if r.get("Counter_Name") != ctr:
                        continue
                    name, v = r["Kernel_Name"], float(r["Counter_Value"])
                    if name.startswith("__amd_rocclr_copyBuffer"):
                        copy.append(v)
                    elif "scale_add_kernel<0>" in name:
                        kern.setdefault(int(r["Grid_Size"]), []).append(v)
            if not copy or not kern:
                log(f"live counters: {ctr} file lacks the copy or the scale-add dispatches")
                return None
            big = kern[max(kern)]
            per[ctr] = (sum(big) / len(big), max(copy))
    gib_kib = float(1 << 20)  # 1 GiB copied = 1 GiB read + 1 GiB written, in KiB
    fetch, fcal = per["FETCH_SIZE"]
    write, wcal = per["WRITE_SIZE"]
    return {"traffic_bytes": int(round(fetch * 1024 * gib_kib / fcal + write * 1024 * gib_kib / wcal)),
            "fetch_kib": round(fetch, 1), "write_kib": round(write, 1),
            "copy_fetch_kib": round(fcal, 1), "copy_write_kib": round(wcal, 1)}


def want_live_counters(args, only, environ) -> bool:
    """Whether this run measures the scale-add kernel's traffic itself: only
    when it times that kernel over the whole buffer, was not told not to, and
    is not itself under rocprofv3 (which sets ROCPROF_OUTPUT_PATH for the
    program it runs, and does not nest)."""
    if args.per_rank_only or args.no_live_counters or (only and "scale_add" not in only):
        return False
    if "ROCPROF_OUTPUT_PATH" in environ:
        log("live counters: skipped under rocprofv3")
        return False
    return True


def counter_pass(args):
    """The child of live_counters: two whole-buffer scale-add launches and a
    plain 1 GiB device copy (torch), nothing else."""
    import torch

    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream(dev)
    g = Group(args.workload, args.align, args.chunk, dev, stream)
    for _ in range(2):
        g.ranged["scale_add"](0, g.m)
    a = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    g.close()


def host_info():
    """Host CPU model (from /proc/cpuinfo, no subprocess), logical CPUs and
    the CPUs this process may run on."""
    model = platform.machine()
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"cpu_model": model, "cpu_count": os.cpu_count(), "usable_cpus": usable}


def cpu_baseline(w, offs, S, inp, k1, align, min_seconds=10.0):
    """The oracle, as it stands, on ranks [0, k1) of the same workload:
    whole passes of all six operations, repeated until min_seconds; and the
    oracle's planner on the whole group."""
    from oracle import ops as O
    from oracle import plan as P

    items = P.items_from_specs(w.tensors)
    t0 = time.perf_counter()
    P.plan(items, w.m, align)
    plan_s = time.perf_counter() - t0
    total = w.m * S
    m = w.m
    y0 = np.zeros(total, np.float32)
    x0 = np.zeros(total, np.float32)
    for g, l in zip(inp.grads, offs):
        y0[l:l + g.size] = g.reshape(-1)
        x0[l:l + g.size] = g.reshape(-1)
    nt = O.num_tiles(w.tensors)
    shapes = [(s.rows, s.cols) for s in w.tensors]

    def one_pass():
        buf = O.pack(inp.params, offs, S, m, np.zeros(total, np.uint16), "bf16", 0, k1)
        O.unpack(buf, shapes, offs, S, m, [np.zeros(s.numel, np.uint16) for s in w.tensors],
                 "bf16", 0, k1)
        y, _ = O.scale_add(y0, x0, 1.0, 1.0, items, offs, S, m, 0, k1)
        O.sqnorm(y, items, offs, S, m, 0, k1)
        O.block_quant(y, w.tensors, offs, S, m, w.qfmt, 0, k1, np.zeros(total, np.uint8),
                      np.zeros(nt, np.float32))
        O.zero(x0, items, offs, S, m, 0, k1)

    passes, t0 = 0, time.perf_counter()
    while True:
        one_pass()
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or passes >= 8:
            break
    # algorithmic bytes of the sample: the ranks' share of every operation
    E_in = sum(max(0, min(l + it.numel, k1 * S) - l) for it, l in zip(items, offs))
    eq_in = sum(max(0, min(l + t.numel, k1 * S) - l) for t, l in zip(w.tensors, offs) if t.q_rows)
    b = (4 * E_in + 2 * k1 * S) + 4 * E_in + 12 * E_in + 4 * E_in + 5 * eq_in + 4 * k1 * S
    hi = host_info()
    return {"value": round(b * passes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"ranks [0,{k1}) of {m} ({k1 * S} buffer positions): {passes} passes of all "
                      f"six operations in {dt:.1f} s, numpy on one host core",
            "host_cpu": hi["cpu_model"], "host_cpus": hi["cpu_count"],
            "host_usable_cpus": hi["usable_cpus"],
            "planner_ms": round(plan_s * 1e3, 2)}


STUDY_MS = (8, 16, 32, 64, 128, 256, 512, 1024)
STUDY_ROWS = (1, 16, 128)


def padding_study(align: int, out_path: str = "") -> None:
    """Planner-only study (host, no GPU): padding % = (m*S - E)/E of each
    group with every matrix at 1-, 16- and 128-row granules over FSDP sizes
    m, for the given tensor order and the best of the three orders, with
    the planner's wall time (the pages' study: veScale-FSDP, section 6.4 and
    "Planning Algorithm").  Prints a markdown table per group; with out_path
    also writes one JSON line per plan."""
    import fsdp_sharded_buffer_amd as R
    import workloads as W

    groups = {n: W.WORKLOADS[n].tensors
              for n in ("llama3_8b_layer", "llama70b_layer", "ragged_mixed", "moe_experts")}
    groups["moe_experts_fused"] = W.fused_experts(W.WORKLOADS["moe_experts"]).tensors
    recs = []
    for name, specs in groups.items():
        E = sum(s.numel for s in specs)
        print(f"\n{name} (E = {E}, A = {align}): padding % given order / best order "
              f"[planner ms, all orders]\n")
        print("| rows | " + " | ".join(f"m={m}" for m in STUDY_MS) + " |")
        print("|---|" + "---|" * len(STUDY_MS))
        for rows in STUDY_ROWS:
            sp = W.regranulated(specs, rows)
            gmax = max(s.gran_rows * s.cols for s in sp if s.gran_rows)
            cells = []
            for m in STUDY_MS:
                res = {}
                t0 = time.perf_counter()
                for k in ("given", "block", "shape"):
                    perm, _, info = R.rs_plan_ordered(sp, m, align, k)
                    res[k] = info
                    recs.append({"group": name, "rows": rows, "m": m, "align": align, "order": k,
                                 "S": info["S"], "pad_frac": info["pad_frac"],
                                 "lower_bound": info["lower_bound"], "seconds": info["seconds"],
                                 "max_granule": gmax})
                ms = (time.perf_counter() - t0) * 1e3
                g = res["given"]["pad_frac"] * 100
                b = min(r["pad_frac"] for r in res.values()) * 100
                mark = "" if -(-E // m) >= gmax else "*"
                cells.append(f"{g:.2f}/{b:.2f}{mark} [{ms:.0f}]")
            print(f"| {rows} | " + " | ".join(cells) + " |", flush=True)
    print("\n* E/m is below the largest granule: some rank holds less than one granule of "
          "data, so S >= granule forces padding.")
    if out_path:
        with open(out_path, "w") as f:
            for r in recs:
                f.write(json.dumps(r) + "\n")


# Practical HBM ceilings: plain 128-bit streaming kernels (include/hbm_ceiling.h)
# for each read:write mix, and the mix each operation moves.
CEILING_LIB = os.path.join(ROOT, "fsdp_sharded_buffer_amd", "libhbm_ceiling.so")
CEILING_KINDS = {   # name: (kind, bytes per fp32 (or u8) element)
    "read": (0, 4), "write": (1, 4), "copy": (2, 8), "axpby_inplace": (3, 12), "axpby": (4, 12),
    "f32_to_bf16": (5, 6), "f32_to_u8": (6, 5), "u8_to_f32": (7, 5)}
OP_MIX = {"pack": "f32_to_bf16", "unpack": "copy", "scale_add": "axpby_inplace", "sqnorm": "read",
          "block_quant": "f32_to_u8", "zero": "write", "block_dequant": "u8_to_f32"}


def measure_ceilings(torch, dev, stream, event_ms, n=1 << 28, slices=1, vecs=(1, 2, 4, 8),
                     kinds=None):
    """Best GB/s of each streaming kind over n fp32 elements (vectors per
    lane, nontemporal hints, workgroup order by XCD and, for conversions,
    wide and narrow forms swept), with the variant kept.  With slices > 1, each timed call is one
    launch per slice of n elements, in turn over `slices` consecutive slices:
    one rank's share, cycled over the ranks as the per-rank launches are."""
    if not os.path.exists(CEILING_LIB):
        raise RuntimeError(f"{CEILING_LIB} is not built; run python -m fsdp_sharded_buffer_amd.build")
    lib = ctypes.CDLL(CEILING_LIB)
    lib.hc_stream.restype = ctypes.c_int
    lib.hc_stream.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                              ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    n -= n % (4096 * max(vecs))
    x = torch.empty(n * slices, dtype=torch.float32, device=dev).normal_()
    y = torch.empty_like(x).normal_()
    z = torch.empty_like(x)
    sp = stream.cuda_stream
    out = {}
    for name, (kind, per) in CEILING_KINDS.items():
        if kinds and name not in kinds:
            continue
        best = None
        forms = (0, 16) if kind >= 5 else (0,)    # conversions: wide and narrow forms
        for form, order, vec, nt in itertools.product(forms, (0, 32, 64), vecs, (0, 1)):
            def f(k=kind + form + order, vec=vec, nt=nt):
                for j in range(slices):
                    o = 4 * n * j
                    if lib.hc_stream(k, x.data_ptr() + o, y.data_ptr() + o, z.data_ptr() + o,
                                     n, vec, nt, sp):
                        raise RuntimeError("hc_stream failed")
            med, _, _ = event_ms(f, 5)
            gbs = per * n * slices / (med * 1e-3) / 1e9
            if best is None or gbs > best["GB/s"]:
                best = {"GB/s": round(gbs, 1), "vec": vec, "nt": nt,
                        "form": "narrow" if form else "wide",
                        "order": {0: "hardware", 32: "xcd runs", 64: "xcd one run"}[order]}
        out[name] = best
        log(f"ceiling {name:14s} {best['GB/s']:8.1f} GB/s ({best}, {slices} x {n} elements)")
    del x, y, z
    torch.cuda.empty_cache()
    return out


class Group:
    """One workload set up on the GPU: plan, layout, inputs and buffers, and
    every operation as a closure over a rank range [a, b)."""

    def __init__(self, name, align, chunk, dev, stream):
        import torch

        import fsdp_sharded_buffer_amd as R
        import workloads as W
        self.w = w = W.WORKLOADS[name]
        log(f"bench: {w.name} m={w.m} elements={w.numel}")
        self.offs, self.pinfo = R.rs_plan(w.tensors, w.m, align)
        S = self.S = self.pinfo["S"]
        self.lay = lay = R.Layout(w.tensors, w.m, S, self.offs, chunk)
        total, m = w.m * S, w.m
        log(f"planned S={S} pad={self.pinfo['pad_frac']*100:.2f}% in "
            f"{self.pinfo['seconds']*1e3:.1f} ms; chunks={lay.info['num_chunks']} "
            f"tiles={lay.info['num_tiles']}")
        self.inp = inp = W.make_inputs(w)
        log("inputs drawn")
        params = [torch.from_numpy(a).to(dev) for a in inp.params]
        pbuf = torch.empty(total, dtype=torch.bfloat16, device=dev)
        outs = [torch.empty(t.numel, dtype=torch.bfloat16, device=dev) for t in w.tensors]
        acc = torch.zeros(total, dtype=torch.float32, device=dev)
        grad = torch.zeros(total, dtype=torch.float32, device=dev)
        for g, l in zip(inp.grads, self.offs):
            grad[l:l + g.size].copy_(torch.from_numpy(g.reshape(-1)))
            acc[l:l + g.size].copy_(torch.from_numpy(g.reshape(-1)))
        found = torch.zeros(m, dtype=torch.int32, device=dev)
        sq = torch.empty(len(w.tensors), dtype=torch.float64, device=dev)
        codes = torch.empty(total, dtype=torch.uint8, device=dev)
        nt = lay.info["num_tiles"]
        scales = torch.empty(nt, dtype=torch.float32, device=dev)
        ptab, otab = R.ptr_table(params), R.ptr_table(outs)
        qfmt = R.RS_Q_FP8_E4M3 if w.qfmt == "fp8_e4m3" else R.RS_Q_INT8
        h, sp = lay.handle, stream.cuda_stream
        deq = torch.empty(total, dtype=torch.float32, device=dev)
        mom = torch.zeros(total, dtype=torch.float32, device=dev)
        codes2 = torch.zeros(total, dtype=torch.uint8, device=dev)
        scales2 = torch.ones(nt, dtype=torch.float32, device=dev)
        var = torch.zeros(total, dtype=torch.float32, device=dev)
        self.bufs = [params, pbuf, outs, acc, grad, found, sq, codes, scales, ptab, otab, deq, mom,
                     codes2, scales2, var]
        # the step's operations, then those measured beside it
        self.ranged = {
            "pack": lambda a, b: R.rs_pack(h, ptab, R.RS_F32, pbuf, R.RS_BF16, a, b, sp),
            "unpack": lambda a, b: R.rs_unpack(h, pbuf, R.RS_BF16, otab, R.RS_BF16, a, b, sp),
            "scale_add": lambda a, b: R.rs_group_scale_add(h, acc, grad, R.RS_F32, 1.0, 1.0, None,
                                                           found, a, b, sp),
            "sqnorm": lambda a, b: R.rs_ragged_sqnorm(h, acc, sq, None, None, lay.ws, a, b, sp),
            "block_quant": lambda a, b: R.rs_block_quant(h, acc, qfmt, codes, scales, a, b, sp),
            "zero": lambda a, b: R.rs_group_zero(h, grad, R.RS_F32, None, a, b, sp),
        }
        self.ranged_extra = {
            "block_dequant": lambda a, b: R.rs_block_dequant(h, codes, qfmt, scales, deq, R.RS_F32,
                                                             a, b, sp),
            "adamw_step": lambda a, b: R.rs_adamw_step(h, deq, acc, mom, var, 1e-4, 0.9, 0.95, 1e-8,
                                                       0.1, 0.5, 0.1, 1.0, None, None, a, b, sp),
            "sgd_step": lambda a, b: R.rs_sgd_step(h, deq, acc, mom, 1e-4, 0.9, 0.0, False, 1.0,
                                                   None, None, a, b, sp),
            "adamw8_step": lambda a, b: R.rs_adamw8_step(h, deq, acc, codes, scales, codes2,
                                                         scales2, qfmt, 1e-4, 0.9, 0.95, 1e-8, 0.1,
                                                         0.5, 0.1, 1.0, None, a, b, sp),
        }
        self.nbytes = op_bytes(w, S, nt)
        self.xbytes = extra_bytes(w, S, nt)
        self.rb = rank_bytes(w, self.offs, S)

    @property
    def m(self):
        return self.w.m

    def close(self):
        self.lay.close()
        self.bufs = self.ranged = self.ranged_extra = None


def time_per_rank(g, names, event_ms, stream, samples, graph=False):
    """Each operation on one rank's shard: launches over [k, k+1), cycling k
    so that each launch reads other memory than the last.  The mean comes
    from whole cycles timed at their ends only; the slowest rank from a pass
    with an event between launches (which adds the events' own cost).  With
    graph, the cycle is also captured once into a HIP graph and replayed
    (stream must be the current stream and not the null stream): the host
    then issues one launch per cycle, so a mean that drops says the eager
    cycle was bound by the host's launch rate."""
    import torch
    m = g.m
    allr = dict(g.ranged, **g.ranged_extra)
    res = {}
    for name in names:
        f = allr[name]
        cycle = lambda f=f: [f(k, k + 1) for k in range(m)]
        med, _, _ = event_ms(cycle, samples)
        gmed = None
        if graph:
            gr = torch.cuda.CUDAGraph()
            torch.cuda.synchronize()
            with torch.cuda.graph(gr, stream=stream):
                cycle()
            gmed, _, _ = event_ms(gr.replay, samples)
            del gr
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(m + 1)]
        times = [[] for _ in range(m)]
        for _ in range(5):
            ev[0].record(stream)
            for k in range(m):
                f(k, k + 1)
                ev[k + 1].record(stream)
            ev[m].synchronize()
            for k in range(m):
                times[k].append(ev[k].elapsed_time(ev[k + 1]))
        each = np.array([np.median(t) for t in times])
        worst = int(np.argmax(each))
        byt = sum(g.rb[k][name] for k in range(m))
        res[name] = {
            "mean_us": round(med / m * 1e3, 2),
            "GB/s": round(byt / (med * 1e-3) / 1e9, 1),
            "slowest_rank": worst, "slowest_us_with_events": round(float(each[worst]) * 1e3, 2),
            "slowest_GB/s_with_events": round(g.rb[worst][name] / (each[worst] * 1e-3) / 1e9, 1)}
        if gmed is not None:
            res[name]["graph_mean_us"] = round(gmed / m * 1e3, 2)
            res[name]["graph_GB/s"] = round(byt / (gmed * 1e-3) / 1e9, 1)
        log(f"per rank {g.w.name} {name:12s} mean {med / m * 1e3:8.1f} us  "
            f"{res[name]['GB/s']:8.1f} GB/s; slowest rank {worst}" +
            (f"; graph {gmed / m * 1e3:8.1f} us" if gmed is not None else ""))
    return res


def event_timer(torch, stream):
    def event_ms(f, n_samples):
        """Median ms per call, HIP events on the launch stream, each sample
        at least ~20 ms of back-to-back calls; also the samples and reps."""
        for _ in range(3):
            f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        f()
        e1.record(stream)
        torch.cuda.synchronize()
        one = max(e0.elapsed_time(e1), 1e-3)
        reps = max(1, int(20.0 / one))
        samples = []
        for _ in range(n_samples):
            e0.record(stream)
            for _ in range(reps):
                f()
            e1.record(stream)
            e1.synchronize()
            samples.append(e0.elapsed_time(e1) / reps)
        return float(np.median(samples)), samples, reps
    return event_ms


def time_whole(g, names, event_ms, samples):
    """Median launch time of each operation over the whole buffer."""
    allops = dict(g.ranged, **g.ranged_extra)
    allbytes = dict(g.nbytes, **g.xbytes)
    out = {}
    for name in names:
        f = allops[name]
        med, smp, reps = event_ms(lambda f=f: f(0, g.m), samples)
        gbs = allbytes[name] / (med * 1e-3) / 1e9
        out[name] = {"us": round(med * 1e3, 2), "min_us": round(min(smp) * 1e3, 2),
                     "p90_us": round(float(np.percentile(smp, 90)) * 1e3, 2),
                     "bytes": allbytes[name], "GB/s": round(gbs, 1),
                     "frac_peak": round(gbs / HBM_PEAK_GBS, 4), "reps": reps}
        log(f"{g.w.name} {name:12s} {med*1e3:9.1f} us  {gbs:8.1f} GB/s  "
            f"{gbs/HBM_PEAK_GBS*100:5.1f}% of peak")
    return out


def with_ceiling(res, ceil):
    """Adds each operation's fraction of its read:write mix's ceiling."""
    if ceil:
        for name, r in res.items():
            mix = OP_MIX.get(name)
            if mix and mix in ceil:
                r["ceiling_mix"] = mix
                r["frac_of_ceiling"] = round(r["GB/s"] / ceil[mix]["GB/s"], 4)
    return res


def rank_ceilings(torch, dev, stream, event_ms, g):
    """The streaming kinds the operations map to, timed on one rank's share
    (S elements) cycled over the m rank slices: the practical ceiling at the
    per-rank launch size, fixed launch costs included."""
    out = measure_ceilings(torch, dev, stream, event_ms, n=g.S, slices=g.m, vecs=(1, 2),
                           kinds=set(OP_MIX.values()) - {"copy"})
    # unpack moves bf16: a copy of S/2 fp32 elements moves the same bytes
    out.update(measure_ceilings(torch, dev, stream, event_ms, n=g.S // 2, slices=g.m, vecs=(1, 2),
                                kinds={"copy"}))
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama3_8b_layer")
    ap.add_argument("--align", type=int, default=16)
    ap.add_argument("--chunk", type=int, default=0)
    ap.add_argument("--samples", type=int, default=15)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-ranks", type=int, default=0)
    ap.add_argument("--only", default="", help="comma list of ops to time per op (default all)")
    ap.add_argument("--no-live-counters", action="store_true",
                    help="skip measuring the scale-add kernel's HBM traffic with two short "
                         "rocprofv3 counter passes (the committed profile is read instead)")
    ap.add_argument("--counter-pass", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (torch) to scale HBM counters")
    ap.add_argument("--per-rank", action="store_true", default=True,
                    help="also time each operation on one rank's shard, cycling over the ranks "
                         "(default)")
    ap.add_argument("--no-per-rank", dest="per_rank", action="store_false")
    ap.add_argument("--per-rank-only", action="store_true",
                    help="only the per-rank cycles (for tracing them): no step, no whole-buffer "
                         "timings, no extras")
    ap.add_argument("--per-rank-graph", action="store_true",
                    help="run on a side stream and also time each per-rank cycle replayed from a "
                         "HIP graph (per_rank[op].graph_mean_us)")
    ap.add_argument("--no-torch-ref", action="store_true",
                    help="skip timing torch's own copy/axpy/fill/fused optimizers for context")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the plain streaming kernels that give each mix's HBM ceiling")
    ap.add_argument("--no-70b", action="store_true",
                    help="skip the Llama-70B-layer measurements beside the default group")
    ap.add_argument("--records", default="",
                    help="write one JSON record per (group, operation, range) to this file")
    ap.add_argument("--padding-study", action="store_true",
                    help="planner-only padding study over granularity and FSDP size (no GPU)")
    ap.add_argument("--study-out", default="", help="JSON lines of the padding study")
    args = ap.parse_args()
    if args.padding_study:
        padding_study(args.align if "--align" in sys.argv else 1, args.study_out)
        return
    if args.counter_pass:
        counter_pass(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the m virtual ranks are slices of one device buffer "
              "and this library has no multi-GPU path; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    # The counter passes run before this process touches the GPU, so the
    # profiler they start (which replaces itself with the program it
    # profiles) descends from a process without GPU state.
    only = [o for o in args.only.split(",") if o]
    live = None
    if want_live_counters(args, only, os.environ):
        live = live_counters(args.workload, args.align, args.chunk)

    import torch

    dev = torch.device("cuda", 0)
    if args.per_rank_graph:  # graphs are captured on a stream of their own, not the null stream
        torch.cuda.set_stream(torch.cuda.Stream(dev))
    stream = torch.cuda.current_stream(dev)
    event_ms = event_timer(torch, stream)
    records = []

    def record(group, op, rng, r, unit_key="GB/s"):
        rec = {"group": group, "op": op, "range": rng}
        rec.update({k: v for k, v in r.items()})
        records.append(rec)

    g = Group(args.workload, args.align, args.chunk, dev, stream)
    w, m, S = g.w, g.m, g.S
    step_names = list(g.ranged)
    extra_names = list(g.ranged_extra)

    value = ms_step = None
    step_bytes = sum(g.nbytes.values())
    per_op, per_extra = {}, {}
    if not args.per_rank_only:
        def step():
            for f in g.ranged.values():
                f(0, m)

        # whole-step throughput: K steps between two synchronisations
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        ms_step = dt / args.steps * 1e3
        value = step_bytes * args.steps / dt / 1e9
        log(f"step: {ms_step:.3f} ms, {value:.1f} GB/s")

        if args.calibrate_copy:
            # a plain copy of known size: its FETCH_SIZE / WRITE_SIZE
            # readings turn counter values into bytes
            a = torch.empty(1 << 28, dtype=torch.float32, device=dev)
            b = torch.empty_like(a)
            for _ in range(3):
                b.copy_(a)
            torch.cuda.synchronize()
            del a, b

        res = time_whole(g, only or (step_names + extra_names), event_ms, args.samples)
        per_op = {k: v for k, v in res.items() if k in g.ranged}
        per_extra = {k: v for k, v in res.items() if k in g.ranged_extra}

    per_rank = None
    if args.per_rank or args.per_rank_only:
        per_rank = time_per_rank(g, step_names + extra_names, event_ms, stream, args.samples,
                                 graph=args.per_rank_graph)
        if not args.no_ceiling and not args.per_rank_only:
            per_rank["ceilings_at_rank_size"] = rank_ceilings(torch, dev, stream, event_ms, g)
            with_ceiling({k: v for k, v in per_rank.items() if k in OP_MIX},
                         per_rank["ceilings_at_rank_size"])

    ceil = None
    if not args.no_ceiling and not args.per_rank_only:
        ceil = measure_ceilings(torch, dev, stream, event_ms)
    with_ceiling(per_op, ceil)
    with_ceiling(per_extra, ceil)
    for name, r in dict(per_op, **per_extra).items():
        record(w.name, name, "all ranks", r)
    for name, r in (per_rank or {}).items():
        if name in OP_MIX or name in g.ranged_extra:
            record(w.name, name, "one rank (cycled)", r)

    roof = None
    timed = dict(per_op, **per_extra)
    if timed:
        dom = "scale_add" if "scale_add" in timed else next(iter(timed))
        allbytes = dict(g.nbytes, **g.xbytes)
        # the dominant kernel as rocprofv3 names it (template argument 0: x in fp32)
        traffic, source = None, None
        if dom == "scale_add":
            if live:
                traffic, source = live["traffic_bytes"], dict(live, kind="rocprofv3 in this run")
            else:
                traffic = read_counters(w.name)
                if traffic is not None:
                    source = {"kind": f"profiles/counters_scale_add_{w.name}.json, same kernel source"}
        roof = {"kernel": "scale_add_kernel<0>" if dom == "scale_add" else dom,
                "bound": "hbm", "achieved": timed[dom]["GB/s"], "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": timed[dom]["frac_peak"], "traffic": traffic,
                "traffic_source": source,
                "bytes_per_launch": allbytes[dom], "avg_launch_us": timed[dom]["us"]}
        if ceil and dom in OP_MIX:
            c = ceil[OP_MIX[dom]]
            roof["ceiling"] = {"kernel": f"hbm_ceiling {OP_MIX[dom]}", "GB/s": c["GB/s"],
                               "frac": round(timed[dom]["GB/s"] / c["GB/s"], 4)}

    # the Llama-70B layer beside the default group: one rank's share of every
    # operation (the operating point of one of its 128 ranks) and the
    # whole-buffer bf16 pack / unpack and FP8 quantisation
    c70 = None
    if args.workload == "llama3_8b_layer" and not args.no_70b and not args.per_rank_only:
        keep_c2 = g
        g = None
        g5 = Group("llama70b_layer", args.align, args.chunk, dev, stream)
        full = with_ceiling(time_whole(g5, ["pack", "unpack", "block_quant"], event_ms,
                                       min(args.samples, 7)), ceil)
        pr5 = time_per_rank(g5, step_names + extra_names, event_ms, stream, min(args.samples, 7),
                            graph=args.per_rank_graph)
        if not args.no_ceiling:
            pr5["ceilings_at_rank_size"] = rank_ceilings(torch, dev, stream, event_ms, g5)
            with_ceiling({k: v for k, v in pr5.items() if k in OP_MIX}, pr5["ceilings_at_rank_size"])
        for name, r in full.items():
            record(g5.w.name, name, "all ranks", r)
        for name, r in pr5.items():
            if name != "ceilings_at_rank_size":
                record(g5.w.name, name, "one rank (cycled)", r)
        c70 = {"workload": f"{g5.w.name}: {g5.w.description}", "elements": g5.w.numel,
               "m": g5.m, "S": g5.S, "whole_buffer": full, "per_rank": pr5}
        g5.close()
        del g5
        torch.cuda.empty_cache()
        g = keep_c2

    # torch's own kernels on one contiguous tensor, same box, same timing:
    # context for the grouped kernels' rates (not a target)
    ref = None
    if not args.no_torch_ref and not args.per_rank_only:
        n = 1 << 28
        a = torch.empty(n, dtype=torch.float32, device=dev).normal_()
        b = torch.empty_like(a).normal_()
        ref = {}
        med, _, _ = event_ms(lambda: b.copy_(a), 5)
        ref["copy_1GiB"] = round(8 * n / (med * 1e-3) / 1e9, 1)
        med, _, _ = event_ms(lambda: b.add_(a, alpha=0.5), 5)
        ref["axpy_inplace_1GiB"] = round(12 * n / (med * 1e-3) / 1e9, 1)
        med, _, _ = event_ms(lambda: b.zero_(), 5)
        ref["fill_1GiB"] = round(4 * n / (med * 1e-3) / 1e9, 1)
        del a, b
        k = 1 << 26
        prm = torch.nn.Parameter(torch.randn(k, device=dev) * 0.02)
        prm.grad = torch.randn(k, device=dev) * 1e-3
        opt = torch.optim.AdamW([prm], lr=1e-4, fused=True)
        med, _, _ = event_ms(opt.step, 5)
        ref["fused_adamw_64M"] = round(28 * k / (med * 1e-3) / 1e9, 1)
        opt = torch.optim.SGD([prm], lr=1e-4, momentum=0.9, fused=True)
        med, _, _ = event_ms(opt.step, 5)
        ref["fused_sgd_64M"] = round(20 * k / (med * 1e-3) / 1e9, 1)
        del prm, opt
        if args.per_rank:
            # one rank's share (S contiguous fp32 elements), cycling over m
            # slices of one buffer as the per-rank launches do: context for
            # the fixed per-launch costs at that size
            A = torch.empty((m, S), dtype=torch.float32, device=dev).normal_()
            B = torch.empty_like(A).normal_()
            share = {"elements": S}
            for name, f, per in (("copy", lambda k: B[k].copy_(A[k]), 8),
                                 ("axpy_inplace", lambda k: B[k].add_(A[k], alpha=0.5), 12),
                                 ("fill", lambda k: B[k].zero_(), 4),
                                 ("l2_norm", lambda k: torch.linalg.vector_norm(A[k]), 4)):
                med, _, _ = event_ms(lambda f=f: [f(k) for k in range(m)], 5)
                share[name] = round(per * S * m / (med * 1e-3) / 1e9, 1)
            ref["rank_share"] = share
            del A, B
        ref["unit"] = "GB/s"
        log(f"torch reference: {ref}")

    cpu = None
    if not args.no_cpu_baseline and not args.per_rank_only:
        k1 = args.cpu_ranks or m
        log(f"cpu baseline: oracle on ranks [0,{k1})")
        cpu = cpu_baseline(w, g.offs, S, g.inp, k1, args.align)
        log(f"cpu baseline {cpu['value']} GB/s ({cpu['sample']})")

    out = {
        "metric": METRIC, "value": None if value is None else round(value, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": None if ms_step is None else round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.description}", "elements": w.numel, "m": m, "S": S,
                   "align": args.align, "chunk_elems": g.lay.info["chunk_elems"],
                   "qfmt": w.qfmt, "step_bytes": step_bytes,
                   "planner_ms": round(g.pinfo["seconds"] * 1e3, 3),
                   "pad_frac": round(g.pinfo["pad_frac"], 5)},
        "frac_peak": None if value is None else round(value / HBM_PEAK_GBS, 4),
        "ops": per_op,
        "next_ops": per_extra,
        "roofline": roof,
        "cpu_baseline": cpu,
        "ceilings": ceil,
        "torch_reference": ref,
        "per_rank": per_rank,
        "configs": {"llama70b_layer": c70} if c70 else None,
        "device": torch.cuda.get_device_name(0),
        "host": host_info(),
    }
    if args.records:
        with open(args.records, "w") as f:
            for r in records:
                f.write(json.dumps(r) + "\n")
    # release everything before the line is printed, so nothing of this
    # process is left running once it has been read
    g.close()
    del g
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
