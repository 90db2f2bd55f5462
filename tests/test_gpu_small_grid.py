"""Launch shapes the small test groups never reach, forced through the
library's environment variables (read once per process) in a child pytest.

* Ranges covered by several launches.  One launch holds at most 2^31 lanes,
  so a call over more workgroups than that is split: the chunk kernels
  stride over a capped grid, and the fill, quantisation, dequantisation and
  8-bit AdamW are issued as consecutive launches.  Real groups reach that
  only past about 34 GB of fp32; RS_MAX_GRID=3 makes every call take the
  split paths, and the small-group parity and optimizer tests of five groups
  run again against the same oracle bar.
* pack, unpack, scale/add and the unmasked zero with their chunks grouped
  by XCD, which they do only on ranges of at least RS_XCD_REMAP_MIN
  elements (2^26 by default), in runs of RS_XCD_RUN chunks (128);
  RS_XCD_REMAP_MIN=1 with short runs turns it on for every parity case of
  those operations.  Dequantisation takes runs of RS_DEQ_XCD_RUN
  workgroups (16) on such ranges when its tiles mostly belong to tensors of
  at least RS_DEQ_XCD_MIN_COLS columns (8192); RS_DEQ_XCD_MIN_COLS=1 with
  the same short runs turns it on for its parity cases too.
"""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GROUPS = ("toy", "ragged_a1_c64", "bands")  # "toy" also selects toy_a1_c64, toy_chunk_max


@pytest.mark.timeout(900)
def test_parity_with_three_workgroup_grid_cap():
    if os.environ.get("RS_MAX_GRID"):
        pytest.skip("already running under a grid cap")
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    expr = "(" + " or ".join(GROUPS) + ") and not every"
    cmd = [sys.executable, "-u", "-m", "pytest", "tests/test_gpu_parity.py",
           "tests/test_gpu_optim.py", "-x", "-q", "-m", "gpu", "-k", expr, "-p",
           "no:cacheprovider", "--timeout", "300", "--timeout-method", "thread"]
    print("child:", " ".join(cmd), "with RS_MAX_GRID=3", flush=True)
    # the child's progress goes straight to this process's output
    r = subprocess.run(cmd, cwd=ROOT, env=dict(os.environ, RS_MAX_GRID="3"), timeout=840)
    assert r.returncode == 0, f"child pytest under RS_MAX_GRID=3 exited with {r.returncode}"


@pytest.mark.timeout(900)
@pytest.mark.parametrize("run,grid_cap", [("2", None), ("8", None), ("2", "5")])
def test_chunks_grouped_by_xcd(run, grid_cap):
    """Pack, unpack, scale/add and the unmasked zero group their chunks by
    XCD on long ranges (at least RS_XCD_REMAP_MIN elements): runs of
    RS_XCD_RUN consecutive chunks per XCD (one run per XCD for the zero);
    dequantisation of wide tensors takes runs of RS_DEQ_XCD_RUN workgroups.
    The small groups reach neither the threshold nor a full round of the
    default 128-chunk runs, so a child process sets RS_XCD_REMAP_MIN=1 and
    short runs (2 or 8 chunks: rounds of 16 or 64, then a partial round),
    and re-runs those operations' parity cases and the two-stream test; once
    more with the grid capped at 5 workgroups (the first item plus the
    strided loop, with a grid below one round)."""
    if any(os.environ.get(v) for v in ("RS_XCD_REMAP_MIN", "RS_XCD_RUN", "RS_MAX_GRID",
                                        "RS_DEQ_XCD_RUN", "RS_DEQ_XCD_MIN_COLS")):
        pytest.skip("already running under a launch-shape override")
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    env = dict(os.environ, RS_XCD_REMAP_MIN="1", RS_XCD_RUN=run, RS_DEQ_XCD_RUN=run,
               RS_DEQ_XCD_MIN_COLS="1")
    if grid_cap:
        env["RS_MAX_GRID"] = grid_cap
    cmd = [sys.executable, "-u", "-m", "pytest", "tests/test_gpu_parity.py", "tests/test_gpu_streams.py",
           "-x", "-q", "-m", "gpu", "-k", "pack or scale_add or zero or disjoint or dequant",
           "-p", "no:cacheprovider", "--timeout", "300", "--timeout-method", "thread"]
    print("child:", " ".join(cmd), f"with RS_XCD_REMAP_MIN=1 RS_XCD_RUN={run} RS_DEQ_XCD_RUN={run}",
          "RS_DEQ_XCD_MIN_COLS=1",
          f"RS_MAX_GRID={grid_cap}" if grid_cap else "", flush=True)
    r = subprocess.run(cmd, cwd=ROOT, env=env, timeout=840)
    assert r.returncode == 0, f"child pytest with XCD runs forced exited with {r.returncode}"
