"""Launch shapes the small test groups never reach, forced through the
library's environment variables (read once per process) in a child pytest.

* Ranges covered by several launches.  One launch holds at most 2^31 lanes,
  so a call over more workgroups than that is split: the chunk kernels
  stride over a capped grid, and the fill, quantisation, dequantisation and
  8-bit AdamW are issued as consecutive launches.  Real groups reach that
  only past about 34 GB of fp32; RS_MAX_GRID=3 makes every call take the
  split paths, and the small-group parity and optimizer tests of five groups
  run again against the same oracle bar.
* scale/add, unpack and the unmasked zero with their chunks grouped by XCD,
  which they do only on ranges of at least RS_XCD_REMAP_MIN elements (2^26
  by default); RS_XCD_REMAP_MIN=1 turns it on for every parity case of
  those operations.
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
@pytest.mark.parametrize("grid_cap", [None, "5"])
def test_chunks_grouped_by_xcd(grid_cap):
    """scale/add, unpack and the unmasked zero give each XCD a contiguous
    run of chunks on long ranges (at least RS_XCD_REMAP_MIN elements).  The
    small groups never reach the threshold, so a child process sets
    RS_XCD_REMAP_MIN=1 and re-runs those operations' parity cases (and the
    two-stream test) with the remap on: once with the normal grid and
    once with the grid capped at 5 workgroups (the remapped first item plus
    the strided loop, and a grid below 8 where the remap is the identity)."""
    if os.environ.get("RS_XCD_REMAP_MIN") or os.environ.get("RS_MAX_GRID"):
        pytest.skip("already running under a remap or grid override")
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    env = dict(os.environ, RS_XCD_REMAP_MIN="1")
    if grid_cap:
        env["RS_MAX_GRID"] = grid_cap
    cmd = [sys.executable, "-u", "-m", "pytest", "tests/test_gpu_parity.py", "tests/test_gpu_streams.py",
           "-x", "-q", "-m", "gpu", "-k", "scale_add or unpack or zero or disjoint or roundtrip",
           "-p", "no:cacheprovider", "--timeout", "300", "--timeout-method", "thread"]
    print("child:", " ".join(cmd), "with RS_XCD_REMAP_MIN=1",
          f"and RS_MAX_GRID={grid_cap}" if grid_cap else "", flush=True)
    r = subprocess.run(cmd, cwd=ROOT, env=env, timeout=840)
    assert r.returncode == 0, f"child pytest with the remap forced exited with {r.returncode}"
