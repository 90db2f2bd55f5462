"""Ranges covered by several launches.  One launch holds at most 2^31 lanes,
so a call over more workgroups than that is split: the chunk kernels stride
over a capped grid, and the fill, quantisation, dequantisation and 8-bit
AdamW are issued as consecutive launches.  Real groups reach that only past
about 34 GB of fp32, so this test lowers the cap to 3 workgroups through
the library's RS_MAX_GRID variable (read once per process) and re-runs the
small-group parity and optimizer tests of five groups in a child process,
where every call then takes the split paths, against the same oracle bar.
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
