"""The C-ABI without Python: tests/native/capi_demo (C++, built by
__graft_entry__.build()) plans a group, uploads its layout, packs, unpacks
and takes norms through include/rs.h alone, checks the results on the host
and checks that an invalid rank range is rejected.  Run as a child process."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(__file__), "native", "capi_demo")


def test_capi_demo_program():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(EXE):
        raise RuntimeError(f"{EXE} is not built; run __graft_entry__.build()")
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "capi demo ok" in r.stdout, r.stdout + r.stderr
