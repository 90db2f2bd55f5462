"""The host half of the library (planner and layout builder) under
AddressSanitizer and UndefinedBehaviorSanitizer: tests/native/host_fuzz.cpp
is compiled with both (host code only) together with rs_plan.cpp and
rs_layout.cpp, and fed random and hostile specs, ranks and offsets.  Any
memory error or undefined behaviour aborts the program.  CPU only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "fsdp_sharded_buffer_amd", "csrc")


@pytest.mark.timeout(600)
def test_planner_and_layout_builder_under_asan_ubsan(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not found")
    exe = str(tmp_path / "host_fuzz")
    cmd = [hipcc, "-O1", "-g", "-std=c++17",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-fno-sanitize-recover=undefined",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "native", "host_fuzz.cpp"),
           os.path.join(CSRC, "rs_plan.cpp"), os.path.join(CSRC, "rs_layout.cpp"),
           "-pthread", "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True)
    env = dict(os.environ, RS_PLAN_THREADS="4", ASAN_OPTIONS="detect_leaks=1")
    r = subprocess.run([exe, "5000"], capture_output=True, text=True, timeout=500, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert "fuzz ok" in r.stdout
