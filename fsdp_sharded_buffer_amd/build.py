"""Build librs.so (C-ABI planner + gfx950 HIP kernels) in-tree with hipcc.

Usage: python -m fsdp_sharded_buffer_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "librs.so")

ARCH = os.environ.get("RS_OFFLOAD_ARCH", "gfx950")

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-ffp-contract=off", "-I", INCLUDE, "-I", CSRC]
# Packed fp32 instructions are disabled for all device code; hipcc forms
# them from ordinary float code otherwise.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fno-gpu-rdc"]

SOURCES = ["rs_plan.cpp", "rs_layout.cpp", "rs_kernels.hip"]


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found; ROCm is required to build librs.so")
    return p


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), "-c"] + (["-x", "hip"] + DEVICE if src.endswith(".hip") else [])
    cmd += [os.path.join(CSRC, src), "-o", obj] + COMMON
    subprocess.run(cmd, check=True)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    subprocess.run([hipcc(), "-shared", "-fPIC", "-pthread", f"--offload-arch={ARCH}", "-o", tmp]
                   + objs, check=True)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


CEILING_SRC = os.path.join(CSRC, "hbm_ceiling.hip")
CEILING_LIB = os.path.join(PKG, "libhbm_ceiling.so")


def build_ceiling(verbose: bool = True) -> str:
    """Measurement-only streaming kernels (include/hbm_ceiling.h) that
    bench.py times as the practical HBM ceiling of each read:write mix."""
    tmp = CEILING_LIB + ".tmp"
    subprocess.run([hipcc(), "-x", "hip"] + DEVICE + [CEILING_SRC, "-shared", "-fPIC", "-o", tmp]
                   + COMMON, check=True)
    os.replace(tmp, CEILING_LIB)
    if verbose:
        print(f"built {CEILING_LIB}")
    return CEILING_LIB


PROBE_SRC = os.path.join(ROOT, "tests", "native", "hw_probes.hip")
PROBE_LIB = os.path.join(ROOT, "tests", "native", "libhw_probes.so")


def build_probe(verbose: bool = True) -> str:
    """Test-only probe of the FP8 conversion instruction (tests/native)."""
    tmp = PROBE_LIB + ".tmp"
    subprocess.run([hipcc(), "-x", "hip"] + DEVICE + [PROBE_SRC, "-shared", "-fPIC", "-o", tmp]
                   + COMMON, check=True)
    os.replace(tmp, PROBE_LIB)
    if verbose:
        print(f"built {PROBE_LIB}")
    return PROBE_LIB


DEMO_SRC = os.path.join(ROOT, "tests", "native", "capi_demo.cpp")
DEMO_EXE = os.path.join(ROOT, "tests", "native", "capi_demo")


def build_capi_demo(verbose: bool = True) -> str:
    """Test-only C++ program that drives librs.so through include/rs.h with
    no Python in the process (tests/native)."""
    tmp = DEMO_EXE + ".tmp"
    subprocess.run([hipcc(), DEMO_SRC, "-O2", "-std=c++17", "-I", INCLUDE, "-L", PKG, "-lrs",
                    "-Wl,-rpath,$ORIGIN/../../fsdp_sharded_buffer_amd", "-o", tmp], check=True)
    os.replace(tmp, DEMO_EXE)
    if verbose:
        print(f"built {DEMO_EXE}")
    return DEMO_EXE


if __name__ == "__main__":
    build()
    build_ceiling()
    build_probe()
    build_capi_demo()
    sys.exit(0)
