"""The block quantisation fast path encodes with gfx950's fp32 -> OCP E4M3
conversion instruction.  It only ever receives finite values with
2^-6 (plus 16 ulp) <= |q| < 464; on every fp32 value of that domain, both
signs, the instruction must give the oracle's saturating round-to-nearest-
even code."""
import ctypes
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

from oracle import casts as OC

from harness import log

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(__file__), "native", "libhw_probes.so")
LO, HI = 0x3C800010, 0x43E80000     # the fast path's |q| bit-pattern domain
CHUNK = 1 << 24


@pytest.mark.timeout(900)
def test_e4m3_instruction_equals_oracle_on_fast_path_domain():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(LIB)
    lib.probe_e4m3_hw.restype = ctypes.c_int
    lib.probe_e4m3_hw.argtypes = [ctypes.c_uint32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_void_p,
                                  ctypes.c_void_p]
    out = torch.empty(CHUNK, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    jobs = []
    for sign in (0, 0x80000000):
        for first in range(LO, HI, CHUNK):
            n = min(CHUNK, HI - first)
            assert lib.probe_e4m3_hw(first, n, sign, out.data_ptr(), stream) == 0
            torch.cuda.synchronize()
            jobs.append((first, n, sign, out[:n].cpu().numpy()))
    log(f"e4m3 instruction check: {len(jobs)} chunks converted on the GPU")

    def check(job):
        first, n, sign, got = job
        bits = (np.arange(first, first + n, dtype=np.uint64).astype(np.uint32) | np.uint32(sign))
        exp = OC.e4m3fn_bits_from_f32(bits.view(np.float32))
        if not np.array_equal(got, exp):
            i = int(np.flatnonzero(got != exp)[0])
            return f"input {bits[i]:#010x}: instruction {got[i]:#04x}, oracle {exp[i]:#04x}"
        return n

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as pool:
        results = list(pool.map(check, jobs))
    bad = [r for r in results if isinstance(r, str)]
    assert not bad, bad[0]
    assert sum(results) == 2 * (HI - LO)

