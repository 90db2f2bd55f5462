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



def _random_f32(rng, n):
    """Random finite fp32 values over the whole range: uniform bit patterns
    (subnormals included), NaN/Inf patterns replaced."""
    u = rng.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32)
    u = np.where((u & 0x7F800000) == 0x7F800000, u & 0x807FFFFF, u)
    return u.view(np.float32)


@pytest.mark.timeout(900)
def test_division_and_sqrt_are_correctly_rounded():
    """The device's fp32 x / y and sqrtf, compiled as the kernels compile
    them, bit-equal to NumPy's IEEE float32 division and square root on
    10^8 seeded pairs over the whole range, subnormals included (NaN results
    compare by class)."""
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib = ctypes.CDLL(LIB)
    lib.probe_div_sqrt.restype = ctypes.c_int
    lib.probe_div_sqrt.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.c_void_p]
    rng = np.random.default_rng(71)
    n = 1 << 24
    stream = torch.cuda.current_stream().cuda_stream
    for it in range(6):
        log(f"div/sqrt batch {it}")
        x = _random_f32(rng, n)
        y = _random_f32(rng, n)
        if it == 0:                         # near-equal magnitudes and tiny quotients too
            y[: n // 2] = (x[: n // 2] * np.float32(1.0000001)).astype(np.float32)
        dx, dy = torch.from_numpy(x).cuda(), torch.from_numpy(y).cuda()
        q = torch.empty_like(dx)
        r = torch.empty_like(dx)
        assert lib.probe_div_sqrt(dx.data_ptr(), dy.data_ptr(), n, q.data_ptr(), r.data_ptr(), stream) == 0
        torch.cuda.synchronize()
        with np.errstate(all="ignore"):
            eq = (x / y).astype(np.float32)
            er = np.sqrt(x).astype(np.float32)
        for got, exp, what in ((q.cpu().numpy(), eq, "division"), (r.cpu().numpy(), er, "sqrt")):
            gn, en = np.isnan(got), np.isnan(exp)
            assert np.array_equal(gn, en), what + ": NaN positions differ"
            bad = (got.view(np.uint32) != exp.view(np.uint32)) & ~gn
            assert not bad.any(), f"{what}: {int(bad.sum())} results differ, e.g. x={x[bad][0]!r}"
