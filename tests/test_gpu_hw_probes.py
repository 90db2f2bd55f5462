"""The block quantisation fast path encodes with gfx950's fp32 -> OCP E4M3
conversion instruction.  It only ever receives finite values with
|q| < 464 (the first midpoint past 448); on every fp32 value of that
domain, zeros and subnormals included, both signs, the instruction must
give the oracle's saturating round-to-nearest-even code.  The fast path
also relies on that code being monotone in |q|, which the oracle's rounding
to a grid is."""
import ctypes
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

from oracle import casts as OC

from harness import log

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(__file__), "native", "libhw_probes.so")
LO, HI = 0x00000000, 0x43E80000     # the fast path's |q| bit-pattern domain
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


def _divc_constants():
    """sqrt(1 - beta2^t) in fp32, as a caller's bias correction gives it, for
    common beta2 and steps; the ends of the accepted range; and seeded random
    normals inside it."""
    cs = []
    for beta2 in (0.95, 0.98, 0.99, 0.995, 0.999, 0.9999):
        for t in (1, 2, 3, 10, 100, 1000, 10 ** 4, 10 ** 5, 10 ** 6):
            bc2 = np.float32(1) - np.float32(beta2) ** np.float32(t)
            cs.append(np.sqrt(np.float32(bc2)).astype(np.float32))
    cs += [np.float32(2.0 ** -16), np.float32(2.0 ** 16), np.float32(1.0)]
    rng = np.random.default_rng(5)
    cs += list((2.0 ** rng.uniform(-16, 16, 12)).astype(np.float32))
    return sorted(set(float(c) for c in cs if np.float32(c) > 0))


@pytest.mark.timeout(900)
def test_division_by_a_constant_is_correctly_rounded():
    """The 8-bit AdamW step divides sqrt(v') by the per-call constant
    sqrt(bc2) with rs_exact.h's three-operation form.  For every fp32 v' (all
    2^32 bit patterns: zeros, subnormals, normals, infinities and NaNs of
    both signs) and each constant above, its quotient has the bits of the
    IEEE quotient (NaN by class)."""
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib = ctypes.CDLL(LIB)
    lib.probe_divc.restype = ctypes.c_int
    lib.probe_divc.argtypes = [ctypes.c_uint32, ctypes.c_int64, ctypes.c_float, ctypes.c_float,
                               ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    stream = torch.cuda.current_stream().cuda_stream
    for c in _divc_constants():
        cf = np.float32(c)
        r = np.float32(1) / cf                  # IEEE fp32 reciprocal, as the host computes it
        bad = torch.zeros(1, dtype=torch.int64, device="cuda")
        first = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        log(f"constant division: c = {float(cf)!r}")
        assert lib.probe_divc(0, 1 << 32, float(cf), float(r), bad.data_ptr(), first.data_ptr(),
                              stream) == 0
        torch.cuda.synchronize()
        nbad = int(bad.item())
        assert nbad == 0, (f"c = {float(cf)!r}: {nbad} quotients differ, first at input "
                           f"{int(first.item()) & 0xffffffff:#010x}")


@pytest.mark.timeout(900)
def test_square_root_is_correctly_rounded():
    """The 8-bit AdamW step takes sqrt(v') with rs_exact.h's sqrt_rn (the
    hardware root, then the neighbour chosen by exact residuals).  On all 2^32
    fp32 patterns it has the bits of the IEEE square root (NaN by class)."""
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib = ctypes.CDLL(LIB)
    lib.probe_sqrt.restype = ctypes.c_int
    lib.probe_sqrt.argtypes = [ctypes.c_uint32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                               ctypes.c_void_p]
    stream = torch.cuda.current_stream().cuda_stream
    bad = torch.zeros(1, dtype=torch.int64, device="cuda")
    first = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    log("square root: all 2^32 inputs")
    assert lib.probe_sqrt(0, 1 << 32, bad.data_ptr(), first.data_ptr(), stream) == 0
    torch.cuda.synchronize()
    nbad = int(bad.item())
    assert nbad == 0, f"{nbad} roots differ, first at input {int(first.item()) & 0xffffffff:#010x}"
