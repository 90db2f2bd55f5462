"""Pins for the oracle's number conversions (CPU only).

Checked against hand-worked values from the format definitions
(tests/golden/casts.json) and against PyTorch's CPU casts, an independent
library implementation (bf16 and float8_e4m3fn; torch does not saturate,
so inputs are clamped to +-448 before its FP8 cast).
"""
import json
import os

import numpy as np
import torch

from oracle import casts as C

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "casts.json")))


def _f(v):
    return np.float32(float(v))


def test_bf16_golden():
    for src, dst, _ in GOLD["bf16"]:
        u = np.array([int(src, 16)], dtype=np.uint32)
        got = C.bf16_bits_from_f32(u.view(np.float32))[0]
        assert got == int(dst, 16), (src, hex(got), dst)


def _bit_sample(stride=257, extra_seed=3):
    # every stride-th bit pattern plus random ones: covers all exponents,
    # both signs and varied rounding bits
    a = np.arange(0, 2 ** 32, stride, dtype=np.uint64).astype(np.uint32)
    rng = np.random.default_rng(extra_seed)
    b = rng.integers(0, 2 ** 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    # ties: low 16 bits exactly 0x8000
    c = (rng.integers(0, 2 ** 16, size=1 << 16, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    return np.concatenate([a, b, c])


def test_bf16_matches_torch_on_bit_sample():
    u = _bit_sample()
    x = u.view(np.float32)
    ours = C.bf16_bits_from_f32(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(ours[~nan], ref[~nan])
    # NaN: quiet, sign kept (torch may pick another payload)
    assert np.all((ours[nan] & 0x7FC0) == 0x7FC0)
    assert np.array_equal(ours[nan] >> 15, (u[nan] >> 31).astype(np.uint16))


def test_bf16_roundtrip_exact():
    b = np.arange(0, 2 ** 16, dtype=np.uint32).astype(np.uint16)
    f = C.bf16_to_f32(b)
    back = C.bf16_bits_from_f32(f)
    nan = np.isnan(f)
    assert np.array_equal(back[~nan], b[~nan])


def test_e4m3_golden():
    for v, code in GOLD["e4m3fn"]:
        got = C.e4m3fn_bits_from_f32(np.array([_f(v)], dtype=np.float32))[0]
        assert got == int(code, 16), (v, hex(got), code)


def test_e4m3_matches_torch_after_clamp():
    u = _bit_sample(stride=1021)
    x = u.view(np.float32)
    ours = C.e4m3fn_bits_from_f32(x)
    xc = np.clip(x, -448.0, 448.0).astype(np.float32)
    ref = torch.from_numpy(xc.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    nan = np.isnan(x)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.all(ours[nan] == 0x7F)


def test_e4m3_all_codes_roundtrip_and_midpoints():
    codes = np.arange(256, dtype=np.uint8)
    vals = C.e4m3fn_to_f64(codes)
    ok = ~np.isnan(vals)
    back = C.e4m3fn_bits_from_f32(vals[ok].astype(np.float32))
    assert np.array_equal(back, codes[ok])
    # midpoints between consecutive positive codes round to the even code
    pos = np.arange(0, 0x7E, dtype=np.int64)
    lo, hi = C.e4m3fn_to_f64(pos), C.e4m3fn_to_f64(pos + 1)
    mid = ((lo + hi) / 2).astype(np.float32)
    assert np.array_equal(mid.astype(np.float64), (lo + hi) / 2)  # exact in fp32
    got = C.e4m3fn_bits_from_f32(mid).astype(np.int64)
    expect = np.where(pos % 2 == 0, pos, pos + 1)
    assert np.array_equal(got, expect)


def test_e4m3_saturates_and_monotone():
    x = np.linspace(-600, 600, 100001, dtype=np.float32)
    c = C.e4m3fn_bits_from_f32(x)
    v = C.e4m3fn_to_f64(c)
    assert np.all(np.abs(v) <= 448)
    assert np.all(np.diff(v) >= 0)


def test_int8_golden_and_torch():
    for v, code in GOLD["int8"]:
        got = C.int8_from_f32(np.array([_f(v)], dtype=np.float32))[0]
        assert int(got) == code, (v, got, code)
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(1 << 18) * 80).astype(np.float32)
    x[:1000] = np.round(x[:1000]) + 0.5   # exact ties
    ours = C.int8_from_f32(x).astype(np.int64)
    ref = torch.clamp(torch.round(torch.from_numpy(x)), -127, 127).to(torch.int64).numpy()
    assert np.array_equal(ours, ref)
