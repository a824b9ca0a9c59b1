"""Pins for the oracle's codecs: E4M3, int8, UE8M0 and bf16.

Each codec is checked against something other than itself: hand-derived
cases from the format definitions (tests/golden), an independent library
(torch's CPU float8_e4m3fn and bfloat16 casts, numpy's rint), and exact
rational arithmetic.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests import _exact, _golden


def test_e4m3_decode_all_codes_match_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    lib_vals = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        got = oracle.e4m3_decode(c)
        if c in (0x7F, 0xFF):
            assert math.isnan(got)
            continue
        assert got == lib_vals[c], (hex(c), got, lib_vals[c])
        assert math.copysign(1.0, got) == math.copysign(1.0, lib_vals[c])


def test_e4m3_decode_all_codes_match_exact_definition():
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert Fraction(oracle.e4m3_decode(c)) == _exact.e4m3_value(c)


def test_e4m3_extremes():
    assert oracle.e4m3_decode(0x7E) == 448.0
    assert oracle.e4m3_decode(0x08) == 2.0 ** -6
    assert oracle.e4m3_decode(0x01) == 2.0 ** -9
    assert oracle.e4m3_decode(0x80) == 0.0 and math.copysign(1, oracle.e4m3_decode(0x80)) < 0


def test_e4m3_roundtrip_every_code():
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert oracle.e4m3_encode(oracle.e4m3_decode(c)) == c, hex(c)


def test_e4m3_golden_cases():
    for key, val in _golden.read("e4m3_codec.txt"):
        x = float(key)
        assert oracle.e4m3_encode(x) == int(val[0], 16), (key, hex(oracle.e4m3_encode(x)))


def test_e4m3_every_midpoint_ties_to_even():
    for c in range(0x7E):
        lo, hi = oracle.e4m3_decode(c), oracle.e4m3_decode(c + 1)
        mid = (lo + hi) / 2  # exact in fp32 for adjacent E4M3 values
        assert np.float32(mid) == mid
        even = c if c % 2 == 0 else c + 1
        assert oracle.e4m3_encode(mid) == even
        assert oracle.e4m3_encode(-mid) == even | 0x80
        below = float(np.nextafter(np.float32(mid), np.float32(0)))
        above = float(np.nextafter(np.float32(mid), np.float32(1000)))
        assert oracle.e4m3_encode(below) == c
        assert oracle.e4m3_encode(above) == c + 1


def test_e4m3_encode_matches_torch_on_random_fp32():
    rng = np.random.default_rng(7)
    n = 20000
    mant = rng.random(n, dtype=np.float32) + np.float32(1.0)
    expo = rng.integers(-12, 9, n)
    sign = np.where(rng.random(n) < 0.5, -1.0, 1.0)
    x = (sign * np.ldexp(mant.astype(np.float64), expo)).astype(np.float32)
    x = np.clip(x, -448, 448)
    lib_codes = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for i in range(n):
        assert oracle.e4m3_encode(float(x[i])) == lib_codes[i], (x[i], lib_codes[i])


def test_e4m3_encode_matches_exhaustive_search():
    rng = np.random.default_rng(8)
    for v in rng.uniform(-448, 448, 300).astype(np.float32):
        assert oracle.e4m3_encode(float(v)) == _exact.e4m3_encode(Fraction(float(v)))
    for v in (rng.uniform(-1, 1, 300) * 2.0 ** -6).astype(np.float32):  # subnormal range
        assert oracle.e4m3_encode(float(v)) == _exact.e4m3_encode(Fraction(float(v)),
                                                                  negative_zero=v < 0)


def test_int8_golden_cases():
    for key, val in _golden.read("int8_codec.txt"):
        assert oracle.i8_encode(float(key)) == int(val[0]), key


def test_int8_matches_numpy_rint():
    rng = np.random.default_rng(9)
    x = rng.uniform(-127, 127, 5000).astype(np.float32)
    x[:200] = np.round(x[:200]) + np.float32(0.5)  # exact halves
    x = np.clip(x, -127, 127)
    ref = np.rint(x.astype(np.float64)).astype(np.int64)
    for i in range(x.size):
        assert oracle.i8_encode(float(x[i])) == ref[i]


def test_ue8m0_golden_cases():
    for key, val in _golden.read("ue8m0_codec.txt"):
        s = float(np.float32(float(key)))
        if key.startswith("0.002232"):
            s = float(np.float32(1.0) / np.float32(448.0))
        assert oracle.ue8m0_encode(s) == int(val[0]), key


def test_ue8m0_is_smallest_power_of_two_not_below():
    rng = np.random.default_rng(10)
    s = np.exp2(rng.uniform(-40, 20, 3000)).astype(np.float32)
    s[:40] = np.exp2(np.arange(-20, 20)).astype(np.float32)  # exact powers
    for v in s:
        e = oracle.ue8m0_encode(float(v))
        p = oracle.ue8m0_decode(e)
        assert p == 2.0 ** (e - 127)
        assert p >= v and p / 2 < v
        assert e == _exact.ue8m0_encode(Fraction(float(v)))


def test_bf16_from_double_matches_torch_for_fp32_inputs():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal(20000) * np.exp2(rng.integers(-30, 30, 20000))).astype(np.float32)
    x[:10] = [0.0, -0.0, 1.0, -1.0, 3.0e38, 1e-40, -1e-41, 2.0 ** -133, 65504.0, 1.00390625]
    lib_bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for i in range(x.size):
        assert oracle.bf16_from_double(float(x[i])) == lib_bits[i], (x[i], hex(lib_bits[i]))


def test_bf16_rounds_once_from_double():
    # Values just above a bf16 midpoint by less than an fp32 ulp: a double -> fp32 -> bf16
    # path would see the exact midpoint and round to even; one rounding must go up.
    rng = np.random.default_rng(12)
    for _ in range(500):
        b = int(rng.integers(0x3F80, 0x4700))  # positive normal bf16, even or odd
        lo = oracle.bf16_to_double(b)
        hi = oracle.bf16_to_double(b + 1)
        mid = (lo + hi) / 2
        assert oracle.bf16_from_double(mid) == (b if b % 2 == 0 else b + 1)
        tiny = mid * 2.0 ** -40
        assert oracle.bf16_from_double(mid + tiny) == b + 1
        assert oracle.bf16_from_double(mid - tiny) == b
        assert oracle.bf16_from_double(-(mid + tiny)) == (b + 1) | 0x8000
        assert Fraction(oracle.bf16_to_double(oracle.bf16_from_double(mid + tiny))) == \
            _exact.bf16(Fraction(mid + tiny))
