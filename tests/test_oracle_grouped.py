"""Pins for the oracle's grouped (mixture-of-experts) scaled GEMM: rows
offsets[e]..offsets[e+1] of the routed activations use expert e's weights and
scales.

Pinned by an exact-rational brute force (with an empty expert), by unit-scale
int8 cases equal to numpy int64 matmuls per segment, by expert isolation
(weights of an expert without rows never matter; changing one expert changes
only its rows), and by agreement with the plain scaled GEMM for one expert.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from quantized_bit_gemm_amd import synth
from tests import _exact


def _experts(qtype, E, N, K, seed):
    qws, sws = [], []
    for e in range(E):
        w = synth.draw(seed, N, K, 10 + e, (N, K), "weight")
        qw, sw = oracle.quant_weight_per_channel(qtype, w)
        qws.append(qw)
        sws.append(sw)
    return np.stack(qws), np.stack(sws)


@pytest.mark.parametrize("qtype", ["fp8", "int8"])
def test_grouped_brute_force_with_an_empty_expert(qtype):
    ot = oracle.FP8 if qtype == "fp8" else oracle.INT8
    T, E, N, K = 5, 3, 8, 16
    offsets = [0, 2, 2, 5]
    a = synth.draw(41, N, K, 1, (T, K), "normal_outliers")
    qa, sa = oracle.quant_per_token(ot, a)
    qw, sw = _experts(ot, E, N, K, 41)
    ref, out, acc = oracle.grouped_scaled_mm(ot, qa, sa, qw, sw, offsets)
    for e in range(E):
        for m in range(offsets[e], offsets[e + 1]):
            for n in range(N):
                d = sum(_exact.dequant(qa[m, k], qtype) * _exact.dequant(qw[e, n, k], qtype)
                        for k in range(K))
                exact = Fraction(float(sa[m])) * Fraction(float(sw[e, n])) * d
                assert ref[m, n] == float(exact)
                got = (np.array([out[m, n]], np.uint16).astype(np.uint32) << 16).view(np.float32)[0]
                assert Fraction(float(got)) == _exact.bf16(exact)
                if qtype == "int8":
                    assert acc[m, n] == int(d)


def test_unit_scales_reduce_to_numpy_per_segment():
    rng = np.random.default_rng(42)
    T, E, N, K = 11, 4, 24, 64
    offsets = np.array([0, 3, 3, 10, 11])
    qa = rng.integers(-127, 128, (T, K)).astype(np.int8)
    qw = rng.integers(-127, 128, (E, N, K)).astype(np.int8)
    _, _, acc = oracle.grouped_scaled_mm(oracle.INT8, qa, np.ones(T, np.float32), qw,
                                         np.ones((E, N), np.float32), offsets)
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        want = qa[lo:hi].astype(np.int64) @ qw[e].astype(np.int64).T
        assert np.array_equal(acc[lo:hi].astype(np.int64), want)


def test_expert_isolation():
    T, E, N, K = 6, 4, 16, 32
    offsets = [0, 1, 1, 4, 6]
    a = synth.draw(43, N, K, 1, (T, K), "normal")
    qa, sa = oracle.quant_per_token(oracle.FP8, a)
    qw, sw = _experts(oracle.FP8, E, N, K, 43)
    ref, _, _ = oracle.grouped_scaled_mm(oracle.FP8, qa, sa, qw, sw, offsets)
    qw2, sw2 = qw.copy(), sw.copy()
    qw2[1] = 0x38  # expert 1 has no rows
    sw2[1] = 3.0
    ref2, _, _ = oracle.grouped_scaled_mm(oracle.FP8, qa, sa, qw2, sw2, offsets)
    assert np.array_equal(ref, ref2)
    qw3 = qw.copy()
    qw3[2] = qw[0]  # expert 2 owns rows 1..3 only
    ref3, _, _ = oracle.grouped_scaled_mm(oracle.FP8, qa, sa, qw3, sw, offsets)
    assert np.array_equal(ref3[[0, 4, 5]], ref[[0, 4, 5]])
    assert not np.array_equal(ref3[1:4], ref[1:4])


@pytest.mark.parametrize("qtype", [oracle.FP8, oracle.INT8])
def test_one_expert_is_the_plain_scaled_gemm(qtype):
    T, N, K = 7, 40, 48
    a = synth.draw(44, N, K, 1, (T, K), "normal_outliers")
    qa, sa = oracle.quant_per_token(qtype, a)
    qw, sw = _experts(qtype, 1, N, K, 44)
    ref, out, _ = oracle.grouped_scaled_mm(qtype, qa, sa, qw, sw, [0, T])
    ref1, out1, _ = oracle.scaled_mm(qtype, qa, sa, qw[0], sw[0])
    assert np.array_equal(ref, ref1) and np.array_equal(out, out1)
