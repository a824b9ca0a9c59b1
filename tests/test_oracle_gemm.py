"""Pins for the oracle's scaled GEMMs (FP8-dynamic, W8A8-INT8, Block-FP8) and
their Split-K / Swap-AB variants.

Pinned by hand-worked GEMMs (tests/golden), a special case that reduces to
numpy's integer / float matmul, an exact-rational brute force at 4x8x16 (and
4x8x256 for blocks), and the identities Split-K == unsplit and Swap-AB ==
transpose of the transposed product.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from quantized_bit_gemm_amd import synth
from tests import _exact, _golden


def bits(vals):
    return synth.to_bf16_bits(np.asarray(vals, dtype=np.float32))


def bf16_value(b):
    return oracle.bf16_to_double(int(b))


def test_worked_fp8_gemm():
    t = _golden.table("worked_fp8_gemm.txt")
    qa, sa = oracle.quant_per_token(oracle.FP8, bits([_golden.floats(t["A"])]))
    qw, sw = oracle.quant_weight_per_channel(
        oracle.FP8, bits([_golden.floats(t["W0"]), _golden.floats(t["W1"])]))
    ref, out, _ = oracle.scaled_mm(oracle.FP8, qa, sa, qw, sw)
    assert list(ref[0]) == _golden.floats(t["ref"])
    assert [bf16_value(b) for b in out[0]] == _golden.floats(t["out"])


def test_worked_int8_gemm():
    t = _golden.table("worked_int8_gemm.txt")
    qa, sa = oracle.quant_per_token(oracle.INT8, bits([_golden.floats(t["A"])]))
    qw, sw = oracle.quant_weight_per_channel(oracle.INT8, bits([_golden.floats(t["W"])]))
    ref, out, acc = oracle.scaled_mm(oracle.INT8, qa, sa, qw, sw)
    assert acc[0, 0] == int(t["acc"][0])
    assert ref[0, 0] == float(t["ref"][0])
    assert bf16_value(out[0, 0]) == float(t["out"][0])


@pytest.mark.parametrize("fmt", [oracle.SCALE_F32, oracle.SCALE_UE8M0])
def test_worked_block_gemm(fmt):
    t = _golden.table("worked_block_gemm.txt")
    a = np.array([float(t["a_value"][0])] * 128 + [float(t["a_value"][1])] * 128, np.float32)
    w = np.array([float(t["w_value"][0])] * 128 + [float(t["w_value"][1])] * 128, np.float32)
    qa, sa = oracle.quant_group(fmt, bits(a[None, :]))
    qw, sw = oracle.quant_weight_block(fmt, bits(np.tile(w, (128, 1))))
    ref, out = oracle.block_scaled_mm(fmt, qa, sa, qw, sw)
    assert np.all(ref == float(t["ref"][0]))
    assert all(bf16_value(b) == float(t["out"][0]) for b in out[0])


def test_unit_scales_reduce_to_numpy_matmul():
    rng = np.random.default_rng(21)
    M, N, K = 5, 24, 96
    # int8: any codes in [-127, 127]
    qa = rng.integers(-127, 128, (M, K)).astype(np.int8)
    qw = rng.integers(-127, 128, (N, K)).astype(np.int8)
    one_m, one_n = np.ones(M, np.float32), np.ones(N, np.float32)
    ref, _, acc = oracle.scaled_mm(oracle.INT8, qa, one_m, qw, one_n)
    want = qa.astype(np.int64) @ qw.astype(np.int64).T
    assert np.array_equal(acc.astype(np.int64), want)
    assert np.array_equal(ref, want.astype(np.float64))
    # fp8: codes decoded by torch's float8 cast, matmul in numpy fp64 (exact here)
    import torch
    ca = rng.integers(0, 256, (M, K)).astype(np.uint8)
    cw = rng.integers(0, 256, (N, K)).astype(np.uint8)
    ca[(ca & 0x7F) == 0x7F] = 0x00  # no NaN codes
    cw[(cw & 0x7F) == 0x7F] = 0x00
    da = torch.from_numpy(ca).view(torch.float8_e4m3fn).double().numpy()
    dw = torch.from_numpy(cw).view(torch.float8_e4m3fn).double().numpy()
    ref, _, _ = oracle.scaled_mm(oracle.FP8, ca, one_m, cw, one_n)
    assert np.array_equal(ref, da @ dw.T)


def test_scales_multiply_rows_and_columns():
    rng = np.random.default_rng(22)
    M, N, K = 3, 16, 64
    qa = rng.integers(-127, 128, (M, K)).astype(np.int8)
    qw = rng.integers(-127, 128, (N, K)).astype(np.int8)
    sa = np.array([2.0 ** -3, 2.0 ** 5, 0.75], np.float32)
    sw = np.exp2(rng.integers(-8, 8, N)).astype(np.float32)
    ref, _, acc = oracle.scaled_mm(oracle.INT8, qa, sa, qw, sw)
    want = (qa.astype(np.int64) @ qw.astype(np.int64).T) * sa[:, None].astype(np.float64) \
        * sw[None, :].astype(np.float64)
    assert np.array_equal(ref, want)


def _exact_gemm(qa, sa, qw, sw, qtype):
    M, K = qa.shape
    N = qw.shape[0]
    ref = [[None] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            d = sum(_exact.dequant(qa[m, k], qtype) * _exact.dequant(qw[n, k], qtype)
                    for k in range(K))
            ref[m][n] = Fraction(float(sa[m])) * Fraction(float(sw[n])) * d
    return ref


@pytest.mark.parametrize("qtype", ["fp8", "int8"])
def test_brute_force_4x8x16(qtype):
    ot = oracle.FP8 if qtype == "fp8" else oracle.INT8
    a = synth.draw(31, 8, 16, 1, (4, 16), "normal_outliers")
    w = synth.draw(31, 8, 16, 0, (8, 16), "weight")
    qa, sa = oracle.quant_per_token(ot, a)
    qw, sw = oracle.quant_weight_per_channel(ot, w)
    ref, out, acc = oracle.scaled_mm(ot, qa, sa, qw, sw)
    exact = _exact_gemm(qa, sa, qw, sw, qtype)
    for m in range(4):
        for n in range(8):
            e = exact[m][n]
            # the product of the exact sum with the exact scale product, rounded once to fp64
            assert ref[m, n] == float(e)
            assert Fraction(bf16_value(out[m, n])) == _exact.bf16(e)
            if qtype == "int8":
                assert acc[m, n] == int(e / (Fraction(float(sa[m])) * Fraction(float(sw[n]))))


@pytest.mark.parametrize("fmt", [oracle.SCALE_F32, oracle.SCALE_UE8M0])
def test_block_brute_force_4x8x256(fmt):
    a = synth.draw(32, 8, 256, 1, (4, 256), "normal")
    w = synth.draw(32, 8, 256, 0, (8, 256), "weight")
    qa, sa = oracle.quant_group(fmt, a)
    qw, sw = oracle.quant_weight_block(fmt, w)
    ref, out = oracle.block_scaled_mm(fmt, qa, sa, qw, sw)

    def sc(arr, i, j):
        v = arr[i, j]
        return Fraction(2) ** (int(v) - 127) if fmt == oracle.SCALE_UE8M0 else Fraction(float(v))

    for m in range(4):
        for n in range(8):
            terms = []
            for g in range(2):
                S = sum(_exact.e4m3_value(int(qa[m, k])) * _exact.e4m3_value(int(qw[n, k]))
                        for k in range(g * 128, (g + 1) * 128))
                terms.append(sc(sa, m, g) * sc(sw, n // 128, g) * S)
            total = sum(terms)
            # fp64 evaluation: each of the len(terms) products and sums rounds once
            bound = 2 * len(terms) * Fraction(1, 2 ** 53) * sum(abs(t) for t in terms)
            assert abs(Fraction(ref[m, n]) - total) <= bound
            assert Fraction(bf16_value(out[m, n])) == _exact.bf16(total)


@pytest.mark.parametrize("qtype", [oracle.FP8, oracle.INT8])
def test_split_k_equals_unsplit_exactly(qtype):
    M, N, K = 3, 16, 1024
    a = synth.draw(33, N, K, 1, (M, K), "normal_outliers")
    w = synth.draw(33, N, K, 0, (N, K), "weight")
    qa, sa = oracle.quant_per_token(qtype, a)
    qw, sw = oracle.quant_weight_per_channel(qtype, w)
    ref1, out1, acc1 = oracle.scaled_mm(qtype, qa, sa, qw, sw)
    for s in (2, 4, 8, 16, 32, 64, 128, 256):
        ref, out, acc = oracle.scaled_mm(qtype, qa, sa, qw, sw, split_k=s)
        assert np.array_equal(ref, ref1) and np.array_equal(out, out1)
        if acc is not None:
            assert np.array_equal(acc, acc1)


@pytest.mark.parametrize("qtype", [oracle.FP8, oracle.INT8])
def test_swap_ab_equals_standard_exactly(qtype):
    M, N, K = 5, 32, 512
    a = synth.draw(34, N, K, 1, (M, K), "student_t")
    w = synth.draw(34, N, K, 0, (N, K), "weight")
    qa, sa = oracle.quant_per_token(qtype, a)
    qw, sw = oracle.quant_weight_per_channel(qtype, w)
    ref1, out1, acc1 = oracle.scaled_mm(qtype, qa, sa, qw, sw)
    for s in (1, 4):
        ref, out, acc = oracle.scaled_mm(qtype, qa, sa, qw, sw, split_k=s, swap_ab=True)
        assert np.array_equal(ref, ref1) and np.array_equal(out, out1)
        if acc is not None:
            assert np.array_equal(acc, acc1)


@pytest.mark.parametrize("fmt", [oracle.SCALE_F32, oracle.SCALE_UE8M0])
def test_block_split_k_and_swap_ab(fmt):
    M, N, K = 3, 256, 1024
    a = synth.draw(35, N, K, 1, (M, K), "normal")
    w = synth.draw(35, N, K, 0, (N, K), "weight")
    qa, sa = oracle.quant_group(fmt, a)
    qw, sw = oracle.quant_weight_block(fmt, w)
    ref1, out1 = oracle.block_scaled_mm(fmt, qa, sa, qw, sw)
    for s in (1, 2, 4, 8):
        for swap in (False, True):
            ref, out = oracle.block_scaled_mm(fmt, qa, sa, qw, sw, split_k=s, swap_ab=swap)
            # re-association of fp64 sums of inexact products: a few ulps at most
            assert np.allclose(ref, ref1, rtol=1e-13, atol=0)
            if s == 1:
                assert np.array_equal(ref, ref1)


def test_int8_accumulator_overflow_is_reported():
    K = 140000  # 127*127*K > 2^31
    qa = np.full((1, K), 127, np.int8)
    qw = np.full((1, K), 127, np.int8)
    one = np.ones(1, np.float32)
    with pytest.raises(OverflowError):
        oracle.scaled_mm(oracle.INT8, qa, one, qw, one)
    ref, _, acc = oracle.scaled_mm(oracle.INT8, qa[:, :133000], one, qw[:, :133000], one)
    assert acc[0, 0] == 127 * 127 * 133000


def test_fp64_sum_is_exact_for_largest_k():
    # Largest-magnitude E4M3 products at K = 25600 (the longest reduction used): the fp64
    # partial sums must stay exact, so the result equals the integer-scaled numpy sum.
    K = 25600
    rng = np.random.default_rng(36)
    ca = rng.integers(0, 0x7F, (2, K)).astype(np.uint8)
    cw = rng.integers(0, 0x7F, (3, K)).astype(np.uint8)
    ca[:, ::3] |= 0x80
    one2, one3 = np.ones(2, np.float32), np.ones(3, np.float32)
    ref, _, _ = oracle.scaled_mm(oracle.FP8, ca, one2, cw, one3)
    # exact integer arithmetic on values scaled by 2^18 (all products are multiples of 2^-18)
    da = np.array([[int(Fraction(oracle.e4m3_decode(int(c))) * 2 ** 9) for c in row] for row in ca],
                  dtype=object)
    dw = np.array([[int(Fraction(oracle.e4m3_decode(int(c))) * 2 ** 9) for c in row] for row in cw],
                  dtype=object)
    for m in range(2):
        for n in range(3):
            exact = sum(int(x) * int(y) for x, y in zip(da[m], dw[n]))
            assert Fraction(ref[m, n]) == Fraction(exact, 2 ** 18)


def test_within_tolerance_bar():
    ref = np.array([1.0, -2.0, 1e-5, 0.0])
    ok, worst = oracle.within_tolerance(ref * (1 + 0.0099), ref)
    assert ok
    ok, _ = oracle.within_tolerance(np.array([1.02, -2.0, 1e-5, 0.0]), ref)
    assert not ok
    ok, _ = oracle.within_tolerance(np.array([1.0, -2.0, 9e-4, 5e-4]), ref)  # abs floor 1e-3
    assert ok


@pytest.mark.parametrize("fmt", [oracle.SCALE_F32, oracle.SCALE_UE8M0])
def test_block_gemm_several_block_rows_exact(fmt):
    # Two weight block rows and three K groups: integer block sums from numpy's int64
    # matmul of the codes' values scaled by 2^9 (torch's float8 decode), scales as rationals.
    import torch
    M, N, K = 2, 256, 384
    a = synth.draw(37, N, K, 1, (M, K), "normal")
    w = synth.draw(37, N, K, 0, (N, K), "weight")
    qa, sa = oracle.quant_group(fmt, a)
    qw, sw = oracle.quant_weight_block(fmt, w)
    ref, out = oracle.block_scaled_mm(fmt, qa, sa, qw, sw)
    ia = (torch.from_numpy(qa).view(torch.float8_e4m3fn).double().numpy() * 512).astype(np.int64)
    iw = (torch.from_numpy(qw).view(torch.float8_e4m3fn).double().numpy() * 512).astype(np.int64)

    def sc(arr, i, j):
        v = arr[i, j]
        return Fraction(2) ** (int(v) - 127) if fmt == oracle.SCALE_UE8M0 else Fraction(float(v))

    S = [ia[:, g * 128:(g + 1) * 128] @ iw[:, g * 128:(g + 1) * 128].T for g in range(3)]
    for m in range(M):
        for n in range(0, N, 5):
            terms = [sc(sa, m, g) * sc(sw, n // 128, g) * Fraction(int(S[g][m, n]), 2 ** 18)
                     for g in range(3)]
            total = sum(terms)
            bound = 2 * len(terms) * Fraction(1, 2 ** 53) * sum(abs(t) for t in terms)
            assert abs(Fraction(ref[m, n]) - total) <= bound
            assert Fraction(bf16_value(out[m, n])) == _exact.bf16(total)
