"""Pins for the oracle's quantizers (per-token FP8/int8, 1x128 groups, weight
blocks, fused RMSNorm and SiLU-and-mul producers).

Pinned by hand-worked fixtures, invariants that the definitions fix, and an
exact-rational brute force on tiny inputs.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from quantized_bit_gemm_amd import synth
from tests import _exact, _golden


def bits(vals):
    return synth.to_bf16_bits(np.asarray(vals, dtype=np.float32))


def test_worked_fp8_quant():
    t = _golden.table("worked_fp8_gemm.txt")
    q, s = oracle.quant_per_token(oracle.FP8, bits([_golden.floats(t["A"])]))
    assert s[0] == float(t["sa"][0])
    assert list(q[0]) == _golden.hexbytes(t["qa"])
    qw, sw = oracle.quant_weight_per_channel(
        oracle.FP8, bits([_golden.floats(t["W0"]), _golden.floats(t["W1"])]))
    assert list(sw) == _golden.floats(t["sw"])
    assert list(qw[0]) == _golden.hexbytes(t["qw0"])
    assert list(qw[1]) == _golden.hexbytes(t["qw1"])


def test_worked_int8_quant():
    t = _golden.table("worked_int8_gemm.txt")
    q, s = oracle.quant_per_token(oracle.INT8, bits([_golden.floats(t["A"])]))
    assert s[0] == float(t["sa"][0])
    assert list(q[0]) == [int(v) for v in t["qa"]]
    qw, sw = oracle.quant_weight_per_channel(oracle.INT8, bits([_golden.floats(t["W"])]))
    assert sw[0] == float(t["sw"][0])
    assert list(qw[0]) == [int(v) for v in t["qw"]]


def _block_inputs(t):
    a = np.array([float(t["a_value"][0])] * 128 + [float(t["a_value"][1])] * 128, np.float32)
    w = np.array([float(t["w_value"][0])] * 128 + [float(t["w_value"][1])] * 128, np.float32)
    return bits(a[None, :]), bits(np.tile(w, (128, 1)))


def test_worked_block_quant_fp32_and_ue8m0():
    t = _golden.table("worked_block_gemm.txt")
    a, w = _block_inputs(t)
    qa, sa = oracle.quant_group(oracle.SCALE_F32, a)
    assert list(sa[0]) == _golden.floats(t["sa"])
    assert set(qa.ravel().tolist()) == set(_golden.hexbytes(t["qa"]))
    qw, sw = oracle.quant_weight_block(oracle.SCALE_F32, w)
    assert list(sw[0]) == _golden.floats(t["sw"])
    assert set(qw[:, :128].ravel().tolist()) == {_golden.hexbytes(t["qw"])[0]}
    assert set(qw[:, 128:].ravel().tolist()) == {_golden.hexbytes(t["qw"])[1]}
    qa8, sa8 = oracle.quant_group(oracle.SCALE_UE8M0, a)
    assert list(sa8[0]) == [int(v) for v in t["sa_ue8m0"]]
    assert np.array_equal(qa8, qa)
    qw8, sw8 = oracle.quant_weight_block(oracle.SCALE_UE8M0, w)
    assert list(sw8[0]) == [int(v) for v in t["sw_ue8m0"]]
    assert np.array_equal(qw8, qw)


def test_ones_group_fp32_vs_ue8m0():
    t = _golden.table("ones_group.txt")
    x = bits(np.ones((1, 128), np.float32))
    q, s = oracle.quant_group(oracle.SCALE_F32, x)
    assert s[0, 0] == np.float32(1.0) / np.float32(448.0)
    assert set(q.ravel().tolist()) == {int(t["fp32_code"][0], 16)}
    q8, s8 = oracle.quant_group(oracle.SCALE_UE8M0, x)
    assert s8[0, 0] == int(t["ue8m0_scale_code"][0])
    assert set(q8.ravel().tolist()) == {int(t["ue8m0_code"][0], 16)}


def test_zero_row_gives_unit_scale_and_zero_codes():
    x = np.zeros((2, 64), np.uint16)
    q, s = oracle.quant_per_token(oracle.FP8, x)
    assert list(s) == [1.0, 1.0] and not q.any()
    q, s = oracle.quant_per_token(oracle.INT8, x)
    assert list(s) == [1.0, 1.0] and not q.any()
    q, s = oracle.quant_group(oracle.SCALE_UE8M0, np.zeros((1, 256), np.uint16))
    assert list(s[0]) == [127, 127] and not q.any()


@pytest.mark.parametrize("kind", ["normal", "normal_outliers", "student_t"])
def test_argmax_element_reaches_the_format_maximum(kind):
    x = synth.draw(99, 1, 1, 0, (400, 256), kind)
    for qtype, top in ((oracle.FP8, 448.0), (oracle.INT8, 127.0)):
        q, s = oracle.quant_per_token(qtype, x)
        xf = synth.bf16_bits_to_f32(x)
        am = np.abs(xf).argmax(axis=1)
        for m in range(x.shape[0]):
            code = q[m, am[m]]
            val = oracle.e4m3_decode(int(code)) if qtype == oracle.FP8 else float(code)
            assert abs(val) == top
            assert s[m] == np.float32(np.abs(xf[m]).max()) / np.float32(top)


def test_rne_error_bound_fp8_and_int8():
    x = synth.draw(98, 1, 1, 0, (64, 512), "normal_outliers")
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    q, s = oracle.quant_per_token(oracle.FP8, x)
    for m in range(x.shape[0]):
        for k in range(0, x.shape[1], 7):
            t = np.float32(xf[m, k]) / s[m]
            t = float(np.clip(t, -448, 448))
            dec = oracle.e4m3_decode(int(q[m, k]))
            e = max(np.floor(np.log2(abs(t))) if t != 0 else -6, -6)
            half_ulp = 2.0 ** (e - 3) / 2
            assert abs(t - dec) <= half_ulp
    qi, si = oracle.quant_per_token(oracle.INT8, x)
    t = (xf.astype(np.float32) / si[:, None]).astype(np.float64)
    assert np.all(np.abs(t - qi) <= 0.5)


def test_ue8m0_scale_covers_group_max():
    x = synth.draw(97, 1, 1, 0, (50, 1024), "normal_outliers")
    q, e = oracle.quant_group(oracle.SCALE_UE8M0, x)
    xf = synth.bf16_bits_to_f32(x).reshape(50, 8, 128)
    amax = np.abs(xf).max(axis=2).astype(np.float64)
    scale = np.exp2(e.astype(np.float64) - 127)
    assert np.all(scale * 448 >= amax)
    # smallest power of two not below fl32(amax/448)
    for m in range(50):
        for g in range(8):
            s32 = np.float32(amax[m, g]) / np.float32(448)
            assert scale[m, g] >= s32 and scale[m, g] / 2 < s32


def _exact_quant_rows(x_bits, qtype, group=None, ue8m0=False):
    M, K = x_bits.shape
    G = group or K
    codes = np.zeros((M, K), dtype=np.int64)
    scales = []
    for m in range(M):
        row_scales = []
        for g in range(K // G):
            vals = [_exact.frac_of_bf16(b) for b in x_bits[m, g * G:(g + 1) * G]]
            c, s, ecode = _exact.quant_values(vals, qtype, ue8m0)
            codes[m, g * G:(g + 1) * G] = c
            row_scales.append(ecode if ue8m0 else s)
        scales.append(row_scales)
    return codes, scales


@pytest.mark.parametrize("qtype", ["fp8", "int8"])
def test_per_token_quant_matches_exact_brute_force(qtype):
    x = synth.draw(96, 4, 16, 0, (4, 16), "normal_outliers")
    q, s = oracle.quant_per_token(oracle.FP8 if qtype == "fp8" else oracle.INT8, x)
    codes, scales = _exact_quant_rows(x, qtype)
    got = q.astype(np.int64) if qtype == "int8" else q.astype(np.int64)
    assert np.array_equal(got, codes)
    for m in range(4):
        assert Fraction(float(s[m])) == scales[m][0]


@pytest.mark.parametrize("ue8m0", [False, True])
def test_group_quant_matches_exact_brute_force(ue8m0):
    x = synth.draw(95, 2, 256, 0, (2, 256), "normal")
    fmt = oracle.SCALE_UE8M0 if ue8m0 else oracle.SCALE_F32
    q, s = oracle.quant_group(fmt, x)
    codes, scales = _exact_quant_rows(x, "fp8", group=128, ue8m0=ue8m0)
    assert np.array_equal(q.astype(np.int64), codes)
    for m in range(2):
        for g in range(2):
            if ue8m0:
                assert int(s[m, g]) == scales[m][g]
            else:
                assert Fraction(float(s[m, g])) == scales[m][g]


def test_weight_block_quant_is_group_quant_of_each_block():
    w = synth.draw(94, 200, 256, 0, (200, 256), "weight")  # partial last block row
    q, s = oracle.quant_weight_block(oracle.SCALE_F32, w)
    assert s.shape == (2, 2)
    wf = synth.bf16_bits_to_f32(w)
    for bn in range(2):
        for bk in range(2):
            blk = wf[bn * 128:(bn + 1) * 128, bk * 128:(bk + 1) * 128]
            assert s[bn, bk] == np.float32(np.abs(blk).max()) / np.float32(448)
    # one block through the exact path
    vals = [_exact.frac_of_bf16(b) for b in w[128:200, 128:256].ravel()]
    c, sc, _ = _exact.quant_values(vals, "fp8")
    assert Fraction(float(s[1, 1])) == sc
    assert np.array_equal(q[128:200, 128:256].ravel().astype(np.int64), np.array(c))


def test_rms_norm_quant_matches_decimal_evaluation():
    x = synth.draw(93, 3, 64, 0, (3, 64), "normal_outliers")
    w = synth.draw(93, 3, 64, 1, (64,), "norm_weight")
    y, q, s = oracle.rms_norm_quant(x, w, 1e-6)
    wf = [_exact.frac_of_bf16(b) for b in w]
    for m in range(3):
        xr = [_exact.frac_of_bf16(b) for b in x[m]]
        ey = _exact.rms_norm_values(xr, wf, float(np.float32(1e-6)))
        for k in range(64):
            assert Fraction(float(y[m, k])) == ey[k]
        c, sc, _ = _exact.quant_values(ey, "fp8")
        assert Fraction(float(s[m])) == sc
        assert list(q[m]) == c


def test_rms_norm_closed_form_constant_rows():
    # A row of equal values c with unit weight normalizes to sign(c) * 1/sqrt(1 + eps/c^2).
    x = bits(np.array([[2.0] * 32, [-0.5] * 32], np.float32))
    w = bits(np.ones(32, np.float32))
    y, q, s = oracle.rms_norm_quant(x, w, 0.0)
    assert np.all(y[0] == 1.0) and np.all(y[1] == -1.0)
    assert np.all(q[0] == 0x7E) and np.all(q[1] == 0xFE)
    assert s[0] == np.float32(1.0) / np.float32(448.0)


def test_silu_mul_quant_matches_decimal_evaluation():
    gu = synth.draw(92, 3, 96, 0, (3, 96), "normal_outliers")
    y, q, s = oracle.silu_mul_quant(gu)
    for m in range(3):
        g = [_exact.frac_of_bf16(b) for b in gu[m, :48]]
        u = [_exact.frac_of_bf16(b) for b in gu[m, 48:]]
        ey = _exact.silu_mul_values(g, u)
        for k in range(48):
            assert Fraction(float(y[m, k])) == ey[k]
        c, sc, _ = _exact.quant_values(ey, "fp8")
        assert Fraction(float(s[m])) == sc
        assert list(q[m]) == c


def test_silu_mul_special_values():
    # silu(0) = 0; gate order: the first half is the gate, the second half the multiplier.
    gu = bits(np.array([[0.0, 4.0, -30.0, 1.0, 3.0, 2.0]], np.float32))
    y, q, s = oracle.silu_mul_quant(gu)
    assert y[0, 0] == 0.0
    assert y[0, 1] == np.float32(4.0 / (1.0 + np.exp(-4.0)) * 3.0)
    assert abs(y[0, 2]) < 1e-11
    swapped = bits(np.array([[1.0, 3.0, 2.0, 0.0, 4.0, -30.0]], np.float32))
    y2, _, _ = oracle.silu_mul_quant(swapped)
    assert not np.array_equal(y, y2)


@pytest.mark.parametrize("kind", ["normal", "normal_outliers", "student_t"])
def test_per_token_quant_matches_library_pipeline(kind):
    # The same steps taken with other people's arithmetic: numpy's IEEE fp32 division and
    # torch's float8_e4m3fn cast (round to nearest even), numpy's rint for int8.
    import torch
    x = synth.draw(91, 1, 1, 0, (256, 4096), kind)
    xf = synth.bf16_bits_to_f32(x)
    amax = np.abs(xf).max(axis=1)
    q, s = oracle.quant_per_token(oracle.FP8, x)
    s_lib = np.where(amax > 0, amax / np.float32(448), np.float32(1)).astype(np.float32)
    assert np.array_equal(s, s_lib)
    t = np.clip(xf / s_lib[:, None], -448, 448).astype(np.float32)
    q_lib = torch.from_numpy(t).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q, q_lib)
    qi, si = oracle.quant_per_token(oracle.INT8, x)
    si_lib = np.where(amax > 0, amax / np.float32(127), np.float32(1)).astype(np.float32)
    assert np.array_equal(si, si_lib)
    ti = np.clip(np.rint(xf / si_lib[:, None]), -127, 127).astype(np.int8)
    assert np.array_equal(qi, ti)


def test_group_quant_matches_library_pipeline():
    import torch
    x = synth.draw(90, 1, 1, 0, (64, 5120), "normal")
    xf = synth.bf16_bits_to_f32(x).reshape(64, 40, 128)
    amax = np.abs(xf).max(axis=2)
    q, s = oracle.quant_group(oracle.SCALE_F32, x)
    s_lib = (amax / np.float32(448)).astype(np.float32)
    assert np.array_equal(s, s_lib)
    t = np.clip(xf / s_lib[:, :, None], -448, 448).astype(np.float32).reshape(64, 5120)
    assert np.array_equal(q, torch.from_numpy(t).to(torch.float8_e4m3fn).view(torch.uint8).numpy())
    q8, e8 = oracle.quant_group(oracle.SCALE_UE8M0, x)
    p = np.exp2(np.ceil(np.log2(s_lib.astype(np.float64)))).astype(np.float32)
    assert np.array_equal(np.exp2(e8.astype(np.float64) - 127).astype(np.float32), p)
    t8 = np.clip(xf / p[:, :, None], -448, 448).astype(np.float32).reshape(64, 5120)
    assert np.array_equal(q8, torch.from_numpy(t8).to(torch.float8_e4m3fn).view(torch.uint8).numpy())


def test_fused_prequant_f64_rounds_to_the_fp32_values():
    x = synth.draw(89, 4, 512, 0, (4, 512), "normal_outliers")
    w = synth.draw(89, 4, 512, 1, (512,), "norm_weight")
    y, q, s = oracle.rms_norm_quant(x, w, 1e-6)
    y64 = oracle.rms_norm_prequant_f64(x, w, 1e-6)
    assert np.array_equal(y64.astype(np.float32), y)
    gu = synth.draw(89, 4, 512, 2, (4, 1024), "normal_outliers")
    y, q, s = oracle.silu_mul_quant(gu)
    y64 = oracle.silu_mul_prequant_f64(gu)
    assert np.array_equal(y64.astype(np.float32), y)


def test_fp32_midpoint_tie_detector():
    one = 1.0
    ulp = 2.0 ** -23
    ties = oracle.fp32_midpoint_ties(np.array([one + ulp / 2, one + ulp / 2 * (1 + 2.0 ** -30),
                                               one + ulp / 4, 3.0]))
    assert list(ties) == [True, True, False, False]


def test_fused_prequant_matches_torch_library_routines():
    """torch's CPU rms_norm and silu in float64 are independent implementations of
    the definitions the producers follow (mean of squares over the row with eps
    inside the root, times the weight; gate times its sigmoid, times up).  At the
    decoder's row lengths the oracle's fp64 values agree to a few ulps, and their
    fp32 roundings agree wherever the value is not an fp32 rounding tie."""
    import torch

    H, I = 4096, 12288
    x = synth.draw(94, 8, H, 0, (8, H), "normal_outliers")
    w = synth.draw(94, 8, H, 1, (H,), "norm_weight")
    y64 = oracle.rms_norm_prequant_f64(x, w, 1e-6)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(oracle.bf16_bits_to_f64(x)), (H,),
                                       weight=torch.from_numpy(oracle.bf16_bits_to_f64(w)),
                                       eps=float(np.float32(1e-6))).numpy()
    assert np.allclose(y64, ref, rtol=1e-12, atol=0.0)
    keep = ~oracle.fp32_midpoint_ties(ref)
    assert np.array_equal(y64.astype(np.float32)[keep], ref.astype(np.float32)[keep])

    gu = synth.draw(94, 8, I, 2, (8, 2 * I), "normal_outliers")
    y64 = oracle.silu_mul_prequant_f64(gu)
    g = torch.from_numpy(oracle.bf16_bits_to_f64(gu[:, :I]))
    u = torch.from_numpy(oracle.bf16_bits_to_f64(gu[:, I:]))
    ref = (torch.nn.functional.silu(g) * u).numpy()
    assert np.allclose(y64, ref, rtol=1e-13, atol=0.0)
    keep = ~oracle.fp32_midpoint_ties(ref)
    assert np.array_equal(y64.astype(np.float32)[keep], ref.astype(np.float32)[keep])


def _fp32_rows(seed, shape):
    """fp32 values that are not bf16 numbers (random low mantissa bits), with outliers."""
    rng = np.random.default_rng(seed)
    y = rng.standard_normal(shape).astype(np.float32)
    y[rng.random(shape) < 0.002] *= np.float32(40)
    bits = y.view(np.uint32) | (rng.integers(1, 1 << 16, size=shape, dtype=np.uint32))
    return bits.view(np.float32)


@pytest.mark.parametrize("qtype", [oracle.FP8, oracle.INT8])
def test_per_token_quant_f32_matches_library_pipeline(qtype):
    # The fp32-input quantizer (the fused producers' last step) against the same steps
    # taken with numpy's IEEE fp32 division and torch's float8_e4m3fn cast / numpy's rint,
    # on values bf16 cannot hold: a version that rounded its input to bf16 first, or that
    # multiplied by a reciprocal, fails here.
    import torch
    y = _fp32_rows(7 + qtype, (256, 4096))
    qmax = np.float32(448 if qtype == oracle.FP8 else 127)
    amax = np.abs(y).max(axis=1)
    q, s = oracle.quant_per_token_f32(qtype, y)
    s_lib = (amax / qmax).astype(np.float32)
    assert np.array_equal(s, s_lib)
    t = np.clip(y / s_lib[:, None], -qmax, qmax).astype(np.float32)
    if qtype == oracle.FP8:
        q_lib = torch.from_numpy(t).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    else:
        q_lib = np.rint(t).astype(np.int8)
    assert np.array_equal(q, q_lib)


def test_per_token_quant_f32_hand_cases():
    # amax 448 gives s = 1.  17 + 2^-8 lies above the midpoint 17 of the E4M3 neighbours
    # 16 (0x58) and 18 (0x59), so it encodes as 0x59; rounded to bf16 first it would be 17.0,
    # which ties to even: 0x58.  A zero row takes s = 1 and zero codes.
    y = np.array([[448.0, 17.0 + 2.0 ** -8, -17.0 - 2.0 ** -8, 0.0],
                  [0.0, 0.0, 0.0, 0.0]], dtype=np.float32)
    q, s = oracle.quant_per_token_f32(oracle.FP8, y)
    assert list(s) == [1.0, 1.0]
    assert list(q[0]) == [0x7E, 0x59, 0xD9, 0x00] and not q[1].any()
    # INT8: amax 127 gives s = 1; 2.5 + 2^-20 rounds to 3 (2.5 alone ties to even: 2).
    yi = np.array([[127.0, 2.5 + 2.0 ** -20, 2.5, -126.5]], dtype=np.float32)
    qi, si = oracle.quant_per_token_f32(oracle.INT8, yi)
    assert si[0] == 1.0 and list(qi[0]) == [127, 3, 2, -126]


def test_group_quant_f32_matches_library_pipeline():
    import torch
    y = _fp32_rows(11, (32, 5120))
    yg = y.reshape(32, 40, 128)
    amax = np.abs(yg).max(axis=2)
    q, s = oracle.quant_group_f32(oracle.SCALE_F32, y)
    s_lib = (amax / np.float32(448)).astype(np.float32)
    assert np.array_equal(s, s_lib)
    t = np.clip(yg / s_lib[:, :, None], -448, 448).astype(np.float32).reshape(32, 5120)
    assert np.array_equal(q, torch.from_numpy(t).to(torch.float8_e4m3fn).view(torch.uint8).numpy())
    q8, e8 = oracle.quant_group_f32(oracle.SCALE_UE8M0, y)
    # the smallest power of two >= the fp32 quotient, from frexp (q = f 2^e, f in [0.5, 1))
    f, e = np.frexp(s_lib.astype(np.float64))
    p = np.ldexp(1.0, np.where(f == 0.5, e - 1, e)).astype(np.float32)
    assert np.array_equal(np.ldexp(1.0, e8.astype(np.int64) - 127).astype(np.float32), p)
    t8 = np.clip(yg / p[:, :, None], -448, 448).astype(np.float32).reshape(32, 5120)
    assert np.array_equal(q8, torch.from_numpy(t8).to(torch.float8_e4m3fn).view(torch.uint8).numpy())


def test_tie_check_accepts_one_reround_and_nothing_else():
    # The GPU-side acceptance rule for the fused producers, exercised on the CPU: a
    # result equal to the oracle's with one tie element re-rounded (here the element
    # that sets the row's amax, so the scale and every code change) is accepted; the
    # same change at a non-tie element, or two re-roundings, is not.
    from tests import _ties
    rng = np.random.default_rng(5)
    y64 = rng.standard_normal((3, 256))
    r = y64.astype(np.float32)
    # make element (1, 7) the row's amax and a tie: exactly halfway to its upper neighbour
    top = np.float32(np.abs(r[1]).max() * 2)
    up = np.nextafter(top, np.float32(np.inf))
    y64[1, 7] = (float(top) + float(up)) / 2
    r = y64.astype(np.float32)
    assert oracle.fp32_midpoint_ties(y64)[1, 7]
    alt = r.copy()
    alt[1, 7] = up if r[1, 7] == top else top
    q_ok, s_ok = oracle.quant_per_token_f32(oracle.FP8, alt)
    q0, s0 = oracle.quant_per_token_f32(oracle.FP8, r)
    assert s_ok[1] != s0[1]  # the re-rounding moved the scale
    quant = _ties.per_token()
    assert _ties.check(y64, q0, s0, quant, 256, "exact") == 0
    assert _ties.check(y64, q_ok, s_ok, quant, 256, "one tie") == 1
    bad = q0.copy()
    bad[2, 3] ^= 1  # a code that no tie explains
    assert _ties.explain(y64, bad, s0, quant, 256)[1] == [2]
    two = np.concatenate([y64, y64])
    q2 = np.concatenate([q_ok, q_ok])
    s2 = np.concatenate([s_ok, s_ok])
    with pytest.raises(AssertionError):
        _ties.check(two, q2, s2, quant, 256, "two ties")
