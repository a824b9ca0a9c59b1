"""The quantizers' rule for non-finite values, pinned on the oracle.

The pages define nothing for NaN or infinite inputs.  The reading here: a
quantization span (a token row, a 1 x 128 group, a 128 x 128 weight block)
whose values to quantize hold a NaN or an infinity gets the NaN scale (fp32
quiet NaN 0x7FC00000; UE8M0 code 0xFF) and the NaN code for every element
(E4M3 0x7F; int8 has no NaN: 0).  Every other span is quantized exactly as if
the non-finite one were absent.  The expected values are the rule itself,
written out; the finite spans are checked against quantizing them alone.
"""
import numpy as np
import pytest

import oracle
from quantized_bit_gemm_amd import synth

NAN_F32 = 0x7FC00000
BF16_NAN, BF16_INF, BF16_NINF = 0x7FC0, 0x7F80, 0xFF80


def _finite(K, n):
    base = np.linspace(-3, 3, K, dtype=np.float32)[None].repeat(n, 0) * np.arange(1, n + 1)[:, None]
    return synth.to_bf16_bits(base.astype(np.float32))


def _rows(K):
    """Five bf16 rows; rows 1-3 hold a NaN, a +inf and a -inf, rows 0 and 4 are finite."""
    rows = _finite(K, 5)
    rows[1, 7] = BF16_NAN
    rows[2, K - 1] = BF16_INF
    rows[3, 0] = BF16_NINF
    return rows


@pytest.mark.parametrize("qtype", [oracle.FP8, oracle.INT8])
def test_per_token_rows_with_nan_or_inf(qtype):
    rows = _rows(256)
    q, s = oracle.quant_per_token(qtype, rows)
    nan_code = 0x7F if qtype == oracle.FP8 else 0
    for r in (1, 2, 3):
        assert s[r:r + 1].view(np.uint32)[0] == NAN_F32
        assert np.all(q[r].view(np.uint8) == nan_code)
    q0, s0 = oracle.quant_per_token(qtype, rows[[0, 4]])
    assert np.array_equal(q[[0, 4]], q0) and np.array_equal(s[[0, 4]].view(np.uint32), s0.view(np.uint32))


@pytest.mark.parametrize("fmt", [oracle.SCALE_F32, oracle.SCALE_UE8M0])
def test_group_with_nan_or_inf(fmt):
    K = 384
    rows = _finite(K, 1).repeat(2, 0)
    ref_q, ref_s = oracle.quant_group(fmt, rows[:1])
    rows[1, 130] = BF16_NAN          # group 1 of row 1
    rows[0, 383] = BF16_NINF         # group 2 of row 0
    q, s = oracle.quant_group(fmt, rows)
    bad = {(1, 1), (0, 2)}
    for r in range(2):
        for g in range(3):
            qs = q[r, 128 * g:128 * (g + 1)]
            if (r, g) in bad:
                assert np.all(qs == 0x7F)
                if fmt == oracle.SCALE_UE8M0:
                    assert s[r, g] == 0xFF
                else:
                    assert s[r:r + 1, g].view(np.uint32)[0] == NAN_F32
            else:
                assert np.array_equal(qs, ref_q[0, 128 * g:128 * (g + 1)])
                assert np.array_equal(np.ascontiguousarray(s[r, g:g + 1]).view(np.uint8),
                                      np.ascontiguousarray(ref_s[0, g:g + 1]).view(np.uint8))


@pytest.mark.parametrize("fmt", [oracle.SCALE_F32, oracle.SCALE_UE8M0])
def test_weight_block_with_inf(fmt):
    N, K = 256, 256
    w = synth.to_bf16_bits((np.random.default_rng(3).standard_normal((N, K)) * 0.02).astype(np.float32))
    q0, s0 = oracle.quant_weight_block(fmt, w)
    w[130, 5] = BF16_INF             # block (1, 0)
    q, s = oracle.quant_weight_block(fmt, w)
    assert np.all(q[128:256, 0:128] == 0x7F)
    if fmt == oracle.SCALE_UE8M0:
        assert s[1, 0] == 0xFF
    else:
        assert s[1:2, 0].view(np.uint32)[0] == NAN_F32
    keep = np.ones((N, K), bool)
    keep[128:256, 0:128] = False
    assert np.array_equal(q[keep], q0[keep])
    sk = np.ones(s.shape, bool)
    sk[1, 0] = False
    assert np.array_equal(np.ascontiguousarray(s).view(np.uint8).reshape(s.shape + (-1,))[sk],
                          np.ascontiguousarray(s0).view(np.uint8).reshape(s0.shape + (-1,))[sk])


def test_fused_producers_follow_the_rule():
    # RMSNorm of a row holding a NaN: every value is NaN, so the row takes the rule
    H = 256
    x = _rows(H)[:2]
    wn = synth.to_bf16_bits(np.ones(H, np.float32))
    _, q, s = oracle.rms_norm_quant(x, wn)
    assert s[1:2].view(np.uint32)[0] == NAN_F32 and np.all(q[1] == 0x7F)
    assert np.isfinite(s[0]) and not np.all(q[0] == 0x7F)
    # SiLU-and-mul of finite but huge inputs: silu(g) * u overflows fp32 to +inf
    I = 128
    gu = np.zeros((2, 2 * I), np.float32)
    gu[:, :I] = 1.0
    gu[:, I:] = 0.5
    gu[1, 3] = 3.0e38
    gu[1, I + 3] = 3.0e38
    _, q, s = oracle.silu_mul_quant(synth.to_bf16_bits(gu))
    assert s[1:2].view(np.uint32)[0] == NAN_F32 and np.all(q[1] == 0x7F)
    assert np.isfinite(s[0])


def test_gemm_rows_of_nan_codes_are_nan():
    qa = np.full((2, 128), 0x38, np.uint8)   # 1.0
    qa[1] = 0x7F
    sa = np.array([1.0, np.float32(np.nan)], np.float32)
    qw = np.full((16, 128), 0x38, np.uint8)
    sw = np.ones(16, np.float32)
    ref, out, _ = oracle.scaled_mm(oracle.FP8, qa, sa, qw, sw)
    assert np.all(ref[0] == 128.0) and np.all(np.isnan(ref[1]))
    assert np.all(out[1] == BF16_NAN)
