"""GPU parity of the quantizers' non-finite rule.

A token row, 1 x 128 group or 128 x 128 weight block whose values to quantize
hold a NaN or an infinity gets the NaN scale and the NaN code everywhere
(E4M3 0x7F; int8 0); the oracle applies the same reading, so codes and scale
bits must match it byte for byte, through every quantizer (standalone,
long-row, group, weight block, fused producers, and the quantization inside a
one-launch GEMM), and the GEMM outputs of such a token are NaN.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_bit_gemm_amd as qbg
from quantized_bit_gemm_amd import synth
from tests import _gpu

pytestmark = pytest.mark.gpu

BF16_NAN, BF16_INF, BF16_NINF = 0x7FC0, 0x7F80, 0xFF80
QT = {oracle.FP8: qbg.QBG_FP8_E4M3, oracle.INT8: qbg.QBG_INT8}
FMT = {oracle.SCALE_F32: qbg.QBG_SCALE_F32, oracle.SCALE_UE8M0: qbg.QBG_SCALE_UE8M0}


def _rows(K, n=6, seed=0):
    """bf16 rows; rows 1, 2, 3 hold a NaN, a +inf, a -inf (rows 0, 4, 5 finite)."""
    x = synth.to_bf16_bits((np.random.default_rng(seed).standard_normal((n, K))).astype(np.float32))
    x[1, 7] = BF16_NAN
    x[2, K - 1] = BF16_INF
    x[3, K // 2] = BF16_NINF
    return x


def _same(got, ref, what):
    g = np.ascontiguousarray(_gpu.host(got)).view(np.uint8)
    r = np.ascontiguousarray(ref).view(np.uint8)
    assert g.shape == r.shape and np.array_equal(g, r), what


@pytest.mark.parametrize("qtype", [oracle.FP8, oracle.INT8])
@pytest.mark.parametrize("K", [1024, 70016])  # register-resident rows and the long-row kernel
def test_per_token(qtype, K):
    x = _rows(K)
    q, s = qbg.qbg_quantize_per_token(_gpu.bf16_tensor(x), QT[qtype])
    rq, rs = oracle.quant_per_token(qtype, x)
    _same(q, rq, "codes")
    _same(s, rs, "scales")
    assert np.all(_gpu.host(s)[1:4].view(np.uint32) == 0x7FC00000)


@pytest.mark.parametrize("fmt", [oracle.SCALE_F32, oracle.SCALE_UE8M0])
def test_group_and_weight_block(fmt):
    x = _rows(384)
    q, s = qbg.qbg_quantize_per_token_group(_gpu.bf16_tensor(x), 128, FMT[fmt])
    rq, rs = oracle.quant_group(fmt, x)
    _same(q, rq, "group codes")
    _same(s, rs, "group scales")
    w = synth.to_bf16_bits((np.random.default_rng(4).standard_normal((272, 256)) * 0.02)
                           .astype(np.float32))
    w[130, 5] = BF16_INF
    w[261, 200] = BF16_NAN  # the partial last block row
    q, s = qbg.qbg_quantize_weight_block(_gpu.bf16_tensor(w), FMT[fmt])
    rq, rs = oracle.quant_weight_block(fmt, w)
    _same(q, rq, "block codes")
    _same(s, rs, "block scales")


def test_fused_producers():
    H = 512
    x = _rows(H)
    wn = synth.to_bf16_bits(np.ones(H, np.float32))
    q, s = qbg.qbg_rms_norm_quantize_per_token(_gpu.bf16_tensor(x), _gpu.bf16_tensor(wn))
    _, rq, rs = oracle.rms_norm_quant(x, wn)
    _same(q, rq, "rms codes")
    _same(s, rs, "rms scales")
    for fmt in (oracle.SCALE_F32, oracle.SCALE_UE8M0):
        q, s = qbg.qbg_rms_norm_quantize_per_token_group(_gpu.bf16_tensor(x), _gpu.bf16_tensor(wn),
                                                          fmt=FMT[fmt])
        _, rq, rs = oracle.rms_norm_group_quant(fmt, x, wn)
        _same(q, rq, "rms group codes")
        _same(s, rs, "rms group scales")
    # SiLU-and-mul: a NaN, and finite inputs whose product overflows fp32
    I = 256
    gu = np.zeros((3, 2 * I), np.float32)
    gu[:, :I] = np.linspace(-2, 2, I)
    gu[:, I:] = 0.5
    gu[1, 3] = 3.0e38
    gu[1, I + 3] = 3.0e38
    gu_bits = synth.to_bf16_bits(gu)
    gu_bits[2, I + 9] = BF16_NAN
    q, s = qbg.qbg_silu_mul_quantize_per_token(_gpu.bf16_tensor(gu_bits))
    _, rq, rs = oracle.silu_mul_quant(gu_bits)
    _same(q, rq, "silu codes")
    _same(s, rs, "silu scales")
    assert np.all(_gpu.host(s)[1:3].view(np.uint32) == 0x7FC00000)
    for fmt in (oracle.SCALE_F32, oracle.SCALE_UE8M0):
        q, s = qbg.qbg_silu_mul_quantize_per_token_group(_gpu.bf16_tensor(gu_bits), fmt=FMT[fmt])
        _, rq, rs = oracle.silu_mul_group_quant(fmt, gu_bits)
        _same(q, rq, "silu group codes")
        _same(s, rs, "silu group scales")


@pytest.mark.parametrize("qtype", [oracle.FP8, oracle.INT8])
def test_gemm_of_a_non_finite_token(qtype):
    """Quantize-then-GEMM and the one-launch modes: the token's outputs are NaN,
    every other output is within tolerance of the oracle."""
    N, K, M = 512, 1024, 6
    x = _rows(K)
    w = synth.weights(synth.TINY_FP8, N, K)
    qw, sw = oracle.quant_weight_per_channel(qtype, w)
    conv = _gpu.u8 if qtype == oracle.FP8 else _gpu.i8
    dqw, dsw = conv(qw), _gpu.f32(sw)
    rq, rs = oracle.quant_per_token(qtype, x)
    ref, _, _ = oracle.scaled_mm(qtype, rq, rs, qw, sw)
    finite = [0, 4, 5]
    base = {"kernel_id": 16, "swap_ab": 1, "split_k": 1, "rotate": 0}
    for fuse in (qbg.QBG_FUSE_SEPARATE, qbg.QBG_FUSE_PUBLISH, qbg.QBG_FUSE_LOCAL):
        out, aq, sa = qbg.qbg_quantize_scaled_mm(_gpu.bf16_tensor(x), dqw, dsw, qtype=QT[qtype],
                                                 config=dict(base, fuse=fuse))
        what = "fuse=%d" % fuse
        _same(aq, rq, what + " codes")
        _same(sa, rs, what + " scales")
        o = _gpu.host(out)
        assert np.all(np.isnan(_gpu.bf16_values(o[1:4]))), what
        ok, worst = oracle.within_tolerance(_gpu.bf16_values(o[finite]), ref[finite])
        assert ok, "%s: worst |g-r|/tol %.3f" % (what, worst)
