"""GPU parity of the quantizers: every code byte and every scale bit must equal
the oracle's on the same bf16 input."""
import numpy as np
import pytest
import torch

import oracle
import quantized_bit_gemm_amd as qbg
from quantized_bit_gemm_amd import synth
from tests import _gpu

pytestmark = pytest.mark.gpu


def _edge_rows(K):
    """Rows with degenerate content: zeros, negative zeros, an exact 448*2^k maximum,
    a single nonzero, all-equal values, tiny subnormal-range values."""
    rows = np.zeros((6, K), np.float32)
    rows[1, :] = -0.0
    rows[2, :] = np.linspace(-1, 1, K, dtype=np.float32) * 3.5
    rows[2, K // 3] = 448.0 * 4
    rows[3, K - 1] = -7.25
    rows[4, :] = 0.3
    rows[5, :] = np.linspace(-1, 1, K, dtype=np.float32) * 1e-30
    return synth.to_bf16_bits(rows)


def test_e4m3_conversion_matches_oracle_on_every_boundary():
    vals = []
    for c in range(0x7F):
        v = oracle.e4m3_decode(c)
        vals += [v, -v]
        if c < 0x7E:
            hi = oracle.e4m3_decode(c + 1)
            mid = np.float32((v + hi) / 2)
            vals += [float(mid), -float(mid),
                     float(np.nextafter(mid, np.float32(0))), float(np.nextafter(mid, np.float32(1e9))),
                     -float(np.nextafter(mid, np.float32(0))), -float(np.nextafter(mid, np.float32(1e9)))]
    rng = np.random.default_rng(1)
    vals += list(rng.uniform(-500, 500, 4000)) + list(rng.uniform(-1, 1, 4000) * 2.0 ** -5)
    vals += [0.0, -0.0, 448.0, 449.0, 464.0, 480.0, 1e9, -1e9, -1e-30, 1e-45]
    x = np.array(vals, np.float32)
    got = _gpu.host(qbg.qbg_convert_f32_to_e4m3(_gpu.f32(x)))
    want = np.array([oracle.e4m3_encode(float(np.clip(v, -448, 448))) for v in x], np.uint8)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(x[i]), hex(got[i]), hex(want[i])) for i in bad[:10]]


@pytest.mark.parametrize("qtype", [oracle.FP8, oracle.INT8])
@pytest.mark.parametrize("K", [16, 1024, 1040, 4096, 12288, 25600, 40960, 70016])
def test_quantize_per_token_bit_exact(qtype, K):
    a = synth.activations(synth.DECODE_FP8, 4096, K, 37)
    x = np.concatenate([a, _edge_rows(K)])
    q, s = qbg.qbg_quantize_per_token(_gpu.bf16_tensor(x), qtype)
    oq, os_ = oracle.quant_per_token(qtype, x)
    gq = _gpu.host(q)
    assert np.array_equal(_gpu.host(s).view(np.uint32), os_.view(np.uint32))
    assert np.array_equal(gq.view(np.uint8), oq.view(np.uint8))


@pytest.mark.parametrize("kind", ["student_t", "normal"])
def test_quantize_per_token_int8_distributions(kind):
    x = synth.draw(synth.DECODE_INT8, 4096, 12288, 1, (32, 12288), kind)
    q, s = qbg.qbg_quantize_per_token(_gpu.bf16_tensor(x), qbg.QBG_INT8)
    oq, os_ = oracle.quant_per_token(oracle.INT8, x)
    assert np.array_equal(_gpu.host(s), os_)
    assert np.array_equal(_gpu.host(q), oq)


@pytest.mark.parametrize("fmt", [oracle.SCALE_F32, oracle.SCALE_UE8M0])
@pytest.mark.parametrize("K", [128, 5120, 8192, 25600])
def test_quantize_group_bit_exact(fmt, K):
    a = synth.activations(synth.DECODE_BLOCK, 5120, K, 33)
    x = np.concatenate([a, _edge_rows(K)])
    q, s = qbg.qbg_quantize_per_token_group(_gpu.bf16_tensor(x), 128, fmt)
    oq, os_ = oracle.quant_group(fmt, x)
    assert np.array_equal(_gpu.host(q), oq)
    gs = _gpu.host(s)
    assert np.array_equal(gs.view(np.uint8), os_.view(np.uint8))


@pytest.mark.parametrize("fmt", [oracle.SCALE_F32, oracle.SCALE_UE8M0])
@pytest.mark.parametrize("N,K", [(256, 1024), (400, 384), (5120, 8192)])
def test_quantize_weight_block_bit_exact(fmt, N, K):
    w = synth.weights(synth.DECODE_BLOCK, N, K)
    q, s = qbg.qbg_quantize_weight_block(_gpu.bf16_tensor(w), fmt)
    oq, os_ = oracle.quant_weight_block(fmt, w)
    assert np.array_equal(_gpu.host(q), oq)
    assert np.array_equal(_gpu.host(s).view(np.uint8), os_.view(np.uint8))


def test_quantize_per_token_as_weight_quantizer():
    w = synth.weights(synth.DECODE_FP8, 4096, 4096)
    q, s = qbg.qbg_quantize_per_token(_gpu.bf16_tensor(w), qbg.QBG_FP8_E4M3)
    oq, os_ = oracle.quant_weight_per_channel(oracle.FP8, w)
    assert np.array_equal(_gpu.host(s), os_)
    assert np.array_equal(_gpu.host(q), oq)
