"""GPU parity of the block-format fused producers (RMSNorm or SiLU-and-mul
followed by 1 x 128 group FP8 quantization, fp32 or UE8M0 scales) and of the
Block-FP8 MLP chain they feed, at the 32B-decoder shapes (hidden 5120,
intermediate 25600, M in {1, 8, 32}).

Quantized tensors and scales must equal the oracle's byte for byte, except for
at most one group per call that the oracle reproduces exactly once one of its
tie elements (an fp64 value within 2^-40 |v| of a binary32 midpoint, where two
correct evaluations of the fp64 step may round differently) is rounded to its
other fp32 neighbour (tests/_ties.py).  The chain is checked stage by stage, each oracle stage applied to the
GPU's own previous output; GEMM outputs are checked on whole sampled 128-row
weight blocks to |g - r| <= max(1e-2 |r|, 1e-3).
"""
import numpy as np
import pytest

import oracle
import quantized_bit_gemm_amd as qbg
from quantized_bit_gemm_amd import synth
from tests import _gpu, _ties

pytestmark = pytest.mark.gpu

FMTS = [oracle.SCALE_F32, oracle.SCALE_UE8M0]
H, I = synth.BLOCK_CHAIN_HIDDEN, synth.BLOCK_CHAIN_INTER


def _check_groups(y64, q, s, fmt, what):
    """Codes and group scales equal to the oracle's up to one tie re-rounding."""
    return _ties.check(y64, _gpu.host(q), _gpu.host(s), _ties.per_group(fmt), 128, what)


@pytest.mark.parametrize("fmt", FMTS)
def test_rms_norm_group_quant(fmt):
    x_all = synth.activations(synth.BLOCK_CHAIN, 2 * I, H, 32)
    wn = synth.norm_weight(H)
    for M in synth.BLOCK_CHAIN_MS + [3]:
        x = x_all[:M].copy()
        if M == 3:
            x[1] = 0  # an all-zero row: every group scale 1 (code 127), codes 0
        q, s = qbg.qbg_rms_norm_quantize_per_token_group(_gpu.bf16_tensor(x), _gpu.bf16_tensor(wn),
                                                         1e-6, 128, fmt)
        _check_groups(oracle.rms_norm_prequant_f64(x, wn, 1e-6), q, s, fmt,
                      "rms fmt=%d M=%d" % (fmt, M))


@pytest.mark.parametrize("fmt", FMTS)
def test_silu_mul_group_quant(fmt):
    gu_all = synth.draw(synth.BLOCK_CHAIN, H, I, 3, (32, 2 * I), "normal")
    for M in synth.BLOCK_CHAIN_MS:
        gu = gu_all[:M]
        q, s = qbg.qbg_silu_mul_quantize_per_token_group(_gpu.bf16_tensor(gu), 128, fmt)
        _check_groups(oracle.silu_mul_prequant_f64(gu), q, s, fmt, "silu fmt=%d M=%d" % (fmt, M))


@pytest.mark.parametrize("L", [128, 384, 40960])
def test_group_producers_small_and_long_rows(L):
    """One group, a ragged number of groups, and a row long enough for 8 register
    chunks per thread; both scale formats."""
    x = synth.draw(synth.BLOCK_CHAIN, L, L, 4, (5, L), "normal_outliers")
    wn = synth.draw(synth.BLOCK_CHAIN, L, L, 5, (L,), "norm_weight")
    gu = synth.draw(synth.BLOCK_CHAIN, L, L, 6, (5, 2 * L), "normal_outliers")
    for fmt in FMTS:
        q, s = qbg.qbg_rms_norm_quantize_per_token_group(_gpu.bf16_tensor(x), _gpu.bf16_tensor(wn),
                                                         1e-6, 128, fmt)
        _check_groups(oracle.rms_norm_prequant_f64(x, wn, 1e-6), q, s, fmt,
                      "rms L=%d fmt=%d" % (L, fmt))
        q, s = qbg.qbg_silu_mul_quantize_per_token_group(_gpu.bf16_tensor(gu), 128, fmt)
        _check_groups(oracle.silu_mul_prequant_f64(gu), q, s, fmt, "silu L=%d fmt=%d" % (L, fmt))


def _block_weights(fmt, N, K):
    w = synth.weights(synth.BLOCK_CHAIN, N, K)
    qw, sw = oracle.quant_weight_block(fmt, w)
    conv = _gpu.u8 if fmt == oracle.SCALE_UE8M0 else _gpu.f32
    return qw, sw, _gpu.u8(qw), conv(sw)


def _sample_blocks(N, seed):
    nb = (N + 127) // 128
    rng = np.random.default_rng(seed)
    return sorted({0, nb - 1, *rng.choice(nb, size=2, replace=False).tolist()})


def _check_block_gemm(out_h, fmt, qa, sa, qw, sw, N, what):
    for blk in _sample_blocks(N, N):
        lo, hi = blk * 128, min(N, blk * 128 + 128)
        ref, _ = oracle.block_scaled_mm(fmt, qa, sa, qw[lo:hi], sw[blk:blk + 1])
        ok, worst = oracle.within_tolerance(_gpu.bf16_values(out_h[:, lo:hi]), ref)
        assert ok, "%s blk=%d: worst |g-r|/tol %.3f" % (what, blk, worst)


@pytest.mark.parametrize("fmt", FMTS)
def test_block_mlp_chain_stagewise(fmt):
    x_all = synth.activations(synth.BLOCK_CHAIN, 2 * I, H, 32)
    wn = synth.norm_weight(H)
    qgu, sgu, dqgu, dsgu = _block_weights(fmt, 2 * I, H)
    qd, sd, dqd, dsd = _block_weights(fmt, H, I)
    for M in synth.BLOCK_CHAIN_MS:
        x = x_all[:M]
        # stage 1: RMSNorm + group quant
        q1, s1 = qbg.qbg_rms_norm_quantize_per_token_group(_gpu.bf16_tensor(x),
                                                           _gpu.bf16_tensor(wn), 1e-6, 128, fmt)
        q1h, s1h = _gpu.host(q1), _gpu.host(s1)
        _ties.check(oracle.rms_norm_prequant_f64(x, wn, 1e-6), q1h, s1h, _ties.per_group(fmt), 128,
                    "chain rms fmt=%d M=%d" % (fmt, M))
        # stage 2: gate_up block GEMM on the GPU's own quantized activations
        gu = qbg.qbg_block_scaled_mm(q1, s1, dqgu, dsgu, fmt=fmt)
        guh = _gpu.host(gu)
        _check_block_gemm(guh, fmt, q1h, s1h, qgu, sgu, 2 * I, "gate_up fmt=%d M=%d" % (fmt, M))
        # stage 3: SiLU-mul + group quant on the GPU's gate_up output
        q2, s2 = qbg.qbg_silu_mul_quantize_per_token_group(gu, 128, fmt)
        q2h, s2h = _gpu.host(q2), _gpu.host(s2)
        t2 = _ties.check(oracle.silu_mul_prequant_f64(guh), q2h, s2h, _ties.per_group(fmt), 128,
                         "chain silu fmt=%d M=%d" % (fmt, M))
        # stage 4: down block GEMM
        out = _gpu.host(qbg.qbg_block_scaled_mm(q2, s2, dqd, dsd, fmt=fmt))
        _check_block_gemm(out, fmt, q2h, s2h, qd, sd, H, "down fmt=%d M=%d" % (fmt, M))
        print("block chain fmt=%d M=%d: tie re-roundings %d" % (fmt, M, t2))
