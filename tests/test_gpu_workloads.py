"""GPU parity at the workloads' full sizes, through the configuration the
table (or the built-in default) selects -- the launch configuration the
benchmark times.

* FP8-dynamic at 8B-decoder shapes, M in {1,2,4,8,16,32} (plus ragged M), as
  quantize-then-GEMM and as the fused one-launch form;
* W8A8-INT8 at the same shapes and 512x1024, M in {1,4,16,32}: int32 exact,
  and the fused form;
* Block-FP8 at 32B-decoder shapes, M in {1,8,32}, fp32 and UE8M0 scales;
* the fused MLP chain (RMSNorm+quant -> gate_up -> SiLU-mul+quant -> down) at
  M in {1,32,128,256}, checked stage by stage.

Every GEMM writes into an output pre-filled with NaN and no NaN may remain, so
a workgroup tile that is never stored fails at full grid size.  At 32 tokens
the oracle recomputes every output column of each shape; at the other token
counts a sample of columns (the first and last 48 and 64 seeded random ones).
Quantized tensors are compared byte for byte; bf16 outputs to the GEMM
tolerance.  The fused producers' codes and scales must be the oracle's except
for at most one fp32 rounding tie per call (tests/_ties.py).
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_bit_gemm_amd as qbg
from quantized_bit_gemm_amd import synth
from tests import _gpu, _ties

pytestmark = pytest.mark.gpu


def sample_cols(N, seed=0):
    rng = np.random.default_rng(seed + N)
    idx = set(range(min(48, N))) | set(range(max(0, N - 48), N))
    idx |= set(rng.choice(N, size=min(64, N), replace=False).tolist())
    return np.array(sorted(idx))


def check_cols(got_bits, ref, what):
    ok, worst = oracle.within_tolerance(_gpu.bf16_values(got_bits), ref)
    assert ok, "%s: worst |g-r|/tol %.3f" % (what, worst)


def cols_for(M, N):
    """Every column at the largest decode token count, a sample elsewhere."""
    return np.arange(N) if M == 32 else sample_cols(N)


def nan_out(M, N):
    return torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=_gpu.dev())


def no_nan(out_bits, what):
    bad = np.isnan(_gpu.bf16_values(out_bits))
    assert not bad.any(), "%s: %d outputs never written (first at %s)" % (
        what, int(bad.sum()), np.argwhere(bad)[0].tolist())


_weights = {}


def _evict():
    while len(_weights) >= 2:
        _weights.pop(next(iter(_weights)))


def per_channel_weights(qtype, workload, N, K):
    key = ("pc", qtype, workload, N, K)
    if key not in _weights:
        _evict()
        w = synth.weights(workload, N, K)
        qw, sw = oracle.quant_weight_per_channel(qtype, w)
        conv = _gpu.u8 if qtype == oracle.FP8 else _gpu.i8
        _weights[key] = (qw, sw, conv(qw), _gpu.f32(sw))
    return _weights[key]


def block_weights(fmt, N, K):
    key = ("blk", fmt, N, K)
    if key not in _weights:
        _evict()
        w = synth.weights(synth.DECODE_BLOCK, N, K)
        qw, sw = oracle.quant_weight_block(fmt, w)
        conv = _gpu.u8 if fmt == oracle.SCALE_UE8M0 else _gpu.f32
        _weights[key] = (qw, sw, _gpu.u8(qw), conv(sw))
    return _weights[key]


@pytest.mark.parametrize("N,K", synth.DECODE_SHAPES)
def test_fp8_decode_shapes(N, K):
    qw, sw, dqw, dsw = per_channel_weights(oracle.FP8, synth.DECODE_FP8, N, K)
    a_all = synth.activations(synth.DECODE_FP8, N, K, 32)
    for M in synth.DECODE_MS + [3, 17]:
        a = a_all[:M]
        cols = cols_for(M, N)
        what = "fp8 N=%d K=%d M=%d" % (N, K, M)
        # the activation path on the GPU: quantizer (bit-exact) then GEMM
        qa_d, sa_d = qbg.qbg_quantize_per_token(_gpu.bf16_tensor(a), qbg.QBG_FP8_E4M3)
        qa, sa = oracle.quant_per_token(oracle.FP8, a)
        assert np.array_equal(_gpu.host(qa_d), qa) and np.array_equal(_gpu.host(sa_d), sa)
        out = _gpu.host(qbg.qbg_scaled_mm(qa_d, sa_d, dqw, dsw, out=nan_out(M, N)))
        no_nan(out, what)
        ref, _, _ = oracle.scaled_mm(oracle.FP8, qa, sa, qw[cols], sw[cols])
        check_cols(out[:, cols], ref, what)
        # the same layer as one fused launch (quantization inside the GEMM launch)
        out_f, qa_f, sa_f = qbg.qbg_quantize_scaled_mm(_gpu.bf16_tensor(a), dqw, dsw,
                                                       out=nan_out(M, N))
        assert np.array_equal(_gpu.host(qa_f), qa) and np.array_equal(_gpu.host(sa_f), sa)
        out_f = _gpu.host(out_f)
        no_nan(out_f, "fused " + what)
        check_cols(out_f[:, cols], ref, "fused " + what)


@pytest.mark.parametrize("N,K", synth.DECODE_SHAPES + synth.TINY_SHAPES)
def test_int8_decode_shapes(N, K):
    qw, sw, dqw, dsw = per_channel_weights(oracle.INT8, synth.DECODE_INT8, N, K)
    a_all = synth.activations(synth.DECODE_INT8, N, K, 32)
    for M in synth.INT8_MS:
        a = a_all[:M]
        cols = cols_for(M, N)
        what = "int8 N=%d K=%d M=%d" % (N, K, M)
        qa_d, sa_d = qbg.qbg_quantize_per_token(_gpu.bf16_tensor(a), qbg.QBG_INT8)
        qa, sa = oracle.quant_per_token(oracle.INT8, a)
        assert np.array_equal(_gpu.host(qa_d), qa) and np.array_equal(_gpu.host(sa_d), sa)
        sentinel = torch.full((M, N), -7, dtype=torch.int32, device=_gpu.dev())
        acc_d = _gpu.host(qbg.qbg_scaled_mm_i32(qa_d, dqw, out=sentinel))
        out = _gpu.host(qbg.qbg_scaled_mm(qa_d, sa_d, dqw, dsw, qtype=qbg.QBG_INT8,
                                          out=nan_out(M, N)))
        no_nan(out, what)
        ref, _, acc = oracle.scaled_mm(oracle.INT8, qa, sa, qw[cols], sw[cols])
        assert np.array_equal(acc_d[:, cols], acc), "int32 " + what
        check_cols(out[:, cols], ref, what)
        out_f, qa_f, sa_f = qbg.qbg_quantize_scaled_mm(_gpu.bf16_tensor(a), dqw, dsw,
                                                       qtype=qbg.QBG_INT8, out=nan_out(M, N))
        assert np.array_equal(_gpu.host(qa_f), qa) and np.array_equal(_gpu.host(sa_f), sa)
        out_f = _gpu.host(out_f)
        no_nan(out_f, "fused " + what)
        check_cols(out_f[:, cols], ref, "fused " + what)


@pytest.mark.parametrize("fmt", [oracle.SCALE_F32, oracle.SCALE_UE8M0])
@pytest.mark.parametrize("N,K", synth.BLOCK_SHAPES)
def test_block_decode_shapes(N, K, fmt):
    qw, sw, dqw, dsw = block_weights(fmt, N, K)
    # the oracle works on whole 128-row weight blocks: sample the first, the last and two
    # seeded random blocks
    nb = (N + 127) // 128
    rng = np.random.default_rng(N + K)
    blocks = sorted({0, nb - 1, *rng.choice(nb, size=2, replace=False).tolist()})
    a_all = synth.activations(synth.DECODE_BLOCK, N, K, 32)
    for M in synth.BLOCK_MS:
        a = a_all[:M]
        qa_d, sa_d = qbg.qbg_quantize_per_token_group(_gpu.bf16_tensor(a), 128, fmt)
        qa, sa = oracle.quant_group(fmt, a)
        assert np.array_equal(_gpu.host(qa_d), qa)
        assert np.array_equal(_gpu.host(sa_d).view(np.uint8), sa.view(np.uint8))
        what = "block fmt=%d N=%d K=%d M=%d" % (fmt, N, K, M)
        out = _gpu.host(qbg.qbg_block_scaled_mm(qa_d, sa_d, dqw, dsw, fmt=fmt, out=nan_out(M, N)))
        no_nan(out, what)
        if M == 32:  # every column
            ref, _ = oracle.block_scaled_mm(fmt, qa, sa, qw, sw)
            check_cols(out, ref, what)
            continue
        for blk in blocks:
            lo, hi = blk * 128, min(N, blk * 128 + 128)
            ref, _ = oracle.block_scaled_mm(fmt, qa, sa, qw[lo:hi], sw[blk:blk + 1])
            check_cols(out[:, lo:hi], ref, "%s blk=%d" % (what, blk))


def test_edge_rows_zero_and_exact_powers():
    N, K = 4096, 4096
    qw, sw, dqw, dsw = per_channel_weights(oracle.FP8, synth.DECODE_FP8, N, K)
    a = synth.activations(synth.DECODE_FP8, N, K, 5).copy()
    a[1] = 0                                          # zero row: scale 1, codes 0, output 0
    a[3, 7] = synth.to_bf16_bits(np.array([448.0 * 8], np.float32))[0]  # exact 448*2^k maximum
    qa_d, sa_d = qbg.qbg_quantize_per_token(_gpu.bf16_tensor(a))
    qa, sa = oracle.quant_per_token(oracle.FP8, a)
    assert np.array_equal(_gpu.host(qa_d), qa) and np.array_equal(_gpu.host(sa_d), sa)
    assert sa[1] == 1.0 and sa[3] == 8.0
    out = _gpu.host(qbg.qbg_scaled_mm(qa_d, sa_d, dqw, dsw))
    assert not np.any(_gpu.bf16_values(out[1]))
    cols = sample_cols(N)
    ref, _, _ = oracle.scaled_mm(oracle.FP8, qa, sa, qw[cols], sw[cols])
    check_cols(out[:, cols], ref, "edge rows")


def test_split_k_is_deterministic_and_guard_bands_untouched():
    N, K, M = 4096, 12288, 32
    qw, sw, dqw, dsw = per_channel_weights(oracle.FP8, synth.DECODE_FP8, N, K)
    a = synth.activations(synth.DECODE_FP8, N, K, M)
    qa_d, sa_d = qbg.qbg_quantize_per_token(_gpu.bf16_tensor(a))
    guard = 4096
    # register tiles, LDS decode tiles (4 and 8 waves) and a large-M tile
    cfgs = [{"kernel_id": 4, "swap_ab": 1, "split_k": s} for s in (2, 8, 32)] + [
        {"kernel_id": 45, "swap_ab": 1, "split_k": 2}, {"kernel_id": 47, "swap_ab": 1, "split_k": 4},
        {"kernel_id": 13, "swap_ab": 0, "split_k": 8}, {"kernel_id": 22, "swap_ab": 0, "split_k": 4}]
    for cfg in cfgs:
        outs = []
        for _ in range(2):
            big = torch.full((M * N + 2 * guard,), float("nan"), dtype=torch.bfloat16,
                             device=_gpu.dev())
            out = big[guard:guard + M * N].view(M, N)
            qbg.qbg_scaled_mm(qa_d, sa_d, dqw, dsw, out=out, config=cfg)
            h = _gpu.host(big)
            assert np.all(h[:guard] == h[0]) and np.all(h[-guard:] == h[0]), "guard band written"
            assert np.isnan(_gpu.bf16_values(h[:1]))[0]
            assert not np.isnan(_gpu.bf16_values(h[guard:guard + M * N])).any(), cfg
            outs.append(h[guard:guard + M * N])
        assert np.array_equal(outs[0], outs[1]), "%s not deterministic" % cfg


@pytest.mark.parametrize("M", synth.CHAIN_MS)
def test_mlp_chain_stagewise(M):
    H, I = synth.CHAIN_HIDDEN, synth.CHAIN_INTER
    x = synth.activations(synth.MLP_CHAIN, 2 * I, H, max(synth.CHAIN_MS))[:M]
    wn = synth.norm_weight(H)
    qgu, sgu, dqgu, dsgu = per_channel_weights(oracle.FP8, synth.MLP_CHAIN, 2 * I, H)
    # stage 1: RMSNorm + quant
    q1, s1 = qbg.qbg_rms_norm_quantize_per_token(_gpu.bf16_tensor(x), _gpu.bf16_tensor(wn), 1e-6)
    q1h, s1h = _gpu.host(q1), _gpu.host(s1)
    t1 = _ties.check(oracle.rms_norm_prequant_f64(x, wn, 1e-6), q1h, s1h, _ties.per_token(), H,
                     "rmsnorm+quant M=%d" % M)
    # stage 2: gate_up GEMM on the GPU's own quantized activations
    gu = qbg.qbg_scaled_mm(q1, s1, dqgu, dsgu)
    guh = _gpu.host(gu)
    cols = sample_cols(2 * I)
    ref, _, _ = oracle.scaled_mm(oracle.FP8, q1h, s1h, qgu[cols], sgu[cols])
    check_cols(guh[:, cols], ref, "gate_up M=%d" % M)
    # stage 3: SiLU-mul + quant on the GPU's gate_up output
    q2, s2 = qbg.qbg_silu_mul_quantize_per_token(gu)
    q2h, s2h = _gpu.host(q2), _gpu.host(s2)
    t2 = _ties.check(oracle.silu_mul_prequant_f64(guh), q2h, s2h, _ties.per_token(), I,
                     "silu+quant M=%d" % M)
    # stage 4: down GEMM
    qd, sd, dqd, dsd = per_channel_weights(oracle.FP8, synth.MLP_CHAIN, H, I)
    out = _gpu.host(qbg.qbg_scaled_mm(q2, s2, dqd, dsd))
    cols = sample_cols(H)
    ref, _, _ = oracle.scaled_mm(oracle.FP8, q2h, s2h, qd[cols], sd[cols])
    check_cols(out[:, cols], ref, "down M=%d" % M)
    print("chain M=%d: tie re-roundings %d / %d" % (M, t1, t2))
