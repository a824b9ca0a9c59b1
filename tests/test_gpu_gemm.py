"""GPU parity of the scaled GEMMs against the oracle.

Both sides get the oracle's quantized operands.  bf16 outputs must satisfy
|g - r| <= max(1e-2 |r|, 1e-3) against the oracle's fp64 value r; the int8
path's int32 accumulators must be equal.  Every tile variant, both Standard
and Swap-AB, and every feasible power-of-two split_k are forced through the
C ABI on small shapes with ragged tails; the full shapes are checked on
sampled output columns.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_bit_gemm_amd as qbg
from quantized_bit_gemm_amd import synth
from tests import _gpu

pytestmark = pytest.mark.gpu


def _operands(qtype, workload, N, K, M, kind=None):
    w = synth.weights(workload, N, K)
    a = synth.activations(workload, N, K, M) if kind is None else \
        synth.draw(workload, N, K, 1, (M, K), kind)
    qa, sa = oracle.quant_per_token(qtype, a)
    qw, sw = oracle.quant_weight_per_channel(qtype, w)
    return a, qa, sa, qw, sw


def _dev_ops(qtype, qa, sa, qw, sw):
    conv = _gpu.u8 if qtype == oracle.FP8 else _gpu.i8
    return conv(qa), _gpu.f32(sa), conv(qw), _gpu.f32(sw)


def _nan_out(M, N):
    """An output buffer pre-filled with NaN, so a launch that skips a store cannot pass."""
    return torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=_gpu.dev())


def _check(got_bits, ref, what):
    ok, worst = oracle.within_tolerance(_gpu.bf16_values(got_bits), ref)
    assert ok, "%s: worst |g-r|/tol = %.3f" % (what, worst)


def _configs(K, quantum, op=qbg.QBG_OP_FP8, M=1, N=512):
    """Every configuration the library accepts for this call."""
    for kid in range(qbg.qbg_kernel_count()):
        for swap in (0, 1):
            s = 1
            while s <= 256:
                if K % s == 0 and (K // s) % quantum == 0:
                    cfg = {"kernel_id": kid, "swap_ab": swap, "split_k": s}
                    try:
                        qbg.qbg_workspace_size(op, M, N, K, cfg)
                    except qbg.QbgError as e:
                        assert e.status == 9, e  # only tile/op or LDS infeasibility is skipped
                        s *= 2
                        continue
                    yield cfg
                s *= 2


@pytest.mark.parametrize("K", [1040, 2048])
@pytest.mark.parametrize("M", [1, 3, 16, 17, 32])
def test_fp8_every_variant_small(M, K):
    N = 528  # ragged: N not a multiple of 32/64; K=1040 is not a multiple of 128
    _, qa, sa, qw, sw = _operands(oracle.FP8, synth.TINY_FP8, N, K, M)
    ref, _, _ = oracle.scaled_mm(oracle.FP8, qa, sa, qw, sw)
    d = _dev_ops(oracle.FP8, qa, sa, qw, sw)
    for cfg in _configs(K, 16, qbg.QBG_OP_FP8, M, N):
        out = qbg.qbg_scaled_mm(*d, qtype=qbg.QBG_FP8_E4M3, config=cfg, out=_nan_out(M, N))
        _check(_gpu.host(out), ref, "M=%d %s" % (M, cfg))


@pytest.mark.parametrize("K", [1040, 4096])
@pytest.mark.parametrize("M", [1, 5, 16, 32])
def test_int8_every_variant_exact_int32(M, K):
    N = 272
    _, qa, sa, qw, sw = _operands(oracle.INT8, synth.DECODE_INT8, N, K, M)
    ref, _, acc = oracle.scaled_mm(oracle.INT8, qa, sa, qw, sw)
    d = _dev_ops(oracle.INT8, qa, sa, qw, sw)
    for cfg in _configs(K, 16, qbg.QBG_OP_INT8, M, N):
        sentinel = torch.full((M, N), -7, dtype=torch.int32, device=_gpu.dev())
        got = _gpu.host(qbg.qbg_scaled_mm_i32(d[0], d[2], config=cfg, out=sentinel))
        assert np.array_equal(got, acc), "M=%d %s" % (M, cfg)
        out = qbg.qbg_scaled_mm(*d, qtype=qbg.QBG_INT8, config=cfg, out=_nan_out(M, N))
        _check(_gpu.host(out), ref, "M=%d %s" % (M, cfg))


@pytest.mark.parametrize("fmt", [oracle.SCALE_F32, oracle.SCALE_UE8M0])
@pytest.mark.parametrize("M", [1, 8, 19, 32])
def test_block_every_variant_small(fmt, M):
    N, K = 400, 1024  # N: a partial 128-row weight block and a ragged 16-row tail
    w = synth.weights(synth.DECODE_BLOCK, N, K)
    a = synth.activations(synth.DECODE_BLOCK, N, K, M)
    qa, sa = oracle.quant_group(fmt, a)
    qw, sw = oracle.quant_weight_block(fmt, w)
    ref, _ = oracle.block_scaled_mm(fmt, qa, sa, qw, sw)
    conv = _gpu.u8 if fmt == oracle.SCALE_UE8M0 else _gpu.f32
    d = (_gpu.u8(qa), conv(sa), _gpu.u8(qw), conv(sw))
    for cfg in _configs(K, 128, qbg.QBG_OP_BLOCK_FP8 if fmt == oracle.SCALE_F32
                        else qbg.QBG_OP_BLOCK_UE8M0, M, N):
        out = qbg.qbg_block_scaled_mm(*d, fmt=fmt, config=cfg, out=_nan_out(M, N))
        _check(_gpu.host(out), ref, "fmt=%d M=%d %s" % (fmt, M, cfg))


@pytest.mark.parametrize("M", [1, 16, 32])
def test_tiny_fp8_full_output(M):
    N, K = synth.TINY_SHAPES[0]
    _, qa, sa, qw, sw = _operands(oracle.FP8, synth.TINY_FP8, N, K, M)
    ref, _, _ = oracle.scaled_mm(oracle.FP8, qa, sa, qw, sw)
    out = qbg.qbg_scaled_mm(*_dev_ops(oracle.FP8, qa, sa, qw, sw))
    _check(_gpu.host(out), ref, "tiny M=%d" % M)


def test_worked_fp8_example_on_gpu():
    from tests import _golden
    t = _golden.table("worked_fp8_gemm.txt")
    qa = np.zeros((1, 16), np.uint8)
    qa[0, :4] = _golden.hexbytes(t["qa"])
    qw = np.zeros((16, 16), np.uint8)
    qw[0, :4] = _golden.hexbytes(t["qw0"])
    qw[1, :4] = _golden.hexbytes(t["qw1"])
    sa = np.array([float(t["sa"][0])], np.float32)
    sw = np.full(16, float(t["sw"][0]), np.float32)
    out = _gpu.host(qbg.qbg_scaled_mm(_gpu.u8(qa), _gpu.f32(sa), _gpu.u8(qw), _gpu.f32(sw)))
    assert list(_gpu.bf16_values(out[0, :2])) == _golden.floats(t["out"])


def _large_m_configs(K, op, M, N):
    for cfg in _configs(K, 16, op, M, N):
        if qbg.qbg_kernel_info(cfg["kernel_id"])["tile_m"] > 32:
            yield cfg


@pytest.mark.parametrize("M", [33, 64, 100, 128, 200, 256])
def test_large_m_tiles_fp8_and_int8(M):
    """Tiles with 64-256 tokens per launch (waves along M): every tile, layout and
    split on a ragged N, including token counts that leave a tile partly empty and
    more tokens than one launch covers."""
    N, K = 528, 2048
    _, qa, sa, qw, sw = _operands(oracle.FP8, synth.TINY_FP8, N, K, M)
    ref, _, _ = oracle.scaled_mm(oracle.FP8, qa, sa, qw, sw)
    d = _dev_ops(oracle.FP8, qa, sa, qw, sw)
    n = 0
    for cfg in _large_m_configs(K, qbg.QBG_OP_FP8, M, N):
        if cfg["split_k"] > 8:
            continue
        out = qbg.qbg_scaled_mm(*d, qtype=qbg.QBG_FP8_E4M3, config=cfg, out=_nan_out(M, N))
        _check(_gpu.host(out), ref, "fp8 M=%d %s" % (M, cfg))
        n += 1
    assert n >= 16
    _, qa, sa, qw, sw = _operands(oracle.INT8, synth.DECODE_INT8, N, K, M)
    _, _, acc = oracle.scaled_mm(oracle.INT8, qa, sa, qw, sw)
    d = _dev_ops(oracle.INT8, qa, sa, qw, sw)
    for cfg in _large_m_configs(K, qbg.QBG_OP_INT8, M, N):
        if cfg["split_k"] not in (1, 4):
            continue
        sentinel = torch.full((M, N), -7, dtype=torch.int32, device=_gpu.dev())
        got = _gpu.host(qbg.qbg_scaled_mm_i32(d[0], d[2], config=cfg, out=sentinel))
        assert np.array_equal(got, acc), "int8 M=%d %s" % (M, cfg)



def test_maximum_k_fp8_and_int32_boundary():
    """The largest K cases: FP8 at K = 65536 with and without a deep split, and int8 at
    K = 133120 (the largest multiple of 16 keeping |acc| <= 127^2 K below 2^31) with
    every product +-127^2, so the exact accumulators reach +-2 147 092 480."""
    M, N, K = 3, 272, 65536
    _, qa, sa, qw, sw = _operands(oracle.FP8, synth.TINY_FP8, N, K, M)
    ref, _, _ = oracle.scaled_mm(oracle.FP8, qa, sa, qw, sw)
    d = _dev_ops(oracle.FP8, qa, sa, qw, sw)
    for cfg in ({"kernel_id": 1, "swap_ab": 1, "split_k": 1},
                {"kernel_id": 16, "swap_ab": 1, "split_k": 64},
                {"kernel_id": 4, "swap_ab": 0, "split_k": 256}):
        out = qbg.qbg_scaled_mm(*d, qtype=qbg.QBG_FP8_E4M3, config=cfg, out=_nan_out(M, N))
        _check(_gpu.host(out), ref, "K=65536 %s" % cfg)
    M, N, K = 2, 64, 133120
    qa = np.full((M, K), 127, np.int8)
    qa[1] = -127
    qw = np.full((N, K), 127, np.int8)
    qw[1::2] = -127
    _, _, acc = oracle.scaled_mm(oracle.INT8, qa, np.ones(M, np.float32), qw,
                                 np.ones(N, np.float32))
    assert abs(int(acc[0, 0])) == 127 * 127 * K
    for cfg in ({"kernel_id": 1, "swap_ab": 1, "split_k": 1},
                {"kernel_id": 16, "swap_ab": 0, "split_k": 8}):
        got = _gpu.host(qbg.qbg_scaled_mm_i32(_gpu.i8(qa), _gpu.i8(qw), config=cfg,
                                              out=torch.full((M, N), -7, dtype=torch.int32,
                                                             device=_gpu.dev())))
        assert np.array_equal(got, acc), cfg


def _cancelling_operands(M, N, K, seed=0):
    """bf16 inputs whose products cancel: token row t holds 448 at K positions 2t and 2t+1,
    every weight row +448 and -448 there, so those two products (+-448^2) cancel exactly
    inside the first 128-wide K block, next to the small products of E4M3 values at the
    other positions.  Per-token and per-channel scales are 1 (amax 448), so the codes are
    the values.  A sum that keeps only the high bits of each K block (as the gfx950 FP8
    matrix cores do) loses the small products beside the large ones."""
    rng = np.random.default_rng(seed)
    small = np.array([1.125, -1.375, 1.625, -1.875, 0.5625, -0.6875], np.float32)
    a = rng.choice(small, (M, K)).astype(np.float32)
    w = rng.choice(small, (N, K)).astype(np.float32)
    a[:, :2 * M] = 0
    for t in range(M):
        a[t, 2 * t] = a[t, 2 * t + 1] = 448.0
    w[:, 0:2 * M:2] = 448.0
    w[:, 1:2 * M:2] = -448.0
    return synth.to_bf16_bits(a), synth.to_bf16_bits(w)


@pytest.mark.parametrize("M", [3, 17, 32])
def test_fp8_cancelling_products_every_variant(M):
    N, K = 272, 1024
    a, w = _cancelling_operands(M, N, K)
    qa, sa = oracle.quant_per_token(oracle.FP8, a)
    qw, sw = oracle.quant_weight_per_channel(oracle.FP8, w)
    assert np.all(sa == 1.0) and np.all(sw == 1.0)
    ref, _, _ = oracle.scaled_mm(oracle.FP8, qa, sa, qw, sw)
    d = _dev_ops(oracle.FP8, qa, sa, qw, sw)
    for cfg in _configs(K, 16, qbg.QBG_OP_FP8, M, N):
        out = qbg.qbg_scaled_mm(*d, qtype=qbg.QBG_FP8_E4M3, config=cfg, out=_nan_out(M, N))
        _check(_gpu.host(out), ref, "cancelling M=%d %s" % (M, cfg))


@pytest.mark.parametrize("fmt", [oracle.SCALE_F32, oracle.SCALE_UE8M0])
def test_block_cancelling_products_every_variant(fmt):
    M, N, K = 17, 256, 1024
    a, w = _cancelling_operands(M, N, K, seed=1)
    qa, sa = oracle.quant_group(fmt, a)
    qw, sw = oracle.quant_weight_block(fmt, w)
    ref, _ = oracle.block_scaled_mm(fmt, qa, sa, qw, sw)
    conv = _gpu.u8 if fmt == oracle.SCALE_UE8M0 else _gpu.f32
    d = (_gpu.u8(qa), conv(sa), _gpu.u8(qw), conv(sw))
    op = qbg.QBG_OP_BLOCK_FP8 if fmt == oracle.SCALE_F32 else qbg.QBG_OP_BLOCK_UE8M0
    for cfg in _configs(K, 128, op, M, N):
        out = qbg.qbg_block_scaled_mm(*d, fmt=fmt, config=cfg, out=_nan_out(M, N))
        _check(_gpu.host(out), ref, "block cancelling fmt=%d %s" % (fmt, cfg))


def _owned_row_tiles():
    """Tile variants whose workgroups own a row count that is no multiple of 16."""
    return [k for k in range(qbg.qbg_kernel_count()) if qbg.qbg_kernel_info(k)["tile_n"] % 16]


@pytest.mark.parametrize("N", [16, 32, 64, 560])
@pytest.mark.parametrize("M", [1, 7, 16, 32])
def test_owned_row_tiles_ragged(N, M):
    """Workgroups owning 24 rows at N that leave the last one 16 or 8 of them
    (N=16: the only workgroup owns fewer rows than its share), FP8 and INT8,
    both layouts, every split the chunk admits."""
    kids = _owned_row_tiles()
    assert kids, "no owned-row tile variant compiled"
    K = 1040
    for qtype, op, workload in ((oracle.FP8, qbg.QBG_OP_FP8, synth.TINY_FP8),
                                (oracle.INT8, qbg.QBG_OP_INT8, synth.DECODE_INT8)):
        _, qa, sa, qw, sw = _operands(qtype, workload, N, K, M)
        ref, _, acc = oracle.scaled_mm(qtype, qa, sa, qw, sw)
        d = _dev_ops(qtype, qa, sa, qw, sw)
        for cfg in _configs(K, 16, op, M, N):
            if cfg["kernel_id"] not in kids:
                continue
            if qtype == oracle.INT8:
                sentinel = torch.full((M, N), -7, dtype=torch.int32, device=_gpu.dev())
                got = _gpu.host(qbg.qbg_scaled_mm_i32(d[0], d[2], config=cfg, out=sentinel))
                assert np.array_equal(got, acc), "N=%d M=%d %s" % (N, M, cfg)
            out = qbg.qbg_scaled_mm(*d, qtype=qbg.QBG_FP8_E4M3 if qtype == oracle.FP8
                                    else qbg.QBG_INT8, config=cfg, out=_nan_out(M, N))
            _check(_gpu.host(out), ref, "N=%d M=%d %s" % (N, M, cfg))
