"""GPU parity at prefill token counts (M up to 8192) for the per-channel GEMM.

Large-M tiles without split-K cover every token in one launch (one grid
dimension over slices of tile_m tokens).  Checked here:
- every large-M tile, Standard and Swap-AB, on a ragged M (1000 = 3 x 256 + 232)
  against the oracle's fp64 GEMM on a seeded sample of rows, and bitwise equal to
  the same call made slice by slice (tile_m tokens per call, the host-sliced form);
- split_k 2 on a large-M tile (host-sliced launches with split-K);
- INT8 int32 accumulators exact against the oracle's int64 sums;
- the prefill tiles (256 x 256 outputs per workgroup on 32x32 matrix-core tiles)
  on ragged M and N against the oracle, every output written, and at 8B-decoder
  shapes on sampled rows and columns;
- the built-in default at M = 8192 on a shape outside the table, and the table's
  configuration at the 8B-decoder prefill shapes, on sampled rows and columns.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_bit_gemm_amd as qbg
from quantized_bit_gemm_amd import synth
from tests import _gpu

pytestmark = pytest.mark.gpu

QT = {oracle.FP8: qbg.QBG_FP8_E4M3, oracle.INT8: qbg.QBG_INT8}
OP = {oracle.FP8: qbg.QBG_OP_FP8, oracle.INT8: qbg.QBG_OP_INT8}


def _large_m_kids():
    """Large-M tiles of the LDS-staged kernel (both layouts, FP8 and INT8)."""
    return [k for k in range(qbg.qbg_kernel_count()) if qbg.qbg_kernel_info(k)["tile_m"] > 32
            and qbg.qbg_kernel_info(k)["k_unroll"] > 0]


def _prefill_kids():
    """Prefill tiles (32x32 matrix-core tiles; FP8, Standard layout, K % 64 == 0)."""
    return [k for k in range(qbg.qbg_kernel_count()) if qbg.qbg_kernel_info(k)["tile_m"] > 32
            and qbg.qbg_kernel_info(k)["k_unroll"] == 0]


def _operands(qtype, M, N, K, seed_wl):
    wl = synth.TINY_FP8 if qtype == oracle.FP8 else synth.DECODE_INT8
    w = synth.weights(seed_wl or wl, N, K)
    qw, sw = oracle.quant_weight_per_channel(qtype, w)
    a = synth.activations(seed_wl or wl, N, K, M)
    qa, sa = oracle.quant_per_token(qtype, a)
    conv = _gpu.u8 if qtype == oracle.FP8 else _gpu.i8
    return qa, sa, qw, sw, conv(qa), _gpu.f32(sa), conv(qw), _gpu.f32(sw)


def _rows(M, n=48, seed=7):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([np.arange(min(M, 8)), np.arange(max(0, M - 8), M),
                                     rng.integers(0, M, n)]))


def _check_rows(qtype, out, qa, sa, qw, sw, rows, what, cols=None):
    c = slice(None) if cols is None else cols
    ref, _, _ = oracle.scaled_mm(qtype, qa[rows], sa[rows], qw[c], sw[c])
    got = _gpu.host(out)[rows][:, c]
    ok, worst = oracle.within_tolerance(_gpu.bf16_values(got), ref)
    assert ok, "%s: worst |g-r|/tol %.3f" % (what, worst)


@pytest.mark.parametrize("qtype", [oracle.FP8, oracle.INT8])
def test_every_large_m_tile_one_launch_and_sliced(qtype):
    M, N, K = 1000, 528, 1040
    qa, sa, qw, sw, dqa, dsa, dqw, dsw = _operands(qtype, M, N, K, None)
    rows = _rows(M)
    for kid in _large_m_kids():
        tm = qbg.qbg_kernel_info(kid)["tile_m"]
        for swap in (0, 1):
            cfg = {"kernel_id": kid, "swap_ab": swap, "split_k": 1, "rotate": swap}
            out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=_gpu.dev())
            qbg.qbg_scaled_mm(dqa, dsa, dqw, dsw, qtype=QT[qtype], out=out, config=cfg)
            what = "M=%d kid=%d swap=%d" % (M, kid, swap)
            _check_rows(qtype, out, qa, sa, qw, sw, rows, what)
            assert not torch.isnan(out.float()).any(), what + ": unwritten outputs"
            sliced = torch.empty_like(out)
            for m0 in range(0, M, tm):
                m1 = min(M, m0 + tm)
                qbg.qbg_scaled_mm(dqa[m0:m1], dsa[m0:m1], dqw, dsw, qtype=QT[qtype],
                                  out=sliced[m0:m1], config=cfg)
            assert torch.equal(out.view(torch.int16), sliced.view(torch.int16)), what


def test_large_m_tile_with_split_k_runs_sliced():
    M, N, K = 600, 528, 2048
    qa, sa, qw, sw, dqa, dsa, dqw, dsw = _operands(oracle.FP8, M, N, K, None)
    kid = _large_m_kids()[0]
    cfg = {"kernel_id": kid, "swap_ab": 1, "split_k": 2}
    out = qbg.qbg_scaled_mm(dqa, dsa, dqw, dsw, config=cfg)
    _check_rows(oracle.FP8, out, qa, sa, qw, sw, _rows(M), "split_k 2 kid %d" % kid)


def test_int8_accumulators_exact_at_prefill_sizes():
    M, N, K = 1000, 528, 1040
    qa, sa, qw, sw, dqa, dsa, dqw, dsw = _operands(oracle.INT8, M, N, K, None)
    rows = _rows(M)
    ref = qa[rows].astype(np.int64) @ qw.astype(np.int64).T
    for kid in _large_m_kids():
        acc = qbg.qbg_scaled_mm_i32(dqa, dqw, config={"kernel_id": kid, "swap_ab": kid % 2})
        assert np.array_equal(_gpu.host(acc)[rows], ref), "kid %d" % kid


def test_default_config_at_8192_tokens():
    M, N, K = 8192, 1040, 1024   # not in the table: the built-in large-M default
    qa, sa, qw, sw, dqa, dsa, dqw, dsw = _operands(oracle.FP8, M, N, K, None)
    cfg, hit = qbg.qbg_config_lookup(qbg.QBG_OP_FP8, M, N, K)
    assert not hit and cfg["tile_m"] > 32 and cfg["split_k"] == 1
    out = qbg.qbg_scaled_mm(dqa, dsa, dqw, dsw)
    _check_rows(oracle.FP8, out, qa, sa, qw, sw, _rows(M, 64), "default M=8192")


@pytest.mark.parametrize("NK", [(6144, 4096), (4096, 12288)])
def test_table_config_at_prefill_shapes(NK):
    N, K = NK
    qw, sw = oracle.quant_weight_per_channel(oracle.FP8, synth.weights(synth.DECODE_FP8, N, K))
    dqw, dsw = _gpu.u8(qw), _gpu.f32(sw)
    cols = np.arange(0, N, 97)
    for M in (512, 2048):
        a = synth.activations(synth.DECODE_FP8, N, K, M)
        qa, sa = oracle.quant_per_token(oracle.FP8, a)
        out = qbg.qbg_scaled_mm(_gpu.u8(qa), _gpu.f32(sa), dqw, dsw)
        _check_rows(oracle.FP8, out, qa, sa, qw, sw, _rows(M, 24), "N=%d K=%d M=%d" % (N, K, M),
                    cols=cols)


@pytest.mark.parametrize("qt,M,N", [(oracle.FP8, 1000, 528), (oracle.INT8, 1000, 528),
                                    (oracle.FP8, 100, 528), (oracle.INT8, 300, 784)])
def test_prefill_tiles_ragged(qt, M, N):
    # 1000 = 3 x 256 + 232 tokens, 528 = 2 x 256 + 16 rows, 784 = 3 x 256 + 16; edge
    # tiles take the per-element stores; 100 tokens fill part of one tile
    K = 1024
    qa, sa, qw, sw, dqa, dsa, dqw, dsw = _operands(qt, M, N, K, None)
    rows = _rows(M)
    assert _prefill_kids()
    for kid in _prefill_kids():
        out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=_gpu.dev())
        qbg.qbg_scaled_mm(dqa, dsa, dqw, dsw, qtype=QT[qt], out=out, config={"kernel_id": kid})
        what = "prefill kid=%d qtype=%d" % (kid, qt)
        assert not torch.isnan(out.float()).any(), what + ": unwritten outputs"
        _check_rows(qt, out, qa, sa, qw, sw, rows, what)


@pytest.mark.parametrize("MN", [(1000, 528), (512, 1024), (100, 784)])
def test_prefill_tiles_int8_accumulators_exact(MN):
    M, N = MN   # ragged tiles (partial-row stores) and whole tiles (16-byte stores)
    K = 1152
    qa, sa, qw, sw, dqa, dsa, dqw, dsw = _operands(oracle.INT8, M, N, K, None)
    ref = qa.astype(np.int64) @ qw.astype(np.int64).T
    for kid in _prefill_kids():
        acc = qbg.qbg_scaled_mm_i32(dqa, dqw, config={"kernel_id": kid})
        assert np.array_equal(_gpu.host(acc), ref), "kid %d" % kid


@pytest.mark.parametrize("NK", [(4096, 4096), (24576, 4096)])
def test_prefill_tiles_at_decoder_shapes(NK):
    N, K = NK
    M = 2048
    qw, sw = oracle.quant_weight_per_channel(oracle.FP8, synth.weights(synth.DECODE_FP8, N, K))
    a = synth.activations(synth.DECODE_FP8, N, K, M)
    qa, sa = oracle.quant_per_token(oracle.FP8, a)
    dqa, dsa, dqw, dsw = _gpu.u8(qa), _gpu.f32(sa), _gpu.u8(qw), _gpu.f32(sw)
    cols = np.arange(0, N, 53)
    for kid in _prefill_kids():
        out = qbg.qbg_scaled_mm(dqa, dsa, dqw, dsw, config={"kernel_id": kid})
        _check_rows(oracle.FP8, out, qa, sa, qw, sw, _rows(M, 24), "kid %d N=%d K=%d" % (kid, N, K),
                    cols=cols)


@pytest.mark.parametrize("fmt", [oracle.SCALE_F32, oracle.SCALE_UE8M0])
@pytest.mark.parametrize("MNK", [(1000, 400, 1024), (300, 784, 2048)])
def test_prefill_tiles_block(fmt, MNK):
    M, N, K = MNK   # ragged token and weight tiles; N = 400 ends in a partial 128-row block
    w = synth.weights(synth.DECODE_BLOCK, N, K)
    a = synth.activations(synth.DECODE_BLOCK, N, K, M)
    qa, sa = oracle.quant_group(fmt, a)
    qw, sw = oracle.quant_weight_block(fmt, w)
    rows = _rows(M)
    ref, _ = oracle.block_scaled_mm(fmt, qa[rows], sa[rows], qw, sw)
    conv = _gpu.u8 if fmt == oracle.SCALE_UE8M0 else _gpu.f32
    d = (_gpu.u8(qa), conv(sa), _gpu.u8(qw), conv(sw))
    op = qbg.QBG_OP_BLOCK_UE8M0 if fmt == oracle.SCALE_UE8M0 else qbg.QBG_OP_BLOCK_FP8
    qf = qbg.QBG_SCALE_UE8M0 if fmt == oracle.SCALE_UE8M0 else qbg.QBG_SCALE_F32
    kids = []
    for kid in _prefill_kids():
        try:
            qbg.qbg_workspace_size(op, M, N, K, {"kernel_id": kid})
            kids.append(kid)
        except qbg.QbgError:
            pass  # fp32 blocks run on the tiles with at most 64 token rows per wave
    assert len(kids) >= 2
    for kid in kids:
        out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=_gpu.dev())
        qbg.qbg_block_scaled_mm(*d, fmt=qf, config={"kernel_id": kid}, out=out)
        what = "prefill block fmt=%d kid=%d M=%d N=%d K=%d" % (fmt, kid, M, N, K)
        assert not torch.isnan(out.float()).any(), what + ": unwritten outputs"
        ok, worst = oracle.within_tolerance(_gpu.bf16_values(_gpu.host(out)[rows]), ref)
        assert ok, "%s: worst |g-r|/tol %.3f" % (what, worst)


def test_prefill_tiles_in_graph_replays():
    """A prefill tile captured in a graph: every replay (new activations between
    replays, outputs reset to NaN) equals the eager call bit for bit."""
    M, N, K = 1000, 528, 1024
    qa, sa, qw, sw, dqa, dsa, dqw, dsw = _operands(oracle.FP8, M, N, K, None)
    for kid in _prefill_kids()[:2]:
        cfg = {"kernel_id": kid}
        out = torch.empty((M, N), dtype=torch.bfloat16, device=_gpu.dev())
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            qbg.qbg_scaled_mm(dqa, dsa, dqw, dsw, out=out, config=cfg)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            qbg.qbg_scaled_mm(dqa, dsa, dqw, dsw, out=out, config=cfg)
        for r in range(3):
            a = synth.draw(synth.TINY_FP8, N, K, 40 + r, (M, K), "normal_outliers")
            qa_r, sa_r = oracle.quant_per_token(oracle.FP8, a)
            dqa.copy_(_gpu.u8(qa_r))
            dsa.copy_(_gpu.f32(sa_r))
            eager = qbg.qbg_scaled_mm(dqa, dsa, dqw, dsw, config=cfg)
            out.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), "kid %d replay %d" % (kid, r)


@pytest.mark.parametrize("N,K", [(16, 128), (48, 256), (16, 512)])
def test_prefill_tiles_one_or_two_stages_and_narrow_n(N, K):
    """The shortest K (one or two 128-byte stages: only the peeled last step pair
    runs) and fewer weight rows than one 128-row block, on every prefill tile and
    every op it runs (Block-FP8 UE8M0 needs K a multiple of 512)."""
    M = 300
    rows = np.arange(M)
    for qt in (oracle.FP8, oracle.INT8):
        qa, sa, qw, sw, dqa, dsa, dqw, dsw = _operands(qt, M, N, K, None)
        for kid in _prefill_kids():
            out = qbg.qbg_scaled_mm(dqa, dsa, dqw, dsw, qtype=QT[qt], config={"kernel_id": kid})
            _check_rows(qt, out, qa, sa, qw, sw, rows, "kid=%d qt=%d N=%d K=%d" % (kid, qt, N, K))
    for fmt in (oracle.SCALE_F32, oracle.SCALE_UE8M0):
        if fmt == oracle.SCALE_UE8M0 and K % 512:
            continue
        w = synth.weights(synth.DECODE_BLOCK, N, K)
        a = synth.activations(synth.DECODE_BLOCK, N, K, M)
        qa, sa = oracle.quant_group(fmt, a)
        qw, sw = oracle.quant_weight_block(fmt, w)
        ref, _ = oracle.block_scaled_mm(fmt, qa, sa, qw, sw)
        conv = _gpu.u8 if fmt == oracle.SCALE_UE8M0 else _gpu.f32
        d = (_gpu.u8(qa), conv(sa), _gpu.u8(qw), conv(sw))
        op = qbg.QBG_OP_BLOCK_UE8M0 if fmt == oracle.SCALE_UE8M0 else qbg.QBG_OP_BLOCK_FP8
        qf = qbg.QBG_SCALE_UE8M0 if fmt == oracle.SCALE_UE8M0 else qbg.QBG_SCALE_F32
        for kid in _prefill_kids():
            try:
                qbg.qbg_workspace_size(op, M, N, K, {"kernel_id": kid})
            except qbg.QbgError:
                continue
            out = qbg.qbg_block_scaled_mm(*d, fmt=qf, config={"kernel_id": kid})
            ok, worst = oracle.within_tolerance(_gpu.bf16_values(_gpu.host(out)), ref)
            assert ok, "block fmt=%d kid=%d N=%d K=%d: worst %.3f" % (fmt, kid, N, K, worst)


# ---- split-K on the prefill tiles: each K chunk's workgroup writes its sums to a
# workspace slot and the last of a tile's chunks to arrive adds them in chunk order.

@pytest.mark.parametrize("qt", [oracle.FP8, oracle.INT8])
@pytest.mark.parametrize("split", [2, 4, 8])
def test_prefill_tiles_split_k(qt, split):
    """Ragged M and N (partial tiles in both), every prefill tile: every output
    written, within tolerance of the oracle, and a second call bitwise equal to the
    first (the sum order is fixed; the arrival counters were reset)."""
    M, N, K = 1000, 528, 1024
    qa, sa, qw, sw, dqa, dsa, dqw, dsw = _operands(qt, M, N, K, None)
    rows = _rows(M)
    for kid in _prefill_kids():
        cfg = {"kernel_id": kid, "split_k": split}
        what = "prefill split=%d kid=%d qtype=%d" % (split, kid, qt)
        outs = []
        for _ in range(2):
            out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=_gpu.dev())
            qbg.qbg_scaled_mm(dqa, dsa, dqw, dsw, qtype=QT[qt], out=out, config=cfg)
            assert not torch.isnan(out.float()).any(), what + ": unwritten outputs"
            outs.append(out)
        assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16)), what + ": not repeatable"
        _check_rows(qt, outs[0], qa, sa, qw, sw, rows, what)


@pytest.mark.parametrize("split", [2, 16])
def test_prefill_tiles_split_k_int8_accumulators_exact(split):
    """The int32 sums through the split-K hand-off equal the oracle's int64 sums."""
    M, N, K = 300, 784, 2048
    qa, sa, qw, sw, dqa, dsa, dqw, dsw = _operands(oracle.INT8, M, N, K, None)
    ref = qa.astype(np.int64) @ qw.astype(np.int64).T
    for kid in _prefill_kids():
        acc = qbg.qbg_scaled_mm_i32(dqa, dqw, config={"kernel_id": kid, "split_k": split})
        assert np.array_equal(_gpu.host(acc), ref), "kid %d split %d" % (kid, split)


def test_prefill_tiles_split_k_at_decoder_shape():
    """512 tokens of the 4096 x 12288 down projection, split 4 (the case split-K is
    for: too few output tiles to fill the chip), sampled rows and columns."""
    M, N, K = 512, 4096, 12288
    qa, sa, qw, sw, dqa, dsa, dqw, dsw = _operands(oracle.FP8, M, N, K, synth.DECODE_FP8)
    rows = _rows(M, 24)
    cols = np.unique(np.concatenate([np.arange(16), np.arange(N - 16, N),
                                     np.random.default_rng(3).choice(N, 48, replace=False)]))
    for kid in _prefill_kids():
        out = qbg.qbg_scaled_mm(dqa, dsa, dqw, dsw, config={"kernel_id": kid, "split_k": 4})
        _check_rows(oracle.FP8, out, qa, sa, qw, sw, rows, "split 4 kid %d" % kid, cols)


def test_prefill_tiles_split_k_in_graph_replays():
    """Split-K on a prefill tile captured in a graph: the workspace and its arrival
    counters are reused by every replay, and each replay equals the eager call."""
    M, N, K = 700, 528, 2048
    qa, sa, qw, sw, dqa, dsa, dqw, dsw = _operands(oracle.FP8, M, N, K, None)
    kid = _prefill_kids()[-1]
    cfg = {"kernel_id": kid, "split_k": 4}
    out = torch.empty((M, N), dtype=torch.bfloat16, device=_gpu.dev())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        qbg.qbg_scaled_mm(dqa, dsa, dqw, dsw, out=out, config=cfg)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qbg.qbg_scaled_mm(dqa, dsa, dqw, dsw, out=out, config=cfg)
    for r in range(3):
        a = synth.draw(synth.TINY_FP8, N, K, 60 + r, (M, K), "normal_outliers")
        qa_r, sa_r = oracle.quant_per_token(oracle.FP8, a)
        dqa.copy_(_gpu.u8(qa_r))
        dsa.copy_(_gpu.f32(sa_r))
        eager = qbg.qbg_scaled_mm(dqa, dsa, dqw, dsw, config=cfg)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), "replay %d" % r


def test_default_config_splits_k_when_tiles_are_few():
    """A shape outside the table with fewer prefill output tiles than CUs and a long K:
    the built-in default takes two K chunks (workspace from the binding), checked on
    sampled rows for FP8 and INT8."""
    M, N, K = 1100, 3072, 10240
    for qt in (oracle.FP8, oracle.INT8):
        c, hit = qbg.qbg_config_lookup(OP[qt], M, N, K)
        assert not hit and c["split_k"] == 2 and c["k_unroll"] == 0
        qa, sa, qw, sw, dqa, dsa, dqw, dsw = _operands(qt, M, N, K, None)
        out = qbg.qbg_scaled_mm(dqa, dsa, dqw, dsw, qtype=QT[qt])
        assert not torch.isnan(out.float()).any()
        _check_rows(qt, out, qa, sa, qw, sw, _rows(M, 16), "default split qtype=%d" % qt)


@pytest.mark.parametrize("fmt", [oracle.SCALE_F32, oracle.SCALE_UE8M0])
@pytest.mark.parametrize("split", [2, 16])
def test_prefill_tiles_block_split_k(fmt, split):
    """Block-FP8 split by whole 128-wide scale groups (each chunk reads its own
    groups' scales or codes): ragged M and N, every prefill tile that runs the
    format, every output written and within tolerance, a second call bitwise equal."""
    M, N, K = 300, 400, 2048
    w = synth.weights(synth.DECODE_BLOCK, N, K)
    a = synth.activations(synth.DECODE_BLOCK, N, K, M)
    qa, sa = oracle.quant_group(fmt, a)
    qw, sw = oracle.quant_weight_block(fmt, w)
    ref, _ = oracle.block_scaled_mm(fmt, qa, sa, qw, sw)
    conv = _gpu.u8 if fmt == oracle.SCALE_UE8M0 else _gpu.f32
    d = (_gpu.u8(qa), conv(sa), _gpu.u8(qw), conv(sw))
    op = qbg.QBG_OP_BLOCK_UE8M0 if fmt == oracle.SCALE_UE8M0 else qbg.QBG_OP_BLOCK_FP8
    qf = qbg.QBG_SCALE_UE8M0 if fmt == oracle.SCALE_UE8M0 else qbg.QBG_SCALE_F32
    n = 0
    for kid in _prefill_kids():
        cfg = {"kernel_id": kid, "split_k": split}
        try:
            qbg.qbg_workspace_size(op, M, N, K, cfg)
        except qbg.QbgError:
            continue  # fp32 blocks run on the tiles with at most 64 token rows per wave
        what = "block split fmt=%d split=%d kid=%d" % (fmt, split, kid)
        outs = []
        for _ in range(2):
            out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=_gpu.dev())
            qbg.qbg_block_scaled_mm(*d, fmt=qf, config=cfg, out=out)
            assert not torch.isnan(out.float()).any(), what + ": unwritten outputs"
            outs.append(out)
        assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16)), what + ": not repeatable"
        ok, worst = oracle.within_tolerance(_gpu.bf16_values(_gpu.host(outs[0])), ref)
        assert ok, "%s: worst |g-r|/tol %.3f" % (what, worst)
        n += 1
    assert n >= 2
