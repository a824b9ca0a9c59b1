"""GPU parity of the grouped (mixture-of-experts) scaled GEMM.

Both sides get the oracle's quantized operands; bf16 outputs must satisfy
|g - r| <= max(1e-2 |r|, 1e-3) against the oracle's fp64 grouped GEMM.  Every
LDS-staged decode tile and both layouts are forced on ragged shapes with
empty experts, an expert with more rows than one tile stages (the slice
loop) and 4- and 16-row stagings; offsets outside [0, T] are clamped without
touching memory around the output; the MoE decode shapes run with seeded
top-8 routing through the table; a captured graph is replayed with new
routing each time.
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


def _experts(qtype, E, N, K, seed):
    qws, sws = [], []
    for e in range(E):
        w = synth.draw(synth.MOE, N, K, 1000 * seed + e, (N, K), "weight")
        qw, sw = oracle.quant_weight_per_channel(qtype, w)
        qws.append(qw)
        sws.append(sw)
    return np.stack(qws), np.stack(sws)


def _rows(qtype, T, K, seed):
    a = synth.draw(synth.MOE, T, K, 500 + seed, (T, K), "normal_outliers")
    return oracle.quant_per_token(qtype, a)


def _dev(qtype, qa, sa, qw, sw, offsets):
    conv = _gpu.u8 if qtype == oracle.FP8 else _gpu.i8
    off = torch.from_numpy(np.asarray(offsets, np.int32)).to(_gpu.dev())
    return conv(qa), _gpu.f32(sa), conv(qw), _gpu.f32(sw), off


def _check(out, ref, what, cols=slice(None)):
    ok, worst = oracle.within_tolerance(_gpu.bf16_values(_gpu.host(out)[:, cols]), ref)
    assert ok, "%s: worst |g-r|/tol %.3f" % (what, worst)


def _grouped_configs(op, T, N, K):
    """Every configuration the library accepts for a grouped call of T rows."""
    for kid in range(qbg.qbg_kernel_count()):
        info = qbg.qbg_kernel_info(kid)
        if info["stages"] == 0 or info["tile_m"] != 32:
            continue
        for swap in (0, 1):
            cfg = {"kernel_id": kid, "swap_ab": swap, "split_k": 1, "rotate": swap}
            try:
                qbg.qbg_workspace_size(op, T, N, K, cfg)
            except qbg.QbgError as e:
                assert e.status == 9, e  # LDS infeasible for this tile at T rows
                continue
            yield cfg


@pytest.mark.parametrize("qtype", [oracle.FP8, oracle.INT8])
@pytest.mark.parametrize("K", [1040, 2048])
def test_grouped_every_tile(qtype, K):
    E, N = 6, 272
    counts = [3, 0, 40, 1, 0, 16]          # empty experts and one with more than 32 rows
    offsets = np.concatenate([[0], np.cumsum(counts)])
    T = int(offsets[-1])
    qa, sa = _rows(qtype, T, K, K)
    qw, sw = _experts(qtype, E, N, K, 1)
    ref, _, _ = oracle.grouped_scaled_mm(qtype, qa, sa, qw, sw, offsets)
    d = _dev(qtype, qa, sa, qw, sw, offsets)
    n = 0
    for cfg in _grouped_configs(qbg.QBG_OP_FP8_GROUPED, T, N, K):
        out = torch.full((T, N), float("nan"), dtype=torch.bfloat16, device=_gpu.dev())
        qbg.qbg_grouped_scaled_mm(*d, qtype=QT[qtype], out=out, config=cfg)
        _check(out, ref, "K=%d %s" % (K, cfg))
        n += 1
    assert n >= 10


@pytest.mark.parametrize("T", [3, 12])
def test_grouped_few_rows(T):
    """4- and 16-row stagings (the launch sizes its activation tile by T)."""
    E, N, K = 5, 128, 1024
    offsets = np.array([0, 0, T // 2, T // 2, T, T])
    qa, sa = _rows(oracle.FP8, T, K, T)
    qw, sw = _experts(oracle.FP8, E, N, K, 2)
    ref, _, _ = oracle.grouped_scaled_mm(oracle.FP8, qa, sa, qw, sw, offsets)
    d = _dev(oracle.FP8, qa, sa, qw, sw, offsets)
    for cfg in _grouped_configs(qbg.QBG_OP_FP8_GROUPED, T, N, K):
        out = torch.full((T, N), float("nan"), dtype=torch.bfloat16, device=_gpu.dev())
        qbg.qbg_grouped_scaled_mm(*d, out=out, config=cfg)
        _check(out, ref, "T=%d %s" % (T, cfg))


def test_grouped_offsets_are_clamped():
    """A last offset beyond T and a decreasing pair: rows stay inside [0, T) and the
    memory around the output is untouched."""
    E, N, K, T = 4, 64, 512, 10
    qa, sa = _rows(oracle.FP8, T, K, 7)
    qw, sw = _experts(oracle.FP8, E, N, K, 3)
    good = np.array([0, 4, 4, 7, T])
    # expert 1: [4, 2) clamps to empty; expert 2: [2, 7) overlaps expert 0's rows 2-3 (two
    # experts write them: not compared); expert 3: [7, T + 1000) clamps to [7, T)
    bad = np.array([0, 4, 2, 7, T + 1000])
    ref, _, _ = oracle.grouped_scaled_mm(oracle.FP8, qa, sa, qw, sw, good)
    d = list(_dev(oracle.FP8, qa, sa, qw, sw, bad))
    guard = 4096
    big = torch.full((T * N + 2 * guard,), float("nan"), dtype=torch.bfloat16, device=_gpu.dev())
    out = big[guard:guard + T * N].view(T, N)
    qbg.qbg_grouped_scaled_mm(*d, out=out)
    h = _gpu.host(big)
    assert np.isnan(_gpu.bf16_values(h[:guard])).all() and np.isnan(_gpu.bf16_values(h[-guard:])).all()
    got = _gpu.bf16_values(h[guard:guard + T * N].reshape(T, N))
    ok, worst = oracle.within_tolerance(got[[0, 1, 7, 8, 9]], ref[[0, 1, 7, 8, 9]])
    assert ok, worst
    ref_e2, _, _ = oracle.grouped_scaled_mm(oracle.FP8, qa[4:7], sa[4:7], qw[2:3], sw[2:3], [0, 3])
    ok, worst = oracle.within_tolerance(got[4:7], ref_e2)
    assert ok, worst


@pytest.mark.parametrize("qtype", [oracle.FP8, oracle.INT8])
def test_grouped_moe_decode_shapes(qtype):
    E, k = synth.MOE_EXPERTS, synth.MOE_TOP_K
    H, I = synth.MOE_HIDDEN, synth.MOE_INTER
    for (N, K) in ((2 * I, H), (H, I)):
        qw, sw = _experts(qtype, E, N, K, 4 + N)
        cols = np.unique(np.concatenate([np.arange(24), np.arange(N - 24, N),
                                         np.random.default_rng(N).choice(N, 48, replace=False)]))
        for M in synth.MOE_MS:
            order, offsets = synth.moe_routing(M, E, k)
            T = len(order)
            a = synth.draw(synth.MOE, M, K, 7, (M, K), "normal")[order]
            qa, sa = oracle.quant_per_token(qtype, a)
            d = _dev(qtype, qa, sa, qw, sw, offsets)
            out = qbg.qbg_grouped_scaled_mm(*d, qtype=QT[qtype])
            ref, _, _ = oracle.grouped_scaled_mm(qtype, qa, sa, qw[:, cols], sw[:, cols], offsets)
            _check(out, ref, "N=%d K=%d M=%d" % (N, K, M), cols)


def test_grouped_graph_replay_with_new_routing():
    E, N, K, M, k = 16, 512, 1024, 8, 4
    T = M * k
    qw, sw = _experts(oracle.FP8, E, N, K, 5)
    dqw, dsw = _gpu.u8(qw), _gpu.f32(sw)
    d = _gpu.dev()
    qa_d = torch.zeros((T, K), dtype=torch.uint8, device=d)
    sa_d = torch.ones((T,), dtype=torch.float32, device=d)
    off_d = torch.zeros((E + 1,), dtype=torch.int32, device=d)
    off_d[-1] = T
    out = torch.empty((T, N), dtype=torch.bfloat16, device=d)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        qbg.qbg_grouped_scaled_mm(qa_d, sa_d, dqw, dsw, off_d, out=out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qbg.qbg_grouped_scaled_mm(qa_d, sa_d, dqw, dsw, off_d, out=out)
    for i in range(4):
        order, offsets = synth.moe_routing(M, E, k, seed=i)
        a = synth.draw(synth.MOE, M, K, 30 + i, (M, K), "normal")[order]
        qa, sa = oracle.quant_per_token(oracle.FP8, a)
        qa_d.copy_(_gpu.u8(qa))
        sa_d.copy_(_gpu.f32(sa))
        off_d.copy_(torch.from_numpy(offsets).to(d))
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref, _, _ = oracle.grouped_scaled_mm(oracle.FP8, qa, sa, qw, sw, offsets)
        _check(out, ref, "replay %d" % i)


# ---- the prefill tiles (32x32 matrix-core tiles, both operands staged) run the
# grouped GEMM too: every workgroup finds its expert from the device offsets.

def _prefill_kids():
    return [k for k in range(qbg.qbg_kernel_count()) if qbg.qbg_kernel_info(k)["k_unroll"] == 0]


@pytest.mark.parametrize("qtype", [oracle.FP8, oracle.INT8])
def test_grouped_prefill_tiles_ragged(qtype):
    """Empty experts, a one-row expert, experts of one, two and three 128-row tiles
    with partial last tiles, N ending inside a 128-row weight tile, on every prefill
    tile."""
    E, N, K = 7, 400, 1152
    counts = [300, 0, 1, 257, 0, 130, 64]
    offsets = np.concatenate([[0], np.cumsum(counts)])
    T = int(offsets[-1])
    qa, sa = _rows(qtype, T, K, 11)
    qw, sw = _experts(qtype, E, N, K, 6)
    ref, _, _ = oracle.grouped_scaled_mm(qtype, qa, sa, qw, sw, offsets)
    d = _dev(qtype, qa, sa, qw, sw, offsets)
    kids = _prefill_kids()
    assert len(kids) >= 2
    for kid in kids:
        out = torch.full((T, N), float("nan"), dtype=torch.bfloat16, device=_gpu.dev())
        qbg.qbg_grouped_scaled_mm(*d, qtype=QT[qtype], out=out, config={"kernel_id": kid})
        what = "prefill grouped qt=%d kid=%d" % (qtype, kid)
        assert not torch.isnan(out.float()).any(), what + ": unwritten outputs"
        _check(out, ref, what)


def test_grouped_prefill_tiles_offsets_are_clamped():
    """Malformed offsets on a prefill tile: rows stay inside [0, T), nothing around
    the output is written, and the well-formed experts' rows are right."""
    E, N, K, T = 4, 272, 512, 300
    qa, sa = _rows(oracle.FP8, T, K, 8)
    qw, sw = _experts(oracle.FP8, E, N, K, 7)
    # expert 1: [140, 20) clamps to empty; expert 2: [20, 200) overlaps expert 0's rows
    # 20-139 (two experts write them: not compared); expert 3: [200, T + 5000) clamps
    # to [200, T)
    bad = np.array([0, 140, 20, 200, T + 5000])
    good = np.array([0, 140, 140, 200, T])
    ref, _, _ = oracle.grouped_scaled_mm(oracle.FP8, qa, sa, qw, sw, good)
    d = list(_dev(oracle.FP8, qa, sa, qw, sw, bad))
    guard = 8192
    for kid in _prefill_kids():
        big = torch.full((T * N + 2 * guard,), float("nan"), dtype=torch.bfloat16, device=_gpu.dev())
        out = big[guard:guard + T * N].view(T, N)
        qbg.qbg_grouped_scaled_mm(*d, out=out, config={"kernel_id": kid})
        h = _gpu.host(big)
        assert np.isnan(_gpu.bf16_values(h[:guard])).all() and np.isnan(_gpu.bf16_values(h[-guard:])).all()
        got = _gpu.bf16_values(h[guard:guard + T * N].reshape(T, N))
        for rows in (slice(0, 20), slice(200, T)):  # written by expert 0, expert 3 alone
            ok, worst = oracle.within_tolerance(got[rows], ref[rows])
            assert ok, (kid, rows, worst)
        # rows 140-199: expert 2 alone
        ref_e2, _, _ = oracle.grouped_scaled_mm(oracle.FP8, qa[140:200], sa[140:200], qw[2:3], sw[2:3], [0, 60])
        ok, worst = oracle.within_tolerance(got[140:200], ref_e2)
        assert ok, (kid, worst)


@pytest.mark.parametrize("qtype", [oracle.FP8, oracle.INT8])
def test_grouped_moe_prefill_shapes(qtype):
    """The MoE MLP shapes at 512 tokens (4096 routed rows, seeded top-8 routing) on
    the table's configuration and on every prefill tile; sampled columns."""
    E, k = synth.MOE_EXPERTS, synth.MOE_TOP_K
    H, I = synth.MOE_HIDDEN, synth.MOE_INTER
    M = 512
    order, offsets = synth.moe_routing(M, E, k)
    T = len(order)
    for (N, K) in ((2 * I, H), (H, I)):
        qw, sw = _experts(qtype, E, N, K, 8 + N)
        cols = np.unique(np.concatenate([np.arange(16), np.arange(N - 16, N),
                                         np.random.default_rng(N).choice(N, 32, replace=False)]))
        a = synth.draw(synth.MOE, M, K, 9, (M, K), "normal")[order]
        qa, sa = oracle.quant_per_token(qtype, a)
        ref, _, _ = oracle.grouped_scaled_mm(qtype, qa, sa, qw[:, cols], sw[:, cols], offsets)
        d = _dev(qtype, qa, sa, qw, sw, offsets)
        for cfg in [None] + [{"kernel_id": kid} for kid in _prefill_kids()]:
            out = qbg.qbg_grouped_scaled_mm(*d, qtype=QT[qtype], config=cfg)
            _check(out, ref, "N=%d K=%d M=%d %s" % (N, K, M, cfg), cols)


def test_grouped_prefill_tile_graph_replay_with_new_routing():
    """The offsets are read on the device: a captured prefill-tile launch replayed
    with new routing (and new rows) matches the oracle on every replay."""
    E, N, K, M, k = 16, 512, 1024, 128, 4
    T = M * k
    kid = _prefill_kids()[-1]
    qw, sw = _experts(oracle.FP8, E, N, K, 9)
    dqw, dsw = _gpu.u8(qw), _gpu.f32(sw)
    d = _gpu.dev()
    qa_d = torch.zeros((T, K), dtype=torch.uint8, device=d)
    sa_d = torch.ones((T,), dtype=torch.float32, device=d)
    off_d = torch.zeros((E + 1,), dtype=torch.int32, device=d)
    off_d[-1] = T
    out = torch.empty((T, N), dtype=torch.bfloat16, device=d)
    cfg = {"kernel_id": kid}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        qbg.qbg_grouped_scaled_mm(qa_d, sa_d, dqw, dsw, off_d, out=out, config=cfg)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qbg.qbg_grouped_scaled_mm(qa_d, sa_d, dqw, dsw, off_d, out=out, config=cfg)
    for i in range(3):
        order, offsets = synth.moe_routing(M, E, k, seed=40 + i)
        a = synth.draw(synth.MOE, M, K, 50 + i, (M, K), "normal")[order]
        qa, sa = oracle.quant_per_token(oracle.FP8, a)
        qa_d.copy_(_gpu.u8(qa))
        sa_d.copy_(_gpu.f32(sa))
        off_d.copy_(torch.from_numpy(offsets).to(d))
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref, _, _ = oracle.grouped_scaled_mm(oracle.FP8, qa, sa, qw, sw, offsets)
        _check(out, ref, "kid %d replay %d" % (kid, i))


def test_grouped_table_prefill_tile_falls_back_for_many_experts():
    """The table picks a prefill tile for 4096 routed rows of the down shape; with more
    experts than those tiles' offset scan takes, a call without a configuration runs
    on the decode tiles instead, and a forced prefill tile is rejected."""
    E, N, K, M, k = 1100, synth.MOE_HIDDEN, synth.MOE_INTER, 512, 8
    c, hit = qbg.qbg_config_lookup(qbg.QBG_OP_FP8_GROUPED, M * k, N, K)
    assert hit and c["k_unroll"] == 0, c
    d = _gpu.dev()
    g = torch.Generator(device=d)
    g.manual_seed(5)
    # finite E4M3 codes: magnitudes 0..125 (0x7F is NaN) with a random sign
    def codes(shape):
        mag = torch.randint(0, 126, shape, generator=g, device=d, dtype=torch.int32)
        sgn = torch.randint(0, 2, shape, generator=g, device=d, dtype=torch.int32) << 7
        return (mag | sgn).to(torch.uint8)
    qw = codes((E, N, K))
    sw = torch.rand((E, N), generator=g, device=d, dtype=torch.float32) * 1e-3 + 1e-4
    order, offsets = synth.moe_routing(M, E, k)
    T = len(order)
    qa = codes((T, K))
    sa = torch.rand((T,), generator=g, device=d, dtype=torch.float32) * 1e-2 + 1e-3
    off = torch.from_numpy(offsets).to(d)
    out = qbg.qbg_grouped_scaled_mm(qa, sa, qw, sw, off)
    cols = np.unique(np.random.default_rng(1).choice(N, 24, replace=False))
    ref, _, _ = oracle.grouped_scaled_mm(oracle.FP8, _gpu.host(qa), _gpu.host(sa),
                                         _gpu.host(qw[:, cols].contiguous()),
                                         _gpu.host(sw[:, cols].contiguous()), offsets)
    _check(out, ref, "E=%d fallback" % E, cols)
    with pytest.raises(qbg.QbgError) as ei:
        qbg.qbg_grouped_scaled_mm(qa, sa, qw, sw, off, config={"kernel_id": c["kernel_id"]})
    assert ei.value.status == 9  # QBG_E_CONFIG


@pytest.mark.parametrize("qtype", [oracle.FP8, oracle.INT8])
def test_grouped_default_at_many_rows_per_expert(qtype):
    """A shape outside the table with 64 routed rows per expert on average: the
    built-in choice is the 64-token prefill tile; every output checked."""
    E, N, K, M, k = 32, 1040, 1536, 512, 4
    order, offsets = synth.moe_routing(M, E, k, seed=3)
    T = len(order)
    assert T >= 32 * E
    qw, sw = _experts(qtype, E, N, K, 12)
    a = synth.draw(synth.MOE, M, K, 13, (M, K), "normal")[order]
    qa, sa = oracle.quant_per_token(qtype, a)
    ref, _, _ = oracle.grouped_scaled_mm(qtype, qa, sa, qw, sw, offsets)
    d = _dev(qtype, qa, sa, qw, sw, offsets)
    out = torch.full((T, N), float("nan"), dtype=torch.bfloat16, device=_gpu.dev())
    qbg.qbg_grouped_scaled_mm(*d, qtype=QT[qtype], out=out)
    assert not torch.isnan(out.float()).any()
    _check(out, ref, "default E=%d T=%d" % (E, T))
