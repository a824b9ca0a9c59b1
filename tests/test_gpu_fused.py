"""GPU parity of the fused quantize + scaled GEMM entry point (qbg_quantize_scaled_mm)
in its three fuse modes: PUBLISH (producer workgroups publish the codes), LOCAL
(every workgroup quantizes the rows itself and keeps its chunk's codes in LDS)
and SEPARATE (quantizer launch, then the GEMM).

Every mode must produce exactly what qbg_quantize_per_token followed by
qbg_scaled_mm produces: the quantized activations and their scales byte for
byte equal to the oracle's per-token quantization of the same bf16 input, and
bf16 outputs within |g - r| <= max(1e-2 |r|, 1e-3) of the oracle's fp64 GEMM
on those operands.  Every LDS-staged tile variant (and for LOCAL every
register-streaming one), Standard and Swap-AB and every feasible split_k is
forced on ragged shapes (PUBLISH and LOCAL; a sample of tiles for SEPARATE);
LOCAL on the register tiles is also checked at the decoder shapes it serves;
with the same tile the one-launch modes give the
two-launch bits exactly; the bounded wait's fall-back (every workgroup
quantizing the rows itself) is forced from the host with the wait-limit hook;
back-to-back calls, token counts above one launch's 32 and graph replays check
that nothing is left behind for the next call.
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
OP = {oracle.FP8: qbg.QBG_OP_FP8_FUSED, oracle.INT8: qbg.QBG_OP_INT8_FUSED}
PLAIN_OP = {oracle.FP8: qbg.QBG_OP_FP8, oracle.INT8: qbg.QBG_OP_INT8}
PUBLISH, LOCAL, SEPARATE = qbg.QBG_FUSE_PUBLISH, qbg.QBG_FUSE_LOCAL, qbg.QBG_FUSE_SEPARATE
MODES = [PUBLISH, LOCAL, SEPARATE]
# a tile each mode runs on: the LDS-staged decode tile (16 rows, 512-byte stage
# rows, 3 stages); SEPARATE also a register-streaming tile
LDS_KID = 16


def _weights(qtype, N, K, workload):
    w = synth.weights(workload, N, K)
    qw, sw = oracle.quant_weight_per_channel(qtype, w)
    conv = _gpu.u8 if qtype == oracle.FP8 else _gpu.i8
    return qw, sw, conv(qw), _gpu.f32(sw)


def _buffers(qtype, M, K, N):
    """Outputs pre-filled with values no correct launch leaves behind."""
    d = _gpu.dev()
    aq = torch.full((M, K), 0x7F, dtype=torch.uint8 if qtype == oracle.FP8 else torch.int8,
                    device=d)
    sa = torch.full((M,), float("nan"), dtype=torch.float32, device=d)
    out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=d)
    return aq, sa, out


def _run_and_check(qtype, x_bits, dqw, dsw, qw, sw, cfg, what, cols=None):
    M, K = x_bits.shape
    N = dqw.shape[0]
    aq, sa, out = _buffers(qtype, M, K, N)
    qbg.qbg_quantize_scaled_mm(_gpu.bf16_tensor(x_bits), dqw, dsw, qtype=QT[qtype], out=out,
                               a_q=aq, a_scale=sa, config=cfg)
    qa_ref, sa_ref = oracle.quant_per_token(qtype, x_bits)
    got_q = _gpu.host(aq)
    if qtype == oracle.INT8:
        got_q = got_q.view(np.int8)
    assert np.array_equal(got_q, qa_ref), "a_q %s" % what
    assert np.array_equal(_gpu.host(sa), sa_ref), "a_scale %s" % what
    c = slice(None) if cols is None else cols
    ref, _, _ = oracle.scaled_mm(qtype, qa_ref, sa_ref, qw[c], sw[c])
    ok, worst = oracle.within_tolerance(_gpu.bf16_values(_gpu.host(out)[:, c]), ref)
    assert ok, "out %s: worst |g-r|/tol %.3f" % (what, worst)
    return out


def _mode_kids(fuse):
    info = {k: qbg.qbg_kernel_info(k) for k in range(qbg.qbg_kernel_count())}
    if fuse == SEPARATE:  # any tile of the plain op: a sample of each kind
        reg = [k for k, i in info.items() if i["stages"] == 0]
        big = [k for k, i in info.items() if i["tile_m"] > 32]
        return [reg[0], reg[-1], LDS_KID, big[0]]
    # LOCAL also runs on the register tiles (where the K chunk is two load groups
    # of every wave; other chunks are rejected and skipped below)
    return [k for k, i in info.items()
            if (i["stages"] > 0 and (fuse == PUBLISH or i["tile_m"] == 32)) or
            (fuse == LOCAL and i["stages"] == 0 and i["tile_m"] == 32)]


def _fused_configs(K, op, M, N, fuse=PUBLISH):
    for kid in _mode_kids(fuse):
        for swap in (0, 1):
            s = 1
            while s <= 256:
                if K % s == 0 and (K // s) % 16 == 0:
                    cfg = {"kernel_id": kid, "swap_ab": swap, "split_k": s, "rotate": s % 2,
                           "fuse": fuse}
                    try:
                        qbg.qbg_workspace_size(op, M, N, K, cfg)
                    except qbg.QbgError as e:
                        assert e.status == 9, e
                        s *= 2
                        continue
                    yield cfg
                s *= 2


@pytest.mark.parametrize("fuse", MODES)
@pytest.mark.parametrize("qtype", [oracle.FP8, oracle.INT8])
@pytest.mark.parametrize("K", [1040, 2048])
@pytest.mark.parametrize("M", [1, 3, 16, 17, 32])
def test_fused_every_variant_small(qtype, M, K, fuse):
    N = 528
    wl = synth.TINY_FP8 if qtype == oracle.FP8 else synth.DECODE_INT8
    qw, sw, dqw, dsw = _weights(qtype, N, K, wl)
    x = synth.activations(wl, N, K, M)
    n = 0
    for cfg in _fused_configs(K, OP[qtype], M, N, fuse):
        _run_and_check(qtype, x, dqw, dsw, qw, sw, cfg, "M=%d K=%d %s" % (M, K, cfg))
        n += 1
    # LOCAL keeps the 2MK bytes of bf16 rows in LDS: no tile takes 32 x 2048 (128 KiB)
    assert n >= (0 if fuse == LOCAL and 2 * M * K > 64 << 10 else 4)


@pytest.mark.parametrize("qtype", [oracle.FP8, oracle.INT8])
def test_fused_equals_two_launches_bitwise(qtype):
    """Same tile variant: each fuse mode and quantize-then-GEMM give identical bits."""
    N, K = 4096, 4096
    wl = synth.DECODE_FP8 if qtype == oracle.FP8 else synth.DECODE_INT8
    qw, sw, dqw, dsw = _weights(qtype, N, K, wl)
    base = [{"kernel_id": LDS_KID, "swap_ab": 1, "split_k": 1, "rotate": 0},
            {"kernel_id": 19, "swap_ab": 0, "split_k": 2, "rotate": 1}]
    for M in (1, 7, 32):
        x = _gpu.bf16_tensor(synth.activations(wl, N, K, M))
        aq, sa = qbg.qbg_quantize_per_token(x, QT[qtype])
        plain, _ = qbg.qbg_config_lookup(PLAIN_OP[qtype], M, N, K)
        cases = [(b, fuse) for b in base for fuse in (PUBLISH, LOCAL)] + [(plain, SEPARATE)]
        for b, fuse in cases:
            b = {k: b[k] for k in ("kernel_id", "swap_ab", "split_k", "rotate")}
            if fuse == LOCAL and 2 * M * K > 64 << 10:
                continue  # the rows do not fit LDS next to this tile's ring
            out_f, aq_f, sa_f = qbg.qbg_quantize_scaled_mm(x, dqw, dsw, qtype=QT[qtype],
                                                           config=dict(b, fuse=fuse))
            out = qbg.qbg_scaled_mm(aq, sa, dqw, dsw, qtype=QT[qtype], config=b)
            what = "M=%d fuse=%d %s" % (M, fuse, b)
            assert torch.equal(aq_f, aq) and torch.equal(sa_f, sa), what
            assert torch.equal(out_f.view(torch.int16), out.view(torch.int16)), what


def test_fused_table_lookup_at_decode_shapes():
    """Whatever the table picks (mode and tile) at the decode shapes is exact."""
    for (N, K) in ((6144, 4096), (4096, 12288)):
        qw, sw, dqw, dsw = _weights(oracle.FP8, N, K, synth.DECODE_FP8)
        cols = np.arange(0, N, 61)
        for M in (1, 4, 16, 32):
            x = synth.activations(synth.DECODE_FP8, N, K, M)
            cfg, _ = qbg.qbg_config_lookup(OP[oracle.FP8], M, N, K)
            _run_and_check(oracle.FP8, x, dqw, dsw, qw, sw, None, "table N=%d K=%d M=%d %s"
                           % (N, K, M, cfg), cols=cols)


@pytest.mark.parametrize("qtype", [oracle.FP8, oracle.INT8])
def test_fused_fallback_every_workgroup_quantizes(qtype):
    """PUBLISH with wait limit 0: no workgroup waits for the producers; each one
    quantizes every row itself (the same bytes), and the results are unchanged."""
    N, K = 1024, 4096
    wl = synth.DECODE_FP8 if qtype == oracle.FP8 else synth.DECODE_INT8
    qw, sw, dqw, dsw = _weights(qtype, N, K, wl)
    prev = qbg.qbg_set_fused_wait_limit(0)
    try:
        for M in (1, 16, 32):
            x = synth.activations(wl, N, K, M)
            cfg = {"kernel_id": LDS_KID, "swap_ab": 1, "split_k": 1, "fuse": PUBLISH}
            for c in (cfg, dict(cfg, split_k=4)):
                _run_and_check(qtype, x, dqw, dsw, qw, sw, c, "fallback M=%d %s" % (M, c))
    finally:
        qbg.qbg_set_fused_wait_limit(prev)


@pytest.mark.parametrize("fuse", MODES)
def test_fused_back_to_back_and_slots_left_zero(fuse):
    """Consecutive calls on the same buffers and workspace with different inputs
    (a stale row, a leftover count or a stale LDS copy would show), split-K
    included, then the slots and counters are zero."""
    N, K = 2048, 4096
    qw, sw, dqw, dsw = _weights(oracle.FP8, N, K, synth.DECODE_FP8)
    kid = 4 if fuse == SEPARATE else LDS_KID
    cfgs = [{"kernel_id": kid, "swap_ab": 1, "split_k": s, "fuse": fuse} for s in (1, 2, 4)]
    # LOCAL serves the smallest token counts (its bf16 rows stay in LDS)
    ms = (4, 4, 1, 3, 2, 4) if fuse == LOCAL else (32, 32, 5, 32, 1, 17)
    need = max(qbg.qbg_workspace_size(qbg.QBG_OP_FP8_FUSED, m, N, K, c)
               for m in ms for c in cfgs)
    ws = torch.zeros(max(need, 64 << 10), dtype=torch.uint8, device=_gpu.dev())
    aq, sa, out = _buffers(oracle.FP8, 32, K, N)
    for i, M in enumerate(ms):
        x_bits = synth.draw(synth.DECODE_FP8, N, K, 10 + i, (M, K), "normal_outliers")
        qbg.qbg_quantize_scaled_mm(_gpu.bf16_tensor(x_bits), dqw, dsw, out=out[:M], a_q=aq[:M],
                                   a_scale=sa[:M], workspace=ws, config=cfgs[i % 3])
        qa_ref, sa_ref = oracle.quant_per_token(oracle.FP8, x_bits)
        assert np.array_equal(_gpu.host(aq[:M]), qa_ref), "call %d" % i
        assert np.array_equal(_gpu.host(sa[:M]), sa_ref), "call %d" % i
        ref, _, _ = oracle.scaled_mm(oracle.FP8, qa_ref, sa_ref, qw, sw)
        ok, worst = oracle.within_tolerance(_gpu.bf16_values(_gpu.host(out[:M])), ref)
        assert ok, "call %d worst %.3f" % (i, worst)
    assert not _gpu.host(ws[:64 << 10]).any(), "synchronization slots not left zero"


@pytest.mark.parametrize("qtype", [oracle.FP8, oracle.INT8])
def test_fused_more_than_one_launch_of_tokens(qtype):
    """Token counts above one launch's 32 run as several launches in every mode
    (K = 1024 keeps LOCAL's 32 bf16 rows, 64 KiB, in LDS)."""
    N, K = 1024, 1024
    wl = synth.DECODE_FP8 if qtype == oracle.FP8 else synth.DECODE_INT8
    qw, sw, dqw, dsw = _weights(qtype, N, K, wl)
    big = next(k for k in range(qbg.qbg_kernel_count()) if qbg.qbg_kernel_info(k)["tile_m"] > 32)
    cfgs = [None, {"kernel_id": LDS_KID, "swap_ab": 1, "split_k": 2, "fuse": LOCAL},
            {"kernel_id": LDS_KID, "swap_ab": 0, "split_k": 1, "fuse": PUBLISH},
            {"kernel_id": big, "swap_ab": 0, "split_k": 1, "fuse": SEPARATE}]
    for M in (33, 80, 256):
        x = synth.activations(wl, N, K, M)
        for c in cfgs:
            _run_and_check(qtype, x, dqw, dsw, qw, sw, c, "M=%d %s" % (M, c))


@pytest.mark.parametrize("fuse", MODES)
def test_fused_graph_replays(fuse):
    """Captured once, replayed with new inputs copied in between replays (eager
    work and synchronization between them); every replay checked."""
    N, K = 4096, 4096
    M = 4 if fuse == LOCAL else 16
    qw, sw, dqw, dsw = _weights(oracle.FP8, N, K, synth.DECODE_FP8)
    d = _gpu.dev()
    cfg = {"kernel_id": 4 if fuse == SEPARATE else LDS_KID, "swap_ab": 1, "split_k": 2,
           "fuse": fuse}
    x = torch.empty((M, K), dtype=torch.bfloat16, device=d)
    aq, sa, out = _buffers(oracle.FP8, M, K, N)
    ws = torch.zeros(max(qbg.qbg_workspace_size(qbg.QBG_OP_FP8_FUSED, M, N, K, cfg), 64 << 10),
                     dtype=torch.uint8, device=d)
    x.copy_(_gpu.bf16_tensor(synth.activations(synth.DECODE_FP8, N, K, M)))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        qbg.qbg_quantize_scaled_mm(x, dqw, dsw, out=out, a_q=aq, a_scale=sa, workspace=ws,
                                   config=cfg)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qbg.qbg_quantize_scaled_mm(x, dqw, dsw, out=out, a_q=aq, a_scale=sa, workspace=ws,
                                   config=cfg)
    for i in range(4):
        x_bits = synth.draw(synth.DECODE_FP8, N, K, 20 + i, (M, K), "normal_outliers")
        x.copy_(_gpu.bf16_tensor(x_bits))
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        qa_ref, sa_ref = oracle.quant_per_token(oracle.FP8, x_bits)
        assert np.array_equal(_gpu.host(aq), qa_ref), "replay %d" % i
        ref, _, _ = oracle.scaled_mm(oracle.FP8, qa_ref, sa_ref, qw, sw)
        ok, worst = oracle.within_tolerance(_gpu.bf16_values(_gpu.host(out)), ref)
        assert ok, "replay %d worst %.3f" % (i, worst)
    assert not _gpu.host(ws[:64 << 10]).any()


@pytest.mark.parametrize("qtype", [oracle.FP8, oracle.INT8])
def test_table_config_at_prefill_sizes(qtype):
    """From 512 tokens the table's fused entries are SEPARATE on a prefill tile: the
    standalone quantizer, then the 32x32-matrix-core GEMM."""
    N, K, M = 4096, 4096, 2048
    wl = synth.DECODE_FP8 if qtype == oracle.FP8 else synth.DECODE_INT8
    qw, sw, dqw, dsw = _weights(qtype, N, K, wl)
    x_bits = synth.draw(wl, N, K, 31, (M, K), "normal_outliers")
    cfg, hit = qbg.qbg_config_lookup(OP[qtype], M, N, K)
    assert hit and cfg["fuse"] == SEPARATE and cfg["k_unroll"] == 0, cfg
    _run_and_check(qtype, x_bits, dqw, dsw, qw, sw, None, "table M=%d" % M,
                   cols=np.arange(0, N, 37))


def _register_local_cases():
    """(N, K, kernel_id) of LOCAL register tiles whose waves take the whole K chunk in
    two load groups (K = 256 x waves_k x k_unroll), at decoder row counts and a ragged one."""
    info = {k: qbg.qbg_kernel_info(k) for k in range(qbg.qbg_kernel_count())}
    out = []
    for N, K in ((4096, 4096), (6144, 4096), (4096, 12288), (560, 4096)):
        kids = [k for k, i in info.items() if i["stages"] == 0 and i["tile_m"] == 32 and
                256 * i["waves_k"] * i["k_unroll"] == K]
        out += [(N, K, k) for k in kids]
    return out


@pytest.mark.parametrize("qtype", [oracle.FP8, oracle.INT8])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 7])
def test_local_register_tiles_decoder_shapes(qtype, M):
    """LOCAL on the register tiles at the 8B-decoder row lengths: codes and scales
    byte-exact, outputs within tolerance on sampled columns (every tile, both layouts).
    A launch whose bf16 rows and codes exceed the CU's LDS (7 rows of 12288) is
    rejected with QBG_E_CONFIG and skipped; every other case runs."""
    cases = _register_local_cases()
    assert {k for _, K, k in cases if K == 12288} and {k for _, K, k in cases if K == 4096}
    wl = synth.DECODE_FP8 if qtype == oracle.FP8 else synth.DECODE_INT8
    last, ran = None, 0
    for N, K, kid in cases:
        if (N, K) != last:
            qw, sw, dqw, dsw = _weights(qtype, N, K, wl)
            x = synth.activations(wl, N, K, M)
            cols = np.unique(np.concatenate([np.arange(0, N, max(1, N // 97)), np.arange(N - 40, N)]))
            last = (N, K)
        for swap in (0, 1):
            cfg = {"kernel_id": kid, "swap_ab": swap, "split_k": 1, "fuse": LOCAL}
            try:
                qbg.qbg_workspace_size(OP[qtype], M, N, K, cfg)
            except qbg.QbgError as e:
                assert e.status == 9 and 3 * M * K > 160 << 10, e  # LDS only
                continue
            _run_and_check(qtype, x, dqw, dsw, qw, sw, cfg,
                           "N=%d K=%d M=%d %s" % (N, K, M, cfg), cols=cols)
            ran += 1
    assert ran > 0
