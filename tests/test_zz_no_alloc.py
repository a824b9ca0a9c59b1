"""The allocation-free GEMM entry point (qbg_scaled_mm_noalloc).

It runs the kernels of qbg_scaled_mm with the library's per-GPU scratch in
place of a caller's workspace, so its outputs must equal qbg_scaled_mm's byte
for byte under the same configuration.  Two calls in a row, the second with a
smaller input, check that the scratch the first call leaves behind (split-K
partials, arrival counters) does not leak into the next.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import quantized_bit_gemm_amd as qbg
from quantized_bit_gemm_amd import synth


def _operands(qtype, N, K, M, dev):
    workload = synth.DECODE_FP8 if qtype == qbg.QBG_FP8_E4M3 else synth.DECODE_INT8
    oq = oracle.FP8 if qtype == qbg.QBG_FP8_E4M3 else oracle.INT8
    qa, sa = oracle.quant_per_token(oq, synth.activations(workload, N, K, M))
    qw, sw = oracle.quant_weight_per_channel(oq, synth.weights(workload, N, K))
    dt = torch.uint8 if qtype == qbg.QBG_FP8_E4M3 else torch.int8
    conv = lambda a: torch.from_numpy(np.ascontiguousarray(a)).view(dt).to(dev)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
    return conv(qa), f32(sa), conv(qw), f32(sw)


def _nan(M, N, dev):
    return torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev)


# (M, N, K, config) of the first and the second call; None = table lookup.
# 72 tokens under kernel 35 run as two launches (64 + 8) in one call; kernel
# 45 is an eight-wave decode tile, kernel 4 the register tile.
_SEQUENCES = [
    [(72, 4096, 12288, None), (5, 2048, 4096, None)],
    [(32, 4096, 12288, {"kernel_id": 45, "swap_ab": 1, "split_k": 4}),
     (3, 1024, 4096, {"kernel_id": 45, "swap_ab": 1, "split_k": 2})],
    [(17, 6144, 4096, {"kernel_id": 4, "swap_ab": 0, "split_k": 8}),
     (1, 512, 1024, {"kernel_id": 4, "swap_ab": 0, "split_k": 4})],
]


@pytest.mark.gpu
@pytest.mark.parametrize("qtype", [qbg.QBG_FP8_E4M3, qbg.QBG_INT8])
@pytest.mark.parametrize("seq", range(len(_SEQUENCES)))
def test_noalloc_matches_workspace_entry_point(qtype, seq):
    dev = torch.device("cuda:0")
    for M, N, K, cfg in _SEQUENCES[seq]:
        print("noalloc qtype=%d M=%d N=%d K=%d cfg=%s" % (qtype, M, N, K, cfg), flush=True)
        d = _operands(qtype, N, K, M, dev)
        op = qbg.QBG_OP_FP8 if qtype == qbg.QBG_FP8_E4M3 else qbg.QBG_OP_INT8
        assert qbg.qbg_workspace_size(op, M, N, K, cfg) > 0, "the case must exercise split-K"
        ref = qbg.qbg_scaled_mm(*d, qtype=qtype, config=cfg, out=_nan(M, N, dev))
        got = qbg.qbg_scaled_mm_noalloc(*d, qtype=qtype, config=cfg, out=_nan(M, N, dev))
        torch.cuda.synchronize()
        r = ref.view(torch.int16).cpu().numpy()
        g = got.view(torch.int16).cpu().numpy()
        assert not np.isnan(ref.float().cpu().numpy()).any(), "reference left NaN"
        assert np.array_equal(g, r), "M=%d N=%d K=%d: %d outputs differ" % (
            M, N, K, int((g != r).sum()))


@pytest.mark.gpu
def test_noalloc_rejects_more_scratch_than_it_holds():
    dev = torch.device("cuda:0")
    M, N, K = 32, 51200, 5120
    cfg = {"kernel_id": 4, "swap_ab": 0, "split_k": 8}
    assert qbg.qbg_workspace_size(qbg.QBG_OP_FP8, M, N, K, cfg) > qbg.QBG_NOALLOC_SCRATCH_BYTES
    a = torch.zeros((M, K), dtype=torch.uint8, device=dev)
    w = torch.zeros((N, K), dtype=torch.uint8, device=dev)
    sa = torch.ones(M, dtype=torch.float32, device=dev)
    sw = torch.ones(N, dtype=torch.float32, device=dev)
    out = _nan(M, N, dev)
    with pytest.raises(qbg.QbgError) as e:
        qbg.qbg_scaled_mm_noalloc(a, sa, w, sw, out=out, config=cfg)
    assert e.value.status == qbg.QBG_E_WORKSPACE and "qbg_scaled_mm_noalloc" in str(e.value)
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all(), "a rejected call must not launch"


def test_noalloc_rejects_before_any_hip_call():
    """Host logic only: the scratch limit is checked before the library makes
    any HIP call, so stand-in pointers that are never dereferenced suffice."""
    L = qbg.lib()
    M, N, K = 32, 51200, 5120
    cfg = qbg.GemmConfig(kernel_id=4, swap_ab=0, split_k=8)
    p = ctypes.c_void_p(1 << 20)
    st = L.qbg_scaled_mm_noalloc(qbg.QBG_FP8_E4M3, p, p, p, p, M, N, K, p, ctypes.byref(cfg), None)
    assert st == qbg.QBG_E_WORKSPACE
    assert b"qbg_scaled_mm_noalloc" in L.qbg_last_error()
    st = L.qbg_scaled_mm_noalloc(7, p, p, p, p, M, N, K, p, None, None)
    assert st == qbg.QBG_E_QTYPE


def test_noalloc_limit_matches_the_header():
    import os
    import re
    hdr = open(os.path.join(os.path.dirname(__file__), "..", "include", "qbg.h")).read()
    expr = re.search(r"#define QBG_NOALLOC_SCRATCH_BYTES \(([0-9 +<()]+)\)", hdr).group(1)
    assert eval(expr, {"__builtins__": {}}) == qbg.QBG_NOALLOC_SCRATCH_BYTES
