"""The in-step selection (steptune) end to end on a small search: a tuner
checkpoint shortlists the SEPARATE candidates, the alone timings the LOCAL
ones, then the paired step timings decide; whatever entries it writes are
valid table lines whose configurations the library accepts and whose outputs
match the oracle."""
import numpy as np
import pytest

import oracle
import quantized_bit_gemm_amd as qbg
from quantized_bit_gemm_amd import steptune, synth, tune
from tests import _gpu

pytestmark = pytest.mark.gpu


def test_steptune_writes_valid_entries(tmp_path):
    # a small tuner checkpoint shortlists the SEPARATE candidates
    ck = tmp_path / "ck.jsonl"
    tune.main(["--ops", "fp8", "--shapes", "4096x4096", "--ms", "1,2", "--kernels", "1,11,19",
               "--max-split", "1", "--reps", "2", "--out", str(tmp_path / "t.txt"),
               "--checkpoint", str(ck)])
    out = tmp_path / "fused.txt"
    steptune.main(["--out", str(out), "--shapes", "4096x4096", "--ms", "1,2", "--max-m", "1",
                   "--modes", "1,2", "--checkpoint", str(ck), "--kernels", "1,11,19,44",
                   "--top", "2", "--pairs", "2", "--reps", "5", "--min-gain-us", "0"])
    lines = [l for l in out.read_text().splitlines() if l.strip()]
    N, K = 4096, 4096
    w = synth.weights(synth.DECODE_FP8, N, K)
    qw, sw = oracle.quant_weight_per_channel(oracle.FP8, w)
    dqw, dsw = _gpu.u8(qw), _gpu.f32(sw)
    for line in lines:
        f = line.split("#")[0].split()
        assert f[0] in ("fp8", "fp8_fused") and (int(f[2]), int(f[3])) == (N, K)
        M = int(f[1])
        cfg = dict(zip(("kernel_id", "swap_ab", "split_k", "rotate", "fuse"), map(int, f[4:9])))
        if f[0] == "fp8":  # the plain entry of a SEPARATE choice: its fused line follows
            assert cfg["fuse"] == 0
            continue
        assert cfg["fuse"] in (qbg.QBG_FUSE_LOCAL, qbg.QBG_FUSE_SEPARATE)
        qbg.qbg_workspace_size(qbg.QBG_OP_FP8_FUSED, M, N, K, cfg)  # accepted
        a = synth.activations(synth.DECODE_FP8, N, K, M)
        out_d, _, _ = qbg.qbg_quantize_scaled_mm(_gpu.bf16_tensor(a), dqw, dsw, config=cfg)
        qa, sa = oracle.quant_per_token(oracle.FP8, a)
        ref, _, _ = oracle.scaled_mm(oracle.FP8, qa, sa, qw, sw)
        ok, worst = oracle.within_tolerance(_gpu.bf16_values(_gpu.host(out_d)), ref)
        assert ok, "%s: worst |g-r|/tol %.3f" % (line, worst)
