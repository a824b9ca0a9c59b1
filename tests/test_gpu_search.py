"""Model-guided configuration search, end to end on the GPU.

The tuner's --search model mode picks which configurations to time with a
tree-ensemble surrogate and times them with the real graph timer; the table
it writes is installed with qbg_config_table_load, the library's lookup must
then return the chosen configuration, and the GEMM that lookup drives must
match the oracle.  There is no timing assertion: only that the search timed
no more than its budget, that its table is what the library loads, and that
the selected kernel computes the right result.
"""
import json

import pytest
import torch

import oracle
import quantized_bit_gemm_amd as qbg
from quantized_bit_gemm_amd import synth, tune
from tests import _gpu

pytestmark = pytest.mark.gpu

# A shape the shipped table does not hold, so the lookup's source is visible.
OP, N, K, M = qbg.QBG_OP_FP8, 2048, 1024, 8


def _candidates():
    n = 0
    for cfg in tune.feasible_configs(qbg, OP, K):
        try:
            qbg.qbg_workspace_size(OP, M, N, K, cfg)
        except qbg.QbgError:
            continue
        n += 1
    return n


def test_model_search_table_drives_the_library(tmp_path):
    assert qbg.qbg_config_lookup(OP, M, N, K)[1] is False, "shape must be outside the shipped table"
    table = str(tmp_path / "searched.txt")
    ck = str(tmp_path / "searched.jsonl")
    print("search: fp8 N=%d K=%d M=%d budget 0.25" % (N, K, M), flush=True)
    tune.main(["--ops", "fp8", "--shapes", "%dx%d" % (N, K), "--ms", str(M), "--out", table,
               "--checkpoint", ck, "--search", "model", "--budget", "0.25", "--reps", "3"])
    with open(ck) as f:
        timed = [json.loads(line) for line in f if line.strip()]
    budget = max(8, int(0.25 * _candidates()))
    assert 8 <= len(timed) <= budget, (len(timed), budget)
    best = min(timed, key=lambda r: r["us"])
    lines = [ln.split("#")[0].split() for ln in open(table) if ln.strip() and not ln.startswith("#")]
    assert lines[0][0] == "qbg-config-table" and len(lines) == 2, lines
    assert lines[1] == ["fp8", str(M), str(N), str(K), str(best["kernel_id"]), str(best["swap_ab"]),
                        str(best["split_k"]), str(best["rotate"]), "0"], (lines[1], best)
    try:
        qbg.qbg_config_table_load(table)
        cfg, from_table = qbg.qbg_config_lookup(OP, M, N, K)
        assert from_table is True
        assert (cfg["kernel_id"], cfg["swap_ab"], cfg["split_k"], cfg["rotate"]) == (
            best["kernel_id"], best["swap_ab"], best["split_k"], best["rotate"])
        # The searched configuration, reached through the table, against the oracle.
        a = synth.activations(synth.DECODE_FP8, N, K, M)
        w = synth.weights(synth.DECODE_FP8, N, K)
        qa, sa = oracle.quant_per_token(oracle.FP8, a)
        qw, sw = oracle.quant_weight_per_channel(oracle.FP8, w)
        ref, _, _ = oracle.scaled_mm(oracle.FP8, qa, sa, qw, sw)
        out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=_gpu.dev())
        qbg.qbg_scaled_mm(_gpu.u8(qa), _gpu.f32(sa), _gpu.u8(qw), _gpu.f32(sw),
                          qtype=qbg.QBG_FP8_E4M3, out=out)
        ok, worst = oracle.within_tolerance(_gpu.bf16_values(_gpu.host(out)), ref)
        assert ok, "searched config %s: worst |g-r|/tol = %.3f" % (cfg, worst)
    finally:
        qbg.qbg_config_table_load(qbg.DEFAULT_TABLE)
    assert qbg.qbg_config_lookup(OP, M, N, K)[1] is False, "the shipped table must be back"
