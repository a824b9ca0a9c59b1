"""The model-based configuration search (search.py), on the CPU.

A synthetic timing landscape over the library's real feasible configuration
space stands in for the GPU: the search must find its optimum while timing a
fraction of the configurations, beat random search with the same budget, and
only ever return a configuration it timed.
"""
import numpy as np
import pytest

import quantized_bit_gemm_amd as qbg
from quantized_bit_gemm_amd import search, tune


def _space(op=qbg.QBG_OP_FP8, M=8, N=6144, K=4096):
    cands = []
    for cfg in tune.feasible_configs(qbg, op, K, 16):
        try:
            qbg.qbg_workspace_size(op, M, N, K, cfg)
        except qbg.QbgError:
            continue
        cands.append(cfg)
    info = {k: qbg.qbg_kernel_info(k) for k in range(qbg.qbg_kernel_count())}
    feats = lambda c: search.config_features(info[c["kernel_id"]], c, M, N, K)
    return cands, feats


def _landscape(cands, feats, seed):
    """A smooth function of the features with per-config noise: a few features matter."""
    rng = np.random.default_rng(seed)
    X = np.array([feats(c) for c in cands])
    Xn = (X - X.mean(0)) / (X.std(0) + 1e-9)
    w = rng.normal(size=X.shape[1]) * (rng.random(X.shape[1]) < 0.4)
    t = np.exp(0.3 * Xn @ w + 0.2 * (Xn[:, 0] - 0.5) ** 2 + 0.02 * rng.normal(size=len(cands)))
    return {id(c): float(v) for c, v in zip(cands, t)}


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_model_search_finds_the_optimum_with_a_quarter_of_the_timings(seed):
    cands, feats = _space()
    assert len(cands) >= 100
    cost = _landscape(cands, feats, seed)
    calls = []
    measure = lambda c: calls.append(id(c)) or cost[id(c)]
    budget = len(cands) // 4
    bi, timed = search.model_search(cands, feats, measure, budget=budget, seed=seed)
    assert len(calls) == len(set(calls)) == len(timed) == budget  # each timed once, no more
    assert bi in timed                                             # never an untimed choice
    best = min(cost.values())
    assert cost[id(cands[bi])] <= best * 1.02


def test_model_search_beats_random_search():
    cands, feats = _space(M=32, N=4096, K=12288)
    budget = len(cands) // 5
    gaps_model, gaps_random = [], []
    for seed in range(6):
        cost = _landscape(cands, feats, 100 + seed)
        best = min(cost.values())
        bi, _ = search.model_search(cands, feats, lambda c: cost[id(c)], budget=budget, seed=seed)
        gaps_model.append(cost[id(cands[bi])] / best)
        pick = np.random.default_rng(seed).choice(len(cands), size=budget, replace=False)
        gaps_random.append(min(cost[id(cands[i])] for i in pick) / best)
    assert np.mean(gaps_model) < np.mean(gaps_random)


def test_full_budget_is_the_grid():
    cands, feats = _space(M=1, N=512, K=1024)
    cost = _landscape(cands, feats, 7)
    bi, timed = search.model_search(cands, feats, lambda c: cost[id(c)], budget=10 ** 6)
    assert len(timed) == len(cands)
    assert cost[id(cands[bi])] == min(cost.values())


def test_no_candidates_is_an_error():
    with pytest.raises(ValueError):
        search.model_search([], lambda c: [0.0], lambda c: 1.0, budget=4)
