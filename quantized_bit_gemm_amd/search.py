"""Model-based configuration search: a tree-ensemble surrogate in place of the
exhaustive grid.

The pages tune each shape ahead of time over the algorithmic variants and
scheduling parameters and describe the search as tree-based ("Helion nel
backend vLLM", ai-radar.it, paragraphs 3 and 7; "Helion DSL added to vLLM to
autotune linear inference backends", signaltitans.com, "Hybrid Dispatch and
Autotuning").  This is that idea as a sequential model-based search:

1. time a seeded random sample of the feasible configurations;
2. fit an extremely-randomized-trees regressor to log(time) over a feature
   vector of each configuration (tile shape, layout, split, rotation, fuse
   mode and the workgroup count it implies for the problem);
3. time the configurations with the lowest lower confidence bound (mean minus
   the spread of the trees' predictions), refit, and repeat until the budget
   of timings is spent;
4. return the fastest configuration actually timed.

No prediction is ever trusted for the result: the table only holds timed
configurations.  The LLM-seeded variant the pages mention is not used.
"""
from __future__ import annotations

import math

import numpy as np


def config_features(info: dict, cfg: dict, M: int, N: int, K: int) -> list:
    """Numeric description of one configuration for problem (M, N, K).
    `info` holds the tile fields of cfg's kernel_id (qbg_kernel_info)."""
    tile_n = info["tile_n"]
    tiles = -(-N // tile_n)
    split = cfg.get("split_k", 1)
    return [
        tile_n, info["waves_n"], info["waves_k"], info["k_unroll"], info["stages"],
        info.get("waves_m", 1), info.get("tile_m", 32), cfg.get("swap_ab", 0),
        math.log2(split), cfg.get("rotate", 0),
        math.log2(tiles * split),                      # workgroups of the launch
        math.log2(max(1, K // split)),                 # K bytes per workgroup
        math.log2(M), math.log2(N), math.log2(K),
        cfg.get("fuse", 0),                            # fused ops: how quantization is done
    ]


def model_search(candidates, features, measure, budget: int, init: int = 0, batch: int = 4,
                 seed: int = 0, kappa: float = 1.0):
    """Search `candidates` (any objects) for the one with the smallest measure().

    features: candidate -> list of floats; measure: candidate -> positive time;
    budget: the most measurements to take.  Returns (best index, {index: time}).
    """
    from sklearn.ensemble import ExtraTreesRegressor

    n = len(candidates)
    if n == 0:
        raise ValueError("no candidates")
    budget = max(1, min(budget, n))
    X = np.asarray([features(c) for c in candidates], dtype=np.float64)
    rng = np.random.default_rng(seed)
    init = min(budget, init or max(4, budget // 3))
    measured = {}
    for i in rng.permutation(n)[:init]:
        measured[int(i)] = float(measure(candidates[int(i)]))
    while len(measured) < budget:
        idx = np.fromiter(measured, dtype=np.int64)
        y = np.log(np.asarray([measured[i] for i in idx]))
        model = ExtraTreesRegressor(n_estimators=64, random_state=seed, min_samples_leaf=1)
        model.fit(X[idx], y)
        rest = np.setdiff1d(np.arange(n), idx)
        per_tree = np.stack([t.predict(X[rest]) for t in model.estimators_])
        lcb = per_tree.mean(axis=0) - kappa * per_tree.std(axis=0)
        take = min(batch, budget - len(measured), len(rest))
        for j in np.argsort(lcb, kind="stable")[:take]:
            i = int(rest[j])
            measured[i] = float(measure(candidates[i]))
    best = min(measured, key=measured.get)
    return best, measured
