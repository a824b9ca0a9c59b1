"""Seeded synthetic inputs for the decode-path workloads.

This module only draws random numbers and rounds them to bf16 (the input
format); it holds none of the quantization or GEMM arithmetic.  The tests,
the oracle runs and the benchmark all draw their inputs from here, so both
sides of every parity check see the same bits.

Recipe (the pages use real Qwen3 projections and serving traffic, which are
not available; these draws stand in for them):

* every tensor gets its own ``numpy.random.Generator`` seeded with
  ``SeedSequence([workload, N, K, stream])``, stream 0 for weights, 1 for
  activations, 2 for the RMSNorm weight;
* values are drawn in fp32 and rounded to bf16 (round to nearest even);
* activations are drawn at the largest token count of the workload, smaller
  token counts take the first rows.

Distributions (per workload):

* ``normal``           N(0, 1)
* ``normal_outliers``  N(0, 1), then each element independently multiplied by
                       50 with probability 0.001 (before the bf16 rounding)
* ``student_t``        0.5 * Student-t with 4 degrees of freedom
* weights              N(0, 0.02)
* RMSNorm weight       1 + N(0, 0.1)
"""
from __future__ import annotations

import numpy as np

# Workload ids used in the seeds.
TINY_FP8 = 1         # FP8-dynamic, N=512, K=1024
DECODE_FP8 = 2       # FP8-dynamic at 8B-decoder linear shapes
DECODE_INT8 = 3      # W8A8-INT8
DECODE_BLOCK = 4     # Block-FP8 at 32B-decoder shapes
MLP_CHAIN = 5        # fused MLP chain
BLOCK_CHAIN = 6      # Block-FP8 MLP chain at the 32B-decoder shapes
MOE = 7              # grouped (mixture-of-experts) GEMM

TINY_SHAPES = [(512, 1024)]
DECODE_SHAPES = [(6144, 4096), (4096, 4096), (24576, 4096), (4096, 12288)]
BLOCK_SHAPES = [(10240, 5120), (5120, 8192), (51200, 5120), (5120, 25600)]
DECODE_MS = [1, 2, 4, 8, 16, 32]
INT8_MS = [1, 4, 16, 32]
BLOCK_MS = [1, 8, 32]
TINY_MS = [1, 16, 32]
CHAIN_MS = [1, 32, 128, 256]
CHAIN_HIDDEN = 4096
CHAIN_INTER = 12288
BLOCK_CHAIN_HIDDEN = 5120
BLOCK_CHAIN_INTER = 25600
BLOCK_CHAIN_MS = [1, 8, 32]
# Mixture-of-experts decode layer of a 30B-A3B-class model: 128 experts, top-8
# routing, hidden 2048, expert intermediate 768 (gate_up 1536 x 2048 and
# down 2048 x 768 per expert).
MOE_EXPERTS = 128
MOE_TOP_K = 8
MOE_HIDDEN = 2048
MOE_INTER = 768
MOE_MS = [1, 8, 32]


def _rng(workload: int, n: int, k: int, stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([workload, n, k, stream]))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even) and return the bits as uint16."""
    import torch  # the conversion is torch's own fp32 -> bf16 cast

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 values (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def draw(workload: int, n: int, k: int, stream: int, shape, kind: str) -> np.ndarray:
    """Draw fp32 values of ``shape`` with distribution ``kind``; returns bf16 bits."""
    g = _rng(workload, n, k, stream)
    size = int(np.prod(shape))
    if kind == "normal":
        v = g.standard_normal(size, dtype=np.float32)
    elif kind == "normal_outliers":
        v = g.standard_normal(size, dtype=np.float32)
        mask = g.random(size, dtype=np.float32) < np.float32(0.001)
        v[mask] *= np.float32(50.0)
    elif kind == "student_t":
        v = (0.5 * g.standard_t(4, size)).astype(np.float32)
    elif kind == "weight":
        v = g.standard_normal(size, dtype=np.float32) * np.float32(0.02)
    elif kind == "norm_weight":
        v = np.float32(1.0) + g.standard_normal(size, dtype=np.float32) * np.float32(0.1)
    else:
        raise ValueError("unknown distribution %r" % kind)
    return to_bf16_bits(v.reshape(shape))


def activation_kind(workload: int) -> str:
    return {TINY_FP8: "normal", DECODE_FP8: "normal_outliers", DECODE_INT8: "student_t",
            DECODE_BLOCK: "normal", MLP_CHAIN: "normal", BLOCK_CHAIN: "normal",
            MOE: "normal"}[workload]


def activations(workload: int, n: int, k: int, m: int) -> np.ndarray:
    """Activation rows [m, k] (bf16 bits) for the (n, k) problem of ``workload``."""
    return draw(workload, n, k, 1, (m, k), activation_kind(workload))


def weights(workload: int, n: int, k: int) -> np.ndarray:
    """Weight master [n, k] (bf16 bits), N(0, 0.02)."""
    return draw(workload, n, k, 0, (n, k), "weight")


def norm_weight(h: int) -> np.ndarray:
    """RMSNorm weight [h] (bf16 bits), 1 + N(0, 0.1)."""
    return draw(MLP_CHAIN, h, h, 2, (h,), "norm_weight")


def moe_routing(m: int, experts: int, top_k: int, seed: int = 0):
    """Seeded routing of m tokens to top_k distinct experts each (uniform).
    Returns (order, offsets): the routed rows grouped by expert -- order[i] is
    the token of routed row i -- and int32 offsets [experts + 1], expert e
    owning rows offsets[e] .. offsets[e+1]-1.  This prepares inputs; it is the
    router's job, outside the GEMM."""
    g = _rng(MOE, m, experts, 100 + seed)
    choice = np.stack([g.choice(experts, size=top_k, replace=False) for _ in range(m)])
    pairs = sorted((int(e), t) for t in range(m) for e in choice[t])
    order = np.array([t for _, t in pairs], dtype=np.int64)
    counts = np.bincount([e for e, _ in pairs], minlength=experts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return order, offsets
