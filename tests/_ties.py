"""Element-exact acceptance of the fused producers' fp32 rounding ties.

The fused producers (RMSNorm or SiLU-and-mul, then FP8 quantization) take
each value to quantize as an fp64 evaluation rounded once to fp32.  Two
correct evaluations of that fp64 step can round differently only where the
fp64 value lies within 2^-40 |v| of the midpoint between two adjacent fp32
numbers: a tie element.

A quantization unit (a token row, or one 1 x 128 group) where the GPU's
codes or scale differ from the oracle's is accepted only if the oracle's own
quantizer, applied to the same fp32 values with ONE tie element of that unit
rounded to its other fp32 neighbour, reproduces the GPU's codes and scale
bit for bit.  That covers both ways a tie shows: a differing code at the tie
element itself, and a differing scale (with every code of the unit re-rounded)
when the tie element sets the unit's amax.  A differing byte anywhere else, or
a differing scale whose amax element is not a tie, is a failure.
"""
import numpy as np

import oracle


def _neighbours(y64):
    """fp32 round-to-nearest of y64, its tie mask, and the other fp32 candidate."""
    r = y64.astype(np.float32)
    ties = oracle.fp32_midpoint_ties(y64)
    up = np.nextafter(r, np.float32(np.inf))
    dn = np.nextafter(r, np.float32(-np.inf))
    r64 = r.astype(np.float64)
    d_up = np.abs(y64 - (r64 + up.astype(np.float64)) / 2)
    d_dn = np.abs(y64 - (r64 + dn.astype(np.float64)) / 2)
    alt = np.where(d_up <= d_dn, up, dn)
    return r, ties, alt


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint8)


def explain(y64, q_gpu, s_gpu, quantize, unit):
    """Tie flips that explain the GPU's quantization of the fp64 values y64.

    quantize(y32 [U, unit]) -> (q [U, unit], s [U, ...]) is the oracle's
    quantizer of fp32 values, one unit per row.  Returns (flips, unexplained):
    flips lists (unit, element) of every accepted re-rounding, unexplained the
    units no single tie re-rounding reproduces.
    """
    y64 = np.asarray(y64, dtype=np.float64)
    U = y64.size // unit
    y = y64.reshape(U, unit)
    qg = np.ascontiguousarray(q_gpu).reshape(U, unit)
    sg = _bits(s_gpu).reshape(U, -1)
    r, ties, alt = _neighbours(y)
    qo, so = quantize(r)
    so = _bits(so).reshape(U, -1)
    bad = np.nonzero((qg != qo).any(axis=1) | (sg != so).any(axis=1))[0]
    flips, unexplained = [], []
    for u in bad:
        found = None
        for e in np.nonzero(ties[u])[0]:
            trial = r[u].copy()
            trial[e] = alt[u, e]
            q1, s1 = quantize(trial[None, :])
            if np.array_equal(q1[0], qg[u]) and np.array_equal(_bits(s1).reshape(-1), sg[u]):
                found = (int(u), int(e))
                break
        if found is None:
            unexplained.append(int(u))
        else:
            flips.append(found)
    return flips, unexplained


def per_token(qtype=oracle.FP8):
    """The oracle's per-token quantizer of fp32 rows."""
    return lambda y32: oracle.quant_per_token_f32(qtype, y32)


def per_group(scale_fmt, group=oracle.GROUP):
    """The oracle's 1 x group quantizer, one group per row."""
    return lambda y32: oracle.quant_group_f32(scale_fmt, y32, group)


def check(y64, q_gpu, s_gpu, quantize, unit, what, max_flips=1):
    """Assert the GPU's quantization is the oracle's up to at most max_flips tie
    re-roundings; returns the number of flips."""
    flips, unexplained = explain(y64, q_gpu, s_gpu, quantize, unit)
    assert not unexplained, "%s: units differ without a tie that explains them: %s" % (
        what, unexplained[:5])
    assert len(flips) <= max_flips, "%s: %d tie re-roundings (at most %d allowed): %s" % (
        what, len(flips), max_flips, flips[:5])
    return len(flips)
