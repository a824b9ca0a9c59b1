"""Exact-arithmetic brute force for tiny inputs (Python Fractions and Decimals).

A second, independent reading of the same definitions the oracle follows,
written without any floating point: rounding to binary32, E4M3, int8, UE8M0
and bf16 is done on exact rationals, and the fused RMSNorm / SiLU steps are
evaluated with 60-digit decimals.  Only usable for a handful of elements.
"""
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np


def _floor_log2(a: Fraction) -> int:
    """Largest e with 2^e <= a, for a > 0."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def _round_half_even(q: Fraction) -> int:
    f = q.numerator // q.denominator
    r = q - f
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and f % 2 == 1):
        f += 1
    return f


def round_binary(x: Fraction, sig_bits: int, min_exp: int) -> Fraction:
    """Round x to nearest (ties even) on a binary grid with sig_bits significant bits.

    min_exp is the exponent of the smallest normal number; below it the grid
    spacing stays 2^(min_exp - sig_bits + 1) (gradual underflow).
    """
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = max(_floor_log2(a), min_exp)
    ulp = Fraction(2) ** (e - sig_bits + 1)
    return sign * _round_half_even(a / ulp) * ulp


def fl32(x: Fraction) -> Fraction:
    return round_binary(x, 24, -126)


def bf16(x: Fraction) -> Fraction:
    return round_binary(x, 8, -126)


def e4m3_value(code: int) -> Fraction:
    s = -1 if code & 0x80 else 1
    e = (code >> 3) & 15
    m = code & 7
    if e == 15 and m == 7:
        raise ValueError("NaN code")
    if e == 0:
        return s * Fraction(m, 8) * Fraction(2) ** -6
    return s * (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)


_E4M3_POS = [(c, e4m3_value(c)) for c in range(0x7F)]  # 0x00..0x7E


def e4m3_encode(x: Fraction, negative_zero: bool = False) -> int:
    """Exhaustive nearest search over all non-negative finite codes; ties to the even code."""
    a = abs(x)
    best = None
    for c, v in _E4M3_POS:
        d = abs(v - a)
        if best is None or d < best[1] or (d == best[1] and c % 2 == 0):
            best = (c, d)
    neg = x < 0 or (x == 0 and negative_zero)
    return best[0] | (0x80 if neg else 0)


def i8_encode(x: Fraction) -> int:
    return max(-127, min(127, _round_half_even(x)))


def ue8m0_encode(s: Fraction) -> int:
    p = _floor_log2(s)
    if Fraction(2) ** p < s:
        p += 1
    return p + 127


def frac_of_bf16(bits) -> Fraction:
    u = int(bits) << 16
    f = np.array([u], dtype=np.uint32).view(np.float32)[0]
    return Fraction(float(f))


def quant_values(vals, qtype: str, ue8m0: bool = False):
    """Quantize exact values sharing one scale -> (codes, scale as Fraction, ue8m0 code or None)."""
    qmax = Fraction(448) if qtype == "fp8" else Fraction(127)
    amax = max(abs(v) for v in vals)
    s = fl32(amax / qmax) if amax > 0 else Fraction(1)
    code = None
    if ue8m0:
        code = ue8m0_encode(s)
        s = Fraction(2) ** (code - 127)
    out = []
    for v in vals:
        t = fl32(v / s)
        t = max(-qmax, min(qmax, t))
        if qtype == "fp8":
            out.append(e4m3_encode(t, negative_zero=(v < 0)))
        else:
            out.append(i8_encode(t))
    return out, s, code


def dequant(code, qtype: str) -> Fraction:
    if qtype == "fp8":
        return e4m3_value(int(code))
    return Fraction(int(code))


# ---- fused pre-quantization steps in 60-digit decimal -----------------------

getcontext().prec = 60


def _dec(fr: Fraction) -> Decimal:
    return Decimal(fr.numerator) / Decimal(fr.denominator)


def _dec_to_frac(d: Decimal) -> Fraction:
    return Fraction(d)


def rms_norm_values(x_row, w, eps: float):
    """y_k = fl32(x_k * w_k / sqrt(mean(x^2) + eps)) with a 60-digit intermediate."""
    xs = [_dec(v) for v in x_row]
    ws = [_dec(v) for v in w]
    ss = sum(v * v for v in xs)
    r = Decimal(1) / (ss / Decimal(len(xs)) + _dec(Fraction(eps))).sqrt()
    return [fl32(_dec_to_frac(xv * r * wv)) for xv, wv in zip(xs, ws)]


def silu_mul_values(g_row, u_row):
    """y = fl32(g / (1 + exp(-g)) * u) with a 60-digit intermediate."""
    out = []
    for g, u in zip(g_row, u_row):
        gd, ud = _dec(g), _dec(u)
        out.append(fl32(_dec_to_frac(gd / (Decimal(1) + (-gd).exp()) * ud)))
    return out


def near_fp32_midpoint(exact: Fraction, rel: float = 2.0 ** -40) -> bool:
    """True if exact lies within rel*|exact| of a midpoint between two binary32 neighbours."""
    if exact == 0:
        return False
    r = fl32(exact)
    a = abs(exact)
    e = max(_floor_log2(a), -126)
    ulp = Fraction(2) ** (e - 23)
    mid_lo = abs(r) - ulp / 2
    mid_hi = abs(r) + ulp / 2
    tol = Fraction(rel) * a
    return abs(a - mid_lo) <= tol or abs(a - mid_hi) <= tol
