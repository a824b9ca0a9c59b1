"""CPU oracle for the 8-bit scaled-matmul decode path (numpy front end).

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  It shares no code with
the HIP library and never imports it.

The arithmetic lives in ``oracle.c`` (plain loops, fp64/int64 accumulation);
this module builds it with gcc when needed and wraps it with numpy arrays.
Every function states the operation it follows; the readings of the pages
that fix the arithmetic are stated in ``oracle.c``.

Parity status: the codecs, quantizers and GEMMs are pinned by the tests in
``tests/test_oracle_*.py`` (format closed forms, hand-worked cases, a
Fraction/Decimal brute force, library special cases and identities).  The
fused RMSNorm and SiLU-and-mul pre-quantization arithmetic is pinned against
a Decimal evaluation of this reading of the pages, a closed form, special
values and torch's float64 CPU rms_norm / silu (independent implementations
of the same definitions), not against any number the pages print (they print
none): parity unpinned with respect to the pages for that step.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

FP8 = 0
INT8 = 1
SCALE_F32 = 0
SCALE_UE8M0 = 1
GROUP = 128

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC",
          "-std=c11", "-Wall"]


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so next to it (gcc)."""
    if force or not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def build_sanitized(out_dir: str) -> str:
    """oracle.c with AddressSanitizer and UndefinedBehaviorSanitizer, built with
    ROCm's clang so that it shares one sanitizer runtime with the library's
    host-sanitizer build (both run under that runtime, preloaded)."""
    clang = "/opt/rocm/llvm/bin/clang"
    os.makedirs(out_dir, exist_ok=True)
    out = os.path.join(out_dir, "liboracle_san.so")
    san = ["-fsanitize" + "=address,undefined", "-fno-sanitize-recover=all", "-shared-libsan",
           "-g", "-fno-omit-frame-pointer"]
    subprocess.check_call([clang, *[f for f in CFLAGS if f != "-O2"], "-O1", *san, _SRC, "-o", out,
                           "-lm"])
    return out


_lib = None


def lib() -> ctypes.CDLL:
    """The oracle library.  QBG_ORACLE_LIB may name another build of oracle.c
    (the mutation tests load deliberately broken copies through it)."""
    global _lib
    if _lib is None:
        path = os.environ.get("QBG_ORACLE_LIB") or build()
        _lib = ctypes.CDLL(path)
        _declare(_lib)
    return _lib


def _declare(L: ctypes.CDLL) -> None:
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I = ctypes.c_int
    L.orc_e4m3_decode.restype = ctypes.c_double
    L.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
    L.orc_e4m3_encode.restype = ctypes.c_uint8
    L.orc_e4m3_encode.argtypes = [ctypes.c_float]
    L.orc_i8_encode.restype = ctypes.c_int8
    L.orc_i8_encode.argtypes = [ctypes.c_float]
    L.orc_ue8m0_decode.restype = ctypes.c_double
    L.orc_ue8m0_decode.argtypes = [ctypes.c_uint8]
    L.orc_ue8m0_encode.restype = ctypes.c_uint8
    L.orc_ue8m0_encode.argtypes = [ctypes.c_float]
    L.orc_bf16_to_double.restype = ctypes.c_double
    L.orc_bf16_to_double.argtypes = [ctypes.c_uint16]
    L.orc_bf16_from_double.restype = ctypes.c_uint16
    L.orc_bf16_from_double.argtypes = [ctypes.c_double]
    L.orc_quant_per_token.restype = None
    L.orc_quant_per_token.argtypes = [I, P, I64, I64, P, P]
    L.orc_quant_per_token_f32.restype = None
    L.orc_quant_per_token_f32.argtypes = [I, P, I64, I64, P, P]
    L.orc_quant_group.restype = None
    L.orc_quant_group.argtypes = [I, P, I64, I64, I64, P, P]
    L.orc_quant_weight_per_channel.restype = None
    L.orc_quant_weight_per_channel.argtypes = [I, P, I64, I64, P, P]
    L.orc_quant_weight_block.restype = None
    L.orc_quant_weight_block.argtypes = [I, P, I64, I64, P, P]
    L.orc_rms_norm_quant.restype = None
    L.orc_rms_norm_quant.argtypes = [P, P, ctypes.c_float, I64, I64, P, P, P]
    L.orc_silu_mul_quant.restype = None
    L.orc_rms_norm_prequant_f64.restype = None
    L.orc_rms_norm_prequant_f64.argtypes = [P, P, ctypes.c_float, I64, I64, P]
    L.orc_silu_mul_prequant_f64.restype = None
    L.orc_silu_mul_prequant_f64.argtypes = [P, I64, I64, P]
    L.orc_silu_mul_quant.argtypes = [P, I64, I64, P, P, P]
    L.orc_quant_group_f32.restype = None
    L.orc_quant_group_f32.argtypes = [I, P, I64, I64, I64, P, P]
    L.orc_rms_norm_group_quant.restype = None
    L.orc_rms_norm_group_quant.argtypes = [P, P, ctypes.c_float, I64, I64, I64, I, P, P, P]
    L.orc_silu_mul_group_quant.restype = None
    L.orc_silu_mul_group_quant.argtypes = [P, I64, I64, I64, I, P, P, P]
    L.orc_scaled_mm.restype = I
    L.orc_scaled_mm.argtypes = [I, P, P, P, P, I64, I64, I64, I64, I, P, P, P]
    L.orc_grouped_scaled_mm.restype = I
    L.orc_grouped_scaled_mm.argtypes = [I, P, P, P, P, P, I64, I64, I64, P, P, P]
    L.orc_block_scaled_mm.restype = None
    L.orc_block_scaled_mm.argtypes = [I, P, P, P, P, I64, I64, I64, I64, I, P, P]


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError("expected %s, got %s" % (dtype, a.dtype))
    return a


# --------------------------------------------------------------------------
# Codecs (scalar)
# --------------------------------------------------------------------------

def e4m3_decode(code: int) -> float:
    return lib().orc_e4m3_decode(code)


def e4m3_encode(x: float) -> int:
    return lib().orc_e4m3_encode(x)


def i8_encode(x: float) -> int:
    return lib().orc_i8_encode(x)


def ue8m0_encode(s: float) -> int:
    return lib().orc_ue8m0_encode(s)


def ue8m0_decode(e: int) -> float:
    return lib().orc_ue8m0_decode(e)


def bf16_from_double(v: float) -> int:
    return lib().orc_bf16_from_double(v)


def bf16_to_double(b: int) -> float:
    return lib().orc_bf16_to_double(b)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64 (a bit shift)."""
    u = (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16)
    return u.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# Quantizers
# --------------------------------------------------------------------------

def quant_per_token(qtype: int, x_bf16: np.ndarray):
    """Per-token quantization of bf16 bits x [M,K] -> (q [M,K], s fp32 [M])."""
    x = _c(x_bf16, np.uint16)
    M, K = x.shape
    q = np.empty((M, K), dtype=np.uint8 if qtype == FP8 else np.int8)
    s = np.empty((M,), dtype=np.float32)
    lib().orc_quant_per_token(qtype, _ptr(x), M, K, _ptr(q), _ptr(s))
    return q, s


def quant_per_token_f32(qtype: int, y: np.ndarray):
    """Per-token quantization of fp32 values y [M,K] -> (q, s)."""
    y = _c(y, np.float32)
    M, K = y.shape
    q = np.empty((M, K), dtype=np.uint8 if qtype == FP8 else np.int8)
    s = np.empty((M,), dtype=np.float32)
    lib().orc_quant_per_token_f32(qtype, _ptr(y), M, K, _ptr(q), _ptr(s))
    return q, s


def quant_group(scale_fmt: int, x_bf16: np.ndarray, group: int = GROUP):
    """1 x group FP8 quantization -> (q [M,K], s [M,K/group] fp32 or uint8)."""
    x = _c(x_bf16, np.uint16)
    M, K = x.shape
    assert K % group == 0
    q = np.empty((M, K), dtype=np.uint8)
    s = np.empty((M, K // group), dtype=np.uint8 if scale_fmt == SCALE_UE8M0 else np.float32)
    lib().orc_quant_group(scale_fmt, _ptr(x), M, K, group, _ptr(q), _ptr(s))
    return q, s


def quant_weight_per_channel(qtype: int, w_bf16: np.ndarray):
    """Per-output-channel weight quantization of W [N,K] -> (q [N,K], s fp32 [N])."""
    w = _c(w_bf16, np.uint16)
    N, K = w.shape
    q = np.empty((N, K), dtype=np.uint8 if qtype == FP8 else np.int8)
    s = np.empty((N,), dtype=np.float32)
    lib().orc_quant_weight_per_channel(qtype, _ptr(w), N, K, _ptr(q), _ptr(s))
    return q, s


def quant_weight_block(scale_fmt: int, w_bf16: np.ndarray):
    """128x128 block FP8 weight quantization -> (q [N,K], s [ceil(N/128), K/128])."""
    w = _c(w_bf16, np.uint16)
    N, K = w.shape
    assert K % GROUP == 0
    nb = (N + GROUP - 1) // GROUP
    q = np.empty((N, K), dtype=np.uint8)
    s = np.empty((nb, K // GROUP), dtype=np.uint8 if scale_fmt == SCALE_UE8M0 else np.float32)
    lib().orc_quant_weight_block(scale_fmt, _ptr(w), N, K, _ptr(q), _ptr(s))
    return q, s


def rms_norm_quant(x_bf16: np.ndarray, w_bf16: np.ndarray, eps: float = 1e-6):
    """Fused RMSNorm + per-token FP8 quant -> (y fp32 [M,H], q [M,H], s [M])."""
    x = _c(x_bf16, np.uint16)
    w = _c(w_bf16, np.uint16)
    M, H = x.shape
    assert w.shape == (H,)
    y = np.empty((M, H), dtype=np.float32)
    q = np.empty((M, H), dtype=np.uint8)
    s = np.empty((M,), dtype=np.float32)
    lib().orc_rms_norm_quant(_ptr(x), _ptr(w), eps, M, H, _ptr(y), _ptr(q), _ptr(s))
    return y, q, s


def silu_mul_quant(gate_up_bf16: np.ndarray):
    """Fused SiLU(gate)*up + per-token FP8 quant -> (y fp32 [M,I], q [M,I], s [M])."""
    gu = _c(gate_up_bf16, np.uint16)
    M, I2 = gu.shape
    assert I2 % 2 == 0
    I = I2 // 2
    y = np.empty((M, I), dtype=np.float32)
    q = np.empty((M, I), dtype=np.uint8)
    s = np.empty((M,), dtype=np.float32)
    lib().orc_silu_mul_quant(_ptr(gu), M, I, _ptr(y), _ptr(q), _ptr(s))
    return y, q, s


def quant_group_f32(scale_fmt: int, y_f32: np.ndarray, group: int = GROUP):
    """1 x group FP8 quantization of fp32 values -> (q [M,K], s [M,K/group])."""
    y = _c(y_f32, np.float32)
    M, K = y.shape
    assert K % group == 0
    q = np.empty((M, K), dtype=np.uint8)
    s = np.empty((M, K // group), dtype=np.uint8 if scale_fmt == SCALE_UE8M0 else np.float32)
    lib().orc_quant_group_f32(scale_fmt, _ptr(y), M, K, group, _ptr(q), _ptr(s))
    return q, s


def rms_norm_group_quant(scale_fmt: int, x_bf16: np.ndarray, w_bf16: np.ndarray,
                         eps: float = 1e-6, group: int = GROUP):
    """Fused RMSNorm + 1 x group FP8 quant -> (y fp32 [M,H], q [M,H], s [M,H/group])."""
    x = _c(x_bf16, np.uint16)
    w = _c(w_bf16, np.uint16)
    M, H = x.shape
    assert w.shape == (H,) and H % group == 0
    y = np.empty((M, H), dtype=np.float32)
    q = np.empty((M, H), dtype=np.uint8)
    s = np.empty((M, H // group), dtype=np.uint8 if scale_fmt == SCALE_UE8M0 else np.float32)
    lib().orc_rms_norm_group_quant(_ptr(x), _ptr(w), eps, M, H, group, scale_fmt, _ptr(y),
                                   _ptr(q), _ptr(s))
    return y, q, s


def silu_mul_group_quant(scale_fmt: int, gate_up_bf16: np.ndarray, group: int = GROUP):
    """Fused SiLU(gate)*up + 1 x group FP8 quant -> (y fp32 [M,I], q [M,I], s [M,I/group])."""
    gu = _c(gate_up_bf16, np.uint16)
    M, I2 = gu.shape
    I = I2 // 2
    assert I2 % 2 == 0 and I % group == 0
    y = np.empty((M, I), dtype=np.float32)
    q = np.empty((M, I), dtype=np.uint8)
    s = np.empty((M, I // group), dtype=np.uint8 if scale_fmt == SCALE_UE8M0 else np.float32)
    lib().orc_silu_mul_group_quant(_ptr(gu), M, I, group, scale_fmt, _ptr(y), _ptr(q), _ptr(s))
    return y, q, s


def rms_norm_prequant_f64(x_bf16: np.ndarray, w_bf16: np.ndarray, eps: float = 1e-6):
    """The fused RMSNorm's fp64 values before their rounding to fp32 [M,H]."""
    x = _c(x_bf16, np.uint16)
    w = _c(w_bf16, np.uint16)
    M, H = x.shape
    y = np.empty((M, H), dtype=np.float64)
    lib().orc_rms_norm_prequant_f64(_ptr(x), _ptr(w), eps, M, H, _ptr(y))
    return y


def silu_mul_prequant_f64(gate_up_bf16: np.ndarray):
    """The fused SiLU-and-mul's fp64 values before their rounding to fp32 [M,I]."""
    gu = _c(gate_up_bf16, np.uint16)
    M, I2 = gu.shape
    y = np.empty((M, I2 // 2), dtype=np.float64)
    lib().orc_silu_mul_prequant_f64(_ptr(gu), M, I2 // 2, _ptr(y))
    return y


def fp32_midpoint_ties(y64: np.ndarray, rel: float = 2.0 ** -40) -> np.ndarray:
    """Elements whose fp64 value lies within rel*|v| of a midpoint between two
    adjacent fp32 numbers: there two correct evaluations may round differently."""
    y64 = np.asarray(y64, dtype=np.float64)
    r = y64.astype(np.float32).astype(np.float64)
    up = np.nextafter(r.astype(np.float32), np.float32(np.inf)).astype(np.float64)
    dn = np.nextafter(r.astype(np.float32), np.float32(-np.inf)).astype(np.float64)
    mid_hi = (r + up) / 2
    mid_lo = (r + dn) / 2
    tol = rel * np.abs(y64)
    return (np.abs(y64 - mid_hi) <= tol) | (np.abs(y64 - mid_lo) <= tol)


# --------------------------------------------------------------------------
# GEMMs
# --------------------------------------------------------------------------

def scaled_mm(qtype: int, qa, sa, qw, sw, split_k: int = 1, swap_ab: bool = False):
    """Per-channel scaled GEMM -> (ref fp64 [M,N], out bf16 bits [M,N], acc int32 or None)."""
    dt = np.uint8 if qtype == FP8 else np.int8
    qa = _c(qa, dt)
    qw = _c(qw, dt)
    sa = _c(sa, np.float32)
    sw = _c(sw, np.float32)
    M, K = qa.shape
    N, K2 = qw.shape
    assert K == K2 and sa.shape == (M,) and sw.shape == (N,)
    assert split_k >= 1 and K % split_k == 0
    ref = np.empty((M, N), dtype=np.float64)
    out = np.empty((M, N), dtype=np.uint16)
    acc = np.empty((M, N), dtype=np.int32) if qtype == INT8 else None
    rc = lib().orc_scaled_mm(qtype, _ptr(qa), _ptr(sa), _ptr(qw), _ptr(sw), M, N, K,
                             split_k, int(bool(swap_ab)), _ptr(ref), _ptr(out), _ptr(acc))
    if rc != 0:
        raise OverflowError("int8 accumulator outside int32")
    return ref, out, acc


def grouped_scaled_mm(qtype: int, qa, sa, qw, sw, offsets):
    """Grouped (mixture-of-experts) per-channel scaled GEMM: rows offsets[e]..offsets[e+1]
    use qw[e] [N,K], sw[e] [N] -> (ref fp64 [T,N], out bf16 bits [T,N], acc int32 or None)."""
    dt = np.uint8 if qtype == FP8 else np.int8
    qa = _c(qa, dt)
    qw = _c(qw, dt)
    sa = _c(sa, np.float32)
    sw = _c(sw, np.float32)
    off = _c(np.asarray(offsets, dtype=np.int64), np.int64)
    T, K = qa.shape
    E, N, K2 = qw.shape
    assert K2 == K and sw.shape == (E, N) and off.shape == (E + 1,)
    assert off[0] == 0 and off[-1] == T and np.all(np.diff(off) >= 0)
    ref = np.empty((T, N), dtype=np.float64)
    out = np.empty((T, N), dtype=np.uint16)
    acc = np.empty((T, N), dtype=np.int32) if qtype == INT8 else None
    st = lib().orc_grouped_scaled_mm(qtype, _ptr(qa), _ptr(sa), _ptr(qw), _ptr(sw), _ptr(off), E,
                                     N, K, _ptr(ref), _ptr(out), _ptr(acc))
    if st != 0:
        raise OverflowError("int8 accumulator leaves int32")
    return ref, out, acc


def block_scaled_mm(scale_fmt: int, qa, sa, qw, sw, split_k: int = 1, swap_ab: bool = False):
    """Block-FP8 scaled GEMM -> (ref fp64 [M,N], out bf16 bits [M,N])."""
    sdt = np.uint8 if scale_fmt == SCALE_UE8M0 else np.float32
    qa = _c(qa, np.uint8)
    qw = _c(qw, np.uint8)
    sa = _c(sa, sdt)
    sw = _c(sw, sdt)
    M, K = qa.shape
    N, K2 = qw.shape
    assert K == K2 and K % GROUP == 0
    ng = K // GROUP
    assert sa.shape == (M, ng) and sw.shape == ((N + GROUP - 1) // GROUP, ng)
    assert split_k >= 1 and ng % split_k == 0
    ref = np.empty((M, N), dtype=np.float64)
    out = np.empty((M, N), dtype=np.uint16)
    lib().orc_block_scaled_mm(scale_fmt, _ptr(qa), _ptr(sa), _ptr(qw), _ptr(sw), M, N, K,
                              split_k, int(bool(swap_ab)), _ptr(ref), _ptr(out))
    return ref, out


def within_tolerance(got: np.ndarray, ref: np.ndarray, rel: float = 1e-2, abs_floor: float = 1e-3):
    """The GEMM parity bar: |g - r| <= max(rel*|r|, abs_floor) elementwise.

    Returns (ok, worst ratio |g-r|/bound).
    """
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    bound = np.maximum(rel * np.abs(ref), abs_floor)
    ratio = np.abs(got - ref) / bound
    worst = float(ratio.max()) if ratio.size else 0.0
    return bool(worst <= 1.0), worst
