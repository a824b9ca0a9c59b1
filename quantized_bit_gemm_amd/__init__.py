"""MI355X-native (gfx950) 8-bit scaled-matmul backend for LLM decode.

A thin Python binding over libqbg.so (include/qbg.h).  Every function here
has the name of the C entry point it calls and only marshals arguments:
PyTorch supplies device memory (outputs are allocated with torch when not
given) and the current HIP stream; all arithmetic runs in the HIP kernels.
There is no CPU fallback: without the built library, or with tensors that
are not on a GPU, every call raises.

Formats on the torch side: bf16 tensors are torch.bfloat16; E4M3 codes and
UE8M0 scale bytes are torch.uint8; int8 codes are torch.int8; scales are
torch.float32.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# QBG_LIBRARY may name another build of the library (the host-sanitizer build,
# _build_san/libqbg_san.so, which has a configs/ link beside it).
LIB_PATH = os.environ.get("QBG_LIBRARY") or os.path.join(_PKG, "libqbg.so")
DEFAULT_TABLE = os.path.join(_PKG, "configs", "gfx950.txt")

QBG_FP8_E4M3 = 0
QBG_INT8 = 1
QBG_SCALE_F32 = 0
QBG_SCALE_UE8M0 = 1
QBG_OP_FP8 = 0
QBG_OP_INT8 = 1
QBG_OP_BLOCK_FP8 = 2
QBG_OP_BLOCK_UE8M0 = 3
QBG_OP_FP8_FUSED = 4
QBG_OP_INT8_FUSED = 5
QBG_OP_FP8_GROUPED = 6
QBG_OP_INT8_GROUPED = 7
# qbg_fuse_mode: how qbg_quantize_scaled_mm combines the quantizer with the GEMM.
QBG_FUSE_PUBLISH = 0
QBG_FUSE_LOCAL = 1
QBG_FUSE_SEPARATE = 2
QBG_E_SHAPE = 2
QBG_E_QTYPE = 4
QBG_E_WORKSPACE = 6
# Per-GPU scratch bytes of qbg_scaled_mm_noalloc (the header's macro).
QBG_NOALLOC_SCRATCH_BYTES = 65536 + (16 << 20)

STATUS_NAMES = {0: "QBG_OK", 1: "QBG_E_NULL", 2: "QBG_E_SHAPE", 3: "QBG_E_ALIGN",
                4: "QBG_E_QTYPE", 5: "QBG_E_SPLITK", 6: "QBG_E_WORKSPACE", 7: "QBG_E_TABLE",
                8: "QBG_E_HIP", 9: "QBG_E_CONFIG"}

# Every symbol include/qbg.h declares.
EXPORTS = [
    "qbg_abi_version", "qbg_status_str", "qbg_last_error", "qbg_quantize_per_token",
    "qbg_quantize_per_token_group", "qbg_quantize_weight_block",
    "qbg_rms_norm_quantize_per_token", "qbg_silu_mul_quantize_per_token",
    "qbg_convert_f32_to_e4m3", "qbg_scaled_mm", "qbg_scaled_mm_noalloc", "qbg_block_scaled_mm", "qbg_scaled_mm_i32",
    "qbg_quantize_scaled_mm", "qbg_set_fused_wait_limit",
    "qbg_rms_norm_quantize_per_token_group", "qbg_silu_mul_quantize_per_token_group",
    "qbg_grouped_scaled_mm",
    "qbg_config_table_load", "qbg_config_table_size", "qbg_config_lookup",
    "qbg_workspace_size", "qbg_workspace_init", "qbg_kernel_count", "qbg_kernel_info",
]


class QbgError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        super().__init__("%s: %s" % (STATUS_NAMES.get(status, str(status)), message))


class GemmConfig(ctypes.Structure):
    """qbg_gemm_config."""
    _fields_ = [("kernel_id", ctypes.c_int32), ("swap_ab", ctypes.c_int32),
                ("split_k", ctypes.c_int32), ("tile_n", ctypes.c_int32),
                ("waves_n", ctypes.c_int32), ("waves_k", ctypes.c_int32),
                ("k_unroll", ctypes.c_int32), ("stages", ctypes.c_int32),
                ("rotate", ctypes.c_int32), ("waves_m", ctypes.c_int32),
                ("tile_m", ctypes.c_int32), ("fuse", ctypes.c_int32)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


_lib = None
_lock = threading.Lock()


def _declare(L):
    P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    ST = ctypes.c_int
    CFG = ctypes.POINTER(GemmConfig)
    sig = {
        "qbg_abi_version": (ctypes.c_int, []),
        "qbg_status_str": (ctypes.c_char_p, [ST]),
        "qbg_last_error": (ctypes.c_char_p, []),
        "qbg_quantize_per_token": (ST, [ST, P, I64, I64, P, P, P]),
        "qbg_quantize_per_token_group": (ST, [P, I64, I64, I32, ST, P, P, P]),
        "qbg_quantize_weight_block": (ST, [P, I64, I64, ST, P, P, P]),
        "qbg_rms_norm_quantize_per_token": (ST, [P, P, ctypes.c_float, I64, I64, P, P, P]),
        "qbg_silu_mul_quantize_per_token": (ST, [P, I64, I64, P, P, P]),
        "qbg_rms_norm_quantize_per_token_group": (ST, [P, P, ctypes.c_float, I64, I64, I32, ST,
                                                       P, P, P]),
        "qbg_silu_mul_quantize_per_token_group": (ST, [P, I64, I64, I32, ST, P, P, P]),
        "qbg_convert_f32_to_e4m3": (ST, [P, P, I64, P]),
        "qbg_scaled_mm": (ST, [ST, P, P, P, P, I64, I64, I64, P, CFG, P, SZ, P]),
        "qbg_scaled_mm_noalloc": (ST, [ST, P, P, P, P, I64, I64, I64, P, CFG, P]),
        "qbg_block_scaled_mm": (ST, [ST, P, P, P, P, I64, I64, I64, P, CFG, P, SZ, P]),
        "qbg_scaled_mm_i32": (ST, [P, P, I64, I64, I64, P, CFG, P, SZ, P]),
        "qbg_quantize_scaled_mm": (ST, [ST, P, P, P, I64, I64, I64, P, P, P, CFG, P, SZ, P]),
        "qbg_set_fused_wait_limit": (I32, [I32]),
        "qbg_grouped_scaled_mm": (ST, [ST, P, P, P, P, P, I64, I64, I64, I64, P, CFG, P]),
        "qbg_config_table_load": (ST, [ctypes.c_char_p]),
        "qbg_config_table_size": (I64, []),
        "qbg_config_lookup": (ST, [ST, I64, I64, I64, CFG, ctypes.POINTER(I32)]),
        "qbg_workspace_size": (ST, [ST, I64, I64, I64, CFG, ctypes.POINTER(SZ)]),
        "qbg_workspace_init": (ST, [P, SZ, P]),
        "qbg_kernel_count": (I32, []),
        "qbg_kernel_info": (ST, [I32, CFG]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args


def lib() -> ctypes.CDLL:
    """The loaded libqbg.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise ImportError("libqbg.so is not built; run "
                                      "`python -m quantized_bit_gemm_amd.build`")
                L = ctypes.CDLL(LIB_PATH)
                _declare(L)
                # The library loads its tuned table itself on the first lookup
                # (QBG_CONFIG_TABLE, else configs/gfx950.txt beside it); a table named
                # in the environment is loaded here as well so that a malformed one
                # raises instead of leaving the built-in defaults.
                table = os.environ.get("QBG_CONFIG_TABLE")
                if table:
                    st = L.qbg_config_table_load(table.encode())
                    if st != 0:
                        raise QbgError(st, L.qbg_last_error().decode())
                _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise QbgError(status, lib().qbg_last_error().decode())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dev(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("qbg runs on the GPU only; got a tensor on %s" % t.device)
        if not t.is_contiguous():
            raise ValueError("qbg needs contiguous tensors")


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype(t, dt, name):
    if t.dtype != dt:
        raise TypeError("%s must be %s, got %s" % (name, dt, t.dtype))


# The library cannot see buffer sizes: every shape and dtype is checked here,
# before a pointer reaches the C ABI, so a mismatch raises instead of reading
# or writing past a device buffer.
_CODES = {QBG_FP8_E4M3: (torch.uint8, torch.float8_e4m3fn), QBG_INT8: (torch.int8,)}


def _codes(qtype):
    if qtype not in _CODES:
        raise ValueError("qtype must be QBG_FP8_E4M3 or QBG_INT8, got %r" % (qtype,))
    return _CODES[qtype]


def _expect(t, shape, dtypes, name):
    """t (if given) must have exactly `shape` and one of `dtypes`."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError("%s must be %s, got %s" % (name, " or ".join(map(str, dtypes)), t.dtype))


def _dims(t, nd, name):
    if t.dim() != nd:
        raise ValueError("%s must have %d dimensions, got shape %s" % (name, nd, tuple(t.shape)))
    return tuple(t.shape)


_F32 = (torch.float32,)
_BF16 = (torch.bfloat16,)


def _scale_types(fmt):
    if fmt not in (QBG_SCALE_F32, QBG_SCALE_UE8M0):
        raise ValueError("fmt must be QBG_SCALE_F32 or QBG_SCALE_UE8M0, got %r" % (fmt,))
    return (torch.uint8,) if fmt == QBG_SCALE_UE8M0 else _F32


def _cfg(config):
    if config is None:
        return None
    if isinstance(config, GemmConfig):
        return ctypes.byref(config)
    c = GemmConfig()
    c.kernel_id = int(config.get("kernel_id", 0))
    c.swap_ab = int(config.get("swap_ab", 0))
    c.split_k = int(config.get("split_k", 1))
    c.rotate = int(config.get("rotate", 0))
    c.fuse = int(config.get("fuse", 0))
    return ctypes.byref(c)


# ---- workspace cache ----------------------------------------------------------

_workspaces = {}


def workspace_for(op: int, M: int, N: int, K: int, config, device) -> torch.Tensor:
    """A zero-initialized workspace big enough for (op, M, N, K, config), cached per
    device and current stream (the library leaves it ready for the next call)."""
    need = qbg_workspace_size(op, M, N, K, config)
    if need == 0:
        return None
    key = (device, torch.cuda.current_stream(device).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < need:
        ws = torch.zeros(max(need, 1 << 20), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


# ---- library information ------------------------------------------------------

def qbg_abi_version() -> int:
    return lib().qbg_abi_version()


def qbg_status_str(status: int) -> str:
    return lib().qbg_status_str(status).decode()


def qbg_last_error() -> str:
    return lib().qbg_last_error().decode()


# ---- quantizers -------------------------------------------------------------

def qbg_quantize_per_token(x: torch.Tensor, qtype: int = QBG_FP8_E4M3, q=None, scale=None):
    """Dynamic per-token quantization of bf16 x [M,K] -> (q [M,K], scale fp32 [M])."""
    M, K = _dims(x, 2, "x")
    _expect(q, (M, K), _codes(qtype), "q")
    _expect(scale, (M,), _F32, "scale")
    _dev(x, q, scale)
    _dtype(x, torch.bfloat16, "x")
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8 if qtype == QBG_FP8_E4M3 else torch.int8,
                        device=x.device)
    if scale is None:
        scale = torch.empty((M,), dtype=torch.float32, device=x.device)
    _check(lib().qbg_quantize_per_token(qtype, _p(x), M, K, _p(q), _p(scale), _stream(x)))
    return q, scale


def qbg_quantize_per_token_group(x: torch.Tensor, group: int = 128,
                                 fmt: int = QBG_SCALE_F32, q=None, scale=None):
    """1 x group FP8 quantization -> (q [M,K] uint8, scale [M,K/group] fp32 or uint8)."""
    M, K = _dims(x, 2, "x")
    if group <= 0 or K % group:
        raise ValueError("K=%d must be a multiple of the group %d" % (K, group))
    _expect(q, (M, K), _codes(QBG_FP8_E4M3), "q")
    _expect(scale, (M, K // group), _scale_types(fmt), "scale")
    _dev(x, q, scale)
    _dtype(x, torch.bfloat16, "x")
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty((M, K // group), device=x.device,
                            dtype=torch.uint8 if fmt == QBG_SCALE_UE8M0 else torch.float32)
    _check(lib().qbg_quantize_per_token_group(_p(x), M, K, group, fmt, _p(q), _p(scale),
                                              _stream(x)))
    return q, scale


def qbg_quantize_weight_block(w: torch.Tensor, fmt: int = QBG_SCALE_F32, q=None, scale=None):
    """128x128 block FP8 quantization of W [N,K] -> (q, scale [ceil(N/128), K/128])."""
    N, K = _dims(w, 2, "w")
    if K % 128:
        raise ValueError("K=%d must be a multiple of 128" % K)
    _expect(q, (N, K), _codes(QBG_FP8_E4M3), "q")
    _expect(scale, ((N + 127) // 128, K // 128), _scale_types(fmt), "scale")
    _dev(w, q, scale)
    _dtype(w, torch.bfloat16, "w")
    if q is None:
        q = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    if scale is None:
        scale = torch.empty(((N + 127) // 128, K // 128), device=w.device,
                            dtype=torch.uint8 if fmt == QBG_SCALE_UE8M0 else torch.float32)
    _check(lib().qbg_quantize_weight_block(_p(w), N, K, fmt, _p(q), _p(scale), _stream(w)))
    return q, scale


def qbg_rms_norm_quantize_per_token(x: torch.Tensor, w: torch.Tensor, eps: float = 1e-6,
                                    q=None, scale=None):
    """Fused RMSNorm + per-token FP8 quantization -> (q [M,H], scale [M])."""
    M, H = _dims(x, 2, "x")
    _expect(w, (H,), _BF16, "w")
    _expect(q, (M, H), _codes(QBG_FP8_E4M3), "q")
    _expect(scale, (M,), _F32, "scale")
    _dev(x, w, q, scale)
    _dtype(x, torch.bfloat16, "x")
    if q is None:
        q = torch.empty((M, H), dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty((M,), dtype=torch.float32, device=x.device)
    _check(lib().qbg_rms_norm_quantize_per_token(_p(x), _p(w), eps, M, H, _p(q), _p(scale),
                                                 _stream(x)))
    return q, scale


def qbg_silu_mul_quantize_per_token(gate_up: torch.Tensor, q=None, scale=None):
    """Fused SiLU(gate) * up + per-token FP8 quantization of gate_up [M,2I] -> (q [M,I], scale)."""
    M, I2 = _dims(gate_up, 2, "gate_up")
    if I2 % 2:
        raise ValueError("gate_up must have an even row length, got %d" % I2)
    I = I2 // 2
    _expect(q, (M, I), _codes(QBG_FP8_E4M3), "q")
    _expect(scale, (M,), _F32, "scale")
    _dev(gate_up, q, scale)
    _dtype(gate_up, torch.bfloat16, "gate_up")
    if q is None:
        q = torch.empty((M, I), dtype=torch.uint8, device=gate_up.device)
    if scale is None:
        scale = torch.empty((M,), dtype=torch.float32, device=gate_up.device)
    _check(lib().qbg_silu_mul_quantize_per_token(_p(gate_up), M, I, _p(q), _p(scale),
                                                 _stream(gate_up)))
    return q, scale


def _group_scales(M, L, group, fmt, device):
    return torch.empty((M, L // group), dtype=torch.uint8 if fmt == QBG_SCALE_UE8M0 else
                       torch.float32, device=device)


def qbg_rms_norm_quantize_per_token_group(x: torch.Tensor, w: torch.Tensor, eps: float = 1e-6,
                                          group: int = 128, fmt: int = QBG_SCALE_F32, q=None,
                                          scale=None):
    """Fused RMSNorm + 1 x group FP8 quantization -> (q [M,H], scale [M,H/group])."""
    M, H = _dims(x, 2, "x")
    if group <= 0 or H % group:
        raise ValueError("H=%d must be a multiple of the group %d" % (H, group))
    _expect(w, (H,), _BF16, "w")
    _expect(q, (M, H), _codes(QBG_FP8_E4M3), "q")
    _expect(scale, (M, H // group), _scale_types(fmt), "scale")
    _dev(x, w, q, scale)
    _dtype(x, torch.bfloat16, "x")
    if q is None:
        q = torch.empty((M, H), dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = _group_scales(M, H, group, fmt, x.device)
    _check(lib().qbg_rms_norm_quantize_per_token_group(_p(x), _p(w), eps, M, H, group, fmt, _p(q),
                                                       _p(scale), _stream(x)))
    return q, scale


def qbg_silu_mul_quantize_per_token_group(gate_up: torch.Tensor, group: int = 128,
                                          fmt: int = QBG_SCALE_F32, q=None, scale=None):
    """Fused SiLU(gate) * up + 1 x group FP8 quantization of gate_up [M,2I]
    -> (q [M,I], scale [M,I/group])."""
    M, I2 = _dims(gate_up, 2, "gate_up")
    I = I2 // 2
    if I2 % 2 or group <= 0 or I % group:
        raise ValueError("gate_up row length %d must be twice a multiple of the group %d" % (I2, group))
    _expect(q, (M, I), _codes(QBG_FP8_E4M3), "q")
    _expect(scale, (M, I // group), _scale_types(fmt), "scale")
    _dev(gate_up, q, scale)
    _dtype(gate_up, torch.bfloat16, "gate_up")
    if q is None:
        q = torch.empty((M, I), dtype=torch.uint8, device=gate_up.device)
    if scale is None:
        scale = _group_scales(M, I, group, fmt, gate_up.device)
    _check(lib().qbg_silu_mul_quantize_per_token_group(_p(gate_up), M, I, group, fmt, _p(q),
                                                       _p(scale), _stream(gate_up)))
    return q, scale


def qbg_convert_f32_to_e4m3(x: torch.Tensor, out=None):
    """The device fp32 -> E4M3 conversion (clamped) applied elementwise; uint8 codes."""
    _expect(out, tuple(x.shape), (torch.uint8,), "out")
    _dev(x, out)
    _dtype(x, torch.float32, "x")
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _check(lib().qbg_convert_f32_to_e4m3(_p(x), _p(out), x.numel(), _stream(x)))
    return out


# ---- GEMMs -------------------------------------------------------------------

def qbg_scaled_mm(a_q, a_scale, w_q, w_scale, qtype: int = QBG_FP8_E4M3, out=None,
                  config=None, workspace=None):
    """Per-token x per-channel scaled GEMM -> bf16 [M,N]."""
    codes = _codes(qtype)
    M, K = _dims(a_q, 2, "a_q")
    N = _dims(w_q, 2, "w_q")[0]
    _expect(a_q, (M, K), codes, "a_q")
    _expect(w_q, (N, K), codes, "w_q")
    _expect(a_scale, (M,), _F32, "a_scale")
    _expect(w_scale, (N,), _F32, "w_scale")
    _expect(out, (M, N), _BF16, "out")
    _dev(a_q, a_scale, w_q, w_scale, out, workspace)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a_q.device)
    op = QBG_OP_FP8 if qtype == QBG_FP8_E4M3 else QBG_OP_INT8
    if workspace is None:
        workspace = workspace_for(op, M, N, K, config, a_q.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().qbg_scaled_mm(qtype, _p(a_q), _p(a_scale), _p(w_q), _p(w_scale), M, N, K,
                               _p(out), _cfg(config), _p(workspace), wsb, _stream(a_q)))
    return out


def qbg_scaled_mm_noalloc(a_q, a_scale, w_q, w_scale, qtype: int = QBG_FP8_E4M3, out=None,
                          config=None):
    """qbg_scaled_mm without a workspace: split-K uses the library's per-GPU
    scratch.  With `out` given, the call allocates no device memory."""
    codes = _codes(qtype)
    M, K = _dims(a_q, 2, "a_q")
    N = _dims(w_q, 2, "w_q")[0]
    _expect(a_q, (M, K), codes, "a_q")
    _expect(w_q, (N, K), codes, "w_q")
    _expect(a_scale, (M,), _F32, "a_scale")
    _expect(w_scale, (N,), _F32, "w_scale")
    _expect(out, (M, N), _BF16, "out")
    _dev(a_q, a_scale, w_q, w_scale, out)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a_q.device)
    _check(lib().qbg_scaled_mm_noalloc(qtype, _p(a_q), _p(a_scale), _p(w_q), _p(w_scale), M, N, K,
                                       _p(out), _cfg(config), _stream(a_q)))
    return out


def qbg_quantize_scaled_mm(x, w_q, w_scale, qtype: int = QBG_FP8_E4M3, out=None, a_q=None,
                           a_scale=None, config=None, workspace=None):
    """Per-token quantization of bf16 x and the scaled GEMM, in the way the
    configuration's `fuse` mode names (QBG_FUSE_PUBLISH / LOCAL: one launch;
    SEPARATE: quantizer launch, then the GEMM).
    Returns (out bf16 [M,N], a_q [M,K], a_scale fp32 [M])."""
    codes = _codes(qtype)
    M, K = _dims(x, 2, "x")
    N = _dims(w_q, 2, "w_q")[0]
    _expect(x, (M, K), _BF16, "x")
    _expect(w_q, (N, K), codes, "w_q")
    _expect(w_scale, (N,), _F32, "w_scale")
    _expect(out, (M, N), _BF16, "out")
    _expect(a_q, (M, K), codes, "a_q")
    _expect(a_scale, (M,), _F32, "a_scale")
    _dev(x, w_q, w_scale, out, a_q, a_scale, workspace)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    if a_q is None:
        a_q = torch.empty((M, K), dtype=torch.uint8 if qtype == QBG_FP8_E4M3 else torch.int8,
                          device=x.device)
    if a_scale is None:
        a_scale = torch.empty((M,), dtype=torch.float32, device=x.device)
    op = QBG_OP_FP8_FUSED if qtype == QBG_FP8_E4M3 else QBG_OP_INT8_FUSED
    if workspace is None:
        workspace = workspace_for(op, M, N, K, config, x.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().qbg_quantize_scaled_mm(qtype, _p(x), _p(w_q), _p(w_scale), M, N, K, _p(a_q),
                                        _p(a_scale), _p(out), _cfg(config), _p(workspace), wsb,
                                        _stream(x)))
    return out, a_q, a_scale


def qbg_grouped_scaled_mm(a_q, a_scale, w_q, w_scale, offsets, qtype: int = QBG_FP8_E4M3,
                          out=None, config=None):
    """Grouped (mixture-of-experts) scaled GEMM: rows offsets[e]..offsets[e+1] of a_q [T,K]
    use w_q[e] [N,K] and w_scale[e] [N] (offsets: int32 [E+1] on the device) -> bf16 [T,N]."""
    codes = _codes(qtype)
    T, K = _dims(a_q, 2, "a_q")
    E, N = _dims(w_q, 3, "w_q")[:2]
    _expect(a_q, (T, K), codes, "a_q")
    _expect(w_q, (E, N, K), codes, "w_q")
    _expect(a_scale, (T,), _F32, "a_scale")
    _expect(w_scale, (E, N), _F32, "w_scale")
    _expect(offsets, (E + 1,), (torch.int32,), "offsets")
    _expect(out, (T, N), _BF16, "out")
    _dev(a_q, a_scale, w_q, w_scale, offsets, out)
    if out is None:
        out = torch.empty((T, N), dtype=torch.bfloat16, device=a_q.device)
    _check(lib().qbg_grouped_scaled_mm(qtype, _p(a_q), _p(a_scale), _p(w_q), _p(w_scale),
                                       _p(offsets), T, E, N, K, _p(out), _cfg(config),
                                       _stream(a_q)))
    return out


def qbg_set_fused_wait_limit(iterations: int) -> int:
    """Test hook: bounded-wait iterations of the fused launch (0: every workgroup
    quantizes the rows itself; negative: default).  Returns the previous value."""
    return lib().qbg_set_fused_wait_limit(iterations)


def qbg_block_scaled_mm(a_q, a_scale, w_q, w_scale, fmt: int = QBG_SCALE_F32, out=None,
                        config=None, workspace=None):
    """Block-FP8 scaled GEMM (1x128 activation groups, 128x128 weight blocks) -> bf16 [M,N]."""
    stype = _scale_types(fmt)
    codes = _codes(QBG_FP8_E4M3)
    M, K = _dims(a_q, 2, "a_q")
    N = _dims(w_q, 2, "w_q")[0]
    if K % 128:
        raise ValueError("K=%d must be a multiple of 128" % K)
    _expect(a_q, (M, K), codes, "a_q")
    _expect(w_q, (N, K), codes, "w_q")
    _expect(a_scale, (M, K // 128), stype, "a_scale")
    _expect(w_scale, ((N + 127) // 128, K // 128), stype, "w_scale")
    _expect(out, (M, N), _BF16, "out")
    _dev(a_q, a_scale, w_q, w_scale, out, workspace)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a_q.device)
    op = QBG_OP_BLOCK_FP8 if fmt == QBG_SCALE_F32 else QBG_OP_BLOCK_UE8M0
    if workspace is None:
        workspace = workspace_for(op, M, N, K, config, a_q.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().qbg_block_scaled_mm(fmt, _p(a_q), _p(a_scale), _p(w_q), _p(w_scale), M, N, K,
                                     _p(out), _cfg(config), _p(workspace), wsb, _stream(a_q)))
    return out


def qbg_scaled_mm_i32(a_q, w_q, out=None, config=None, workspace=None):
    """The int8 GEMM's exact int32 accumulator [M,N] (test hook)."""
    codes = _codes(QBG_INT8)
    M, K = _dims(a_q, 2, "a_q")
    N = _dims(w_q, 2, "w_q")[0]
    _expect(a_q, (M, K), codes, "a_q")
    _expect(w_q, (N, K), codes, "w_q")
    _expect(out, (M, N), (torch.int32,), "out")
    _dev(a_q, w_q, out, workspace)
    if out is None:
        out = torch.empty((M, N), dtype=torch.int32, device=a_q.device)
    if workspace is None:
        workspace = workspace_for(QBG_OP_INT8, M, N, K, config, a_q.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().qbg_scaled_mm_i32(_p(a_q), _p(w_q), M, N, K, _p(out), _cfg(config),
                                   _p(workspace), wsb, _stream(a_q)))
    return out


# ---- configurations -----------------------------------------------------------

def qbg_config_table_load(path: str) -> None:
    _check(lib().qbg_config_table_load(path.encode()))


def qbg_config_table_size() -> int:
    return lib().qbg_config_table_size()


def qbg_config_lookup(op: int, M: int, N: int, K: int):
    """(config dict, from_table) used for (op, M, N, K)."""
    c = GemmConfig()
    hit = ctypes.c_int32(0)
    _check(lib().qbg_config_lookup(op, M, N, K, ctypes.byref(c), ctypes.byref(hit)))
    return c.as_dict(), bool(hit.value)


def qbg_workspace_size(op: int, M: int, N: int, K: int, config=None) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().qbg_workspace_size(op, M, N, K, _cfg(config), ctypes.byref(n)))
    return n.value


def qbg_workspace_init(workspace: torch.Tensor) -> None:
    _dev(workspace)
    _check(lib().qbg_workspace_init(_p(workspace), workspace.numel() * workspace.element_size(),
                                    _stream(workspace)))


def qbg_kernel_count() -> int:
    return lib().qbg_kernel_count()


def qbg_kernel_info(kernel_id: int) -> dict:
    c = GemmConfig()
    _check(lib().qbg_kernel_info(kernel_id, ctypes.byref(c)))
    return c.as_dict()
