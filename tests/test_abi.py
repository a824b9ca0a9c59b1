"""The C ABI on the CPU: the library loads without a GPU, exports every symbol
include/qbg.h declares, and rejects bad arguments with the documented status
before any HIP call.  Configuration-table loading, lookup and workspace
sizing are host logic and are tested here too."""
import ctypes
import os
import re

import pytest

import quantized_bit_gemm_amd as qbg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qbg.h")

OK, E_NULL, E_SHAPE, E_ALIGN, E_QTYPE, E_SPLITK, E_WORKSPACE, E_TABLE, E_HIP, E_CONFIG = range(10)
FAKE = 0x7F0000000000  # a 256-byte aligned address that is never dereferenced by these calls


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qbg_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return qbg.lib()


def P(v):
    return ctypes.c_void_p(v)


def cfg(kid=0, swap=0, split=1, fuse=0):
    c = qbg.GemmConfig()
    c.kernel_id, c.swap_ab, c.split_k, c.fuse = kid, swap, split, fuse
    return ctypes.byref(c)


@pytest.fixture(autouse=True)
def restore_table(L):
    yield
    path = qbg.DEFAULT_TABLE
    if os.path.exists(path):
        assert L.qbg_config_table_load(path.encode()) == OK


def test_library_exports_every_declared_symbol(L):
    declared = header_functions()
    assert len(declared) >= 19
    assert sorted(qbg.EXPORTS) == declared
    for name in declared:
        assert hasattr(L, name), name


def test_abi_version_matches_header(L):
    m = re.search(r"#define QBG_ABI_VERSION (\d+)", open(HEADER).read())
    assert L.qbg_abi_version() == int(m.group(1))


def test_status_strings(L):
    for s in range(10):
        assert L.qbg_status_str(s)
    assert L.qbg_status_str(0) == b"ok"
    assert L.qbg_status_str(99) == b"unknown status"


def test_quantizer_validation(L):
    z = P(None)
    x, q, s = P(FAKE), P(FAKE + 4096), P(FAKE + 8192)
    assert L.qbg_quantize_per_token(7, x, 1, 16, q, s, z) == E_QTYPE
    assert L.qbg_quantize_per_token(0, z, 1, 16, q, s, z) == E_NULL
    assert L.qbg_quantize_per_token(0, x, 0, 16, q, s, z) == E_SHAPE
    assert L.qbg_quantize_per_token(0, x, 1, 24, q, s, z) == E_SHAPE
    assert L.qbg_quantize_per_token(0, P(FAKE + 8), 1, 16, q, s, z) == E_ALIGN
    assert L.qbg_quantize_per_token_group(x, 1, 256, 64, 0, q, s, z) == E_SHAPE
    assert L.qbg_quantize_per_token_group(x, 1, 200, 128, 0, q, s, z) == E_SHAPE
    assert L.qbg_quantize_per_token_group(x, 1, 256, 128, 5, q, s, z) == E_QTYPE
    assert L.qbg_quantize_weight_block(x, 100, 256, 0, q, s, z) == E_SHAPE
    assert L.qbg_rms_norm_quantize_per_token(x, x, 1e-6, 1, 65552, q, s, z) == E_SHAPE
    assert L.qbg_rms_norm_quantize_per_token(x, x, -1.0, 1, 4096, q, s, z) == E_SHAPE
    # eps must be positive: with eps 0 an all-zero row would divide by zero
    for eps in (0.0, float("inf"), float("nan")):
        assert L.qbg_rms_norm_quantize_per_token(x, x, eps, 1, 4096, q, s, z) == E_SHAPE
        assert L.qbg_rms_norm_quantize_per_token_group(x, x, eps, 1, 4096, 128, 0, q, s,
                                                       z) == E_SHAPE
    # grid bounds: rows of a per-token call, groups of a group call
    assert L.qbg_quantize_per_token(0, x, (1 << 22) + 1, 16, q, s, z) == E_SHAPE
    assert L.qbg_quantize_per_token_group(x, 1 << 20, 32768, 128, 0, q, s, z) == E_SHAPE
    assert L.qbg_silu_mul_quantize_per_token(x, 1, 40, q, s, z) == E_SHAPE
    assert L.qbg_convert_f32_to_e4m3(z, z, -1, z) == E_SHAPE
    assert b"16" in L.qbg_last_error() or L.qbg_last_error()


def _mm(L, M=4, N=64, K=256, qtype=0, a=FAKE, sa=FAKE + 1 << 20, w=FAKE + (2 << 20),
        sw=FAKE + (3 << 20), out=FAKE + (4 << 20), c=None, ws=None, wsb=0):
    return L.qbg_scaled_mm(qtype, P(a), P(sa), P(w), P(sw), M, N, K, P(out), c, P(ws), wsb,
                           P(None))


def test_gemm_validation(L):
    assert _mm(L, qtype=3) == E_QTYPE
    assert _mm(L, a=None) == E_NULL
    assert _mm(L, sw=None) == E_NULL
    assert _mm(L, M=0) == E_SHAPE
    assert _mm(L, M=8193) == E_SHAPE
    assert _mm(L, N=24) == E_SHAPE
    assert _mm(L, K=8) == E_SHAPE
    # weight matrices of 2^32 bytes or more: the kernels address them with 32-bit offsets
    assert _mm(L, N=1 << 20, K=4096) == E_SHAPE
    assert _mm(L, N=65536, K=65536) == E_SHAPE
    assert _mm(L, a=FAKE + 4) == E_ALIGN
    assert _mm(L, out=FAKE + 2) == E_ALIGN
    assert _mm(L, c=cfg(kid=qbg.qbg_kernel_count())) == E_CONFIG
    assert _mm(L, c=cfg(kid=-1)) == E_CONFIG
    assert _mm(L, c=cfg(swap=2)) == E_CONFIG
    assert _mm(L, c=cfg(split=3)) == E_SPLITK
    assert _mm(L, c=cfg(split=512)) == E_SPLITK
    assert _mm(L, K=48, c=cfg(split=2)) == E_SPLITK        # 24-wide chunks
    assert _mm(L, K=256, c=cfg(split=4)) == E_WORKSPACE     # no workspace given
    need = qbg.qbg_workspace_size(qbg.QBG_OP_FP8, 4, 64, 256, {"kernel_id": 0, "split_k": 4})
    assert _mm(L, K=256, c=cfg(split=4), ws=FAKE + (8 << 20), wsb=need - 1) == E_WORKSPACE
    assert _mm(L, K=256, c=cfg(split=4), ws=FAKE + (8 << 20) + 16, wsb=need) == E_ALIGN
    # split-K on a prefill tile: one arrival counter per output tile of the whole launch,
    # at most 16320 of them (8192 x 16384 on 64 x 128 tiles is 16384 tiles)
    small = next(k for k in range(qbg.qbg_kernel_count()) if qbg.qbg_kernel_info(k)["k_unroll"] == 0
                 and qbg.qbg_kernel_info(k)["tile_m"] == 64 and qbg.qbg_kernel_info(k)["tile_n"] == 128)
    assert _mm(L, M=8192, N=16384, K=4096, c=cfg(kid=small, split=2), ws=FAKE + (8 << 20),
               wsb=1 << 40) == E_SHAPE
    assert _mm(L, M=8192, N=16384, K=4096, c=cfg(kid=small, split=2)) == E_SHAPE


def test_block_and_i32_validation(L):
    z = P(None)
    a = P(FAKE)
    # An LDS-staged tile (16 rows, 1 KB stage rows, 3 stages: 144 KiB of stages at M=32)
    # serves a block op only while the K chunk's staged scales (4 bytes per token and
    # 128-group) still fit the CU's 160 KiB of LDS.
    lds_kid = next(k for k in range(qbg.qbg_kernel_count())
                   if qbg.qbg_kernel_info(k)["stages"] == 3 and qbg.qbg_kernel_info(k)["tile_n"] == 16
                   and qbg.qbg_kernel_info(k)["k_unroll"] == 8)
    blk = qbg.QBG_OP_BLOCK_FP8
    assert L.qbg_block_scaled_mm(0, a, a, a, a, 32, 128, 32768, a, cfg(kid=lds_kid), z, 0,
                                 z) == E_CONFIG   # 256 groups x 32 tokens x 4 B = 32 KiB more
    with pytest.raises(qbg.QbgError) as ei:
        qbg.qbg_workspace_size(blk, 32, 128, 32768, {"kernel_id": lds_kid})
    assert ei.value.status == E_CONFIG
    # split 2 would need exactly 160 KiB, leaving nothing for the kernel's static LDS
    with pytest.raises(qbg.QbgError):
        qbg.qbg_workspace_size(blk, 32, 128, 32768, {"kernel_id": lds_kid, "split_k": 2})
    assert qbg.qbg_workspace_size(blk, 32, 128, 32768, {"kernel_id": lds_kid, "split_k": 4}) > 0
    assert qbg.qbg_workspace_size(qbg.QBG_OP_FP8, 32, 128, 32768, {"kernel_id": lds_kid}) == 0
    assert qbg.qbg_workspace_size(blk, 4, 128, 32768, {"kernel_id": lds_kid}) == 0
    assert L.qbg_block_scaled_mm(9, a, a, a, a, 1, 128, 256, a, None, z, 0, z) == E_QTYPE
    assert L.qbg_block_scaled_mm(0, a, a, a, a, 1, 128, 200, a, None, z, 0, z) == E_SHAPE
    assert L.qbg_block_scaled_mm(0, a, z, a, a, 1, 128, 256, a, None, z, 0, z) == E_NULL
    assert L.qbg_block_scaled_mm(0, a, a, a, a, 1, 128, 256, a, cfg(split=4), z, 0, z) == E_SPLITK
    # UE8M0 scales are bytes: no 4-byte alignment needed for them
    assert L.qbg_block_scaled_mm(1, a, P(FAKE + 1), a, a, 1, 128, 256, P(FAKE + 3), None, z, 0,
                                 z) == E_ALIGN  # the bf16 output still must be aligned
    assert L.qbg_scaled_mm_i32(z, a, 1, 16, 16, a, None, z, 0, z) == E_NULL
    assert L.qbg_scaled_mm_i32(a, a, 1, 16, 16, a, cfg(split=32), z, 0, z) == E_SPLITK


@pytest.mark.skipif(__import__("torch").cuda.device_count() > 0,
                    reason="the no-device launch path is only exercised on a host without a GPU")
def test_valid_call_without_device_reports_hip_error(L):
    st = _mm(L, c=cfg())
    assert st == E_HIP
    assert L.qbg_last_error()


def test_workspace_sizes(L):
    assert qbg.qbg_workspace_size(qbg.QBG_OP_FP8, 32, 4096, 4096, {"kernel_id": 0, "split_k": 1}) == 0
    n = qbg.qbg_workspace_size(qbg.QBG_OP_FP8, 32, 4096, 4096, {"kernel_id": 0, "split_k": 8})
    assert n == 65536 + 8 * 32 * 4096 * 4
    # token slices of 32: the workspace of M=256 is that of 32
    assert qbg.qbg_workspace_size(qbg.QBG_OP_INT8, 256, 4096, 4096,
                                  {"kernel_id": 0, "split_k": 8}) == n
    m3 = qbg.qbg_workspace_size(qbg.QBG_OP_FP8, 3, 528, 2048, {"kernel_id": 0, "split_k": 2})
    assert m3 == 65536 + ((2 * 3 * 528 * 4 + 255) // 256) * 256


def test_kernel_info(L):
    n = qbg.qbg_kernel_count()
    assert n >= 8
    seen = set()
    for k in range(n):
        info = qbg.qbg_kernel_info(k)
        # tile_n is a multiple of 16, except on register-streaming tiles (stages 0)
        # whose workgroups own fewer rows than their 16-row sub-tiles hold
        # (and on LDS-staged decode tiles of the plain per-channel ops)
        assert info["tile_n"] % 16 == 0 or (info["tile_m"] == 32 and info["tile_n"] % 4 == 0)
        assert info["tile_n"] >= 16 or (info["stages"] == 0 and info["tile_n"] >= 8)
        assert info["waves_n"] >= 1 and info["waves_k"] >= 1
        # k_unroll 0 marks the prefill tiles (LDS-staged, 64 or more tokens)
        assert info["k_unroll"] >= 1 or (info["stages"] > 0 and info["tile_m"] >= 64)
        seen.add((info["tile_n"], info["waves_n"], info["waves_k"], info["k_unroll"],
                  info["stages"], info["waves_m"], info["tile_m"]))
    assert len(seen) == n, "tile variants must be distinct"
    with pytest.raises(qbg.QbgError):
        qbg.qbg_kernel_info(n)


def _write(tmp_path, text, name="t.txt"):
    p = tmp_path / name
    p.write_text(text)
    return str(p)


def test_table_load_and_lookup(L, tmp_path):
    path = _write(tmp_path, "qbg-config-table 1 gfx950\n"
                            "# comment\n"
                            "fp8 4 4096 4096 3 1 1   # 5.9 us\n"
                            "int8 32 4096 12288 5 0 2\n"
                            "block_fp8 8 5120 8192 1 1 4\n"
                            "block_ue8m0 1 51200 5120 0 0 1\n")
    qbg.qbg_config_table_load(path)
    assert qbg.qbg_config_table_size() == 4
    c, hit = qbg.qbg_config_lookup(qbg.QBG_OP_FP8, 3, 4096, 4096)  # bucket next_pow2(3) = 4
    assert hit and (c["kernel_id"], c["swap_ab"], c["split_k"]) == (3, 1, 1)
    c, hit = qbg.qbg_config_lookup(qbg.QBG_OP_FP8, 5, 4096, 4096)  # bucket 8: not in the table
    assert not hit
    c, hit = qbg.qbg_config_lookup(qbg.QBG_OP_INT8, 17, 4096, 12288)
    assert hit and (c["kernel_id"], c["split_k"]) == (5, 2)
    assert c["tile_n"] == qbg.qbg_kernel_info(5)["tile_n"]
    c, hit = qbg.qbg_config_lookup(qbg.QBG_OP_BLOCK_UE8M0, 1, 51200, 5120)
    assert hit
    c, hit = qbg.qbg_config_lookup(qbg.QBG_OP_BLOCK_FP8, 1, 51200, 5120)
    assert not hit  # keyed by op


@pytest.mark.parametrize("text", [
    "",
    "qbg-config-table 1 gfx942\n",
    "not-a-table 1 gfx950\n",
    "qbg-config-table 1 gfx950\nfp8 4 4096 4096 3 1\n",
    "qbg-config-table 1 gfx950\nfp8 4 4096 4096 3 1 1 9\n",
    "qbg-config-table 2 gfx950\nfp8 4 4096 4096 3 1 1\n",
    "qbg-config-table 2 gfx950\nfp8 4 4096 4096 3 1 1 2\n",
    "qbg-config-table 3 gfx950\nfp8 4 4096 4096 3 1 1 0\n",
    "qbg-config-table 1 gfx950\nfp16 4 4096 4096 3 1 1\n",
    "qbg-config-table 1 gfx950\nfp8 3 4096 4096 3 1 1\n",
    "qbg-config-table 1 gfx950\nfp8 4 4100 4096 3 1 1\n",
    "qbg-config-table 1 gfx950\nfp8 4 4096 4096 99 1 1\n",
    "qbg-config-table 1 gfx950\nfp8 4 4096 4096 3 1 3\n",
    "qbg-config-table 1 gfx950\nblock_fp8 4 4096 4096 3 1 64\n",
])
def test_bad_tables_are_rejected_and_keep_the_previous_table(L, tmp_path, text):
    good = _write(tmp_path, "qbg-config-table 1 gfx950\nfp8 1 512 1024 2 0 1\n", "good.txt")
    qbg.qbg_config_table_load(good)
    bad = _write(tmp_path, text, "bad.txt")
    assert L.qbg_config_table_load(bad.encode()) == E_TABLE
    assert L.qbg_last_error()
    assert qbg.qbg_config_table_size() == 1
    c, hit = qbg.qbg_config_lookup(qbg.QBG_OP_FP8, 1, 512, 1024)
    assert hit and c["kernel_id"] == 2


def test_version2_table_carries_rotation(L, tmp_path):
    path = _write(tmp_path, "qbg-config-table 2 gfx950\nfp8 1 4096 4096 16 1 1 1\n"
                            "fp8 2 4096 4096 16 1 1 0\n")
    qbg.qbg_config_table_load(path)
    c, hit = qbg.qbg_config_lookup(qbg.QBG_OP_FP8, 1, 4096, 4096)
    assert hit and c["rotate"] == 1 and c["stages"] > 0
    c, hit = qbg.qbg_config_lookup(qbg.QBG_OP_FP8, 2, 4096, 4096)
    assert hit and c["rotate"] == 0


def test_missing_table_file(L, tmp_path):
    assert L.qbg_config_table_load(str(tmp_path / "nope.txt").encode()) == E_TABLE
    assert L.qbg_config_table_load(None) == E_NULL


def test_default_config_is_valid_for_every_workload_shape():
    shapes = {qbg.QBG_OP_FP8: [(512, 1024), (6144, 4096), (4096, 4096), (24576, 4096), (4096, 12288)],
              qbg.QBG_OP_INT8: [(6144, 4096), (4096, 4096), (24576, 4096), (4096, 12288)],
              qbg.QBG_OP_BLOCK_FP8: [(10240, 5120), (5120, 8192), (51200, 5120), (5120, 25600)],
              qbg.QBG_OP_BLOCK_UE8M0: [(10240, 5120), (5120, 8192), (51200, 5120), (5120, 25600)]}
    for op, lst in shapes.items():
        for (N, K) in lst:
            for M in (1, 3, 32, 128, 256, 1000, 8192):
                c, _ = qbg.qbg_config_lookup(op, M, N, K)
                qbg.qbg_workspace_size(op, M, N, K, c)  # raises if the config is infeasible


def test_default_config_above_32_tokens_is_one_large_m_launch():
    for op in (qbg.QBG_OP_FP8, qbg.QBG_OP_INT8, qbg.QBG_OP_FP8_FUSED):
        c, hit = qbg.qbg_config_lookup(op, 3000, 12352, 4096)  # not in any table
        assert not hit and c["tile_m"] == 256 and c["split_k"] == 1
        assert qbg.qbg_workspace_size(op, 3000, 12352, 4096, c) == 0  # no partials
        # from 1024 tokens the per-channel ops run on a prefill tile (k_unroll 0)
        assert c["k_unroll"] == 0
        c, _ = qbg.qbg_config_lookup(op, 500, 12352, 4096)
        assert c["tile_m"] == 256 and c["k_unroll"] > 0
        c, _ = qbg.qbg_config_lookup(op, 32, 12352, 4096)
        assert c["tile_m"] == 32
    c, _ = qbg.qbg_config_lookup(qbg.QBG_OP_FP8, 3000, 12352, 4160)  # K not a multiple of 128
    assert c["k_unroll"] > 0
    # fewer output tiles than CUs and a long K: two K chunks (partials in the workspace)
    for op in (qbg.QBG_OP_FP8, qbg.QBG_OP_INT8, qbg.QBG_OP_FP8_FUSED):
        c, hit = qbg.qbg_config_lookup(op, 1100, 3072, 10240)
        assert not hit and c["k_unroll"] == 0 and c["split_k"] == 2
        assert qbg.qbg_workspace_size(op, 1100, 3072, 10240, c) > 65536
        c, _ = qbg.qbg_config_lookup(op, 1100, 12352, 10240)  # enough tiles
        assert c["split_k"] == 1
        c, _ = qbg.qbg_config_lookup(op, 1100, 3072, 4096)    # short K loop
        assert c["split_k"] == 1
    c, hit = qbg.qbg_config_lookup(qbg.QBG_OP_BLOCK_FP8, 3000, 12352, 4096)  # the prefill tile
    assert not hit and c["tile_m"] == 128 and c["k_unroll"] == 0
    c, _ = qbg.qbg_config_lookup(qbg.QBG_OP_BLOCK_FP8, 500, 12352, 4096)  # decode launches
    assert c["tile_m"] == 32
    c, hit = qbg.qbg_config_lookup(qbg.QBG_OP_BLOCK_UE8M0, 3000, 12352, 4096)  # the prefill tile
    assert not hit and c["tile_m"] == 128 and c["k_unroll"] == 0
    c, _ = qbg.qbg_config_lookup(qbg.QBG_OP_BLOCK_UE8M0, 3000, 12352, 4224)  # K % 512 != 0
    assert c["tile_m"] == 32


def test_shipped_table_loads():
    if not os.path.exists(qbg.DEFAULT_TABLE):
        pytest.skip("no tuned table shipped")
    qbg.qbg_config_table_load(qbg.DEFAULT_TABLE)
    assert qbg.qbg_config_table_size() > 0


def test_binding_rejects_host_tensors():
    import torch
    x = torch.zeros((2, 16), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        qbg.qbg_quantize_per_token(x)


def test_binding_checks_shapes_and_dtypes_before_the_c_call():
    # The C ABI cannot see buffer sizes, so the binding rejects every mismatch of shape or
    # dtype (ValueError / TypeError naming the tensor) before a pointer reaches it.  Meta
    # tensors carry shapes and dtypes without memory; well-formed arguments get as far as
    # the device check.
    import torch

    def t(shape, dt):
        return torch.empty(shape, dtype=dt, device="meta")

    u8, i8, f32, bf, i32 = torch.uint8, torch.int8, torch.float32, torch.bfloat16, torch.int32
    M, N, K = 4, 64, 256
    aq, sa, wq, sw = t((M, K), u8), t((M,), f32), t((N, K), u8), t((N,), f32)

    def raises(exc, match, fn, *a, **k):
        with pytest.raises(exc, match=match):
            fn(*a, **k)

    raises(ValueError, "GPU only", qbg.qbg_scaled_mm, aq, sa, wq, sw)
    raises(ValueError, "w_q must have shape", qbg.qbg_scaled_mm, aq, sa, t((N, 128), u8), sw)
    raises(ValueError, "a_scale must have shape", qbg.qbg_scaled_mm, aq, t((M + 1,), f32), wq, sw)
    raises(ValueError, "w_scale must have shape", qbg.qbg_scaled_mm, aq, sa, wq, t((N // 2,), f32))
    raises(ValueError, "out must have shape", qbg.qbg_scaled_mm, aq, sa, wq, sw, out=t((M, N + 16), bf))
    raises(TypeError, "out must be", qbg.qbg_scaled_mm, aq, sa, wq, sw, out=t((M, N), f32))
    raises(TypeError, "a_q must be", qbg.qbg_scaled_mm, aq, sa, wq, sw, qtype=qbg.QBG_INT8)
    raises(TypeError, "w_scale must be", qbg.qbg_scaled_mm, aq, sa, wq, t((N,), bf))
    raises(ValueError, "qtype", qbg.qbg_scaled_mm, aq, sa, wq, sw, qtype=5)
    raises(ValueError, "a_q must have 2", qbg.qbg_scaled_mm, t((K,), u8), sa, wq, sw)
    # the int32 test hook
    raises(TypeError, "out must be", qbg.qbg_scaled_mm_i32, t((M, K), i8), t((N, K), i8),
           out=t((M, N), f32))
    raises(ValueError, "w_q must have shape", qbg.qbg_scaled_mm_i32, t((M, K), i8), t((N, K + 16), i8))
    raises(ValueError, "GPU only", qbg.qbg_scaled_mm_i32, t((M, K), i8), t((N, K), i8))
    # the fused entry point
    x = t((M, K), bf)
    raises(ValueError, "GPU only", qbg.qbg_quantize_scaled_mm, x, wq, sw)
    raises(TypeError, "x must be", qbg.qbg_quantize_scaled_mm, t((M, K), f32), wq, sw)
    raises(ValueError, "a_q must have shape", qbg.qbg_quantize_scaled_mm, x, wq, sw, a_q=t((M, K - 16), u8))
    raises(ValueError, "a_scale must have shape", qbg.qbg_quantize_scaled_mm, x, wq, sw,
           a_scale=t((2 * M,), f32))
    # Block-FP8: group and block scale grids, both scale formats
    bs, bw = t((M, K // 128), f32), t(((N + 127) // 128, K // 128), f32)
    raises(ValueError, "GPU only", qbg.qbg_block_scaled_mm, aq, bs, wq, bw)
    raises(ValueError, "a_scale must have shape", qbg.qbg_block_scaled_mm, aq, t((M, 1), f32), wq, bw)
    raises(ValueError, "w_scale must have shape", qbg.qbg_block_scaled_mm, aq, bs, wq, t((2, 2), f32))
    raises(TypeError, "a_scale must be", qbg.qbg_block_scaled_mm, aq, bs, wq, bw,
           fmt=qbg.QBG_SCALE_UE8M0)
    raises(ValueError, "multiple of 128", qbg.qbg_block_scaled_mm, t((M, 200), u8), bs,
           t((N, 200), u8), bw)
    # grouped: offsets hold E + 1 entries, scales [E, N]
    E = 8
    gq, gs, gw, gws = t((16, K), u8), t((16,), f32), t((E, N, K), u8), t((E, N), f32)
    raises(ValueError, "GPU only", qbg.qbg_grouped_scaled_mm, gq, gs, gw, gws, t((E + 1,), i32))
    raises(ValueError, "offsets must have shape", qbg.qbg_grouped_scaled_mm, gq, gs, gw, gws,
           t((E,), i32))
    raises(TypeError, "offsets must be", qbg.qbg_grouped_scaled_mm, gq, gs, gw, gws,
           t((E + 1,), torch.int64))
    raises(ValueError, "w_scale must have shape", qbg.qbg_grouped_scaled_mm, gq, gs, gw,
           t((E, N + 16), f32), t((E + 1,), i32))
    raises(ValueError, "w_q must have 3", qbg.qbg_grouped_scaled_mm, gq, gs, t((N, K), u8), gws,
           t((E + 1,), i32))
    # quantizers: caller-provided outputs
    raises(ValueError, "q must have shape", qbg.qbg_quantize_per_token, x, q=t((M, K + 16), u8))
    raises(TypeError, "q must be", qbg.qbg_quantize_per_token, x, qbg.QBG_INT8, q=t((M, K), u8))
    raises(ValueError, "scale must have shape", qbg.qbg_quantize_per_token_group, x,
           scale=t((M, 1), f32))
    raises(ValueError, "w must have shape", qbg.qbg_rms_norm_quantize_per_token, x, t((K + 16,), bf))
    raises(ValueError, "even row length", qbg.qbg_silu_mul_quantize_per_token, t((M, 2 * 16 + 1), bf))
    raises(ValueError, "GPU only", qbg.qbg_silu_mul_quantize_per_token, t((M, 2 * K), bf))


def test_tuner_table_writer_picks_fastest(tmp_path):
    from quantized_bit_gemm_amd import tune
    results = {}
    for kid, us in ((0, 9.0), (3, 5.5), (5, 7.0)):
        r = {"op": "fp8", "M": 4, "N": 4096, "K": 4096, "kernel_id": kid, "swap_ab": 1,
             "split_k": 1, "rotate": 1, "us": us, "TBs": 1.0}
        results[tune.config_key(r["op"], 4, 4096, 4096, r)] = r
    out = str(tmp_path / "table.txt")
    best = tune.write_table(out, results)
    assert best[("fp8", 4, 4096, 4096)]["kernel_id"] == 3
    qbg.qbg_config_table_load(out)
    c, hit = qbg.qbg_config_lookup(qbg.QBG_OP_FP8, 4, 4096, 4096)
    assert hit and c["kernel_id"] == 3 and c["rotate"] == 1


def test_tuner_checkpoint_resume(tmp_path):
    from quantized_bit_gemm_amd import tune
    ck = tmp_path / "ck.jsonl"
    ck.write_text('{"op": "int8", "M": 1, "N": 16, "K": 64, "kernel_id": 2, "swap_ab": 0, '
                  '"split_k": 1, "us": 3.0, "TBs": 0.1}\n\n')
    done = tune.load_checkpoint(str(ck))
    assert ("int8", 1, 16, 64, 2, 0, 1, 0, 0) in done


def test_tuner_fused_candidates_cover_the_fuse_modes():
    from quantized_bit_gemm_amd import tune
    info = {k: qbg.qbg_kernel_info(k) for k in range(qbg.qbg_kernel_count())}
    # default: the two-launch form only, on every tile of the plain op
    cands = tune.feasible_configs(qbg, qbg.QBG_OP_FP8_FUSED, 4096, max_split=1)
    assert {c["fuse"] for c in cands} == {qbg.QBG_FUSE_SEPARATE}
    assert {c["kernel_id"] for c in cands} == set(info)
    cands = tune.feasible_configs(qbg, qbg.QBG_OP_FP8_FUSED, 4096, max_split=1, fuse_modes=(0, 1, 2))
    local = {c["kernel_id"] for c in cands if c["fuse"] == qbg.QBG_FUSE_LOCAL}
    pub = {c["kernel_id"] for c in cands if c["fuse"] == qbg.QBG_FUSE_PUBLISH}
    # LOCAL: the LDS-staged decode tiles, and the register tiles whose waves hold
    # the 4096-byte chunk in exactly two load groups (256 x waves_k x k_unroll)
    assert local == ({k for k, i in info.items() if i["stages"] > 0 and i["tile_m"] == 32} |
                     {k for k, i in info.items() if i["stages"] == 0 and i["tile_m"] == 32 and
                      256 * i["waves_k"] * i["k_unroll"] == 4096})
    reg_local = [c for c in cands if c["fuse"] == qbg.QBG_FUSE_LOCAL and
                 info[c["kernel_id"]]["stages"] == 0]
    assert reg_local and all(c["rotate"] == 0 for c in reg_local)
    assert pub == {k for k, i in info.items() if i["stages"] > 0}
    assert all("fuse" not in c for c in tune.feasible_configs(qbg, qbg.QBG_OP_FP8, 4096, 1))


def _qmm(L, M=4, N=64, K=256, qtype=0, x=FAKE, w=FAKE + (2 << 20), sw=FAKE + (3 << 20),
         aq=FAKE + (5 << 20), sa=FAKE + (6 << 20), out=FAKE + (4 << 20), c=None,
         ws=FAKE + (8 << 20), wsb=1 << 20):
    return L.qbg_quantize_scaled_mm(qtype, P(x), P(w), P(sw), M, N, K, P(aq), P(sa), P(out), c,
                                    P(ws), wsb, P(None))


def _lds_kids():
    return [k for k in range(qbg.qbg_kernel_count()) if qbg.qbg_kernel_info(k)["stages"] > 0]


def test_fused_validation(L):
    lds = _lds_kids()[0]
    reg = next(k for k in range(qbg.qbg_kernel_count()) if qbg.qbg_kernel_info(k)["stages"] == 0)
    assert _qmm(L, qtype=2) == E_QTYPE
    assert _qmm(L, x=None) == E_NULL
    assert _qmm(L, aq=None) == E_NULL
    assert _qmm(L, sa=None) == E_NULL
    assert _qmm(L, M=0) == E_SHAPE
    assert _qmm(L, K=40) == E_SHAPE
    assert _qmm(L, x=FAKE + 8) == E_ALIGN
    assert _qmm(L, c=cfg(kid=reg)) == E_CONFIG           # no PUBLISH on register-streaming tiles
    # LOCAL on a register tile needs a K chunk of two load groups per wave (tile 0: 2048 bytes)
    assert 256 * qbg.qbg_kernel_info(reg)["waves_k"] * qbg.qbg_kernel_info(reg)["k_unroll"] != 256
    assert _qmm(L, c=cfg(kid=reg, fuse=1)) == E_CONFIG
    assert _qmm(L, K=4096, c=cfg(kid=reg, fuse=1)) == E_CONFIG
    assert _qmm(L, M=17, K=2048, c=cfg(kid=reg, fuse=1)) == E_CONFIG   # at most 16 tokens
    assert _qmm(L, c=cfg(kid=lds, fuse=3)) == E_CONFIG   # no such fuse mode
    assert _qmm(L, c=cfg(kid=lds, fuse=-1)) == E_CONFIG
    assert _qmm(L, c=cfg(kid=lds, split=2, fuse=1), ws=None, wsb=0) == E_WORKSPACE  # split-K partials
    assert _qmm(L, c=cfg(kid=reg, split=2, fuse=2), ws=None, wsb=0) == E_WORKSPACE
    assert _qmm(L, c=cfg(kid=lds), ws=None, wsb=0) == E_WORKSPACE   # needed even without split-K
    assert _qmm(L, c=cfg(kid=lds), wsb=(64 << 10) - 4) == E_WORKSPACE
    assert _qmm(L, c=cfg(kid=lds), ws=FAKE + (8 << 20) + 16) == E_ALIGN
    assert _qmm(L, c=cfg(kid=lds, split=3)) == E_SPLITK


def test_fused_workspace_and_lookup(L):
    for op in (qbg.QBG_OP_FP8_FUSED, qbg.QBG_OP_INT8_FUSED):
        # the 64 KiB slot region is always needed; split-K adds its partials
        assert qbg.qbg_workspace_size(op, 4, 64, 256, {"kernel_id": _lds_kids()[0]}) == 64 << 10
        assert qbg.qbg_workspace_size(op, 4, 64, 256, {"kernel_id": _lds_kids()[0],
                                                         "split_k": 2}) > 64 << 10
        # LOCAL and SEPARATE need no slots: only split-K partials
        for fuse in (qbg.QBG_FUSE_LOCAL, qbg.QBG_FUSE_SEPARATE):
            base = {"kernel_id": _lds_kids()[0], "fuse": fuse}
            assert qbg.qbg_workspace_size(op, 4, 64, 256, base) == 0
            assert qbg.qbg_workspace_size(op, 4, 64, 256, dict(base, split_k=2)) > 0
        c, _ = qbg.qbg_config_lookup(op, 3, 12352, 4096)  # not in any table: the default
        assert c["fuse"] == qbg.QBG_FUSE_SEPARATE        # quantizer launch, then the plain GEMM
        qbg.qbg_workspace_size(op, 3, 12352, 4096, c)
    assert qbg.qbg_workspace_size(qbg.QBG_OP_FP8, 4, 64, 256, {"kernel_id": 0}) == 0
    with pytest.raises(qbg.QbgError) as ei:   # the fuse mode belongs to the fused ops only
        qbg.qbg_workspace_size(qbg.QBG_OP_FP8, 4, 64, 256, {"kernel_id": 0, "fuse": 1})
    assert ei.value.status == E_CONFIG
    with pytest.raises(qbg.QbgError) as ei:
        qbg.qbg_workspace_size(8, 4, 64, 256, None)
    assert ei.value.status == E_QTYPE


def test_fused_table_entries(L, tmp_path):
    lds = _lds_kids()[0]
    p = tmp_path / "t.txt"
    p.write_text("qbg-config-table 2 gfx950\nfp8_fused 4 4096 4096 %d 1 2 1\n"
                 "int8_fused 1 4096 4096 %d 0 1 0\n" % (lds, lds))
    assert L.qbg_config_table_load(str(p).encode()) == OK
    c, hit = qbg.qbg_config_lookup(qbg.QBG_OP_FP8_FUSED, 3, 4096, 4096)
    assert hit and (c["kernel_id"], c["swap_ab"], c["split_k"], c["rotate"]) == (lds, 1, 2, 1)
    c, hit = qbg.qbg_config_lookup(qbg.QBG_OP_INT8_FUSED, 1, 4096, 4096)
    assert hit and c["kernel_id"] == lds
    c, hit = qbg.qbg_config_lookup(qbg.QBG_OP_FP8, 4, 4096, 4096)  # other ops are not affected
    assert not hit
    reg = next(k for k in range(qbg.qbg_kernel_count()) if qbg.qbg_kernel_info(k)["stages"] == 0)
    p.write_text("qbg-config-table 2 gfx950\nfp8_fused 4 4096 4096 %d 1 1 0\n" % reg)
    assert L.qbg_config_table_load(str(p).encode()) == E_TABLE
    # version 3 carries the fuse mode: a register tile is fine for SEPARATE only
    p.write_text("qbg-config-table 3 gfx950\nfp8_fused 4 4096 4096 %d 1 1 0 2\n"
                 "int8_fused 1 4096 4096 %d 0 2 1 1\nfp8 1 4096 4096 %d 0 1 0 0\n" % (reg, lds, reg))
    assert L.qbg_config_table_load(str(p).encode()) == OK
    c, hit = qbg.qbg_config_lookup(qbg.QBG_OP_FP8_FUSED, 4, 4096, 4096)
    assert hit and (c["kernel_id"], c["fuse"]) == (reg, qbg.QBG_FUSE_SEPARATE)
    c, hit = qbg.qbg_config_lookup(qbg.QBG_OP_INT8_FUSED, 1, 4096, 4096)
    assert hit and (c["kernel_id"], c["split_k"], c["fuse"]) == (lds, 2, qbg.QBG_FUSE_LOCAL)
    for bad in ("fp8_fused 4 4096 4096 %d 1 1 0 1\n" % reg,   # LOCAL on a register tile whose
                                                               # waves take 2048-byte chunks
                "fp8 1 4096 4096 %d 0 1 0 1\n" % reg,         # fuse on a plain op
                "fp8_fused 4 4096 4096 %d 1 1 0\n" % lds):    # v3 wants nine fields
        p.write_text("qbg-config-table 3 gfx950\n" + bad)
        assert L.qbg_config_table_load(str(p).encode()) == E_TABLE, bad


def test_fused_wait_limit_hook(L):
    prev = L.qbg_set_fused_wait_limit(0)
    try:
        assert L.qbg_set_fused_wait_limit(17) == 0
        assert L.qbg_set_fused_wait_limit(-1) == 17
        assert L.qbg_set_fused_wait_limit(5) == 4096   # negative restored the default
    finally:
        L.qbg_set_fused_wait_limit(prev)


def test_block_producer_validation(L):
    z = P(None)
    x, w, q, s = P(FAKE), P(FAKE + 4096), P(FAKE + 8192), P(FAKE + 65536)
    f = L.qbg_rms_norm_quantize_per_token_group
    assert f(x, w, 1e-6, 2, 5120, 128, 7, q, s, z) == E_QTYPE
    assert f(z, w, 1e-6, 2, 5120, 128, 0, q, s, z) == E_NULL
    assert f(x, w, 1e-6, 2, 5120, 64, 0, q, s, z) == E_SHAPE      # group must be 128
    assert f(x, w, 1e-6, 2, 5184, 128, 0, q, s, z) == E_SHAPE     # H not a multiple of 128
    assert f(x, w, 1e-6, 2, 65664, 128, 0, q, s, z) == E_SHAPE    # longer than 65536
    assert f(x, w, -1.0, 2, 5120, 128, 0, q, s, z) == E_SHAPE
    assert f(P(FAKE + 8), w, 1e-6, 2, 5120, 128, 0, q, s, z) == E_ALIGN
    assert f(x, w, 1e-6, 2, 5120, 128, 0, q, P(FAKE + 65537), z) == E_ALIGN  # fp32 scales
    g = L.qbg_silu_mul_quantize_per_token_group
    assert g(x, 2, 25600, 128, 3, q, s, z) == E_QTYPE
    assert g(x, 2, 25600, 128, 0, z, s, z) == E_NULL
    assert g(x, 2, 25600, 256, 0, q, s, z) == E_SHAPE
    assert g(x, 2, 25616, 128, 0, q, s, z) == E_SHAPE
    assert g(x, 0, 25600, 128, 0, q, s, z) == E_SHAPE
    assert g(x, 2, 25600, 128, 0, P(FAKE + 12), s, z) == E_ALIGN


def test_large_m_tiles_rejected_for_block_and_fused_ops():
    big = [k for k in range(qbg.qbg_kernel_count()) if qbg.qbg_kernel_info(k)["tile_m"] > 32]
    assert big
    for kid in big:
        prefill = qbg.qbg_kernel_info(kid)["k_unroll"] == 0  # these run Block-FP8
        for op in (qbg.QBG_OP_FP8_FUSED,) + (() if prefill else (qbg.QBG_OP_BLOCK_FP8, qbg.QBG_OP_BLOCK_UE8M0)):
            with pytest.raises(qbg.QbgError) as ei:
                qbg.qbg_workspace_size(op, 64, 1024, 1024, {"kernel_id": kid})
            assert ei.value.status == E_CONFIG
        with pytest.raises(qbg.QbgError) as ei:   # LOCAL keeps 32 tokens resident at most
            qbg.qbg_workspace_size(qbg.QBG_OP_FP8_FUSED, 64, 1024, 1024,
                                   {"kernel_id": kid, "fuse": qbg.QBG_FUSE_LOCAL})
        assert ei.value.status == E_CONFIG
        # the two-launch form runs the plain op, which has the large-M tiles
        qbg.qbg_workspace_size(qbg.QBG_OP_FP8_FUSED, 64, 1024, 1024,
                               {"kernel_id": kid, "fuse": qbg.QBG_FUSE_SEPARATE})


def test_local_fusion_lds_bound():
    """LOCAL keeps the M bf16 rows (2MK bytes) and tile_m x (K / split_k) code
    bytes in LDS next to the stage ring: 32 rows of 12288 never fit, 4 rows fit
    once K is split, one row fits whole."""
    kid = next(k for k in range(qbg.qbg_kernel_count())
               if qbg.qbg_kernel_info(k)["stages"] > 0 and qbg.qbg_kernel_info(k)["tile_m"] == 32)
    c = {"kernel_id": kid, "fuse": qbg.QBG_FUSE_LOCAL}
    for M, split in ((32, 1), (32, 16), (4, 1)):
        with pytest.raises(qbg.QbgError) as ei:
            qbg.qbg_workspace_size(qbg.QBG_OP_FP8_FUSED, M, 4096, 12288, dict(c, split_k=split))
        assert ei.value.status == E_CONFIG, (M, split)
    qbg.qbg_workspace_size(qbg.QBG_OP_FP8_FUSED, 4, 4096, 12288, dict(c, split_k=4))
    qbg.qbg_workspace_size(qbg.QBG_OP_FP8_FUSED, 1, 4096, 12288, c)


def test_grouped_validation(L):
    z = P(None)
    a, sa, w, sw = P(FAKE), P(FAKE + (1 << 20)), P(FAKE + (2 << 20)), P(FAKE + (3 << 20))
    off, out = P(FAKE + (4 << 20)), P(FAKE + (5 << 20))
    lds = next(k for k in range(qbg.qbg_kernel_count())
               if qbg.qbg_kernel_info(k)["stages"] > 0 and qbg.qbg_kernel_info(k)["tile_m"] == 32)
    reg = next(k for k in range(qbg.qbg_kernel_count()) if qbg.qbg_kernel_info(k)["stages"] == 0)
    big = next(k for k in range(qbg.qbg_kernel_count())
               if qbg.qbg_kernel_info(k)["tile_m"] > 32 and qbg.qbg_kernel_info(k)["k_unroll"] > 0)
    pre = next(k for k in range(qbg.qbg_kernel_count()) if qbg.qbg_kernel_info(k)["k_unroll"] == 0)
    g = L.qbg_grouped_scaled_mm

    def call(qt=0, a_=a, T=64, E=8, N=256, K=512, c=None, off_=off, out_=out):
        return g(qt, a_, sa, w, sw, off_, T, E, N, K, out_, c, z)
    assert call(qt=2) == E_QTYPE
    assert call(a_=z) == E_NULL
    assert call(off_=z) == E_NULL
    assert call(T=-1) == E_SHAPE
    assert call(T=65537) == E_SHAPE
    assert call(E=0) == E_SHAPE
    assert call(N=40) == E_SHAPE
    assert call(K=24) == E_SHAPE
    assert call(a_=P(FAKE + 8)) == E_ALIGN
    assert call(off_=P(FAKE + (4 << 20) + 2)) == E_ALIGN
    assert call(c=cfg(kid=reg)) == E_CONFIG
    assert call(c=cfg(kid=big)) == E_CONFIG       # large-M tiles: plain GEMMs only
    assert call(c=cfg(kid=lds, split=2)) == E_SPLITK
    # prefill tiles: Standard layout, at most 1024 experts (each wave scans the offsets)
    assert call(T=0, c=cfg(kid=pre)) == OK
    assert call(T=0, K=640, c=cfg(kid=pre)) == OK
    assert call(T=0, c=cfg(kid=pre, swap=1)) == E_CONFIG
    assert call(T=0, c=cfg(kid=pre, split=2)) == E_CONFIG
    assert call(T=0, E=1025, c=cfg(kid=pre)) == E_CONFIG
    assert call(T=0, E=1025, c=cfg(kid=lds)) == OK
    assert call(T=0, c=cfg(kid=lds)) == OK        # no routed rows: validated, nothing launched
    c, _ = qbg.qbg_config_lookup(qbg.QBG_OP_FP8_GROUPED, 1024, 1536, 2048)
    assert c["stages"] > 0 and c["split_k"] == 1
    assert qbg.qbg_workspace_size(qbg.QBG_OP_INT8_GROUPED, 4096, 1536, 2048, None) == 0


def test_prefill_tiles_reject_what_they_do_not_run(L):
    kids = [k for k in range(qbg.qbg_kernel_count()) if qbg.qbg_kernel_info(k)["k_unroll"] == 0]
    assert kids, "prefill tiles are compiled"
    for kid in kids:
        assert qbg.qbg_workspace_size(qbg.QBG_OP_FP8, 8192, 528, 1024, {"kernel_id": kid}) == 0
        for cfg, K in (({"kernel_id": kid, "swap_ab": 1}, 1024),
                       ({"kernel_id": kid, "split_k": 16}, 1024),   # chunks of 64
                       ({"kernel_id": kid, "split_k": 32}, 8192),   # more than 16 chunks
                       ({"kernel_id": kid}, 1040)):   # K not a multiple of 128
            with pytest.raises(qbg.QbgError) as ei:
                qbg.qbg_workspace_size(qbg.QBG_OP_FP8, 512, 528, K, cfg)
            assert ei.value.status == E_CONFIG, (cfg, K)
        # split-K: the plain FP8 / INT8 GEMMs (and the fused ops' quantize-then-GEMM);
        # the workspace holds the arrival counters and every chunk's whole tiles
        info = qbg.qbg_kernel_info(kid)
        tm, tn = info["tile_m"], info["tile_n"]
        for op in (qbg.QBG_OP_FP8, qbg.QBG_OP_INT8):
            for split in (2, 8):
                need = qbg.qbg_workspace_size(op, 1000, 528, 1024, {"kernel_id": kid, "split_k": split})
                tiles = -(-1000 // tm) * -(-528 // tn)
                assert need == 65536 + -(-(tiles * split * tm * tn * 4) // 256) * 256, (kid, split)
        assert qbg.qbg_workspace_size(qbg.QBG_OP_FP8_FUSED, 1000, 528, 1024,
                                      {"kernel_id": kid, "split_k": 2, "fuse": qbg.QBG_FUSE_SEPARATE}) > 65536
        # Block-FP8 splits by whole 128-wide scale groups; the grouped GEMM does not split
        assert qbg.qbg_workspace_size(qbg.QBG_OP_BLOCK_UE8M0, 1000, 528, 1024,
                                      {"kernel_id": kid, "split_k": 2}) > 65536
        with pytest.raises(qbg.QbgError) as ei:
            qbg.qbg_workspace_size(qbg.QBG_OP_FP8_GROUPED, 1000, 528, 1024, {"kernel_id": kid, "split_k": 2})
        assert ei.value.status in (E_CONFIG, E_SPLITK)
        assert qbg.qbg_workspace_size(qbg.QBG_OP_INT8, 512, 528, 1024, {"kernel_id": kid}) == 0
        for op in (qbg.QBG_OP_FP8_FUSED, qbg.QBG_OP_INT8_FUSED):
            with pytest.raises(qbg.QbgError):
                qbg.qbg_workspace_size(op, 512, 528, 1024, {"kernel_id": kid})
        for op in (qbg.QBG_OP_FP8_GROUPED, qbg.QBG_OP_INT8_GROUPED):  # experts found on the device
            assert qbg.qbg_workspace_size(op, 4096, 528, 1024, {"kernel_id": kid}) == 0
        # Block-FP8 with fp32 scales: the tiles with at most 64 token rows per wave
        info = qbg.qbg_kernel_info(kid)
        if info["tile_m"] // info["waves_m"] <= 64:
            assert qbg.qbg_workspace_size(qbg.QBG_OP_BLOCK_FP8, 512, 528, 1152, {"kernel_id": kid}) == 0
        else:
            with pytest.raises(qbg.QbgError):
                qbg.qbg_workspace_size(qbg.QBG_OP_BLOCK_FP8, 512, 528, 1024, {"kernel_id": kid})
        # Block-FP8 with UE8M0 scales: K a multiple of 512, the tile's codes in LDS
        assert qbg.qbg_workspace_size(qbg.QBG_OP_BLOCK_UE8M0, 512, 528, 1024, {"kernel_id": kid}) == 0
        # K = 65536: a 256-token tile's codes (256 x 512 bytes) no longer fit beside its ring
        big_ks = (1 << 16,) if qbg.qbg_kernel_info(kid)["tile_m"] == 256 else ()
        for K in (1152,) + big_ks:
            with pytest.raises(qbg.QbgError) as ei:
                qbg.qbg_workspace_size(qbg.QBG_OP_BLOCK_UE8M0, 512, 528, K, {"kernel_id": kid})
            assert ei.value.status == E_CONFIG, K
        # quantizer launch + plain GEMM: the prefill tile serves the fused ops
        for op in (qbg.QBG_OP_FP8_FUSED, qbg.QBG_OP_INT8_FUSED):
            assert qbg.qbg_workspace_size(op, 512, 528, 1024,
                                          {"kernel_id": kid, "fuse": qbg.QBG_FUSE_SEPARATE}) == 0


def test_fused_separate_entries_mirror_the_plain_op():
    """A fused op's SEPARATE entry is the quantizer launch, then the plain op's GEMM:
    its tile, layout, split and rotation equal the plain op's entry for the same key."""
    if not os.path.exists(qbg.DEFAULT_TABLE):
        pytest.skip("no tuned table shipped")
    rows = {}
    for line in open(qbg.DEFAULT_TABLE):
        if not line.strip() or line.startswith(("#", "qbg-config-table")):
            continue
        f = line.split("#")[0].split()
        rows[(f[0], int(f[1]), int(f[2]), int(f[3]))] = f[4:9]
    n = 0
    for key, v in rows.items():
        if key[0] in ("fp8_fused", "int8_fused") and int(v[4]) == qbg.QBG_FUSE_SEPARATE:
            plain = rows.get((key[0][: -len("_fused")],) + key[1:])
            assert plain is not None and plain[:4] == v[:4], (key, v, plain)
            n += 1
    assert n > 0


def test_every_shipped_entry_is_a_valid_configuration_for_its_key():
    """Each table row, forced as the configuration of a call at its own token bucket
    and shape, passes the library's validation (tile support, layout, split and
    chunk rules, LDS size) and sizes its workspace; a split prefill tile stays within
    the 16320 arrival counters."""
    if not os.path.exists(qbg.DEFAULT_TABLE):
        pytest.skip("no tuned table shipped")
    ops = {"fp8": 0, "int8": 1, "block_fp8": 2, "block_ue8m0": 3, "fp8_fused": 4,
           "int8_fused": 5, "fp8_grouped": 6, "int8_grouped": 7}
    n = 0
    for line in open(qbg.DEFAULT_TABLE):
        if not line.strip() or line.startswith(("#", "qbg-config-table")):
            continue
        f = line.split("#")[0].split()
        op, m, N, K = ops[f[0]], int(f[1]), int(f[2]), int(f[3])
        cfg = {"kernel_id": int(f[4]), "swap_ab": int(f[5]), "split_k": int(f[6]),
               "rotate": int(f[7]), "fuse": int(f[8])}
        need = qbg.qbg_workspace_size(op, min(m, 8192), N, K, cfg)  # raises if rejected
        assert need >= 0
        info = qbg.qbg_kernel_info(cfg["kernel_id"])
        if info["k_unroll"] == 0 and cfg["split_k"] > 1:
            tiles = -(-min(m, 8192) // info["tile_m"]) * -(-N // info["tile_n"])
            assert tiles <= 16320, (f, tiles)
        n += 1
    assert n > 400


def _fresh_process(code, env_extra):
    """Run `code` in a new interpreter that loads libqbg.so through raw ctypes only."""
    import subprocess
    import sys
    env = dict(os.environ)
    env.pop("QBG_CONFIG_TABLE", None)
    env.update(env_extra)
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    return r.stdout.split()


_LOOKUP = r'''
import ctypes, sys
sys.path.insert(0, %r)
from quantized_bit_gemm_amd import LIB_PATH, GemmConfig   # constants only: no library load
L = ctypes.CDLL(LIB_PATH)
L.qbg_config_table_size.restype = ctypes.c_int64
L.qbg_config_lookup.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                ctypes.POINTER(GemmConfig), ctypes.POINTER(ctypes.c_int32)]
c = GemmConfig(); hit = ctypes.c_int32(-1)
st = L.qbg_config_lookup(0, 32, 4096, 4096, ctypes.byref(c), ctypes.byref(hit))
print(st, hit.value, c.kernel_id, c.split_k, L.qbg_config_table_size())
''' % ROOT


def test_library_loads_its_shipped_table_without_the_binding():
    if not os.path.exists(qbg.DEFAULT_TABLE):
        pytest.skip("no tuned table shipped")
    st, hit, kid, split, size = map(int, _fresh_process(_LOOKUP, {}))
    assert st == OK and hit == 1 and size > 0
    # the same entry the binding reports
    c, from_table = qbg.qbg_config_lookup(qbg.QBG_OP_FP8, 32, 4096, 4096)
    assert from_table and (c["kernel_id"], c["split_k"]) == (kid, split)


def test_library_table_from_environment(tmp_path):
    p = _write(tmp_path, "qbg-config-table 3 gfx950\nfp8 32 4096 4096 0 1 2 0 0\n")
    st, hit, kid, split, size = map(int, _fresh_process(_LOOKUP, {"QBG_CONFIG_TABLE": p}))
    assert (st, hit, kid, split, size) == (OK, 1, 0, 2, 1)
    # set but empty: no table, the built-in default
    st, hit, kid, split, size = map(int, _fresh_process(_LOOKUP, {"QBG_CONFIG_TABLE": ""}))
    assert st == OK and hit == 0 and size == 0
    # a malformed table leaves the built-in defaults
    bad = _write(tmp_path, "qbg-config-table 3 gfx950\nfp8 32 4096\n", "bad.txt")
    st, hit, kid, split, size = map(int, _fresh_process(_LOOKUP, {"QBG_CONFIG_TABLE": bad}))
    assert st == OK and hit == 0 and size == 0


_LOOKUP_TWO = r'''
import ctypes, sys
sys.path.insert(0, %r)
from quantized_bit_gemm_amd import LIB_PATH, GemmConfig   # constants only: no library load
L = ctypes.CDLL(LIB_PATH)
L.qbg_config_lookup.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                ctypes.POINTER(GemmConfig), ctypes.POINTER(ctypes.c_int32)]
for M in (16, 32):
    c = GemmConfig(); hit = ctypes.c_int32(-1)
    st = L.qbg_config_lookup(0, M, 4096, 4096, ctypes.byref(c), ctypes.byref(hit))
    print(st, hit.value, c.kernel_id, c.swap_ab, c.split_k, c.rotate)
''' % ROOT


def test_lookup_environment_flags():
    if not os.path.exists(qbg.DEFAULT_TABLE):
        pytest.skip("no tuned table shipped")

    def run(env):
        v = list(map(int, _fresh_process(_LOOKUP_TWO, env)))
        return v[:6], v[6:]

    # QBG_MAX_TUNED_M: 16 tokens from the table, 32 beyond the tuned window (the default)
    m16, m32 = run({"QBG_MAX_TUNED_M": "16"})
    assert (m16[0], m16[1], m32[0], m32[1]) == (OK, 1, OK, 0)
    # QBG_FORCE_CONFIG overrides every lookup
    m16, m32 = run({"QBG_FORCE_CONFIG": "0,1,2,1"})
    assert m16 == m32 == [OK, 0, 0, 1, 2, 1]
    # malformed values are ignored: both lookups come from the table
    for env in ({"QBG_FORCE_CONFIG": "0,1"}, {"QBG_FORCE_CONFIG": "a,b,c"},
                {"QBG_MAX_TUNED_M": "abc"}, {"QBG_MAX_TUNED_M": "0"}):
        m16, m32 = run(env)
        assert m16[:2] == [OK, 1] and m32[:2] == [OK, 1], env
