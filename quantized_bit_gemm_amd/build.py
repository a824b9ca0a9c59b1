"""Build libqbg.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage: python -m quantized_bit_gemm_amd.build [--sanitize]  (or build()).
Objects go to _build/ at the repository root; the shared library is written
next to this file so that it travels with the source tree.

--sanitize builds _build_san/libqbg_san.so instead: the same
sources with AddressSanitizer and UndefinedBehaviorSanitizer on the host code
only (argument validation, the table parser, the launch set-up); device code
is compiled as usual.  It runs on the CPU with clang's ASan runtime preloaded
(tests/run_sanitizers.py).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libqbg.so")
# (source, object stem, extra flags): the GEMM family is compiled as eight
# parts in parallel (see QBG_GEMM_PART in gemm_kernels.hip).
GEMM_PARTS = 8
SOURCES = ([("quant_kernels.hip", "quant_kernels", []), ("qbg_api.hip", "qbg_api", [])] +
           [("gemm_kernels.hip", "gemm_kernels_p%d" % i, ["-DQBG_GEMM_PART=%d" % i])
            for i in range(GEMM_PARTS)])
ARCH = "gfx950"

# -ffp-contract=off: the quantizers' bit-exactness relies on unfused fp32
# arithmetic; the GEMM uses explicit fma where it wants one.
# The packed-fp32 target feature is switched off for all device code.
HIPFLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-Wall", "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libqbg)")


# Host-only sanitizer flags, each after -Xarch_host so device code stays as is.
SAN_CHECKS = ("address", "undefined")
SAN_FLAGS = [f for c in SAN_CHECKS for f in ("-Xarch_host", "-fsanitize" + "=" + c)]
SAN_HOST = ["-Xarch_host", "-g", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-fno-sanitize-recover=all"]
BUILD_SAN = os.path.join(ROOT, "_build_san")
LIB_SAN = os.path.join(BUILD_SAN, "libqbg_san.so")


def _compile(job) -> str:
    src, stem, extra, sanitize = job
    obj = os.path.join(BUILD_SAN if sanitize else BUILD, stem + ".o")
    san = SAN_FLAGS + SAN_HOST if sanitize else []
    cmd = [hipcc(), *HIPFLAGS, *san, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, out))
    if out:
        sys.stderr.write(out + "\n")
    return obj


def build(verbose: bool = True, sanitize: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libqbg.so (libqbg_san.so
    with sanitize); returns its path."""
    os.makedirs(BUILD_SAN if sanitize else BUILD, exist_ok=True)
    workers = min(len(SOURCES), int(os.environ.get("MAX_JOBS", "0")) or os.cpu_count() or 4)
    with ThreadPoolExecutor(max_workers=workers) as ex:
        objs = list(ex.map(_compile, [job + (sanitize,) for job in SOURCES]))
    lib = LIB_SAN if sanitize else LIB
    if sanitize:  # the library loads configs/ from beside itself
        link = os.path.join(BUILD_SAN, "configs")
        if not os.path.lexists(link):
            os.symlink(os.path.join(PKG, "configs"), link)
    tmp = lib + ".tmp%d" % os.getpid()
    san = SAN_FLAGS + ["-shared-libsan"] if sanitize else []
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", *san, *objs, "-o", tmp]
    subprocess.check_call(cmd)
    os.replace(tmp, lib)
    if verbose:
        print("built", lib)
    return lib


if __name__ == "__main__":
    build(sanitize="--sanitize" in sys.argv[1:])
