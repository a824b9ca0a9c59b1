"""Run the CPU test suite under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds the library's host-sanitizer variant (_build_san/libqbg_san.so: host
code instrumented, device code as usual) and the oracle with the same
sanitizers (_build_san/liboracle_san.so), then runs `pytest tests -m "not gpu"`
in a child process with clang's ASan runtime preloaded and both libraries
selected through QBG_LIBRARY and QBG_ORACLE_LIB.  Any sanitizer report aborts
the run (no recovery), so a green suite means no report.  Leak detection is
off: the Python interpreter and torch keep allocations until exit.

Usage: python tests/run_sanitizers.py [extra pytest args]
"""
import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def main(argv):
    import oracle
    from quantized_bit_gemm_amd import build

    lib = build.build(sanitize=True)
    olib = oracle.build_sanitized(build.BUILD_SAN)
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt:
        raise SystemExit("clang's ASan runtime not found under /opt/rocm/llvm")
    env = dict(os.environ, LD_PRELOAD=rt[-1], QBG_LIBRARY=lib, QBG_ORACLE_LIB=olib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-m", "not gpu", "-q", "-x",
           "-p", "no:cacheprovider", *argv]
    print("[sanitizers] %s" % " ".join(cmd), flush=True)
    return subprocess.call(cmd, env=env, cwd=ROOT)


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
