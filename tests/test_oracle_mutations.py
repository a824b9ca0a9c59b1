"""Planted mistakes: each mutant copy of oracle.c must fail the oracle's pins.

Every mutation below is a plausible slip (a dropped term, a wrong sign or
index, a transposed operand, a different rounding).  A mutant is built with
gcc into a temporary directory and the pin tests are re-run against it in a
subprocess; the test passes only if the pins catch every mutant.  Everything
happens on the CPU.
"""
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTATIONS = [
    ("subnormal exponent", "ldexp((double)m / 8.0, -6)", "ldexp((double)m / 8.0, -7)"),
    ("ties to odd", "((c + 1) & 1) == 0", "((c + 1) & 1) == 1"),
    ("sign dropped on encode", "(signbit(x) ? 0x80 : 0)", "(x < 0.0f ? 0x80 : 0)"),
    ("reciprocal multiply for x/s", "float t = v[i * stride] / s;",
     "float t = v[i * stride] * (1.0f / s);"),
    ("reciprocal multiply for the scale", "(amax > 0.0f) ? amax / qmax : 1.0f",
     "(amax > 0.0f) ? amax * (1.0f / qmax) : 1.0f"),
    ("negative clamp sign", "if (t < -qmax) t = -qmax;", "if (t < -qmax) t = qmax;"),
    ("int8 truncation", "double r = rint((double)x);", "double r = trunc((double)x);"),
    ("UE8M0 rounds to nearest power", "int p = (f == 0.5) ? e - 1 : e;",
     "int p = (f < 0.75) ? e - 1 : e;"),
    ("bf16 truncation", "double r = rint(a / ulp) * ulp;", "double r = floor(a / ulp) * ulp;"),
    ("weight scale dropped", "double r = ((double)sa[m] * (double)sw[n]) * d;",
     "double r = ((double)sa[m]) * d;"),
    ("reversed weight index", "dec8(qtype, qw, n * K + k)", "dec8(qtype, qw, n * K + (K - 1 - k))"),
    ("swap-ab scale roles", "double r = ((double)sw[n] * (double)sa[m]) * d;",
     "double r = ((double)sw[m % N] * (double)sa[n % M]) * d;"),
    ("split-k chunk dropped", "for (int64_t c = 0; c < S; ++c)",
     "for (int64_t c = 0; c + 1 < S; ++c)"),
    ("rmsnorm eps dropped", "sqrt(ss / (double)H + (double)eps)", "sqrt(ss / (double)H)"),
    ("rmsnorm mean over H-1", "ss / (double)H +", "ss / (double)(H - 1) +"),
    ("rmsnorm weight dropped", "* r) * orc_bf16_to_double(w[k]);", "* r) * 1.0;"),
    ("silu sign", "exp(-g)", "exp(g)"),
    ("gate and up read from the same half", "double g = orc_bf16_to_double(gu[m * 2 * I + k]);",
     "double g = orc_bf16_to_double(gu[m * 2 * I + I + k]);"),
    ("group scale layout transposed", "((float*)s)[m * ng + g] = sf;",
     "((float*)s)[g * M + m] = sf;"),
    ("block weight scale index", "(n / G) * ng + g", "(n / G) + g * ((N + G - 1) / G)"),
    ("block activation scale index", "scale_at(scale_fmt, sa, m * ng + g)",
     "scale_at(scale_fmt, sa, g * M + m)"),
    ("fp32-input group quantizer ignores UE8M0",
     "quant_span(ORC_FP8, scale_fmt, y + m * K + g * G, G, 1,",
     "quant_span(ORC_FP8, ORC_SCALE_F32, y + m * K + g * G, G, 1,"),
    ("fp32-input group span one short", "y + m * K + g * G, G, 1,", "y + m * K + g * G, G - 1, 1,"),
    ("grouped GEMM reads expert 0's weights",
     "const char* we = (const char*)qw + (size_t)(e * N * K) * wsz;",
     "const char* we = (const char*)qw;"),
    ("grouped GEMM reads expert 0's scales", "const float* se = sw + e * N;",
     "const float* se = sw;"),
]

PIN_TESTS = ["tests/test_oracle_codecs.py", "tests/test_oracle_quant.py",
             "tests/test_oracle_gemm.py", "tests/test_oracle_block_producers.py",
             "tests/test_oracle_grouped.py"]


def _run_mutant(tmpdir, idx, original, mutated):
    src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    assert original in src, "mutation anchor not found: %r" % original
    mdir = os.path.join(tmpdir, "m%d" % idx)
    os.makedirs(mdir)
    csrc = os.path.join(mdir, "oracle.c")
    with open(csrc, "w") as f:
        f.write(src.replace(original, mutated))
    so = os.path.join(mdir, "liboracle.so")
    subprocess.check_call(["gcc", *oracle.CFLAGS, csrc, "-o", so, "-lm"],
                          stderr=subprocess.DEVNULL)
    env = dict(os.environ, QBG_ORACLE_LIB=so, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        *PIN_TESTS], cwd=ROOT, env=env, stdout=subprocess.PIPE,
                       stderr=subprocess.STDOUT, timeout=600)
    return r.returncode


def test_every_planted_mistake_is_caught():
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    tmpdir = tempfile.mkdtemp(prefix="oracle_mutants_")
    try:
        with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
            # control: an unmodified copy built the same way must pass the pins
            control = ex.submit(_run_mutant, tmpdir, len(MUTATIONS), "", "")
            futs = {name: ex.submit(_run_mutant, tmpdir, i, a, b)
                    for i, (name, a, b) in enumerate(MUTATIONS)}
            survivors = [name for name, f in futs.items() if f.result() == 0]
            assert control.result() == 0, "the unmodified oracle fails its own pins"
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    assert not survivors, "planted mistakes not caught by the pins: %s" % survivors
