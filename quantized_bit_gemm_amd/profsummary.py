"""Summaries of rocprofv3 result databases for the GEMM family.

rocprofv3 (ROCm 7) writes SQLite databases; this module reads the kernel
trace (per-dispatch durations) and PMC runs (FETCH_SIZE / WRITE_SIZE per
dispatch) and writes a short text summary.  HBM bytes are the raw counters
(KiB) scaled by what the same counter reads for a plain device copy of known
size made in the same run (bench.py --calibrate-copy).

Usage:
  python -m quantized_bit_gemm_amd.profsummary trace  <results.db> [--command CMD]
  python -m quantized_bit_gemm_amd.profsummary pmc    <fetch.db> <write.db> --copy-mib 256
  python -m quantized_bit_gemm_amd.profsummary eager  <results.db> --details details.json --reps R

`eager` reads the last R x len(details) GEMM dispatches of a run made with
bench.py --eager-pass R --details details.json (every GEMM launched alone,
synchronized), so each duration is the kernel's own execution time, and
reports per (N, K, M) the mean duration and algorithmic bytes / duration.
"""
from __future__ import annotations

import argparse
import collections
import sqlite3
import statistics

import hashlib
import os

GEMM_KERNELS = ("gemm_kernel", "gemm_lds_kernel", "gemm_lds_grouped_kernel",
                "gemm_prefill_kernel")  # all GEMM launches
_PKG = os.path.dirname(os.path.abspath(__file__))
# Files whose content determines the GEMM kernels a benchmark step launches.
GEMM_SOURCES = ["csrc/gemm_kernels.hip", "csrc/qbg_device.h", "csrc/qbg_launch.h",
                "configs/gfx950.txt"]


def gemm_source_hash() -> str:
    h = hashlib.sha256()
    for rel in GEMM_SOURCES:
        with open(os.path.join(_PKG, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read())
    return h.hexdigest()
QUANT = "quant_per_token_kernel"


def is_gemm(short_name: str) -> bool:
    return short_name.startswith(GEMM_KERNELS)


def short(name: str) -> str:
    n = name
    for p in ("void ", "qbg::(anonymous namespace)::", "(anonymous namespace)::"):
        n = n.replace(p, "")
    return n.split("(")[0]


def trace_summary(db: str):
    c = sqlite3.connect(db)
    rows = c.execute("select name, duration from kernels").fetchall()
    per = collections.defaultdict(list)
    for name, dur in rows:
        per[short(name)].append(dur / 1e3)
    total = sum(sum(v) for v in per.values())
    lines = ["%-62s %7s %10s %9s %6s" % ("kernel", "calls", "total_us", "avg_us", "pct")]
    for k, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        lines.append("%-62s %7d %10.1f %9.3f %5.1f%%" % (k[:62], len(v), sum(v), statistics.mean(v),
                                                         100 * sum(v) / total))
    gemm = [d for k, v in per.items() if is_gemm(k) for d in v]
    quant = [d for k, v in per.items() if k.startswith(QUANT) for d in v]
    agg = {"gemm_calls": len(gemm), "gemm_avg_us": statistics.mean(gemm) if gemm else 0.0,
           "quant_calls": len(quant), "quant_avg_us": statistics.mean(quant) if quant else 0.0}
    return lines, agg


def _counter(db: str):
    c = sqlite3.connect(db)
    return c.execute("select kernel_name, dispatch_id, counter_name, value from counters_collection"
                     ).fetchall()


def pmc_summary(fetch_db: str, write_db: str, copy_mib: int):
    copy_kib = copy_mib * 1024.0

    def calib(rows):
        # the calibration copy is the largest device copy of the run
        copies = [v for (n, d, cn, v) in rows if "copyBuffer" in n]
        return copy_kib / max(copies)

    fr, wr = _counter(fetch_db), _counter(write_db)
    kf, kw = calib(fr), calib(wr)
    per = collections.defaultdict(lambda: [[], []])
    for rows, idx in ((fr, 0), (wr, 1)):
        for n, d, cn, v in rows:
            if is_gemm(short(n)):
                per[short(n)][idx].append(v)
    lines = ["FETCH_SIZE scale %.4f (calibration copy of %d MiB read %.0f KiB raw)" %
             (kf, copy_mib, copy_kib / kf),
             "WRITE_SIZE scale %.4f (calibration copy of %d MiB wrote %.0f KiB raw)" %
             (kw, copy_mib, copy_kib / kw),
             "%-62s %6s %14s %14s" % ("kernel", "calls", "fetch_MB/call", "write_MB/call")]
    all_f, all_w = [], []
    for k, (f, w) in sorted(per.items()):
        mf = statistics.mean(f) * kf * 1024 / 1e6 if f else 0.0
        mw = statistics.mean(w) * kw * 1024 / 1e6 if w else 0.0
        all_f += f
        all_w += w
        lines.append("%-62s %6d %14.3f %14.3f" % (k[:62], len(f), mf, mw))
    traffic = (statistics.mean(all_f) * kf + statistics.mean(all_w) * kw) * 1024 if all_f else 0.0
    return lines, {"fetch_scale": kf, "write_scale": kw, "gemm_traffic_bytes_per_launch": traffic}


def eager_summary(db: str, details: str, reps: int):
    import json

    calls = json.load(open(details))
    c = sqlite3.connect(db)
    rows = c.execute("select name, start, duration from kernels order by start").fetchall()
    gemm = [(short(n), d) for n, st, d in rows if is_gemm(short(n))]
    n = len(calls)
    tail = gemm[-reps * n:]
    if len(tail) != reps * n:
        raise SystemExit("expected %d GEMM dispatches, found %d" % (reps * n, len(tail)))
    lines = ["%5s %5s %3s  %9s  %8s  %6s  %s" % ("N", "K", "M", "kernel_us", "TB/s", "%8TB/s",
                                                   "kernel")]
    tot_b, tot_t = 0.0, 0.0
    for i, call in enumerate(calls):
        ds = [tail[r * n + i][1] / 1e3 for r in range(reps)]
        us = statistics.mean(ds)
        tbs = call["bytes"] / us / 1e6
        tot_b += call["bytes"]
        tot_t += us
        lines.append("%5d %5d %3d  %9.2f  %8.3f  %5.1f%%  %s" % (
            call["N"], call["K"], call["M"], us, tbs, 100 * tbs / 8.0, tail[i][0][:48]))
    agg = {"kernel_only_TBs": tot_b / tot_t / 1e6, "kernel_only_frac_of_8TBs": tot_b / tot_t / 8e6,
           "mean_kernel_us": tot_t / n}
    return lines, agg


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("db")
    p = sub.add_parser("pmc")
    p.add_argument("fetch_db")
    p.add_argument("write_db")
    p.add_argument("--copy-mib", type=int, required=True)
    sub.add_parser("hash")
    e = sub.add_parser("eager")
    e.add_argument("db")
    e.add_argument("--details", required=True)
    e.add_argument("--reps", type=int, required=True)
    args = ap.parse_args(argv)
    if args.cmd == "hash":
        print(gemm_source_hash())
        return
    if args.cmd == "trace":
        lines, agg = trace_summary(args.db)
    elif args.cmd == "eager":
        lines, agg = eager_summary(args.db, args.details, args.reps)
    else:
        lines, agg = pmc_summary(args.fetch_db, args.write_db, args.copy_mib)
    print("\n".join(lines))
    for k, v in agg.items():
        print("%s: %s" % (k, round(v, 4) if isinstance(v, float) else v))


if __name__ == "__main__":
    main()
