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
  python -m quantized_bit_gemm_amd.profsummary sets   <sets.json> --trace <db> [--pmc <db> ...]
                                                      [--reps R] [--out FILE] [--command CMD ...]

`eager` reads the last R x len(details) GEMM dispatches of a run made with
bench.py --eager-pass R --details details.json (every GEMM launched alone,
synchronized), so each duration is the kernel's own execution time, and
reports per (N, K, M) the mean duration and algorithmic bytes / duration.

`sets` reads runs of tableprof.py launch (every launch set of a list called
W + R times, one GEMM dispatch per call, synchronized; the first W of each set
are dropped): the kernel trace gives each
set's mean duration, each PMC database the mean of its counters per dispatch
(FETCH_SIZE and WRITE_SIZE scaled to bytes by the run's calibration copy).
For a `select` list (winner and runner-up per table entry) it writes one row
per entry; for a `cases` list one row per case.
"""
from __future__ import annotations

import argparse
import collections
import sqlite3
import statistics

import hashlib
import json
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


def table_hash() -> str:
    with open(os.path.join(_PKG, "configs", "gfx950.txt"), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def _gemm_trace(db: str):
    c = sqlite3.connect(db)
    rows = c.execute("select name, start, duration from kernels order by start").fetchall()
    return [(short(n), d / 1e3) for n, st, d in rows if is_gemm(short(n))]


def _gemm_pmc(db: str):
    """GEMM dispatches in dispatch order as (kernel, {counter: value}), and the
    counters of the largest device copy (the calibration copy)."""
    per = collections.OrderedDict()
    for n, d, cn, v in sorted(_counter(db), key=lambda r: r[1]):
        e = per.setdefault(d, [short(n), collections.defaultdict(float)])
        e[1][cn] += v
    gemm = [(k, dict(c)) for k, c in per.values() if is_gemm(k)]
    copies = [c for k, c in per.values() if "copyBuffer" in k]
    return gemm, copies


def sets_summary(sets_path: str, trace_db: str, pmc_dbs, reps: int, copy_mib: int,
                 warmup: int = 0):
    """Per launch set: the last `reps` of its warmup + reps dispatches."""
    sets = json.load(open(sets_path))
    n = len(sets)
    per = warmup + reps
    trace = _gemm_trace(trace_db)
    if len(trace) != n * per:
        raise SystemExit("%s: expected %d GEMM dispatches (%d sets x %d), found %d" %
                         (trace_db, n * per, n, per, len(trace)))
    rows = []
    for i, s in enumerate(sets):
        ds = [d for _, d in trace[i * per + warmup:(i + 1) * per]]
        rows.append({"set": s, "kernel": trace[i * per][0], "us": statistics.mean(ds),
                     "us_min": min(ds), "counters": {}})
    scales = {}
    for db in pmc_dbs:
        gemm, copies = _gemm_pmc(db)
        if len(gemm) != n * per:
            raise SystemExit("%s: expected %d GEMM dispatches, found %d" % (db, n * per, len(gemm)))
        for i, r in enumerate(rows):
            chunk = [c for _, c in gemm[i * per + warmup:(i + 1) * per]]
            for name in chunk[0]:
                base = name.split("_sum")[0]
                val = statistics.mean(c[name] for c in chunk)
                if base in ("FETCH_SIZE", "WRITE_SIZE"):
                    if base not in scales:
                        raw = max(c.get(name, 0.0) for c in copies) if copies else 0.0
                        if raw <= 0:
                            raise SystemExit("%s: no calibration copy for %s" % (db, name))
                        scales[base] = copy_mib * 1024.0 / raw
                    r["counters"][base + "_MB"] = val * scales[base] * 1024 / 1e6
                else:
                    r["counters"][name] = val
    return rows, scales


def _cfg_str(c):
    return "%d/%d/%d" % (c["kernel_id"], c["swap_ab"], c["split_k"])


def render_sets(rows, scales, commands):
    from quantized_bit_gemm_amd import tune

    lines = ["# source_sha256: %s" % gemm_source_hash(), "# table_sha256: %s" % table_hash()]
    lines += ["# command: %s" % c for c in commands]
    for k, v in sorted(scales.items()):
        lines.append("# %s scale %.4f (bytes per raw KiB, from the calibration copy)" % (k, v))
    entries = [r for r in rows if r["set"]["role"] in ("winner", "runner-up")]
    if entries:
        lines.append("# config = kernel_id/swap_ab/split_k; us = mean kernel-trace duration; "
                     "fetch = FETCH_SIZE MB per dispatch; alg = algorithmic MB per call;")
        lines.append("# sel = the select step's graph-timed us (winner, runner-up)")
        lines.append("%-11s %5s %5s %2s %6s | %-9s %7s %7s | %-9s %7s %7s | %6s %s" % (
            "op", "N", "K", "M", "alg", "winner", "us", "fetch", "runner-up", "us", "fetch",
            "ru/win", "sel"))
        wins = 0
        for w, ru in zip(entries[0::2], entries[1::2]):
            s = w["set"]
            alg = tune.gemm_bytes(tune.OPS[s["op"]], s["M"], s["N"], s["K"]) / 1e6
            fw = w["counters"].get("FETCH_SIZE_MB", float("nan"))
            fr = ru["counters"].get("FETCH_SIZE_MB", float("nan"))
            wins += w["us"] <= ru["us"]
            lines.append("%-11s %5d %5d %2d %6.2f | %-9s %7.2f %7.2f | %-9s %7.2f %7.2f | %6.3f "
                         "%.2f,%.2f" % (s["op"], s["N"], s["K"], s["M"], alg,
                                        _cfg_str(w["set"]["config"]), w["us"], fw,
                                        _cfg_str(ru["set"]["config"]), ru["us"], fr,
                                        ru["us"] / w["us"], s.get("select_us", 0),
                                        ru["set"].get("select_us", 0)))
        lines.append("entries: %d; winner faster in the kernel trace: %d" % (len(entries) // 2, wins))
    cases = [r for r in rows if r["set"]["role"] == "case"]
    if cases:
        names = sorted({k for r in cases for k in r["counters"]})
        lines.append("# per case: mean kernel-trace us and the mean of each counter per dispatch")
        for r in cases:
            s = r["set"]
            lines.append("%s N=%d K=%d M=%d config %s kernel %s: %.2f us (min %.2f)" % (
                s["op"], s["N"], s["K"], s["M"], _cfg_str(s["config"]), r["kernel"], r["us"],
                r["us_min"]))
            for k in names:
                if k in r["counters"]:
                    lines.append("    %-36s %16.1f" % (k, r["counters"][k]))
    return lines


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
    st = sub.add_parser("sets")
    st.add_argument("sets")
    st.add_argument("--trace", required=True)
    st.add_argument("--pmc", action="append", default=[])
    st.add_argument("--reps", type=int, default=10)
    st.add_argument("--warmup", type=int, default=0,
                    help="dispatches to drop at the start of every set (tableprof launch --warmup)")
    st.add_argument("--copy-mib", type=int, default=512)
    st.add_argument("--command", action="append", default=[])
    st.add_argument("--out", default="")
    args = ap.parse_args(argv)
    if args.cmd == "sets":
        rows, scales = sets_summary(args.sets, args.trace, args.pmc, args.reps, args.copy_mib,
                                    args.warmup)
        text = "\n".join(render_sets(rows, scales, args.command)) + "\n"
        if args.out:
            with open(args.out, "w") as f:
                f.write(text)
        print(text, end="")
        return
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
