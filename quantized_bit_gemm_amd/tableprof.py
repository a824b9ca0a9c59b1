"""Launch sets for rocprofv3 evidence behind the configuration table.

The table holds, per (op, M bucket, N, K), the configuration the tuner timed
fastest ("Helion nel backend vLLM", ai-radar.it, paragraphs 3 and 7: the
per-shape configurations are chosen ahead of time by measurement).  This
module produces the launches that let a profiler check each decode entry:

  select  For every decode entry (per-channel FP8 and INT8 at the 8B-decoder
          shapes, Block-FP8 with fp32 and with UE8M0 scales at the
          32B-decoder shapes; buckets 1 to 32) time, with the tuner's graph
          timer, the entry's configuration and its neighbourhood: every tile
          variant at the entry's layout and split_k, and the entry's tile at
          every split_k and both layouts.  The runner-up is the fastest
          configuration that differs from the entry in kernel_id, swap_ab or
          split_k.  Writes the list of launch sets (winner and runner-up per
          entry) as JSON.
  cases   Write a launch-set list from explicit cases (op:NxK:M:kid,swap,split).
  launch  Run every set of a list `warmup` + `reps` times, each call on its own weight
          copy (1 GiB of copies per shape, so each call streams its weights
          from HBM; the copies are read once after they are built) and synchronized,
          after one plain device copy of
          --calibrate-mib MiB that scales the byte counters.  This is the
          dispatch sequence that rocprofv3 records; profsummary `sets` maps
          it back to the sets.

Usage (on the GPU, from the repository root):
  python -m quantized_bit_gemm_amd.tableprof select --out sets.json
  rocprofv3 --kernel-trace -d DIR -o trace -- python3 -m quantized_bit_gemm_amd.tableprof launch sets.json
  rocprofv3 --pmc FETCH_SIZE -d DIR -o fetch -- python3 -m quantized_bit_gemm_amd.tableprof launch sets.json
  python -m quantized_bit_gemm_amd.profsummary sets sets.json --trace DIR/trace_results.db \\
      --pmc DIR/fetch_results.db --out profiles/....txt
"""
from __future__ import annotations

import argparse
import json
import sys
import time

from quantized_bit_gemm_amd import tune

DECODE_OPS = {
    "fp8": [(6144, 4096), (4096, 4096), (24576, 4096), (4096, 12288)],
    "int8": [(6144, 4096), (4096, 4096), (24576, 4096), (4096, 12288)],
    "block_fp8": [(10240, 5120), (5120, 8192), (51200, 5120), (5120, 25600)],
    "block_ue8m0": [(10240, 5120), (5120, 8192), (51200, 5120), (5120, 25600)],
}
DECODE_MS = [1, 2, 4, 8, 16, 32]
KEYS = ("kernel_id", "swap_ab", "split_k", "rotate")


def _cfg(c):
    return {k: int(c.get(k, 0)) for k in KEYS}


def _differs(a, b):
    return any(a[k] != b[k] for k in ("kernel_id", "swap_ab", "split_k"))


def neighbourhood(qbg, op, M, N, K, win):
    """The entry's configuration and the alternatives timed against it."""
    out = [win]
    for cfg in tune.feasible_configs(qbg, op, K):
        same_layout = cfg["swap_ab"] == win["swap_ab"] and cfg["split_k"] == win["split_k"]
        same_tile = cfg["kernel_id"] == win["kernel_id"]
        if not (same_layout or same_tile) or cfg["rotate"] != win["rotate"]:
            continue
        c = _cfg(cfg)
        if not _differs(c, win):
            continue
        try:
            qbg.qbg_workspace_size(op, M, N, K, c)
        except qbg.QbgError:
            continue
        out.append(c)
    return out


def select(args):
    import torch

    import quantized_bit_gemm_amd as qbg

    dev = torch.device("cuda", 0)
    sets = []
    for opname in args.ops.split(","):
        op = tune.OPS[opname]
        for (N, K) in DECODE_OPS[opname]:
            prob = tune.Problem(torch, qbg, op, N, K, max(DECODE_MS), dev)
            for M in DECODE_MS:
                t0 = time.time()
                win_full, from_table = qbg.qbg_config_lookup(op, M, N, K)
                if not from_table:
                    raise SystemExit("%s N=%d K=%d M=%d has no table entry" % (opname, N, K, M))
                win = _cfg(win_full)
                cands = neighbourhood(qbg, op, M, N, K, win)
                timed = [(prob.time_config(M, c, args.reps), c) for c in cands]
                win_us = timed[0][0]
                ru_us, ru = min(timed[1:], key=lambda t: t[0])
                entry = {"op": opname, "N": N, "K": K, "M": M}
                sets.append(dict(entry, role="winner", config=win, select_us=round(win_us, 3)))
                sets.append(dict(entry, role="runner-up", config=ru, select_us=round(ru_us, 3),
                                 candidates=len(cands)))
                print("[tableprof] %-11s N=%5d K=%5d M=%2d winner %s %.2f us, runner-up %s %.2f us "
                      "(%d timed, %.1fs)" % (opname, N, K, M, win, win_us, ru, ru_us, len(cands),
                                            time.time() - t0), flush=True)
            del prob
            torch.cuda.empty_cache()
    with open(args.out, "w") as f:
        json.dump(sets, f, indent=0)
    print("[tableprof] wrote %d launch sets to %s" % (len(sets), args.out))


def cases(args):
    sets = []
    for spec in args.case:
        opname, shape, m, cfg = spec.split(":")
        N, K = (int(v) for v in shape.split("x"))
        kid, swap, split = (int(v) for v in cfg.split(","))
        sets.append({"op": opname, "N": N, "K": K, "M": int(m), "role": "case",
                     "config": {"kernel_id": kid, "swap_ab": swap, "split_k": split, "rotate": 0}})
    with open(args.out, "w") as f:
        json.dump(sets, f, indent=0)
    print("[tableprof] wrote %d launch sets to %s" % (len(sets), args.out))


def launch(args):
    import torch

    import quantized_bit_gemm_amd as qbg

    dev = torch.device("cuda", 0)
    sets = json.load(open(args.sets))
    if args.calibrate_mib:
        n = args.calibrate_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        print("[tableprof] calibration copy of %d MiB" % args.calibrate_mib, flush=True)
    # Sets run in list order; a shape's operands are built when its first set comes.
    prob, prob_key = None, None
    for i, s in enumerate(sets):
        key = (s["op"], s["N"], s["K"])
        if key != prob_key:
            prob = None
            torch.cuda.empty_cache()
            prob = tune.Problem(torch, qbg, tune.OPS[s["op"]], s["N"], s["K"], max(DECODE_MS), dev)
            prob_key = key  # (Problem reads every weight copy once after building it)
        cfg = s["config"]
        op = tune.OPS[s["op"]]
        need = qbg.qbg_workspace_size(op, s["M"], s["N"], s["K"], cfg)
        ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev) if need else None
        torch.cuda.synchronize()
        for r in range(args.warmup + args.reps):
            prob.launch(r, s["M"], cfg, ws)
            torch.cuda.synchronize()
        print("[tableprof] set %d/%d %s N=%d K=%d M=%d %s %s done" % (
            i + 1, len(sets), s["op"], s["N"], s["K"], s["M"], s["role"], cfg), flush=True)
    print("[tableprof] launched %d sets x (%d + %d) calls" % (len(sets), args.warmup, args.reps))


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("select")
    s.add_argument("--ops", default=",".join(DECODE_OPS))
    s.add_argument("--reps", type=int, default=3)
    s.add_argument("--out", required=True)
    c = sub.add_parser("cases")
    c.add_argument("case", nargs="+", help="op:NxK:M:kernel_id,swap_ab,split_k")
    c.add_argument("--out", required=True)
    la = sub.add_parser("launch")
    la.add_argument("sets")
    la.add_argument("--reps", type=int, default=10)
    la.add_argument("--warmup", type=int, default=2,
                    help="calls before the counted ones in every set (dropped by the summary)")
    la.add_argument("--calibrate-mib", type=int, default=512)
    args = ap.parse_args(argv)
    {"select": select, "cases": cases, "launch": launch}[args.cmd](args)


if __name__ == "__main__":
    sys.exit(main())
