"""Fuse-mode selection inside the FP8 decode step.

tune.py times each configuration alone: a graph of the same call on rotating
weight copies.  For the fused quantize+GEMM op that ranking does not carry over
to a step of independent calls of different shapes, where the one-launch LOCAL
mode (every workgroup quantizes the activation rows itself) wins by 1-2 us
alone but often loses.  This script decides the fused entries of the table
inside the step itself:

1. it builds the decode step (per shape and token count one
   qbg_quantize_scaled_mm call on its own weight copy, all captured in one HIP
   graph, the configurations from the loaded table);
2. for each call with at most --max-m tokens it times every one-launch
   candidate alone (tune.Problem) and keeps the --top fastest; with --modes 2
   it also shortlists, for every call, the --top fastest other GEMM
   configurations of a tune.py checkpoint, run behind the quantizer (SEPARATE);
3. it times the step with that call's configuration replaced by each kept
   candidate against the unchanged step, in --pairs alternating pairs of
   --reps replays each, and keeps the candidate whose step time is lower in
   every pair by the largest median margin, if that margin exceeds
   --min-gain-us;
4. it times the step with every kept replacement at once against the
   unchanged step, and writes the kept entries as table lines (or none, if the
   combination does not win in every pair); a kept SEPARATE configuration is
   written for the plain fp8 op as well, whose entry that GEMM is.

This is the pages' ahead-of-time per-shape choice among algorithmic variants
("Helion nel backend vLLM", ai-radar.it, paragraphs 3 and 7), made in the
context the table serves.

Usage:
  python -m quantized_bit_gemm_amd.steptune --out fused_entries.txt \
      [--shapes 6144x4096,...] [--ms 1,2,4,8,16,32] [--max-m 4]
"""
from __future__ import annotations

import argparse
import json
import sys
import time

import numpy as np

DECODE_SHAPES = [(6144, 4096), (4096, 4096), (24576, 4096), (4096, 12288)]
DECODE_MS = [1, 2, 4, 8, 16, 32]
KEYS = ("kernel_id", "swap_ab", "split_k", "rotate", "fuse")


def log(*a):
    print("[steptune]", *a, file=sys.stderr, flush=True)


class Step:
    """The decode step: one fused call per (shape, M), each on its own weight copy."""

    def __init__(self, torch, qbg, synth, shapes, ms, dev):
        self.torch, self.qbg, self.dev = torch, qbg, dev
        self.calls = []
        for (N, K) in shapes:
            w = synth.weights(synth.DECODE_FP8, N, K)
            wt = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).to(dev)
            qw, sw = qbg.qbg_quantize_per_token(wt, qbg.QBG_FP8_E4M3)
            del wt
            a = synth.activations(synth.DECODE_FP8, N, K, max(ms))
            at = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
            for i, M in enumerate(ms):
                fcfg, _ = qbg.qbg_config_lookup(qbg.QBG_OP_FP8_FUSED, M, N, K)
                self.calls.append({
                    "N": N, "K": K, "M": M, "cfg": {k: fcfg[k] for k in KEYS},
                    "x": at[:M], "w": (qw, sw) if i == 0 else (qw.clone(), sw.clone()),
                    "qa": torch.empty((M, K), dtype=torch.uint8, device=dev),
                    "sa": torch.empty((M,), dtype=torch.float32, device=dev),
                    "out": torch.empty((M, N), dtype=torch.bfloat16, device=dev)})
        torch.cuda.synchronize()

    def graph(self, cfgs):
        torch, qbg = self.torch, self.qbg
        wss = []
        for c, cfg in zip(self.calls, cfgs):
            need = qbg.qbg_workspace_size(qbg.QBG_OP_FP8_FUSED, c["M"], c["N"], c["K"], cfg)
            wss.append(torch.zeros(max(need, 256), dtype=torch.uint8, device=self.dev) if need else None)

        def run():
            for c, cfg, ws in zip(self.calls, cfgs, wss):
                qbg.qbg_quantize_scaled_mm(c["x"], c["w"][0], c["w"][1], qtype=qbg.QBG_FP8_E4M3,
                                           out=c["out"], a_q=c["qa"], a_scale=c["sa"],
                                           config=cfg, workspace=ws)
        run()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            run()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            run()
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        return g, wss

    def time(self, g, reps):
        torch = self.torch
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps  # us per step

    def paired(self, base, cfgs, pairs, reps):
        """Per-pair step time differences (variant - base), us."""
        g, ws = self.graph(cfgs)
        d = []
        for _ in range(pairs):
            b = self.time(base, reps)
            v = self.time(g, reps)
            d.append(v - b)
        del g, ws
        return d


def candidates(qbg, M, N, K, modes, kernels=None):
    """One-launch configurations of the fused op for (M, N, K): every LDS-staged
    decode tile (or those in `kernels`), both layouts, both rotations, split 1-2."""
    out = []
    for kid in range(qbg.qbg_kernel_count()):
        info = qbg.qbg_kernel_info(kid)
        if info["stages"] == 0 or info["tile_m"] != 32 or (kernels and kid not in kernels):
            continue
        for fuse in modes:
            for swap in (0, 1):
                for rot in (0, 1):
                    for split in (1, 2):
                        c = {"kernel_id": kid, "swap_ab": swap, "split_k": split, "rotate": rot,
                             "fuse": fuse}
                        try:
                            qbg.qbg_workspace_size(qbg.QBG_OP_FP8_FUSED, M, N, K, c)
                        except qbg.QbgError:
                            continue
                        out.append(c)
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--out", required=True, help="table lines of the kept fused entries")
    ap.add_argument("--shapes", default="", help="comma list NxK (default: the 8B decode shapes)")
    ap.add_argument("--ms", default=",".join(map(str, DECODE_MS)))
    ap.add_argument("--max-m", type=int, default=4, help="largest token count given candidates")
    ap.add_argument("--modes", default="1",
                    help="fuse modes to try: 0 PUBLISH, 1 LOCAL (shortlisted by timing them "
                         "alone), 2 SEPARATE with another GEMM configuration (shortlisted "
                         "from --checkpoint)")
    ap.add_argument("--checkpoint", default="",
                    help="tune.py JSONL checkpoint of the plain fp8 op (SEPARATE shortlist)")
    ap.add_argument("--kernels", default="", help="restrict candidates to these kernel ids")
    ap.add_argument("--top", type=int, default=3, help="alone-timed candidates per call")
    ap.add_argument("--pairs", type=int, default=5)
    ap.add_argument("--reps", type=int, default=40)
    ap.add_argument("--min-gain-us", type=float, default=0.3)
    args = ap.parse_args(argv)

    import torch
    import quantized_bit_gemm_amd as qbg
    from quantized_bit_gemm_amd import synth, tune

    dev = torch.device("cuda", 0)
    shapes = DECODE_SHAPES if not args.shapes else [
        tuple(int(v) for v in s.split("x")) for s in args.shapes.split(",")]
    ms = [int(v) for v in args.ms.split(",")]
    modes = [int(v) for v in args.modes.split(",")]
    kernels = {int(v) for v in args.kernels.split(",")} if args.kernels else None
    t0 = time.time()

    # 2. shortlist per call: one-launch candidates timed alone; SEPARATE candidates
    # (another GEMM configuration behind the quantizer) from the tuner's timings
    short = {}
    one_launch = [m for m in modes if m != 2]
    if 2 in modes:
        if not args.checkpoint:
            raise SystemExit("--modes 2 needs --checkpoint")
        rows = {}
        with open(args.checkpoint) as f:
            for line in f:
                r = json.loads(line)
                if r.get("op") != "fp8" or r.get("fuse", 0) != 0:
                    continue
                key = (r["N"], r["K"], r["M"])
                cfg = (r["kernel_id"], r["swap_ab"], r["split_k"], r.get("rotate", 0))
                if kernels and cfg[0] not in kernels:
                    continue
                best = rows.setdefault(key, {})
                if cfg not in best or r["us"] < best[cfg]:
                    best[cfg] = r["us"]
        for (N, K) in shapes:
            for M in ms:
                cur, _ = qbg.qbg_config_lookup(qbg.QBG_OP_FP8, M, N, K)
                cur = (cur["kernel_id"], cur["swap_ab"], cur["split_k"], cur["rotate"])
                ranked = sorted(rows.get((N, K, M), {}).items(), key=lambda t: t[1])
                picks = [dict(zip(KEYS, cfg + (2,))) for cfg, _ in ranked if cfg != cur][:args.top]
                short.setdefault((N, K, M), []).extend(picks)
    for (N, K) in shapes:
        todo = [M for M in ms if M <= args.max_m] if one_launch else []
        if not todo:
            continue
        prob = tune.Problem(torch, qbg, qbg.QBG_OP_FP8_FUSED, N, K, max(todo), dev)
        for M in todo:
            res = [(prob.time_config(M, c, reps=3), c)
                   for c in candidates(qbg, M, N, K, one_launch, kernels)]
            res.sort(key=lambda t: t[0])
            short.setdefault((N, K, M), []).extend(c for _, c in res[:args.top])
            log("N=%d K=%d M=%d: %d candidates, best alone %.2f us (%.0fs)" % (
                N, K, M, len(res), res[0][0] if res else float("nan"), time.time() - t0))
        del prob
        torch.cuda.empty_cache()

    # 3. each shortlisted candidate inside the step, against the unchanged step
    step = Step(torch, qbg, synth, shapes, ms, dev)
    base_cfgs = [c["cfg"] for c in step.calls]
    base, base_ws = step.graph(base_cfgs)
    for _ in range(3):
        step.time(base, args.reps)
    log("step with the table's entries: %.2f us" % step.time(base, args.reps))
    keep = {}
    for i, c in enumerate(step.calls):
        key = (c["N"], c["K"], c["M"])
        best = None
        for cand in short.get(key, []):
            cfgs = list(base_cfgs)
            cfgs[i] = cand
            d = step.paired(base, cfgs, args.pairs, args.reps)
            med = float(np.median(d))
            log("N=%d K=%d M=%d %d/%d/%d/r%d/f%d: step %+.2f us (pairs %s)" % (
                c["N"], c["K"], c["M"], cand["kernel_id"], cand["swap_ab"], cand["split_k"],
                cand["rotate"], cand["fuse"], med, " ".join("%+.2f" % v for v in d)))
            if max(d) < 0 and -med >= args.min_gain_us and (best is None or med < best[0]):
                best = (med, cand)
        if best is not None:
            keep[i] = best

    # 4. all kept replacements together
    lines = []
    if keep:
        cfgs = list(base_cfgs)
        for i, (_, cand) in keep.items():
            cfgs[i] = cand
        d = step.paired(base, cfgs, args.pairs, args.reps)
        log("all %d replacements: step %+.2f us (pairs %s)" % (
            len(keep), float(np.median(d)), " ".join("%+.2f" % v for v in d)))
        if max(d) < 0:
            for i, (med, cand) in sorted(keep.items()):
                c = step.calls[i]
                cols = (c["M"], c["N"], c["K"], cand["kernel_id"], cand["swap_ab"],
                        cand["split_k"], cand["rotate"])
                if cand["fuse"] == 2:  # the plain op's entry runs the same GEMM
                    lines.append("fp8 %d %d %d %d %d %d %d 0   # in the decode step: %+.2f us" % (
                        cols + (med,)))
                lines.append("fp8_fused %d %d %d %d %d %d %d %d   # in the decode step: %+.2f us" % (
                    cols + (cand["fuse"], med)))
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + ("\n" if lines else ""))
    log("wrote %d entries to %s (%.0fs)" % (len(lines), args.out, time.time() - t0))


if __name__ == "__main__":
    main()
