"""Offline tuner for the GEMM configuration table.

For every (op, M bucket, N, K) it forces each feasible configuration -- tile
variant x Standard/Swap-AB x power-of-two split_k x rotation, and for the
fused quantize+GEMM ops the fuse mode (by default only the two-launch
SEPARATE mode; --fuse-modes 0,1,2 adds the one-launch PUBLISH and LOCAL
modes) -- through the C ABI and times it inside a HIP graph, then keeps the
fastest.  Timed alone, LOCAL beats SEPARATE by about 1.5 us at one or two
tokens; inside the decode benchmark's step, next to other shapes' GEMMs, it
mostly loses, so it is not a default candidate here: steptune.py decides the
one-launch entries inside the step itself.  This is the pages'
ahead-of-time per-shape tuning over the algorithmic variants and the
scheduling parameters ("Helion nel backend vLLM", ai-radar.it, paragraphs 3
and 7; "Helion DSL added to vLLM to autotune linear inference backends",
signaltitans.com, "Hybrid Dispatch and Autotuning"), done as an exhaustive
grid because the space here is small.

Timing: L back-to-back launches per graph, each on its own copy of the
quantized weights, with enough copies that the weights cycled through exceed
1 GiB (four times the 256 MB Infinity Cache), so every launch streams its
weights from HBM; the per-launch time is the median over repeated replays.
The fused ops also read their own copy of the bf16 activations per launch:
a call's input arrives cold from HBM, as in the decode benchmark (a buffer
re-read by every launch would sit in the cache and favour the one-launch
mode, which reads it from every workgroup).

Results are appended to a JSONL checkpoint as they are measured, so an
interrupted run resumes where it stopped; the table is written at the end.

With --search model only a budget of the configurations is timed, chosen by
a tree-ensemble surrogate (search.py); --search grid (default) times all.

Usage:
  python -m quantized_bit_gemm_amd.tune --ops fp8 --out configs/gfx950.txt \
      --checkpoint tune.jsonl [--shapes 4096x4096,...] [--ms 1,2,4,8,16,32] \
      [--search model --budget 0.25]

A deployment starts from the shipped table (configs/gfx950.txt) and falls back
to the built-in default for shapes it lacks; a user tunes their own shapes
with this script and points QBG_CONFIG_TABLE at the result.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

OPS = {"fp8": 0, "int8": 1, "block_fp8": 2, "block_ue8m0": 3, "fp8_fused": 4, "int8_fused": 5,
       "fp8_grouped": 6, "int8_grouped": 7}
FUSED = (4, 5)
GROUPED = (6, 7)
# Grouped (mixture-of-experts) ops: --ms are token counts; each token is routed to
# TOP_K of EXPERTS experts, so a call carries T = TOP_K * M rows and the table key
# is next_pow2(T).
EXPERTS, TOP_K = 128, 8
OP_NAMES = {v: k for k, v in OPS.items()}
DEFAULT_SHAPES = {
    "fp8": [(6144, 4096), (4096, 4096), (24576, 4096), (4096, 12288), (512, 1024),
            (24576, 4096), (4096, 12288)],
    "int8": [(6144, 4096), (4096, 4096), (24576, 4096), (4096, 12288), (512, 1024)],
    "block_fp8": [(10240, 5120), (5120, 8192), (51200, 5120), (5120, 25600)],
    "block_ue8m0": [(10240, 5120), (5120, 8192), (51200, 5120), (5120, 25600)],
}
DEFAULT_SHAPES["fp8_fused"] = DEFAULT_SHAPES["fp8"]
DEFAULT_SHAPES["int8_fused"] = DEFAULT_SHAPES["int8"]
DEFAULT_SHAPES["fp8_grouped"] = [(1536, 2048), (2048, 768)]  # per-expert gate_up, down
DEFAULT_SHAPES["int8_grouped"] = DEFAULT_SHAPES["fp8_grouped"]
DEFAULT_MS = [1, 2, 4, 8, 16, 32]
ROTATE_BYTES = 1 << 30


FUSE_PUBLISH, FUSE_LOCAL, FUSE_SEPARATE = 0, 1, 2


def feasible_configs(qbg, op, K, max_split=256, min_chunk=128, fuse_modes=(FUSE_SEPARATE,)):
    """Candidate configurations (validated later against the shape).  A fused op
    gets one candidate per fuse mode: PUBLISH runs on the LDS-staged tiles, LOCAL
    on the LDS-staged decode tiles and on the register tiles (there only with a
    K chunk of exactly two load groups per wave, without rotation), SEPARATE on
    any tile of the plain op."""
    quantum = 128 if op in (2, 3) else 16
    out = []
    max_split_op = 1 if op in GROUPED else max_split  # the grouped launch has no split-K
    for kid in range(qbg.qbg_kernel_count()):
        info = qbg.qbg_kernel_info(kid)
        if op in FUSED:
            modes = [m for m in fuse_modes
                     if m == FUSE_SEPARATE or (info["stages"] > 0 and
                                               (m == FUSE_PUBLISH or info["tile_m"] == 32))
                     or (m == FUSE_LOCAL and info["stages"] == 0 and info["tile_m"] == 32)]
        else:
            modes = [0]
            if op in GROUPED and info["stages"] == 0:
                continue  # the grouped launch runs on the LDS-staged variants
        for fuse in modes:
            for swap in (0, 1):
                s = 1
                while s <= max_split_op:
                    reg_local = op in FUSED and fuse == FUSE_LOCAL and info["stages"] == 0
                    if reg_local and K // s != 256 * info["waves_k"] * info["k_unroll"]:
                        s *= 2
                        continue
                    if K % s == 0 and (K // s) % quantum == 0 and (K // s) >= min(min_chunk, K):
                        for rot in ((0,) if reg_local else (0, 1)):
                            c = {"kernel_id": kid, "swap_ab": swap, "split_k": s, "rotate": rot}
                            if op in FUSED:
                                c["fuse"] = fuse
                            out.append(c)
                    s *= 2
    return out


def config_key(opname, M, N, K, cfg):
    return (opname, M, N, K, cfg["kernel_id"], cfg["swap_ab"], cfg["split_k"],
            cfg.get("rotate", 0), cfg.get("fuse", 0))


class Problem:
    """Device-resident operands of one (op, N, K) with rotating weight copies."""

    def __init__(self, torch, qbg, op, N, K, max_m, dev):
        self.torch, self.qbg, self.op, self.N, self.K = torch, qbg, op, N, K
        g = torch.Generator(device=dev)
        g.manual_seed(N * 131 + K)
        if op in GROUPED:
            self._init_grouped(torch, qbg, N, K, max_m, dev, g)
            return
        # Weights: random codes quantized on the GPU from a bf16 master.
        w = (torch.randn((N, K), generator=g, device=dev, dtype=torch.float32) * 0.02).to(torch.bfloat16)
        a = torch.randn((max_m, K), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
        if op in (0, 1) + FUSED:
            qt = qbg.QBG_FP8_E4M3 if op in (0, 4) else qbg.QBG_INT8
            qw, sw = qbg.qbg_quantize_per_token(w, qt)
            self.qa, self.sa = qbg.qbg_quantize_per_token(a, qt)
        else:
            fmt = qbg.QBG_SCALE_F32 if op == 2 else qbg.QBG_SCALE_UE8M0
            qw, sw = qbg.qbg_quantize_weight_block(w, fmt)
            self.qa, self.sa = qbg.qbg_quantize_per_token_group(a, 128, fmt)
        del w
        wbytes = N * K
        self.copies = max(2, min(64, (ROTATE_BYTES + wbytes - 1) // wbytes))
        self.w = [(qw, sw)] + [(qw.clone(), sw.clone()) for _ in range(self.copies - 1)]
        self.xs = [a] + [a.clone() for _ in range(self.copies - 1)] if op in FUSED else [a]
        self.out = torch.empty((max_m, N), dtype=torch.bfloat16, device=dev)
        self._settle()

    def _settle(self):
        """Read every weight copy once (a reduction, not a GEMM): building the
        copies wrote them, and the first calls timed otherwise pay for those dirty
        lines leaving the memory-side cache (2-3 us on a 100 MB shape)."""
        torch = self.torch
        for qw, _ in self.w:
            qw.view(torch.uint8).sum(dtype=torch.int64)
        torch.cuda.synchronize()

    def _init_grouped(self, torch, qbg, N, K, max_m, dev, g):
        from quantized_bit_gemm_amd import synth

        qt = qbg.QBG_FP8_E4M3 if self.op == 6 else qbg.QBG_INT8
        w = (torch.randn((EXPERTS * N, K), generator=g, device=dev) * 0.02).to(torch.bfloat16)
        qw, sw = qbg.qbg_quantize_per_token(w, qt)
        del w
        qw, sw = qw.view(EXPERTS, N, K), sw.view(EXPERTS, N)
        T = TOP_K * max_m
        a = torch.randn((T, K), generator=g, device=dev).to(torch.bfloat16)
        self.qa, self.sa = qbg.qbg_quantize_per_token(a, qt)
        wbytes = EXPERTS * N * K
        self.copies = max(2, min(16, (ROTATE_BYTES + wbytes - 1) // wbytes))
        self.w = [(qw, sw)] + [(qw.clone(), sw.clone()) for _ in range(self.copies - 1)]
        self.routes = {}
        self.out = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
        self._synth = synth
        self._settle()

    def offsets(self, M):
        """Routing of M tokens (T = TOP_K * M rows): device offsets and active experts."""
        if M not in self.routes:
            _, off = self._synth.moe_routing(M, EXPERTS, TOP_K)
            active = int((off[1:] > off[:-1]).sum())
            self.routes[M] = (self.torch.from_numpy(off).to(self.out.device), active)
        return self.routes[M]

    def launch(self, i, M, cfg, ws):
        qbg = self.qbg
        qw, sw = self.w[i % self.copies]
        if self.op in GROUPED:
            off, _ = self.offsets(M)
            T = TOP_K * M
            qbg.qbg_grouped_scaled_mm(self.qa[:T], self.sa[:T], qw, sw, off,
                                      qtype=qbg.QBG_FP8_E4M3 if self.op == 6 else qbg.QBG_INT8,
                                      out=self.out[:T], config=cfg)
            return
        qa, sa = self.qa[:M], self.sa[:M]
        if self.op in FUSED:
            qbg.qbg_quantize_scaled_mm(self.xs[i % self.copies][:M], qw, sw,
                                       qtype=qbg.QBG_FP8_E4M3 if self.op == 4 else qbg.QBG_INT8,
                                       out=self.out[:M], a_q=qa, a_scale=sa, config=cfg,
                                       workspace=ws)
        elif self.op in (0, 1):
            qbg.qbg_scaled_mm(qa, sa, qw, sw, qtype=self.op, out=self.out[:M], config=cfg,
                              workspace=ws)
        else:
            fmt = qbg.QBG_SCALE_F32 if self.op == 2 else qbg.QBG_SCALE_UE8M0
            qbg.qbg_block_scaled_mm(qa, sa, qw, sw, fmt=fmt, out=self.out[:M], config=cfg,
                                    workspace=ws)

    def time_config(self, M, cfg, reps=5):
        torch, qbg = self.torch, self.qbg
        rows = TOP_K * M if self.op in GROUPED else M
        need = qbg.qbg_workspace_size(self.op, rows, self.N, self.K, cfg)
        ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=self.out.device) if need else None
        L = self.copies
        self.launch(0, M, cfg, ws)  # eager once: surfaces argument errors before capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for i in range(L):
                self.launch(i, M, cfg, ws)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for i in range(L):
                self.launch(i, M, cfg, ws)
        g.replay()
        torch.cuda.synchronize()
        # Each sample times R back-to-back replays between two events, so the
        # latency of submitting a graph is spread over R * L launches rather
        # than L (with 100 MB weights L is 11, and one submission's latency
        # would add 1-2 us to every launch).
        R = max(2, (96 + L - 1) // L)
        times = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(R):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e3 / (R * L))  # us per launch
        del g
        return float(np.median(times))


def gemm_bytes(op, M, N, K, active=None):
    """Algorithmic bytes of one call (the fused ops add the quantizer's 3MK + 4M; a
    grouped call reads the weights of its `active` experts for its M routed rows)."""
    if op in GROUPED:
        return active * (N * K + 4 * N) + M * K + 4 * M + 2 * M * N
    b = N * K + M * K + 2 * M * N
    if op in FUSED:
        return b + 4 * N + 4 * M + 3 * M * K + 4 * M
    if op in (0, 1):
        return b + 4 * N + 4 * M
    s = 4 if op == 2 else 1
    return b + s * ((N + 127) // 128) * (K // 128) + s * M * (K // 128)


def load_checkpoint(path):
    done = {}
    if path and os.path.exists(path):
        with open(path) as f:
            for line in f:
                line = line.strip()
                if not line:
                    continue
                r = json.loads(line)
                r.setdefault("rotate", 0)
                r.setdefault("fuse", 0)
                done[config_key(r["op"], r["M"], r["N"], r["K"], r)] = r
    return done


def write_table(path, results):
    """Best timed configuration per (op, M, N, K) as the text table libqbg loads."""
    best = {}
    for r in results.values():
        key = (r["op"], r["M"], r["N"], r["K"])
        if key not in best or r["us"] < best[key]["us"]:
            best[key] = r
    lines = ["qbg-config-table 3 gfx950",
             "# op m_bucket N K kernel_id swap_ab split_k rotate fuse   # us/call, HBM TB/s"]
    for key in sorted(best):
        r = best[key]
        lines.append("%s %d %d %d %d %d %d %d %d   # %.2f us %.3f TB/s" % (
            r["op"], r["M"], r["N"], r["K"], r["kernel_id"], r["swap_ab"], r["split_k"],
            r.get("rotate", 0), r.get("fuse", 0), r["us"], r["TBs"]))
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return best


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--ops", default="fp8")
    ap.add_argument("--shapes", default="", help="comma list NxK (default: the op's shapes)")
    ap.add_argument("--ms", default=",".join(map(str, DEFAULT_MS)))
    ap.add_argument("--out", required=True, help="table to write")
    ap.add_argument("--checkpoint", default="", help="JSONL checkpoint (appended, resumable)")
    ap.add_argument("--max-split", type=int, default=256)
    ap.add_argument("--kernels", default="", help="restrict to these kernel ids (comma list)")
    ap.add_argument("--reps", type=int, default=5)
    ap.add_argument("--search", choices=["grid", "model"], default="grid")
    ap.add_argument("--budget", type=float, default=0.25,
                    help="model search: fraction of the feasible configurations to time")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--fuse-modes", default="2",
                    help="fused ops: fuse modes to try (0 PUBLISH, 1 LOCAL, 2 SEPARATE)")
    args = ap.parse_args(argv)
    fuse_modes = tuple(int(x) for x in args.fuse_modes.split(",") if x)

    import torch

    import quantized_bit_gemm_amd as qbg
    from quantized_bit_gemm_amd import search

    dev = torch.device("cuda", 0)
    ms = [int(x) for x in args.ms.split(",") if x]
    results = load_checkpoint(args.checkpoint)
    ck = open(args.checkpoint, "a") if args.checkpoint else None
    kernels = {int(x) for x in args.kernels.split(",") if x} if args.kernels else None
    for opname in args.ops.split(","):
        op = OPS[opname]
        shapes = ([tuple(int(v) for v in s.split("x")) for s in args.shapes.split(",") if s]
                  or list(dict.fromkeys(DEFAULT_SHAPES[opname])))
        for (N, K) in shapes:
            prob = Problem(torch, qbg, op, N, K, max(ms), dev)
            for M in ms:
                t0 = time.time()
                rows = TOP_K * M if op in GROUPED else M  # the table key's token count
                cands = []
                # SEPARATE is the quantizer launch plus the plain GEMM: its best tile
                # is the plain op's, so only the plain op's table entry is timed.
                sep = None
                if op in FUSED and FUSE_SEPARATE in fuse_modes:
                    plain, _ = qbg.qbg_config_lookup(qbg.QBG_OP_FP8 if op == 4 else qbg.QBG_OP_INT8,
                                                     rows, N, K)
                    sep = {k: plain[k] for k in ("kernel_id", "swap_ab", "split_k", "rotate")}
                    cands.append(dict(sep, fuse=FUSE_SEPARATE))
                for cfg in feasible_configs(qbg, op, K, args.max_split, fuse_modes=fuse_modes):
                    if kernels is not None and cfg["kernel_id"] not in kernels:
                        continue
                    if sep is not None and cfg.get("fuse") == FUSE_SEPARATE:
                        continue
                    try:
                        qbg.qbg_workspace_size(op, rows, N, K, cfg)  # validates the config
                    except qbg.QbgError:
                        continue
                    cands.append(cfg)

                def measure(cfg, M=M, rows=rows, N=N, K=K, prob=prob, opname=opname, op=op):
                    key = config_key(opname, rows, N, K, cfg)
                    if key not in results:
                        us = prob.time_config(M, cfg, args.reps)
                        active = prob.offsets(M)[1] if op in GROUPED else None
                        results[key] = {"op": opname, "M": rows, "N": N, "K": K, **cfg,
                                        "us": round(us, 3),
                                        "TBs": round(gemm_bytes(op, rows, N, K, active) / us / 1e6, 4)}
                        if ck:
                            ck.write(json.dumps(results[key]) + "\n")
                            ck.flush()
                    return results[key]["us"]

                if args.search == "model":
                    info = {k: qbg.qbg_kernel_info(k) for k in {c["kernel_id"] for c in cands}}
                    bi, timed = search.model_search(
                        cands, lambda c: search.config_features(info[c["kernel_id"]], c, rows, N, K),
                        measure, budget=max(8, int(args.budget * len(cands))), seed=args.seed)
                    chosen = [cands[i] for i in timed]
                    if sep is not None and 0 not in timed:
                        measure(cands[0])  # the two-launch baseline is always timed
                        chosen.append(cands[0])
                else:
                    chosen = cands
                    for c in chosen:
                        measure(c)
                best = None
                for cfg in chosen:
                    r = results[config_key(opname, rows, N, K, cfg)]
                    if best is None or r["us"] < best["us"]:
                        best = r
                print("[tune] %-11s N=%5d K=%5d M=%3d best kernel=%2d swap=%d split=%3d fuse=%d "
                      "%8.2f us %.3f TB/s (%.1fs)" % (opname, N, K, M, best["kernel_id"],
                                                     best["swap_ab"], best["split_k"],
                                                     best.get("fuse", 0), best["us"],
                                                     best["TBs"], time.time() - t0), flush=True)
            del prob
            torch.cuda.empty_cache()
    if ck:
        ck.close()
    write_table(args.out, results)
    print("[tune] wrote", args.out)


if __name__ == "__main__":
    main()
