#!/usr/bin/env python3
"""Benchmark of the 8-bit scaled-matmul decode path on one MI355X.

Workload (default): FP8-dynamic scaled GEMM at 8B-decoder linear shapes,
(N, K) in {(6144,4096), (4096,4096), (24576,4096), (4096,12288)} and token
counts M in {1, 2, 4, 8, 16, 32}; activations bf16 N(0,1) with 0.1% x50
outliers, weights N(0,0.02) quantized per output channel to E4M3.

One step = one pass of the hot path over that batch: for every (N, K, M),
per-token FP8 quantization of the bf16 activations and the scaled GEMM, one
qbg_quantize_scaled_mm call each with the configuration the tuned table
selects (Standard or Swap-AB, split_k, tile variant, fuse mode; the shipped
table runs the one- and two-token calls of every shape as one launch that
quantizes inside the GEMM, chosen inside this step
(the line's config.one_launch_calls counts them), and every other call as the
quantizer launch, then the GEMM), captured
once in a HIP graph and replayed.  Inputs are resident in HBM before timing.  Each GEMM of
a step reads its own copy of the weights (six copies per shape, 1.15 GB per
step), so no weight byte can be served from the 256 MB Infinity Cache.

value = algorithmic bytes of the step / step time (TB/s), where a GEMM moves
N*K + M*K + 4N + 4M + 2MN bytes and a quantizer 3MK + 4M bytes.

The same line also carries (unless --no-other-configs) the GEMM-only time of
each (N, K, M) of the workload ("per_shape") and the GEMM-only throughput of the
other configurations ("other_configs": FP8 at 512x1024, W8A8-INT8, Block-FP8
with fp32 and with UE8M0 scales, and the MLP chain's two GEMMs at 128 and 256
tokens in TFLOP/s against the dense fp8 matrix-core peak), each call timed on
weight copies totalling at least 1 GiB with the table's configuration, and the
geometric mean of the per-call roofline fractions of each list.

--workload block_chain measures the Block-FP8 MLP chain of a 32B decoder
instead (hidden 5120, intermediate 25600): for each scale format (fp32,
UE8M0) and M in {1, 8, 32}, RMSNorm + 1x128 group quant, the gate_up block
GEMM (51200x5120), SiLU-and-mul + group quant and the down block GEMM
(5120x25600); 24 launches per step, 786 MB of weights.  A block GEMM moves
N*K + M*K + s*ceil(N/128)*K/128 + s*M*K/128 + 2MN bytes (s = 4 or 1), the
producers read their bf16 inputs and write codes and group scales.

--workload mlp_chain measures the fused FP8 MLP chain (hidden 4096,
intermediate 12288): for M in {1, 32, 128, 256}, RMSNorm + per-token quant,
gate_up scaled GEMM (24576x4096), SiLU-and-mul + per-token quant and down
scaled GEMM (4096x12288); the GEMMs are also reported in TFLOP/s against the
dense fp8 matrix-core peak (5.0 PFLOP/s), the bound above M = 32.

--workload moe measures a mixture-of-experts decode MLP of a 30B-A3B-class
model (128 experts, top-8 routing, hidden 2048, expert intermediate 768):
for M in {1, 8, 32} tokens (8M routed rows, seeded routing), per-token quant
of the routed rows, the grouped gate_up GEMM (1536x2048 per expert),
SiLU-and-mul + quant and the grouped down GEMM (2048x768 per expert).  Only
the weights of experts that received rows count as algorithmic bytes.

--workload int8_decode and --workload block_decode measure the other decode
configurations the same way (quantization + GEMM per (N, K, M), through the
fused entry point for INT8, every GEMM on its own weight copy): W8A8-INT8 at the 8B-decoder shapes with M in {1, 4, 16, 32}
and Student-t activations, and Block-FP8 at the 32B-decoder shapes
{(10240,5120), (5120,8192), (51200,5120), (5120,25600)} with M in {1, 8, 32}
for fp32 and UE8M0 scales.

--workload prefill measures the same FP8-dynamic quantization + GEMM at
prefill token counts M in {512, 2048, 8192} on the 8B-decoder shapes, where
the GEMMs pass the matrix-core ridge; the roofline is reported in TFLOP/s
against the dense fp8 peak (5.0 PFLOP/s).  No CPU baseline (one oracle call
at 8192 tokens takes minutes).

Printed: one JSON line on stdout (details on stderr).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_TBS = 8.0  # MI355X HBM3E, TB/s
SHAPES = [(6144, 4096), (4096, 4096), (24576, 4096), (4096, 12288)]
MS = [1, 2, 4, 8, 16, 32]
PREFILL_MS = [512, 2048, 8192]  # --workload prefill token counts
MFMA_FP8_PEAK_TFLOPS = 5000.0  # MI355X dense fp8 matrix-core peak
COPIES = len(MS)  # one weight copy per token count of a shape


def gemm_bytes(M, N, K):
    return N * K + M * K + 4 * N + 4 * M + 2 * M * N


def quant_bytes(M, K):
    return 3 * M * K + 4 * M


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--workload", choices=["fp8_decode", "int8_decode", "block_decode",
                                           "block_chain", "mlp_chain", "moe", "prefill"],
                    default="fp8_decode")
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip timing the CPU oracle")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum CPU time of the oracle's timed sample")
    ap.add_argument("--details", default="",
                    help="write the configuration of every (N, K, M) of the step as JSON")
    ap.add_argument("--no-details", action="store_true",
                    help="accepted for compatibility; per-shape timings come from the tuner")
    ap.add_argument("--eager-pass", type=int, default=0, metavar="R",
                    help="after timing, launch every GEMM of the step R times on its own "
                         "(synchronized, no graph), for kernel traces of kernel-only durations")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="before timing, run one plain device copy of MIB MiB (a kernel of "
                         "known traffic for scaling hardware byte counters)")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the per-shape list and the other configurations' GEMM timings")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def make_inputs(torch, qbg, synth, dev):
    """Device-resident inputs: per shape, COPIES quantized weight copies and bf16 activations."""
    data = []
    for (N, K) in SHAPES:
        w = synth.weights(synth.DECODE_FP8, N, K)
        wt = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).to(dev)
        qw, sw = qbg.qbg_quantize_per_token(wt, qbg.QBG_FP8_E4M3)  # per output channel
        del wt
        copies = [(qw, sw)] + [(qw.clone(), sw.clone()) for _ in range(COPIES - 1)]
        a = synth.activations(synth.DECODE_FP8, N, K, max(MS))
        at = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        data.append({"N": N, "K": K, "w": copies, "a": at, "a_host": a, "w_host": w})
    torch.cuda.synchronize()
    return data


def build_calls(torch, qbg, data, dev):
    """Preallocated buffers and resolved configurations for every (shape, M) of a step:
    the fused entry point's (the step) and the plain GEMM's (its GEMM launch alone)."""
    calls = []
    for d in data:
        N, K = d["N"], d["K"]
        for i, M in enumerate(MS):
            cfg, from_table = qbg.qbg_config_lookup(qbg.QBG_OP_FP8, M, N, K)
            fcfg, _ = qbg.qbg_config_lookup(qbg.QBG_OP_FP8_FUSED, M, N, K)
            ws_bytes = max(qbg.qbg_workspace_size(qbg.QBG_OP_FP8, M, N, K, cfg),
                           qbg.qbg_workspace_size(qbg.QBG_OP_FP8_FUSED, M, N, K, fcfg))
            ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device=dev) if ws_bytes else None
            calls.append({
                "N": N, "K": K, "M": M, "cfg": cfg, "from_table": from_table, "fcfg": fcfg,
                "local": fcfg["fuse"] == qbg.QBG_FUSE_LOCAL,
                "x": d["a"][:M], "qa": torch.empty((M, K), dtype=torch.uint8, device=dev),
                "sa": torch.empty((M,), dtype=torch.float32, device=dev),
                "w": d["w"][i], "out": torch.empty((M, N), dtype=torch.bfloat16, device=dev),
                "ws": ws,
            })
    return calls


def run_step(qbg, calls, gemm_only=False, only=None):
    """One step (gemm_only: the table's plain GEMM of every call alone, on the codes
    the step left -- also for a call the step runs as one LOCAL launch, so the
    roofline always measures the same GEMM kernel family)."""
    for c in calls:
        if only is not None and not only(c):
            continue
        if gemm_only:
            qbg.qbg_scaled_mm(c["qa"], c["sa"], c["w"][0], c["w"][1], qtype=qbg.QBG_FP8_E4M3,
                              out=c["out"], config=c["cfg"], workspace=c["ws"])
        else:
            qbg.qbg_quantize_scaled_mm(c["x"], c["w"][0], c["w"][1], qtype=qbg.QBG_FP8_E4M3,
                                       out=c["out"], a_q=c["qa"], a_scale=c["sa"],
                                       config=c["fcfg"], workspace=c["ws"])


def launch_bytes(c):
    """Algorithmic bytes of a call's plain GEMM launch."""
    return gemm_bytes(c["M"], c["N"], c["K"])


def capture(torch, fn):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # eager warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def time_graph(torch, g, reps, warmup):
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(reps):
        g.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / 1e3  # seconds for `reps` replays


def measured_traffic():
    """HBM bytes per GEMM launch from the committed rocprofv3 PMC summary, if it
    was taken on the GEMM sources and configuration table in this tree; else None."""
    from quantized_bit_gemm_amd import profsummary

    path = os.path.join(ROOT, "profiles", "gemm_fp8_decode_shapes_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_sha256") != profsummary.gemm_source_hash():
        return None
    try:
        return round(float(vals["gemm_traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def cpu_baseline(data, min_seconds=10.0):
    """The CPU oracle on the same workload: per-token quantization of the
    activations and the scaled GEMM for every (N, K, M) of a step (weights
    quantized by the oracle beforehand, untimed), repeated until at least
    min_seconds of CPU work have been timed."""
    import oracle

    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count()
    prepared = []
    for d in data:
        qw, sw = oracle.quant_weight_per_channel(oracle.FP8, d["w_host"])
        prepared.append((d, qw, sw))
    total_bytes = 0
    passes = 0
    t = time.perf_counter()
    while True:
        for d, qw, sw in prepared:
            for M in MS:
                a = d["a_host"][:M]
                qa, sa = oracle.quant_per_token(oracle.FP8, a)
                oracle.scaled_mm(oracle.FP8, qa, sa, qw, sw)
                total_bytes += gemm_bytes(M, d["N"], d["K"]) + quant_bytes(M, d["K"])
        passes += 1
        dt = time.perf_counter() - t
        if dt >= min_seconds:
            break
    return {"value": round(total_bytes / dt / 1e12, 6), "unit": "TB/s", "cores": threads,
            "kind": "oracle",
            "sample": "%d full step(s): per-token FP8 quant + FP8 scaled GEMM for all 24 (N,K,M) "
                      "of the workload, %.1f s of CPU work" % (passes, dt)}


# ---- per-shape and other-configuration GEMM timings (default run) ---------------

def per_call_timings(torch, qbg, dev, op, shapes, ms, flops_peak=None):
    """GEMM-only time per launch of each (N, K, M) with the configuration the table
    selects, timed like the tuner: a graph of launches, each on its own copy of the
    weights (copies totalling >= 1 GiB, so none is served from the Infinity Cache),
    replayed back to back between two events.  Returns a list of per-call records."""
    from quantized_bit_gemm_amd import tune

    out = []
    for (N, K) in shapes:
        prob = tune.Problem(torch, qbg, op, N, K, max(ms), dev)
        for M in ms:
            cfg, hit = qbg.qbg_config_lookup(op, M, N, K)
            us = prob.time_config(M, cfg, reps=5)
            b = tune.gemm_bytes(op, M, N, K)
            rec = {"N": N, "K": K, "M": M, "us": round(us, 3), "bytes": b, "TBs": round(b / us / 1e6, 4),
                   "frac": round(b / us / 1e6 / HBM_PEAK_TBS, 4), "kernel_id": cfg["kernel_id"],
                   "split_k": cfg["split_k"], "swap_ab": cfg["swap_ab"], "from_table": bool(hit)}
            if flops_peak:
                tf = 2.0 * M * N * K / us / 1e6
                rec["TFLOPs"] = round(tf, 1)
                rec["mfma_frac"] = round(tf / flops_peak, 4)
            out.append(rec)
        del prob
        torch.cuda.empty_cache()
    return out


def summarize(recs, what):
    """Aggregate TB/s (algorithmic bytes over summed launch time) of a list of calls."""
    tot_us = sum(r["us"] for r in recs)
    tbs = sum(r["bytes"] for r in recs) / tot_us / 1e6
    return {"workload": what, "gemm_TBs": round(tbs, 4), "frac": round(tbs / HBM_PEAK_TBS, 4),
            "geomean_frac": geomean_frac(recs), "launches": len(recs),
            "avg_launch_us": round(tot_us / len(recs), 3), "calls": recs}


def geomean_frac(recs):
    """Geometric mean over calls of each call's fraction of the HBM roofline (the
    pages report per-shape results as geometric means)."""
    return round(math.exp(sum(math.log(r["frac"]) for r in recs) / len(recs)), 4)


def other_configs(torch, qbg, synth, dev):
    """GEMM-only timings of the other configurations, one record list each."""
    res = {}
    log("[bench] other configurations: FP8 tiny (512x1024)")
    res["fp8_tiny"] = summarize(per_call_timings(torch, qbg, dev, qbg.QBG_OP_FP8, synth.TINY_SHAPES,
                                                 [1, 16, 32]),
                                "FP8-dynamic scaled GEMM 512x1024 (launch-bound)")
    log("[bench] other configurations: W8A8-INT8")
    res["int8_decode"] = summarize(per_call_timings(torch, qbg, dev, qbg.QBG_OP_INT8, synth.DECODE_SHAPES,
                                                    synth.INT8_MS),
                                   "W8A8-INT8 scaled GEMM, 8B-decoder linear shapes")
    for op, name in ((qbg.QBG_OP_BLOCK_FP8, "fp32"), (qbg.QBG_OP_BLOCK_UE8M0, "ue8m0")):
        log("[bench] other configurations: Block-FP8 (%s scales)" % name)
        res["block_fp8_" + name] = summarize(
            per_call_timings(torch, qbg, dev, op, synth.BLOCK_SHAPES, synth.BLOCK_MS),
            "Block-FP8 scaled GEMM (%s scales), 32B-decoder shapes" % name)
    log("[bench] other configurations: FP8 MLP-chain GEMMs at 128 and 256 tokens")
    chain = per_call_timings(torch, qbg, dev, qbg.QBG_OP_FP8, [(2 * MC_I, MC_H), (MC_H, MC_I)], [128, 256],
                             flops_peak=MFMA_FP8_PEAK_TFLOPS)
    tot_us = sum(r["us"] for r in chain)
    tf = sum(2.0 * r["M"] * r["N"] * r["K"] for r in chain) / tot_us / 1e6
    res["mlp_chain_gemms_128_256"] = {"workload": "FP8 gate_up (24576x4096) and down (4096x12288) "
                                                  "at 128 and 256 tokens", "TFLOPs": round(tf, 1),
                                      "mfma_frac": round(tf / MFMA_FP8_PEAK_TFLOPS, 4), "calls": chain}
    return res


# ---- INT8 and Block-FP8 decode (--workload int8_decode / block_decode) ----------

def other_decode(args, torch, qbg, synth, dev, kind):
    to_dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    calls = []
    if kind == "int8_decode":
        wl, shapes, ms, fmts = synth.DECODE_INT8, synth.DECODE_SHAPES, synth.INT8_MS, [None]
    elif kind == "prefill":
        wl, shapes, ms, fmts = synth.DECODE_FP8, synth.DECODE_SHAPES, PREFILL_MS, [None]
    else:
        wl, shapes, ms, fmts = synth.DECODE_BLOCK, synth.BLOCK_SHAPES, synth.BLOCK_MS, [0, 1]
    # per-channel workloads: INT8 decode, FP8 prefill
    pq = qbg.QBG_INT8 if kind == "int8_decode" else qbg.QBG_FP8_E4M3
    pop = qbg.QBG_OP_INT8 if kind == "int8_decode" else qbg.QBG_OP_FP8
    pfop = qbg.QBG_OP_INT8_FUSED if kind == "int8_decode" else qbg.QBG_OP_FP8_FUSED
    log("[bench] %s: generating inputs" % kind)
    for (N, K) in shapes:
        w_host = synth.weights(wl, N, K)
        a_host = synth.activations(wl, N, K, max(ms))
        wt = to_dev(w_host)
        x = to_dev(a_host)
        for fmt in fmts:
            if fmt is None:
                base = qbg.qbg_quantize_per_token(wt, pq)
                op = pop
            else:
                base = qbg.qbg_quantize_weight_block(wt, fmt)
                op = qbg.QBG_OP_BLOCK_FP8 if fmt == 0 else qbg.QBG_OP_BLOCK_UE8M0
            for i, M in enumerate(ms):  # one weight copy per token count
                w = base if i == 0 else (base[0].clone(), base[1].clone())
                cfg, _ = qbg.qbg_config_lookup(op, M, N, K)
                nb = qbg.qbg_workspace_size(op, M, N, K, cfg)
                fcfg = None  # per-channel: the fused entry point's configuration
                if fmt is None:
                    fcfg, _ = qbg.qbg_config_lookup(pfop, M, N, K)
                    nb = max(nb, qbg.qbg_workspace_size(pfop, M, N, K, fcfg))
                calls.append({"N": N, "K": K, "M": M, "fmt": fmt, "op": op, "x": x[:M], "w": w,
                              "cfg": cfg, "fcfg": fcfg,
                              "local": fcfg is not None and fcfg["fuse"] == qbg.QBG_FUSE_LOCAL,
                              "qa": torch.empty((M, K), dtype=torch.int8 if pq == qbg.QBG_INT8
                                                else torch.uint8, device=dev),
                              "sa": torch.empty((M,), dtype=torch.float32, device=dev),
                              "ws": torch.zeros(nb, dtype=torch.uint8, device=dev)
                              if nb else None,
                              "out": torch.empty((M, N), dtype=torch.bfloat16, device=dev),
                              "w_host": w_host, "a_host": a_host[:M]})
        del wt
    torch.cuda.synchronize()

    def quant(c):
        if c["fmt"] is None:
            return qbg.qbg_quantize_per_token(c["x"], pq)
        return qbg.qbg_quantize_per_token_group(c["x"], 128, c["fmt"])

    def gemm(c, qa, sa):
        if c["fmt"] is None:
            qbg.qbg_scaled_mm(qa, sa, *c["w"], qtype=pq, out=c["out"], config=c["cfg"],
                              workspace=c["ws"])
        else:
            qbg.qbg_block_scaled_mm(qa, sa, *c["w"], fmt=c["fmt"], out=c["out"], config=c["cfg"],
                                    workspace=c["ws"])

    def step_call(c):
        # per-channel: the fused entry point (one launch or quantizer + GEMM, as the table says)
        if c["fmt"] is None:
            qbg.qbg_quantize_scaled_mm(c["x"], *c["w"], qtype=pq, out=c["out"],
                                       a_q=c["qa"], a_scale=c["sa"], config=c["fcfg"],
                                       workspace=c["ws"])
        else:
            gemm(c, *quant(c))

    def gemm_launch(c, q):
        # the call's plain GEMM alone (also for a call the step runs as one launch)
        gemm(c, *q)

    def g_bytes(c):
        M, N, K = c["M"], c["N"], c["K"]
        if c["fmt"] is None:
            return gemm_bytes(M, N, K)
        return block_gemm_bytes(M, N, K, 4 if c["fmt"] == 0 else 1)

    def launch_b(c):
        return g_bytes(c)

    def q_bytes(c):
        M, K = c["M"], c["K"]
        if c["fmt"] is None:
            return quant_bytes(M, K)
        return 3 * M * K + (4 if c["fmt"] == 0 else 1) * M * (K // 128)

    step_bytes = sum(g_bytes(c) + q_bytes(c) for c in calls)
    gemm_total = sum(launch_b(c) for c in calls)
    launches = sum(1 if c["local"] else 2 for c in calls)
    g = capture(torch, lambda: [step_call(c) for c in calls])
    t = time_graph(torch, g, args.steps, args.warmup)
    ms_step = t / args.steps * 1e3
    value = step_bytes / (t / args.steps) / 1e12
    log("[bench] %s step: %.3f ms, %.3f TB/s over %.1f MB (%d launches)" % (
        kind, ms_step, value, step_bytes / 1e6, launches))
    pre = [quant(c) for c in calls]
    reps = max(args.steps, 20)
    gg = capture(torch, lambda: [gemm_launch(c, q) for c, q in zip(calls, pre)])
    t_gemm = time_graph(torch, gg, reps, args.warmup) / reps
    gemm_tbs = gemm_total / t_gemm / 1e12
    log("[bench] GEMMs alone: %.3f ms per step, %.3f TB/s" % (t_gemm * 1e3, gemm_tbs))
    flops = sum(2 * c["M"] * c["N"] * c["K"] for c in calls)
    gemm_tflops = flops / t_gemm / 1e12
    if kind == "prefill":
        log("[bench] GEMMs alone: %.1f TFLOP/s (%.1f %% of the dense fp8 peak)" % (
            gemm_tflops, 100 * gemm_tflops / MFMA_FP8_PEAK_TFLOPS))
    if kind == "int8_decode":
        workload = "W8A8-INT8 scaled GEMM, 8B-decoder linear shapes"
        cfgd = {"shapes_NK": shapes, "M": ms}
    elif kind == "prefill":
        workload = "FP8-dynamic scaled GEMM at prefill token counts, 8B-decoder linear shapes"
        cfgd = {"shapes_NK": shapes, "M": ms}
    else:
        workload = "Block-FP8 scaled GEMM (1x128 x 128x128), 32B-decoder shapes"
        cfgd = {"shapes_NK": shapes, "M": ms, "scale_formats": ["fp32", "ue8m0"]}
    result = {
        "metric": "scaled_mm achieved HBM TB/s (% roofline) at M=1-32, Qwen3-shaped NxK",
        "value": round(value, 4), "unit": "TB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "int8" if kind == "int8_decode" else "fp8_e4m3", "data": "synthetic",
        "config": {"workload": workload, **cfgd, "launches_per_step": launches,
                   "step_bytes": step_bytes},
        "roofline": {"bound": "hbm", "achieved": round(gemm_tbs * 1e3, 1), "peak": HBM_PEAK_TBS * 1e3,
                     "unit": "GB/s", "frac": round(gemm_tbs / HBM_PEAK_TBS, 4), "traffic": None,
                     "algorithmic_bytes_per_launch": round(gemm_total / len(calls)),
                     "kernel": "%s GEMM (all %d launches of a step)" % (
                         "block scaled" if kind == "block_decode" else "scaled", len(calls)),
                     "avg_launch_us": round(t_gemm / len(calls) * 1e6, 3)},
        "cpu_baseline": None,
    }
    if kind == "prefill":  # past the ridge: the matrix cores bound the GEMMs
        result["roofline"] = {
            "bound": "mfma", "achieved": round(gemm_tflops, 1),
            "peak": MFMA_FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(gemm_tflops / MFMA_FP8_PEAK_TFLOPS, 4), "traffic": None,
            "algorithmic_flops_per_launch": round(flops / len(calls)),
            "kernel": "scaled GEMM (all %d launches of a step)" % len(calls),
            "avg_launch_us": round(t_gemm / len(calls) * 1e6, 3)}
    if not args.no_cpu_baseline and kind != "prefill":
        log("[bench] timing the CPU oracle")
        result["cpu_baseline"] = other_decode_cpu(calls, g_bytes, q_bytes, args.cpu_seconds)
    return result


def other_decode_cpu(calls, g_bytes, q_bytes, min_seconds):
    """The CPU oracle on the calls of the step, cycling in step order until min_seconds of
    CPU work have been timed (weights quantized by the oracle when first needed, untimed)."""
    import oracle

    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count()
    wq = {}
    total, n, t = 0, 0, time.perf_counter()
    done = False
    while not done:
        for c in calls:
            key = (c["N"], c["K"], c["fmt"])
            if key not in wq:
                t_skip = time.perf_counter()
                wq[key] = (oracle.quant_weight_per_channel(oracle.INT8, c["w_host"])
                           if c["fmt"] is None else oracle.quant_weight_block(c["fmt"], c["w_host"]))
                t += time.perf_counter() - t_skip  # weight quantization is not timed
            qw, sw = wq[key]
            if c["fmt"] is None:
                qa, sa = oracle.quant_per_token(oracle.INT8, c["a_host"])
                oracle.scaled_mm(oracle.INT8, qa, sa, qw, sw)
            else:
                qa, sa = oracle.quant_group(c["fmt"], c["a_host"])
                oracle.block_scaled_mm(c["fmt"], qa, sa, qw, sw)
            total += g_bytes(c) + q_bytes(c)
            n += 1
            if time.perf_counter() - t >= min_seconds:
                done = True
                break
    dt = time.perf_counter() - t
    return {"value": round(total / dt / 1e12, 6), "unit": "TB/s", "cores": threads,
            "kind": "oracle",
            "sample": "%d quantize+GEMM calls cycling through the step's %d (N, K, M) in "
                      "step order, %.1f s of CPU work" % (n, len(calls), dt)}


# ---- Block-FP8 MLP chain (--workload block_chain) ------------------------------

BC_H, BC_I = 5120, 25600
BC_MS = [1, 8, 32]
BC_FMTS = [0, 1]  # fp32 scales, UE8M0 scales


def block_gemm_bytes(M, N, K, s):
    return N * K + M * K + s * ((N + 127) // 128) * (K // 128) + s * M * (K // 128) + 2 * M * N


def block_chain_bytes(M, s):
    """Algorithmic bytes of one chain pass: producers and both block GEMMs."""
    H, I = BC_H, BC_I
    rms = 2 * M * H + 2 * H + M * H + s * M * (H // 128)
    silu = 2 * M * 2 * I + M * I + s * M * (I // 128)
    return rms + silu + block_gemm_bytes(M, 2 * I, H, s) + block_gemm_bytes(M, H, I, s)


def block_chain(args, torch, qbg, synth, dev):
    log("[bench] block chain: generating inputs")
    x = synth.activations(synth.BLOCK_CHAIN, 2 * BC_I, BC_H, max(BC_MS))
    wn = synth.norm_weight(BC_H)
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
    wnt = torch.from_numpy(wn.view(np.int16)).view(torch.bfloat16).to(dev)
    host_w = {}
    weights = {}
    for fmt in BC_FMTS:
        for name, (N, K) in (("gu", (2 * BC_I, BC_H)), ("down", (BC_H, BC_I))):
            if name not in host_w:
                host_w[name] = synth.weights(synth.BLOCK_CHAIN, N, K)
            wt = torch.from_numpy(host_w[name].view(np.int16)).view(torch.bfloat16).to(dev)
            weights[fmt, name] = qbg.qbg_quantize_weight_block(wt, fmt)
            del wt
    torch.cuda.synchronize()
    calls = []
    for fmt in BC_FMTS:
        for M in BC_MS:
            c = {"fmt": fmt, "M": M, "x": xt[:M], "gu": torch.empty((M, 2 * BC_I), dtype=torch.bfloat16,
                                                                    device=dev),
                 "out": torch.empty((M, BC_H), dtype=torch.bfloat16, device=dev), "ws": {}}
            for name, (N, K) in (("gu", (2 * BC_I, BC_H)), ("down", (BC_H, BC_I))):
                cfg, _ = qbg.qbg_config_lookup(2 + fmt, M, N, K)
                nb = qbg.qbg_workspace_size(2 + fmt, M, N, K, cfg)
                c["ws"][name] = torch.zeros(nb, dtype=torch.uint8, device=dev) if nb else None
                c["cfg_" + name] = cfg
            calls.append(c)

    def step(gemm_only=False, pre=None):
        for i, c in enumerate(calls):
            fmt, M = c["fmt"], c["M"]
            if gemm_only:
                q1, s1, q2, s2 = pre[i]
            else:
                q1, s1 = qbg.qbg_rms_norm_quantize_per_token_group(c["x"], wnt, 1e-6, 128, fmt)
            qw, sw = weights[fmt, "gu"]
            qbg.qbg_block_scaled_mm(q1, s1, qw, sw, fmt=fmt, out=c["gu"], config=c["cfg_gu"],
                                    workspace=c["ws"]["gu"])
            if not gemm_only:
                q2, s2 = qbg.qbg_silu_mul_quantize_per_token_group(c["gu"], 128, fmt)
            qw, sw = weights[fmt, "down"]
            qbg.qbg_block_scaled_mm(q2, s2, qw, sw, fmt=fmt, out=c["out"], config=c["cfg_down"],
                                    workspace=c["ws"]["down"])

    step_bytes = sum(block_chain_bytes(c["M"], 4 if c["fmt"] == 0 else 1) for c in calls)
    gemm_total = sum(block_gemm_bytes(c["M"], 2 * BC_I, BC_H, 4 if c["fmt"] == 0 else 1) +
                     block_gemm_bytes(c["M"], BC_H, BC_I, 4 if c["fmt"] == 0 else 1) for c in calls)
    log("[bench] capturing the block chain step (%d launches)" % (4 * len(calls)))
    g = capture(torch, step)
    t = time_graph(torch, g, args.steps, args.warmup)
    ms = t / args.steps * 1e3
    value = step_bytes / (t / args.steps) / 1e12
    log("[bench] block chain step: %.3f ms, %.3f TB/s over %.1f MB" % (ms, value, step_bytes / 1e6))
    # the block GEMMs alone, on activations quantized once beforehand
    pre = []
    for c in calls:
        q1, s1 = qbg.qbg_rms_norm_quantize_per_token_group(c["x"], wnt, 1e-6, 128, c["fmt"])
        q2, s2 = qbg.qbg_silu_mul_quantize_per_token_group(
            torch.zeros((c["M"], 2 * BC_I), dtype=torch.bfloat16, device=dev), 128, c["fmt"])
        pre.append((q1, s1, q2, s2))
    reps = max(args.steps, 20)
    gg = capture(torch, lambda: step(gemm_only=True, pre=pre))
    t_gemm = time_graph(torch, gg, reps, args.warmup) / reps
    gemm_tbs = gemm_total / t_gemm / 1e12
    log("[bench] block GEMMs alone: %.3f ms per step, %.3f TB/s" % (t_gemm * 1e3, gemm_tbs))
    result = {
        "metric": "scaled_mm achieved HBM TB/s (% roofline) at M=1-32, Qwen3-shaped NxK",
        "value": round(value, 4), "unit": "TB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3", "data": "synthetic",
        "config": {"workload": "Block-FP8 MLP chain, 32B-decoder shapes (hidden 5120, "
                               "intermediate 25600)", "M": BC_MS, "scale_formats": ["fp32", "ue8m0"],
                   "launches_per_step": 4 * len(calls), "step_bytes": step_bytes},
        "roofline": {"bound": "hbm", "achieved": round(gemm_tbs * 1e3, 1), "peak": HBM_PEAK_TBS * 1e3,
                     "unit": "GB/s", "frac": round(gemm_tbs / HBM_PEAK_TBS, 4), "traffic": None,
                     "algorithmic_bytes_per_launch": round(gemm_total / (2 * len(calls))),
                     "kernel": "block scaled GEMM (all %d launches of a step)" % (2 * len(calls)),
                     "avg_launch_us": round(t_gemm / (2 * len(calls)) * 1e6, 3)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle")
        result["cpu_baseline"] = block_chain_cpu(x, wn, host_w, args.cpu_seconds)
    return result


def block_chain_cpu(x, wn, host_w, min_seconds):
    """The CPU oracle on the block chain: weights block-quantized beforehand (untimed),
    then passes of the chain (both formats, every M) until min_seconds have been timed."""
    import oracle

    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count()
    wq = {(fmt, n): oracle.quant_weight_block(fmt, w) for fmt in BC_FMTS for n, w in host_w.items()}
    total, passes, t = 0, 0, time.perf_counter()
    while True:
        for fmt in BC_FMTS:
            for M in BC_MS:
                _, q1, s1 = oracle.rms_norm_group_quant(fmt, x[:M], wn, 1e-6)
                qw, sw = wq[fmt, "gu"]
                _, gu = oracle.block_scaled_mm(fmt, q1, s1, qw, sw)
                _, q2, s2 = oracle.silu_mul_group_quant(fmt, gu)
                qw, sw = wq[fmt, "down"]
                oracle.block_scaled_mm(fmt, q2, s2, qw, sw)
                total += block_chain_bytes(M, 4 if fmt == 0 else 1)
        passes += 1
        dt = time.perf_counter() - t
        if dt >= min_seconds:
            break
    return {"value": round(total / dt / 1e12, 6), "unit": "TB/s", "cores": threads,
            "kind": "oracle",
            "sample": "%d full step(s) of the block chain (both scale formats, M 1/8/32), "
                      "%.1f s of CPU work" % (passes, dt)}


# ---- FP8 MLP chain (--workload mlp_chain) --------------------------------------

MC_H, MC_I = 4096, 12288
MC_MS = [1, 32, 128, 256]


def mlp_chain(args, torch, qbg, synth, dev):
    log("[bench] mlp chain: generating inputs")
    x = synth.activations(synth.MLP_CHAIN, 2 * MC_I, MC_H, max(MC_MS))
    wn = synth.norm_weight(MC_H)
    to_dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    xt, wnt = to_dev(x), to_dev(wn)
    # one weight copy per token count: 600 MB per step, so no GEMM reads its
    # weights from the 256 MB Infinity Cache
    base = {}
    for name, (N, K) in (("gu", (2 * MC_I, MC_H)), ("down", (MC_H, MC_I))):
        wt = to_dev(synth.weights(synth.MLP_CHAIN, N, K))
        base[name] = qbg.qbg_quantize_per_token(wt, qbg.QBG_FP8_E4M3)
        del wt
    calls = []
    for i, M in enumerate(MC_MS):
        c = {"M": M, "x": xt[:M], "gu": torch.empty((M, 2 * MC_I), dtype=torch.bfloat16, device=dev),
             "out": torch.empty((M, MC_H), dtype=torch.bfloat16, device=dev), "ws": {}, "cfg": {},
             "w": {k: (v if i == 0 else (v[0].clone(), v[1].clone())) for k, v in base.items()}}
        for name, (N, K) in (("gu", (2 * MC_I, MC_H)), ("down", (MC_H, MC_I))):
            cfg, _ = qbg.qbg_config_lookup(qbg.QBG_OP_FP8, M, N, K)
            nb = qbg.qbg_workspace_size(qbg.QBG_OP_FP8, M, N, K, cfg)
            c["ws"][name] = torch.zeros(nb, dtype=torch.uint8, device=dev) if nb else None
            c["cfg"][name] = cfg
        calls.append(c)

    def gemms(c, q1, s1, q2, s2):
        qbg.qbg_scaled_mm(q1, s1, *c["w"]["gu"], out=c["gu"], config=c["cfg"]["gu"],
                          workspace=c["ws"]["gu"])
        qbg.qbg_scaled_mm(q2, s2, *c["w"]["down"], out=c["out"], config=c["cfg"]["down"],
                          workspace=c["ws"]["down"])

    def step():
        for c in calls:
            q1, s1 = qbg.qbg_rms_norm_quantize_per_token(c["x"], wnt, 1e-6)
            qbg.qbg_scaled_mm(q1, s1, *c["w"]["gu"], out=c["gu"], config=c["cfg"]["gu"],
                              workspace=c["ws"]["gu"])
            q2, s2 = qbg.qbg_silu_mul_quantize_per_token(c["gu"])
            qbg.qbg_scaled_mm(q2, s2, *c["w"]["down"], out=c["out"], config=c["cfg"]["down"],
                              workspace=c["ws"]["down"])

    def gemm_bytes_mc(M):
        return gemm_bytes(M, 2 * MC_I, MC_H) + gemm_bytes(M, MC_H, MC_I)

    prod_bytes = lambda M: (3 * M * MC_H + 2 * MC_H + 4 * M) + (2 * M * 2 * MC_I + M * MC_I + 4 * M)
    step_bytes = sum(gemm_bytes_mc(M) + prod_bytes(M) for M in MC_MS)
    g = capture(torch, step)
    t = time_graph(torch, g, args.steps, args.warmup)
    ms = t / args.steps * 1e3
    value = step_bytes / (t / args.steps) / 1e12
    log("[bench] mlp chain step: %.3f ms, %.3f TB/s over %.1f MB" % (ms, value, step_bytes / 1e6))
    # per-M GEMM pair (activations quantized once beforehand)
    pre = {}
    for c in calls:
        q1, s1 = qbg.qbg_rms_norm_quantize_per_token(c["x"], wnt, 1e-6)
        q2, s2 = qbg.qbg_silu_mul_quantize_per_token(c["gu"])
        pre[c["M"]] = (q1, s1, q2, s2)
    reps = max(args.steps, 20)
    per_m = {}
    # each M's GEMM pair is timed on the four weight copies in turn (600 MB per replay)
    for c in calls:
        gg = capture(torch, lambda c=c: [gemms(dict(c, w=o["w"]), *pre[c["M"]]) for o in calls])
        tt = time_graph(torch, gg, reps, args.warmup) / reps / len(calls)
        M = c["M"]
        flops = 2.0 * M * (2 * MC_I * MC_H + MC_H * MC_I)
        per_m[M] = {"gemm_us": round(tt * 1e6, 2), "TBs": round(gemm_bytes_mc(M) / tt / 1e12, 3),
                    "TFLOPs": round(flops / tt / 1e12, 1),
                    "mfma_frac": round(flops / tt / 1e12 / MFMA_FP8_PEAK_TFLOPS, 4)}
        log("[bench]   M=%3d gate_up+down %8.2f us  %.3f TB/s  %.1f TFLOP/s (%.1f%% of fp8 peak)" % (
            M, tt * 1e6, per_m[M]["TBs"], per_m[M]["TFLOPs"], 100 * per_m[M]["mfma_frac"]))
    big = per_m[max(MC_MS)]
    result = {
        "metric": "scaled_mm achieved HBM TB/s (% roofline) at M=1-32, Qwen3-shaped NxK",
        "value": round(value, 4), "unit": "TB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3", "data": "synthetic",
        "config": {"workload": "Fused FP8 MLP chain (hidden 4096, intermediate 12288)",
                   "M": MC_MS, "launches_per_step": 4 * len(calls), "step_bytes": step_bytes,
                   "gemm_per_M": per_m},
        "roofline": {"bound": "mfma", "achieved": big["TFLOPs"], "peak": MFMA_FP8_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": big["mfma_frac"], "traffic": None,
                     "kernel": "scaled GEMM pair at M=%d (gate_up + down)" % max(MC_MS)},
        "cpu_baseline": None,
    }
    return result


# ---- mixture-of-experts MLP (--workload moe) ------------------------------------

def moe(args, torch, qbg, synth, dev):
    E, k, H, I = synth.MOE_EXPERTS, synth.MOE_TOP_K, synth.MOE_HIDDEN, synth.MOE_INTER
    log("[bench] moe: generating inputs")
    to_dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    sets = []
    for copy in range(2):  # two weight sets (1.2 GB): consecutive calls never share weights
        ws = {}
        for name, (N, K) in (("gu", (2 * I, H)), ("down", (H, I))):
            w = torch.randn((E * N, K), generator=torch.Generator(device=dev).manual_seed(
                copy * 7 + N), device=dev).mul_(0.02).to(torch.bfloat16)
            qw, sw = qbg.qbg_quantize_per_token(w, qbg.QBG_FP8_E4M3)
            ws[name] = (qw.view(E, N, K), sw.view(E, N))
            del w
        sets.append(ws)
    calls = []
    for i, M in enumerate(synth.MOE_MS):
        order, offsets = synth.moe_routing(M, E, k)
        T = len(order)
        x = to_dev(synth.draw(synth.MOE, M, H, 7, (M, H), "normal")[order])
        active = int((offsets[1:] > offsets[:-1]).sum())
        c = {"M": M, "T": T, "x": x, "off": torch.from_numpy(offsets).to(dev), "active": active,
             "w": sets[i % 2], "gu": torch.empty((T, 2 * I), dtype=torch.bfloat16, device=dev),
             "out": torch.empty((T, H), dtype=torch.bfloat16, device=dev)}
        calls.append(c)

    def step(gemm_only=False, pre=None):
        for c in calls:
            if gemm_only:
                q1, s1, q2, s2 = pre[c["M"]]
            else:
                q1, s1 = qbg.qbg_quantize_per_token(c["x"], qbg.QBG_FP8_E4M3)
            qbg.qbg_grouped_scaled_mm(q1, s1, *c["w"]["gu"], c["off"], out=c["gu"])
            if not gemm_only:
                q2, s2 = qbg.qbg_silu_mul_quantize_per_token(c["gu"])
            qbg.qbg_grouped_scaled_mm(q2, s2, *c["w"]["down"], c["off"], out=c["out"])

    def gemm_b(c):
        T, a = c["T"], c["active"]
        return (a * (2 * I * H + 4 * 2 * I) + T * H + 4 * T + 2 * T * 2 * I +
                a * (H * I + 4 * H) + T * I + 4 * T + 2 * T * H)

    def prod_b(c):
        T = c["T"]
        return (3 * T * H + 4 * T) + (2 * T * 2 * I + T * I + 4 * T)

    step_bytes = sum(gemm_b(c) + prod_b(c) for c in calls)
    gemm_total = sum(gemm_b(c) for c in calls)
    g = capture(torch, step)
    t = time_graph(torch, g, args.steps, args.warmup)
    ms = t / args.steps * 1e3
    value = step_bytes / (t / args.steps) / 1e12
    log("[bench] moe step: %.3f ms, %.3f TB/s over %.1f MB" % (ms, value, step_bytes / 1e6))
    pre = {}
    for c in calls:
        q1, s1 = qbg.qbg_quantize_per_token(c["x"], qbg.QBG_FP8_E4M3)
        q2, s2 = qbg.qbg_silu_mul_quantize_per_token(c["gu"])
        pre[c["M"]] = (q1, s1, q2, s2)
    reps = max(args.steps, 20)
    gg = capture(torch, lambda: step(gemm_only=True, pre=pre))
    t_gemm = time_graph(torch, gg, reps, args.warmup) / reps
    gemm_tbs = gemm_total / t_gemm / 1e12
    log("[bench] grouped GEMMs alone: %.3f ms per step, %.3f TB/s (active experts: %s)" % (
        t_gemm * 1e3, gemm_tbs, [c["active"] for c in calls]))
    return {
        "metric": "scaled_mm achieved HBM TB/s (% roofline) at M=1-32, Qwen3-shaped NxK",
        "value": round(value, 4), "unit": "TB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3", "data": "synthetic",
        "config": {"workload": "Mixture-of-experts decode MLP (128 experts, top-8, hidden 2048, "
                               "expert intermediate 768)", "M": synth.MOE_MS,
                   "routed_rows": [c["T"] for c in calls],
                   "active_experts": [c["active"] for c in calls],
                   "launches_per_step": 4 * len(calls), "step_bytes": step_bytes},
        "roofline": {"bound": "hbm", "achieved": round(gemm_tbs * 1e3, 1), "peak": HBM_PEAK_TBS * 1e3,
                     "unit": "GB/s", "frac": round(gemm_tbs / HBM_PEAK_TBS, 4), "traffic": None,
                     "algorithmic_bytes_per_launch": round(gemm_total / (2 * len(calls))),
                     "kernel": "grouped scaled GEMM (all %d launches of a step)" % (2 * len(calls)),
                     "avg_launch_us": round(t_gemm / (2 * len(calls)) * 1e6, 3)},
        "cpu_baseline": None,
    }


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    import quantized_bit_gemm_amd as qbg
    from quantized_bit_gemm_amd import synth

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    qbg.lib()
    if args.workload in ("int8_decode", "block_decode", "prefill"):
        print(json.dumps(other_decode(args, torch, qbg, synth, dev, args.workload)), flush=True)
        return
    if args.workload == "block_chain":
        print(json.dumps(block_chain(args, torch, qbg, synth, dev)), flush=True)
        return
    if args.workload == "mlp_chain":
        print(json.dumps(mlp_chain(args, torch, qbg, synth, dev)), flush=True)
        return
    if args.workload == "moe":
        print(json.dumps(moe(args, torch, qbg, synth, dev)), flush=True)
        return
    log("[bench] generating inputs")
    data = make_inputs(torch, qbg, synth, dev)
    calls = build_calls(torch, qbg, data, dev)
    step_bytes = sum(gemm_bytes(c["M"], c["N"], c["K"]) + quant_bytes(c["M"], c["K"]) for c in calls)
    gemm_total = sum(launch_bytes(c) for c in calls)
    launches = sum(1 if c["local"] else 2 for c in calls)

    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] calibration copy: %d bytes read, %d bytes written" % (n, n))
        del src, dst

    log("[bench] capturing the step graph (%d launches)" % launches)
    step_graph = capture(torch, lambda: run_step(qbg, calls))
    torch.cuda.synchronize()
    t_steps = time_graph(torch, step_graph, args.steps, args.warmup)
    ms_per_step = t_steps / args.steps * 1e3
    value = step_bytes / (t_steps / args.steps) / 1e12
    log("[bench] step: %.3f ms, %.3f TB/s over %.1f MB" % (ms_per_step, value, step_bytes / 1e6))

    # Dominant kernel: the scaled GEMM.  Time the GEMM launches alone (graph of the
    # 24 GEMM launches of a step); HIP events on the replay stream.
    reps = max(args.steps, 20)
    gemm_graph = capture(torch, lambda: run_step(qbg, calls, gemm_only=True))
    t_gemm = time_graph(torch, gemm_graph, reps, args.warmup) / reps
    gemm_tbs = gemm_total / t_gemm / 1e12
    log("[bench] GEMMs alone: %.3f ms per step, %.3f TB/s" % (t_gemm * 1e3, gemm_tbs))
    if args.details:
        with open(args.details, "w") as f:
            json.dump([{"N": c["N"], "K": c["K"], "M": c["M"],
                        "cfg": c["cfg"], "fused_cfg": c["fcfg"],
                        "from_table": c["from_table"], "bytes": launch_bytes(c)}
                       for c in calls], f, indent=1)
    if args.eager_pass:
        # each GEMM alone: a kernel trace of this part shows kernel-only durations
        log("[bench] eager pass: %d x %d GEMM launches, each synchronized" % (args.eager_pass,
                                                                              len(calls)))
        for _ in range(args.eager_pass):
            for c in calls:
                run_step(qbg, [c], gemm_only=True)
                torch.cuda.synchronize()

    result = {
        "metric": "scaled_mm achieved HBM TB/s (% roofline) at M=1-32, Qwen3-shaped NxK",
        "value": round(value, 4), "unit": "TB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3", "data": "synthetic",
        "config": {"workload": "FP8-dynamic scaled GEMM, 8B-decoder linear shapes",
                   "shapes_NK": SHAPES, "M": MS, "launches_per_step": launches,
                   "one_launch_calls": sum(c["local"] for c in calls),
                   "step_bytes": step_bytes, "weight_copies_per_shape": COPIES},
        "roofline": {"bound": "hbm", "achieved": round(gemm_tbs * 1e3, 1), "peak": HBM_PEAK_TBS * 1e3,
                     "unit": "GB/s", "frac": round(gemm_tbs / HBM_PEAK_TBS, 4),
                     "traffic": measured_traffic(),
                     "algorithmic_bytes_per_launch": round(gemm_total / len(calls)),
                     "kernel": "the table's plain GEMM at each of the 24 (N, K, M) of a step "
                               "(a call the step runs as one LOCAL launch is timed as its "
                               "plain GEMM)",
                     "avg_launch_us": round(t_gemm / len(calls) * 1e6, 3)},
        "cpu_baseline": None,
    }
    if not args.no_other_configs:
        # each (N, K, M) of this workload alone, then the other configurations
        log("[bench] per-shape GEMM timings")
        per_shape = per_call_timings(torch, qbg, dev, qbg.QBG_OP_FP8, SHAPES, MS)
        result["per_shape"] = [{k: r[k] for k in ("N", "K", "M", "us", "frac", "TBs", "kernel_id",
                                                  "split_k")} for r in per_shape]
        result["per_shape_geomean_frac"] = geomean_frac(per_shape)
        result["other_configs"] = other_configs(torch, qbg, synth, dev)
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle")
        result["cpu_baseline"] = cpu_baseline(data, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
