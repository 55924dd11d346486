#!/usr/bin/env python3
"""Benchmark of one HTTM global-attention layer (merge + attention + unmerge) on one GPU.

A step is one full layer call (httm_layer: similarity + argmax, top-r
grouping, K/V merge, query merge + deviation, cross-head outlier select,
restore, ragged attention, unmerge) over one batch of synthetic tokens that
are already resident in HBM.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--workload vggt30] [--no-cpu-baseline]

By default W and K are sized from a one-step probe so that the warmup and
the timed region each cover about 0.5 s of GPU work (clocks ramp up over the
first few hundred milliseconds of load); the JSON line reports the W and K
actually used.

Workload default: 30 frames x (37x37 patches + 5 special tokens) = 41,220
tokens, 16 heads x 64 channels, bf16; blocks n_s=128 x n_t=30; queries merged
90 % with 10 % outliers restored; keys/values merged 50 %.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import gen  # noqa: E402

METRIC = "HTTM global-attn layer tokens/s (merge+attn+unmerge), 30–500 frames"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
MFMA_F32_PEAK_TFLOPS = 157.3


def log(*a):
    print(*a, file=sys.stderr, flush=True)


ATTN_SRC = os.path.join(ROOT, "token_merged_global_amd", "csrc", "k_attn.hip")
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "attn_fast_hbm_traffic_vggt30.md")
GA_SRC = os.path.join(ROOT, "token_merged_global_amd", "csrc", "k_ga.hip")
GA_TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "ga_match_hbm_traffic_vggt30.md")


def measured_traffic(workload: str, dtype: str, profile: str = TRAFFIC_PROFILE, src: str = ATTN_SRC):
    """HBM bytes per launch of a kernel from a committed rocprofv3 counter summary.

    Returned only while the kernel's source is the one the counters were
    taken with (sha256 recorded in the summary) and for that workload;
    otherwise None.
    """
    if dtype != "bf16" or not os.path.exists(profile):
        return None
    txt = open(profile).read()
    sha = re.search(r"source_sha256:\s*([0-9a-f]{64})", txt)
    wl = re.search(r"workload:\s*(\S+)", txt)
    nb = re.search(r"bytes_per_launch:\s*([0-9]+)", txt)
    if not (sha and wl and nb) or wl.group(1) != workload:
        return None
    cur = hashlib.sha256(open(src, "rb").read()).hexdigest()
    return int(nb.group(1)) if cur == sha.group(1) else None


def describe(w) -> str:
    if getattr(w, "partition", 0) == 1:
        return (f"{w.name}: {w.frames} frames x ({w.grid_h}x{w.grid_w}+{w.n_special}) = {w.n_tokens} tokens, "
                f"{w.heads} heads x {w.d_head}, {w.dtype}, geometry-aware partition ({w.protect_pct:g}% "
                f"protected, global match) + {w.outlier_pct:g}% outliers")
    return (f"{w.name}: {w.frames} frames x ({w.grid_h}x{w.grid_w}+{w.n_special}) = {w.n_tokens} tokens, "
            f"{w.heads} heads x {w.d_head}, {w.dtype}, n_s={w.n_s} n_t={w.n_t}, q merge {w.q_ratio:g} + "
            f"{w.outlier_pct:g}% outliers, kv merge {w.kv_ratio:g}")


def cpu_baseline(w, x, heads: int):
    """The oracle, untouched, on a bounded sample: the first `heads` heads of the layer."""
    import oracle as O
    from threadpoolctl import threadpool_info

    ws = w.with_(heads=heads)
    p = O.Params.from_workload(ws)
    t0 = time.perf_counter()
    O.layer(x["q"][:heads], x["k"][:heads], x["v"][:heads], p)
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    scale = w.heads / heads
    return {"value": w.n_tokens / (dt * scale), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"full oracle layer on {heads} of {w.heads} heads of the same workload "
                       f"(outlier budget over those heads), {dt:.2f} s wall, scaled x{scale:g} to {w.heads} heads; "
                       f"numpy/BLAS threads {threads}, cpu {platform.processor() or platform.machine()}")}


# (n_s, n_t) shapes of the block sweep: block sizes near 256, 800 and 3840
# tokens, each as spatial-only (n_t = 1) and temporal stacks.
SWEEP_SHAPES = [(256, 1), (86, 3), (26, 10), (800, 1), (267, 3), (80, 10), (27, 30),
                (1369, 1), (1280, 3), (384, 10), (128, 30)]


def sweep_blocks(args, H, torch) -> None:
    """Cost and merge quality of block shapes and stackings on one set of inputs.

    HTTM page, key design 2 and its spatial/temporal trade-off: per shape the
    layer time, the merged lengths, the mean query deviation (how far queries
    sit from their merged token) and the relative RMS error of the layer
    output against exact unmerged attention on the same inputs.
    """
    base = gen.WORKLOADS[args.workload]
    x = gen.layer_inputs(base, seed=args.seed)
    tdt = torch.bfloat16 if base.dtype == "bf16" else torch.float32
    q, k, v = (torch.from_numpy(x[t]).to(tdt).cuda() for t in "qkv")
    exact = H.attention_dense(H.Plan.from_workload(base), q, k, v).float()
    torch.cuda.synchronize()
    enorm = float(exact.norm())
    stream = torch.cuda.current_stream()
    for n_s, n_t in SWEEP_SHAPES:
        for order in ((0, 1) if n_t > 1 else (0,)):
            w = base.with_(n_s=n_s, n_t=min(n_t, base.frames), block_order=order)
            plan = H.Plan.from_workload(w)
            ws = H.workspace(plan)
            out = torch.empty_like(q)
            for _ in range(20):
                H.layer(plan, q, k, v, ws=ws, out=out, stream=stream)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = 50
            e0.record(stream)
            for _ in range(reps):
                H.layer(plan, q, k, v, ws=ws, out=out, stream=stream)
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            delta = H.debug_read(plan, ws, "delta")
            lq = np.diff(H.debug_read(plan, ws, "cu_q"))
            err = float((out.float() - exact).norm()) / enorm
            print(json.dumps({"n_s": n_s, "n_t": w.n_t, "n_b": n_s * w.n_t, "block_order": order,
                              "ms_per_layer": round(ms, 4), "tokens_per_s": w.n_tokens / (ms * 1e-3),
                              "q_len_mean": float(lq.mean()), "kv_len": plan.info["kv_len"],
                              "mean_delta": float(delta.mean()), "out_rel_rms_err": err}), flush=True)
            del ws, out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=0,
                    help="timed steps (default: enough for ~0.5 s of GPU work, at least 10)")
    ap.add_argument("--warmup", type=int, default=0,
                    help="untimed warmup steps (default: enough for ~0.5 s, at least 3, so clocks have ramped)")
    ap.add_argument("--workload", default="vggt30", choices=sorted(gen.WORKLOADS))
    ap.add_argument("--seed", type=int, default=gen.DEFAULT_SEED)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=8)
    ap.add_argument("--dense-reps", type=int, default=3)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run a plain device copy of this size (HBM counter calibration)")
    ap.add_argument("--kv-ratio", type=float, default=None, help="override the workload's K/V merge ratio")
    ap.add_argument("--q-ratio", type=float, default=None, help="override the workload's query merge ratio")
    ap.add_argument("--outlier-pct", type=float, default=None, help="override the workload's outlier budget")
    ap.add_argument("--cached-layers", type=int, default=None,
                    help="also time layers that reuse the merge indices (default: workload layers - 1)")
    ap.add_argument("--partition", default="httm", choices=["httm", "ga"],
                    help="httm: temporal blocks (default); ga: geometry-aware three-class partition")
    ap.add_argument("--protect-pct", type=float, default=10.0, help="ga: percent of each frame's patches protected")
    ap.add_argument("--sweep-blocks", action="store_true",
                    help="instead of the benchmark: block shape / stacking sweep (one JSON line per shape)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the HTTM layer here runs on a single MI355X "
              "(multi-GPU head sharding is a design note, not built); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import token_merged_global_amd as H

    if args.sweep_blocks:
        sweep_blocks(args, H, torch)
        return

    w = gen.WORKLOADS[args.workload]
    over = {k: v for k, v in (("kv_ratio", args.kv_ratio), ("q_ratio", args.q_ratio),
                                ("outlier_pct", args.outlier_pct)) if v is not None}
    if over:
        w = w.with_(**over)
    ga = args.partition == "ga"
    if ga:
        w = w.with_(name=w.name + "_ga", partition=1, protect_pct=args.protect_pct)
    n_cached = (w.layers - 1) if args.cached_layers is None else args.cached_layers
    log(f"[bench] generating {describe(w)}")
    x = gen.layer_inputs(w, seed=args.seed)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = [torch.from_numpy(x[t]).to(tdt).cuda() for t in "qkv"]
    q, k, v = dev
    plan = H.Plan.from_workload(w)
    ws = H.workspace(plan)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()

    # step-time probe (untimed for the result): sizes the default warmup and step counts
    H.layer(plan, q, k, v, ws=ws, out=out, stream=stream)
    torch.cuda.synchronize()
    p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    p0.record(stream)
    H.layer(plan, q, k, v, ws=ws, out=out, stream=stream)
    p1.record(stream)
    torch.cuda.synchronize()
    probe_ms = max(p0.elapsed_time(p1), 1e-3)
    if args.warmup <= 0:
        args.warmup = max(3, int(500.0 / probe_ms))
    if args.steps <= 0:
        args.steps = max(10, int(500.0 / probe_ms))
    log(f"[bench] warmup {args.warmup} steps (probe {probe_ms:.3f} ms/step)")
    for _ in range(args.warmup):
        H.layer(plan, q, k, v, ws=ws, out=out, stream=stream)
    torch.cuda.synchronize()

    # timed region: K layer calls; HIP events around the attention kernel only
    # (and, with the geometry-aware partition, around its global match kernel)
    H.set_timing(["attn", "ga_match"] if ga else ["attn"])
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        H.layer(plan, q, k, v, ws=ws, out=out, stream=stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_total = ev0.elapsed_time(ev1)
    attn_t, calls = H.get_timing()
    ms_step = ms_total / args.steps
    value = w.n_tokens / (ms_step * 1e-3)
    log(f"[bench] {args.steps} steps: {ms_step:.4f} ms/step, {value:.4g} tokens/s, attn {attn_t['attn']:.4f} ms")

    cu = H.debug_read(plan, ws, "cu_q")
    lq = np.diff(cu)
    lk = plan.info["kv_len"]
    lkh = H.debug_read(plan, ws, "kv_len").astype(np.float64) if ga else np.full(w.heads, float(lk))
    attn_flop = 4.0 * w.d_head * float((lkh * lq).sum())
    ga_info = None
    if ga:
        # global match: 2*d*|S|*|D| per head and stream
        role = H.debug_read(plan, ws, "ga_role").reshape(2, w.heads, -1)
        ns = (role == 0).sum(axis=2).astype(np.float64)
        nd = (role == 1).sum(axis=2).astype(np.float64)
        ga_info = {"match_flop": float((2.0 * w.d_head * ns * nd).sum()),
                   "sources_per_head_mean": float(ns.mean()), "destinations_per_head_mean": float(nd.mean()),
                   "kv_len_min": int(lkh.min()), "kv_len_max": int(lkh.max())}
    attn_ms = attn_t["attn"]
    peak = MFMA_BF16_PEAK_TFLOPS if w.dtype == "bf16" else MFMA_F32_PEAK_TFLOPS
    achieved = attn_flop / (attn_ms * 1e-3) / 1e12
    attn_roof = {"bound": "mfma", "kernel": "attn_fast" if w.dtype == "bf16" else "attn_f32",
                 "achieved": achieved, "peak": peak, "unit": "TFLOP/s", "frac": achieved / peak,
                 "traffic": measured_traffic(w.name, "bf16" if w.dtype == "bf16" else "f32"),
                 "traffic_unit": "bytes per launch (HBM, rocprofv3 FETCH_SIZE x2.0 + WRITE_SIZE x1.0)",
                 "algorithmic": (f"4*d*sum_h(L_k,h*L_q,h) = {attn_flop:.4g} FLOP per launch" if ga else
                                 f"4*d*L_k*sum_h(L_q,h) = 4*{w.d_head}*{lk}*{int(lq.sum())} = {attn_flop:.4g} FLOP per launch"),
                 "avg_launch_ms": attn_ms, "launches_timed": calls}
    roofline, other_roofline = attn_roof, None
    if ga and attn_t["ga_match"] > 0:
        match_ms = attn_t["ga_match"]
        m_ach = ga_info["match_flop"] / (match_ms * 1e-3) / 1e12
        match_roof = {"bound": "mfma", "kernel": "ga_match_bf16" if w.dtype == "bf16" else "ga_match_f32",
                      "achieved": m_ach, "peak": peak, "unit": "TFLOP/s", "frac": m_ach / peak,
                      "traffic": measured_traffic(w.name, "bf16" if w.dtype == "bf16" else "f32",
                                                  GA_TRAFFIC_PROFILE, GA_SRC),
                      "traffic_unit": "bytes per launch (HBM, rocprofv3 FETCH_SIZE x2.0 + WRITE_SIZE x1.0)",
                      "algorithmic": f"2*d*sum_(stream,h)(|S|*|D|) = {ga_info['match_flop']:.4g} FLOP per launch",
                      "avg_launch_ms": match_ms, "launches_timed": calls}
        log(f"[bench] global match {match_ms:.4f} ms ({m_ach:.1f} TFLOP/s), attention {attn_ms:.4f} ms")
        # the dominant kernel (the longer launch) carries the roofline; the other rides along
        if match_ms > attn_ms:
            roofline, other_roofline = match_roof, attn_roof
        else:
            other_roofline = match_roof

    # per-stage breakdown (separate untimed pass; events around every stage, 30 calls)
    H.set_timing(None)
    for _ in range(30):
        H.layer(plan, q, k, v, ws=ws, out=out, stream=stream)
    stages, _ = H.get_timing()
    H.set_timing([])
    torch.cuda.synchronize()

    # layers that reuse this layer's merge indices (LiteVGGT-style cache)
    cached = None
    if n_cached > 0:
        idx = H.CachedIndex(plan)
        H.layer(plan, q, k, v, ws=ws, out=out, index=idx, stream=stream)
        H.layer_cached(plan, idx, q, k, v, ws=ws, out=out, stream=stream)
        torch.cuda.synchronize()
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        for _ in range(args.steps):
            H.layer_cached(plan, idx, q, k, v, ws=ws, out=out, stream=stream)
        c1.record(stream)
        torch.cuda.synchronize()
        cms = c0.elapsed_time(c1) / args.steps
        stack_ms = ms_step + n_cached * cms
        cached = {"cached_layers": n_cached, "cached_ms_per_layer": cms,
                  "stack_ms": stack_ms, "stack_tokens_per_s": (1 + n_cached) * w.n_tokens / (stack_ms * 1e-3),
                  "cached_tokens_per_s": w.n_tokens / (cms * 1e-3)}
        log(f"[bench] cached layer {cms:.4f} ms; stack of {1 + n_cached}: {stack_ms:.3f} ms")
        del idx

    # speedup over the same engine's unmerged attention
    dense_ms = None
    if args.dense_reps > 0:
        dws = H.workspace(plan, "dense")
        dout = torch.empty_like(q)
        H.attention_dense(plan, q, k, v, ws=dws, out=dout)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.dense_reps):
            H.attention_dense(plan, q, k, v, ws=dws, out=dout, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        dense_ms = e0.elapsed_time(e1) / args.dense_reps
        del dws, dout

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib * (1 << 20)
        a = torch.empty(n, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: {args.copy_calibration_mib} MiB device copy")

    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline: oracle on {args.cpu_heads} heads")
        cpu = cpu_baseline(w, x, args.cpu_heads)

    res = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic: seeded VGGT-shaped tokens (smoothed spatial field + per-frame drift + noise), inputs resident in HBM",
        "config": {"workload": describe(w), "frames": w.frames, "tokens": w.n_tokens, "heads": w.heads,
                   "d_head": w.d_head, "n_s": w.n_s, "n_t": w.n_t, "q_ratio": w.q_ratio, "kv_ratio": w.kv_ratio,
                   "outlier_pct": w.outlier_pct, "seed": args.seed,
                   **({"partition": "geometry-aware", "protect_pct": w.protect_pct} if ga else {})},
        "roofline": roofline,
        **({"roofline_other_kernel": other_roofline} if other_roofline else {}),
        "cpu_baseline": cpu,
        "stages_ms": stages,
        "cached": cached,
        "geometry_aware": ga_info,
        "speedup_vs_unmerged_attention": (dense_ms / ms_step) if dense_ms else None,
        "unmerged_attention_ms": dense_ms,
        "lengths": {"kv_len": lk, "q_len_mean": float(lq.mean()), "q_len_min": int(lq.min()),
                    "q_len_max": int(lq.max()), "q_ratio_final": float(lq.mean() / w.n_tokens),
                    "kv_ratio_final": lk / w.n_tokens},
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
