#!/usr/bin/env python3
"""
Benchmark of the routed MoE FFN layer on one MI355X.

A step is one pass of the whole hot path on one batch of seeded synthetic
input already resident in HBM: moe_plan_create (route, capacity, dispatch)
then moe_forward (classify, dequantise-once, gate/up tiles with clamped
SwiGLU, down tiles, combine). W untimed warm-up steps, then exactly K timed
steps between two device synchronisations.

Default workload: the 13,312-token prompt over 256 4-bit experts
(d_model 4096, expert d_ff 2048, top-8, Zipf(1.1) popularity), the size at
which the dequant-once FP16 route of Strata PR #4366 was measured.
``--config N`` selects another named workload (1..7; 6 and 7 are
decode-shaped calls of 1..8 tokens, ``--T``). ``--router`` times moe_route
instead (router map x . Wr^T, plan and routing statistics) on the same
prompt's router: 13,312 tokens (``--T``), d_model 4096, 256 experts, top-8,
fp16.

Prints one JSON line: the metric (routed-expert TFLOP/s, 6 D F flops per
kept pair), pairs/s, the dominant kernel's roofline (HIP events around its
launches on the library's stream, over the timed region), and the CPU oracle
timed on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0, "f32": 157.3}
PEAK_HBM_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "mixture_experts_routed_route_amd", "csrc")
# source file of each phase's kernel: a committed counter summary applies to
# the phase only while this file (and the shared header) is unchanged
KERNEL_SRC = {"gateup_full": "gemm_full.hip", "down_full": "gemm_full.hip",
              "gateup_thin16": "forward_kernels.hip",
              "down_thin16": "forward_kernels.hip",
              "gateup_thin64": "gemm_wide.hip",
              "down_thin64": "gemm_wide.hip",
              "dequant_once": "forward_kernels.hip",
              "combine": "forward_kernels.hip",
              "classify": "forward_kernels.hip",
              "router_gemm": "router.hip",
              "bwd_weights": "gemm_wgrad.hip", "bwd_data": "gemm_full.hip",
              "bwd_recompute": "gemm_full.hip"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=4)
    ap.add_argument("--capacity-factor", type=float, default=None)
    ap.add_argument("--T", type=int, default=None)
    ap.add_argument("--pairs-per-expert", type=int, default=None)
    ap.add_argument("--splitk-max-pairs", type=float, default=None)
    ap.add_argument("--fat-rows", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--no-phase-events", action="store_true")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache pass (K more steps, each after "
                         "a 1 GiB write that evicts L2 and the 256 MB MALL)")
    ap.add_argument("--one-stream", action="store_true",
                    help="MOE_OPT_ONE_STREAM: every launch on the caller's "
                         "stream (no second stream for the thin groups)")
    ap.add_argument("--tiled-decode", action="store_true",
                    help="MOE_OPT_TILED_DECODE: a one-token call runs the "
                         "split-K tile and the combine "
                         "instead of the matrix-vector kernels")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the graph pass (plan + forward captured once "
                         "into a HIP graph, K replays timed)")
    ap.add_argument("--weights", default=None, choices=("q4b32", "q4a32", "q4a64"),
                    help="4-bit format of workloads 4 and 7 (default q4b32)")
    ap.add_argument("--backward", action="store_true",
                    help="time moe_backward on the workload's plan (16-bit "
                         "workloads; default the prefill one)")
    ap.add_argument("--router", action="store_true",
                    help="time moe_route (router map + plan + statistics)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run one plain elementwise copy of MIB MiB "
                         "(dst = src * 1 in f32: MIB MiB read, MIB MiB "
                         "written) for scaling counter readings")
    return ap.parse_args()


def source_sha(kernel: str) -> str:
    h = hashlib.sha256()
    for f in (KERNEL_SRC[kernel], "moe_internal.h"):
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, kernel: str):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(PROFILES, f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except Exception:
        return None
    if rec.get("source_sha") != source_sha(kernel):
        return None
    return rec.get("bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: this build "
              "runs the layer on one GPU (expert parallelism over several "
              "GPUs is a design note only); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mixture_experts_routed_route_amd as moe
    import workloads as W

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.router:
        return bench_router(args, dev, torch, moe, W)
    if args.backward:
        return bench_backward(args, dev, torch, moe, W)
    wl = W.config(args.config, capacity_factor=args.capacity_factor, T=args.T,
                  pairs_per_expert=args.pairs_per_expert, w_dtype=args.weights)
    T, D, F, E, k, ns = (wl[n] for n in ("T", "D", "F", "E", "k", "n_shared"))
    logits = wl["logits"].to(dev)
    x = wl["x"].to(dev)

    def dv(w):
        return tuple(t.to(dev) for t in w) if isinstance(w, tuple) else w.to(dev)

    wg, wu, wd = dv(wl["w_gate"]), dv(wl["w_up"]), dv(wl["w_down"])
    # an explicit switch point is applied exactly (the sweep of the switch
    # point compares the two tiles at every size)
    exact = args.splitk_max_pairs is not None
    one = moe.MOE_OPT_ONE_STREAM if args.one_stream else 0
    if args.tiled_decode:
        one |= moe.MOE_OPT_TILED_DECODE

    def options(flags=0):
        o = moe.make_options(splitk_max_pairs=args.splitk_max_pairs,
                             fat_rows=args.fat_rows, exact_routes=exact)
        o.flags |= one | flags
        return o

    opts = options()
    plan_ws = torch.empty(moe.moe_plan_workspace_bytes(T, E, k,
                                                       wl["capacity_factor"], ns),
                          dtype=torch.uint8, device=dev)
    p = moe.moe_plan_create(logits, k, wl["capacity_factor"], ns,
                            workspace=plan_ws)
    wdt = {"f32": moe.MOE_F32, "bf16": moe.MOE_BF16, "f16": moe.MOE_F16,
           "q4b32": moe.MOE_Q4B32, "q4a32": moe.MOE_Q4A32,
           "q4a64": moe.MOE_Q4A64}[wl["w_dtype"]]
    xdt = {"f32": moe.MOE_F32, "bf16": moe.MOE_BF16, "f16": moe.MOE_F16}[wl["x_dtype"]]
    fwd_ws = torch.empty(moe.moe_forward_workspace_bytes(p, D, F, xdt, wdt, opts),
                         dtype=torch.uint8, device=dev)
    y = torch.empty(T, D, dtype=torch.float32, device=dev)

    def step(o):
        pl = moe.moe_plan_create(logits, k, wl["capacity_factor"], ns,
                                 workspace=plan_ws)
        moe.moe_forward(pl, x, wg, wu, wd, options=o, out=y, workspace=fwd_ws)
        return pl

    copy_calibration(args, torch, dev)
    for _ in range(args.warmup):
        pl = step(opts)
    torch.cuda.synchronize()

    # routing facts of this workload (one host read, outside the timing)
    st = moe.moe_plan_stats_get(pl, opts)
    counts = moe.moe_plan_get_views(pl)["counts"].cpu().numpy().astype(np.int64)
    kept_pairs = int(counts.sum())                       # shared included
    touched = int((counts > 0).sum())

    # routes per expert (the library's rule, restated for accounting)
    q4 = wl["w_dtype"].startswith("q4")
    fat_rows = opts.fat_rows if q4 else 0
    if 0 < fat_rows < 17:
        fat_rows = 17
    if q4 and T < fat_rows:
        fat_rows_eff = 0
    else:
        fat_rows_eff = fat_rows
    S = float(opts.splitk_max_pairs)
    if q4:
        full_mask = (counts >= fat_rows_eff) if fat_rows_eff > 0 else counts < 0
    elif wl["w_dtype"] == "f32":
        full_mask = counts < 0
    else:
        full_mask = counts.astype(np.float64) > S
        if not exact:
            # an underfilled full route hands experts of <= 256 rows over
            tiles = int(((counts[full_mask] + 255) // 256).sum())
            ncu = torch.cuda.get_device_properties(0).multi_processor_count
            if tiles * (F // 128) < ncu:
                full_mask &= counts > 256
    sk_mask = (counts > 0) & ~full_mask
    rows_full = int(counts[full_mask].sum())
    phase_units = route_units(counts, full_mask, sk_mask, D, F, wl, T, kept_pairs)

    # Per-phase times with every launch on one stream (a pass of its own,
    # 10 steps, outside the timed region): in the timed steps the thin
    # groups' launches run on the library's second stream beside the full
    # tiles, and their event spans there include waiting for compute units;
    # each phase's roofline fraction comes from this pass, where the phases
    # run one after another.
    solo = None
    routes = None
    dom = None
    if not args.no_phase_events:
        o_solo = options(moe.MOE_OPT_ONE_STREAM | moe.MOE_OPT_PHASE_EVENTS)
        moe.moe_phase_times(reset=True)
        for _ in range(min(args.steps, 10)):
            step(o_solo)
        torch.cuda.synchronize()
        solo_ms, solo_calls = moe.moe_phase_times(reset=True)
        solo = {name: v / max(solo_calls, 1) for name, v in solo_ms.items()}
        routes = {}
        for name, (bound, amount, extra) in phase_units.items():
            ms = solo.get(name, 0.0)
            if ms <= 0 or amount <= 0:
                continue
            routes[name] = roofline_entry(bound, amount, ms, wl["x_dtype"], extra)
        # the dominant kernel, timed in the steps themselves below; where the
        # library forks its second stream (its rule, restated: thin groups
        # beside full-tile ones, T k D F above 2^33) the thin phases run
        # there, their spans stretched by the full tiles beside them
        thin = {"gateup_thin16", "down_thin16", "gateup_thin64", "down_thin64"}
        forked = (not args.one_stream and T * k * D * F > 2 ** 33
                  and any(solo.get(n, 0) > 0 for n in ("gateup_full", "down_full"))
                  and any(solo.get(n, 0) > 0 for n in thin))
        cand = [n for n in solo if solo[n] > 0 and n in phase_units
                and phase_units[n][1] > 0 and not (forked and n in thin)]
        dom = max(cand, key=lambda n: solo[n]) if cand else None

    # The timed steps: HIP events only around the dominant phase (each
    # recorded pair makes the GPU drain the work before it, a few
    # microseconds a phase), on the stream that phase runs on.
    o_timed = (options(moe.MOE_OPT_PHASE_EVENTS |
                       moe.MOE_OPT_PHASE_ONLY(moe.PHASES.index(dom)))
               if dom is not None else opts)
    moe.moe_phase_times(reset=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        pl = step(o_timed)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    timed_ms, timed_calls = moe.moe_phase_times(reset=True)
    flops = W.flops_per_pair(D, F) * kept_pairs
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    pairs_s = kept_pairs / (ms_per_step * 1e-3)

    roofline = None
    if dom is not None:
        dom_ms = timed_ms[dom] / max(timed_calls, 1)
        bound, amount, extra = phase_units[dom]
        roofline = dict(kernel=dom, **roofline_entry(bound, amount, dom_ms,
                                                     wl["x_dtype"], extra))
        roofline["traffic"] = load_traffic(wl["name"], dom)
        roofline["algorithmic_per_launch"] = amount
        roofline["avg_launch_ms"] = round(dom_ms, 4)
        roofline["phase_ms_per_step_one_stream"] = {
            n: round(v, 4) for n, v in solo.items() if v > 0}

    # Cold-cache pass (outside the timed region above): each step follows
    # a 1 GiB write, so x, the weights and the plan start in HBM, not in L2
    # or the MALL; HIP events on the stream the library runs on time each
    # step alone.
    cold = None
    if not args.no_cold:
        flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        evs = [(torch.cuda.Event(enable_timing=True),
                torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for i, (ea, eb) in enumerate(evs):
            flush.fill_(i & 255)
            ea.record()
            step(opts)
            eb.record()
        torch.cuda.synchronize()
        ts = sorted(ea.elapsed_time(eb) for ea, eb in evs)
        cold = {"median_ms": round(ts[len(ts) // 2], 4), "min_ms": round(ts[0], 4),
                "steps": len(ts),
                "method": "1 GiB written before each step; HIP events per step"}
        del flush

    # Graph pass (outside the timed region above): one step captured into a
    # HIP graph and replayed, so the host's per-call work (argument checks,
    # launches) is paid once; what remains is the kernels and the gaps
    # between them. Short prompts and decode calls are launch-bound.
    graph = None
    if not args.no_graph:
        side = torch.cuda.Stream(device=dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            step(opts)
        torch.cuda.current_stream(dev).wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(opts)
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        gms = (time.perf_counter() - t0) * 1e3 / args.steps
        graph = {"ms_per_step": round(gms, 4), "replays": args.steps,
                 "method": "plan + forward captured once (torch.cuda.CUDAGraph "
                           "on the library's stream), replays timed back to back"}
        del g

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, args.cpu_seconds)

    out = {
        "metric": "routed-expert TFLOP/s per MoE layer (6*D*F per kept pair)",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl["x_dtype"],
        "data": "synthetic (seeded; workloads.py)",
        "config": {"workload": wl["name"], "T": T, "d_model": D, "d_ff": F,
                   "experts": E, "top_k": k, "shared": ns,
                   "weights": wl["w_dtype"],
                   "capacity_factor": wl["capacity_factor"],
                   "parallelism": "single GPU"},
        "pairs_per_s": round(pairs_s, 1),
        "kept_pairs": kept_pairs,
        "drop_fraction": st["drop_fraction"],
        "route_counts": {"touched_experts": touched,
                         "full_or_fat_experts": int(full_mask.sum()),
                         "splitk_experts": int(sk_mask.sum()),
                         "rows_full": rows_full,
                         "splitk_max_pairs": S, "fat_rows": fat_rows},
        "roofline": roofline,
        "routes": routes,
        "routes_timing": (None if routes is None else
                          "each phase alone, every launch on one stream (a "
                          "pass of its own)"),
        "cold": cold,
        "graph": graph,
        "cpu_baseline": cpu,
        "hardware": hardware(torch),
    }
    print(json.dumps(out), flush=True)


def route_units(counts, full_mask, sk_mask, D, F, wl, T, kept_pairs):
    """Algorithmic work of each forward phase, per step: (bound, amount,
    details). Full tile: 4 D F (gate/up) and 2 D F (down) flops per pair of
    a full-route expert. Thin groups (an expert's split-K rows cut into
    groups of <= 64; a group of <= 16 rows runs in the 16-row launch, the
    others in the 64-row one): per group its expert's weights of the stage
    once, its activation rows in and its output rows out. Dequant-once: each
    fat matrix read packed and written as fp16 once. Combine: each kept
    pair's output row read once, y written once."""
    import numpy as np

    import workloads as W
    bw = W.weight_bytes_per_expert(1, 1, wl["w_dtype"]) / 3.0   # B per weight
    xb = W.dtype_bytes(wl["x_dtype"])
    yb = 2 if wl["x_dtype"] == "f16" else 4          # per-pair output rows
    rows_full = int(counts[full_mask].sum())
    g16 = g64 = r16 = r64 = 0
    for c in counts[sk_mask]:
        c = int(c)
        ng = (c + 63) // 64
        last = c - 64 * (ng - 1)
        g64 += ng - 1 + (1 if last > 16 else 0)
        r64 += 64 * (ng - 1) + (last if last > 16 else 0)
        if last <= 16:
            g16 += 1
            r16 += last
    gu_w, d_w = 2.0 * D * F * bw, 1.0 * D * F * bw
    units = {
        "gateup_full": ("mfma", 4.0 * D * F * rows_full, {"rows": rows_full}),
        "down_full": ("mfma", 2.0 * D * F * rows_full, {"rows": rows_full}),
        "gateup_thin16": ("hbm", g16 * gu_w + r16 * (D + F) * xb,
                          {"groups": g16, "rows": r16}),
        "gateup_thin64": ("hbm", g64 * gu_w + r64 * (D + F) * xb,
                          {"groups": g64, "rows": r64}),
        "down_thin16": ("hbm", g16 * d_w + r16 * (F * xb + D * yb),
                        {"groups": g16, "rows": r16}),
        "down_thin64": ("hbm", g64 * d_w + r64 * (F * xb + D * yb),
                        {"groups": g64, "rows": r64}),
        "combine": ("hbm", kept_pairs * D * yb + T * D * 4, {"pairs": kept_pairs}),
    }
    if wl["w_dtype"].startswith("q4"):
        n_fat = int(full_mask.sum())
        units["dequant_once"] = ("hbm", n_fat * 3.0 * D * F * (bw + 2.0),
                                 {"experts": n_fat})
    return units


def roofline_entry(bound, amount, ms, x_dtype, extra=None):
    sec = ms * 1e-3
    if bound == "mfma":
        achieved, peak, unit = amount / sec / 1e12, PEAK_TFLOPS[x_dtype], "TFLOP/s"
    else:
        achieved, peak, unit = amount / sec / 1e9, PEAK_HBM_GBS, "GB/s"
    out = {"bound": bound, "achieved": round(achieved, 2), "peak": peak,
           "unit": unit, "frac": round(achieved / peak, 4), "ms": round(ms, 4),
           "amount": amount}
    if extra:
        out.update(extra)
    return out


def copy_calibration(args, torch, dev):
    """One plain elementwise copy of --copy-calibration MiB (f32, dst = src
    * 1) for scaling the counters of a profiled run."""
    if not args.copy_calibration:
        return
    n = (args.copy_calibration << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    del src, dst


def bench_router(args, dev, torch, moe, W):
    """moe_route on the long prompt's router: logits = x . Wr^T (fp16, f32
    accumulation), the plan over them and the routing statistics."""
    T = args.T or 13312
    D, E, k = 4096, 256, 8
    wl = W.make_router(T, D, E, k, "f16", seed=0, spread=0.5)
    x, w = wl["x"].to(dev), wl["w_router"].to(dev)
    nbytes = moe.moe_route_workspace_bytes_for(T, E, k, D)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    logits = torch.empty(T, E, dtype=torch.float32, device=dev)
    stats = torch.empty(8, dtype=torch.float32, device=dev)

    def step(flags=0):
        return moe.moe_route(x, w, k, workspace=ws, flags=flags,
                             logits=logits, stats=stats)

    copy_calibration(args, torch, dev)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # every phase's events in a pass of their own (10 calls); the timed
    # calls record events around the router kernel only (each recorded
    # pair drains the queue)
    per_all = None
    if not args.no_phase_events:
        moe.moe_phase_times(reset=True)
        for _ in range(min(args.steps, 10)):
            step(moe.MOE_OPT_PHASE_EVENTS)
        torch.cuda.synchronize()
        phase_ms, calls = moe.moe_phase_times(reset=True)
        per_all = {n: phase_ms[n] / max(calls, 1)
                   for n in ("router_gemm", "route_plan", "router_stats")}
    flags = (0 if args.no_phase_events else
             moe.MOE_OPT_PHASE_EVENTS | moe.MOE_OPT_PHASE_ONLY(moe.PHASES.index("router_gemm")))
    moe.moe_phase_times(reset=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(flags)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    flops = 2.0 * T * D * E
    roofline = None
    if flags:
        phase_ms, calls = moe.moe_phase_times(reset=True)
        gemm_ms = phase_ms["router_gemm"] / max(calls, 1)
        # x read once, Wr once, logits written once
        amount = T * D * 2 + E * D * 2 + T * E * 4
        achieved = amount / (gemm_ms * 1e-3) / 1e9
        roofline = {"kernel": "router_gemm", "bound": "hbm",
                    "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                    "traffic": load_traffic("long_prompt_router", "router_gemm"),
                    "algorithmic_per_launch": amount,
                    "avg_launch_ms": round(gemm_ms, 4),
                    "mfma_TFLOPs": round(flops / (gemm_ms * 1e-3) / 1e12, 1),
                    "phase_ms_per_step_all_events": {n: round(v, 4)
                                                     for n, v in per_all.items()}}
    st = stats.cpu().numpy().tolist()
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_router(wl, args.cpu_seconds)
    out = {
        "metric": "router TFLOP/s (2*D*E per token; router map, plan and "
                  "routing statistics timed together)",
        "value": round(flops / (ms * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic (seeded; workloads.make_router)",
        "config": {"workload": "long_prompt_router", "T": T, "d_model": D,
                   "experts": E, "top_k": k, "parallelism": "single GPU"},
        "tokens_per_s": round(T / (ms * 1e-3), 1),
        "route_stats": dict(zip(moe.ROUTE_STATS, st[:5])),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "hardware": hardware(torch),
    }
    print(json.dumps(out), flush=True)


def bench_backward(args, dev, torch, moe, W):
    """moe_backward on a 16-bit workload's plan (default: the prefill layer,
    4096 tokens, d_model 2048, d_ff 768, 128 experts, top-8, bf16): dx, the
    three weight gradients, the routing-weight and logit gradients of
    sum(dy * y) for a seeded dy ~ N(0, 1). Flops per kept pair: 16 D F, the
    products the backward runs (the recomputed gate/up products, dH, dX over
    both weights and the three weight gradients, 2 D F each, gate/up and dX
    twice); the routing-weight gradients are dots, not a product."""
    import numpy as np

    cfg = args.config if args.config != 4 else 3
    wl = W.config(cfg, capacity_factor=args.capacity_factor, T=args.T,
                  pairs_per_expert=args.pairs_per_expert)
    if wl["w_dtype"] not in ("bf16", "f16"):
        raise SystemExit("--backward needs a bf16 or f16 workload (2, 3, 5, 6)")
    T, D, F, E, k, ns = (wl[n] for n in ("T", "D", "F", "E", "k", "n_shared"))
    x = wl["x"].to(dev)
    wg, wu, wd = (wl[n].to(dev) for n in ("w_gate", "w_up", "w_down"))
    dy = torch.randn(T, D, generator=torch.Generator().manual_seed(1)).to(dev)
    plan = moe.moe_plan_create(wl["logits"].to(dev), k, wl["capacity_factor"], ns)
    ws = None

    def step(flags=0):
        o = moe.make_options()
        o.flags |= flags
        return moe.moe_backward(plan, x, wg, wu, wd, dy, options=o,
                                want_dtw=True, want_dlogits=True, workspace=ws)

    out = step()
    torch.cuda.synchronize()
    ws = torch.empty(moe.library().moe_backward_workspace_bytes(
        plan.handle, D, F, moe._TORCH_TO_MOE[x.dtype]), dtype=torch.uint8, device=dev)
    copy_calibration(args, torch, dev)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    counts = moe.moe_plan_get_views(plan)["counts"].cpu().numpy().astype(np.int64)
    P = int(counts.sum())
    flops = 16.0 * D * F * P
    # every phase's events in a pass of their own (10 calls), which also
    # picks the dominant phase; the timed calls record events around that
    # phase only (each recorded pair drains the queue)
    per_all, dom = None, None
    n_exp = E + ns
    # recompute: the gate and up products, 4 D F flops a pair; data
    # gradients: dH' and dX over both weights, 6 D F (matrix cores);
    # weight gradients: writing the f32 gradients of every
    # expert (3 E' D F x 4 B) plus reading the per-pair operands once
    # outweighs their 6 D F flops a pair at the HBM / MFMA ridge
    amount = {"bwd_recompute": ("mfma", 4.0 * D * F * P),
              "bwd_data": ("mfma", 6.0 * D * F * P),
              "bwd_weights": ("hbm", 3.0 * n_exp * D * F * 4
                              + P * (2.0 * D + 3.0 * F) * W.dtype_bytes(wl["x_dtype"]))}
    if not args.no_phase_events:
        moe.moe_phase_times(reset=True)
        for _ in range(min(args.steps, 10)):
            step(moe.MOE_OPT_PHASE_EVENTS)
        torch.cuda.synchronize()
        phase_ms, calls = moe.moe_phase_times(reset=True)
        per_all = {n: phase_ms[n] / max(calls, 1)
                   for n in ("bwd_recompute", "bwd_data", "bwd_weights", "bwd_routing")}
        dom = max(amount, key=lambda n: per_all[n])
    flags = (0 if dom is None else
             moe.MOE_OPT_PHASE_EVENTS | moe.MOE_OPT_PHASE_ONLY(moe.PHASES.index(dom)))
    moe.moe_phase_times(reset=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(flags)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    roofline = None
    if dom is not None:
        phase_ms, calls = moe.moe_phase_times(reset=True)
        per = {dom: phase_ms[dom] / max(calls, 1)}
        bound, amt = amount[dom]
        if bound == "mfma":
            achieved = amt / (per[dom] * 1e-3) / 1e12
            peak, u = PEAK_TFLOPS[wl["x_dtype"]], "TFLOP/s"
        else:
            achieved = amt / (per[dom] * 1e-3) / 1e9
            peak, u = PEAK_HBM_GBS, "GB/s"
        roofline = {"kernel": dom, "bound": bound, "achieved": round(achieved, 2),
                    "peak": peak, "unit": u, "frac": round(achieved / peak, 4),
                    "traffic": load_traffic(wl["name"], dom),
                    "algorithmic_per_launch": amt,
                    "avg_launch_ms": round(per[dom], 4),
                    "phase_ms_per_step_all_events": {n: round(v, 4)
                                                     for n, v in per_all.items()}}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_backward(wl, dy.cpu(), args.cpu_seconds)
    line = {
        "metric": "backward TFLOP/s per MoE layer (16*D*F per kept pair)",
        "value": round(flops / (ms * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": wl["x_dtype"],
        "data": "synthetic (seeded; workloads.py)",
        "config": {"workload": wl["name"] + "_backward", "T": T, "d_model": D,
                   "d_ff": F, "experts": E, "top_k": k, "shared": ns,
                   "parallelism": "single GPU"},
        "kept_pairs": P,
        "pairs_per_s": round(P / (ms * 1e-3), 1),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "hardware": hardware(torch),
    }
    print(json.dumps(line), flush=True)


def cpu_baseline_backward(wl, dy, target_s):
    """The oracle's dx path (each kept pair: g, u, h, the pair output, dH
    and dx, 12 D F flops) on the first tokens, doubling until about
    target_s seconds."""
    import numpy as np

    import oracle

    ids, w = oracle.route(wl["logits"], wl["k"])
    pl = oracle.plan(ids, wl["E"], wl["capacity_factor"], wl["n_shared"])
    n, done, total_t, pairs = 4, 0, 0.0, 0
    T = wl["T"]
    dyn = dy.numpy().astype(np.float64)
    while done < T and total_t < target_s:
        toks = np.arange(done, min(T, done + n))
        t0 = time.perf_counter()
        oracle.backward(wl["x"], wl["w_gate"], wl["w_up"], wl["w_down"], ids, w,
                        pl["keep"], dyn, E=wl["E"], n_shared=wl["n_shared"],
                        x_dtype=wl["x_dtype"], w_dtype=wl["w_dtype"],
                        c=wl["swiglu_limit"], tokens=toks, want=("dx",))
        total_t += time.perf_counter() - t0
        pairs += int(pl["keep"][toks].sum()) + wl["n_shared"] * len(toks)
        done += len(toks)
        n *= 2
    return {"value": round(12.0 * wl["D"] * wl["F"] * pairs / total_t / 1e12, 6),
            "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"dx of the first {done} tokens ({pairs} kept pairs) in "
                      f"{total_t:.1f} s; the oracle's dx path, 12 D F flops a pair"}


def cpu_baseline_router(wl, target_s):
    """The oracle's router map and statistics on the first tokens, doubling
    until about target_s seconds; TFLOP/s of the map (2 D E per token)."""
    import oracle

    T, D, E, k = wl["T"], wl["D"], wl["E"], wl["k"]
    n, done, total_t = 16, 0, 0.0
    while done < T and total_t < target_s:
        m = min(T, done + n) - done
        t0 = time.perf_counter()
        lg = oracle.router_logits(wl["x"][done:done + m], wl["w_router"],
                                  wl["dtype"])
        oracle.router_stats(lg.astype("float32"), k)
        total_t += time.perf_counter() - t0
        done += m
        n *= 2
    return {"value": round(2.0 * D * E * done / total_t / 1e12, 6),
            "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"router map + statistics of the first {done} of {T} "
                      f"tokens in {total_t:.1f} s"}


def cpu_baseline(wl, target_s):
    """The oracle, as it stands, on a bounded sample of the same workload:
    route + plan over all T tokens, then the layer on the first tokens
    until about target_s seconds of work; reported in TFLOP/s."""
    import numpy as np

    import oracle
    import workloads as W

    t0 = time.perf_counter()
    ids, w = oracle.route(wl["logits"], wl["k"])
    pl = oracle.plan(ids, wl["E"], wl["capacity_factor"], wl["n_shared"])
    t_plan = time.perf_counter() - t0
    T = wl["T"]
    n = 8
    total_t, total_pairs, done = 0.0, 0, 0
    while done < T and total_t < target_s:
        toks = np.arange(done, min(T, done + n))
        t0 = time.perf_counter()
        oracle.layer(wl["x"], wl["w_gate"], wl["w_up"], wl["w_down"], ids, w,
                     pl["keep"], E=wl["E"], n_shared=wl["n_shared"],
                     x_dtype=wl["x_dtype"], w_dtype=wl["w_dtype"],
                     c=wl["swiglu_limit"], tokens=toks)
        total_t += time.perf_counter() - t0
        total_pairs += int(pl["keep"][toks].sum()) + wl["n_shared"] * len(toks)
        done += len(toks)
        n *= 2
    flops = W.flops_per_pair(wl["D"], wl["F"]) * total_pairs
    return {"value": round(flops / total_t / 1e12, 6), "unit": "TFLOP/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"route+plan of all {T} tokens ({t_plan:.2f} s), then "
                      f"the layer on the first {done} tokens ({total_pairs} "
                      f"kept pairs) in {total_t:.1f} s",
            "pairs_per_s": round(total_pairs / total_t, 2)}


def hardware(torch):
    props = torch.cuda.get_device_properties(0)
    return {"device": props.name,
            "arch": getattr(props, "gcnArchName", ""),
            "cus": props.multi_processor_count,
            "hbm_gib": round(props.total_memory / 2 ** 30, 1),
            "torch": torch.__version__, "hip": torch.version.hip,
            "host_cpu": platform.processor() or platform.machine(),
            "host_threads": len(os.sched_getaffinity(0))}


if __name__ == "__main__":
    main()
