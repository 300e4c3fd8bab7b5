#!/usr/bin/env python
"""Benchmark of the single-GPU Muon optimizer step on MI355X.

One "step" is one muon_step_batched call over the whole matrix set (for
the periodic-RowNorm workload, one call of the schedule: refresh when
t mod K == 0, RowNorm otherwise).  Inputs are synthetic, seeded and already
resident in HBM when the timed region starts.

The headline is the Qwen2.5-7B 28-layer matrix set (or --config), timed
with the launch profiler off; a second pass of the same number of steps with
the per-launch HIP-event profiler on gives per-kernel times and the
roofline of the dominant kernel class.  The other four workloads follow as
"extra" entries (ms per step, TFLOP/s, dominant kernel roofline; refresh,
RowNorm and cycle times for the periodic-RowNorm workload), each with its
buffers freed before the next.  The float64 CPU oracle is timed on a bounded
sample of the headline workload.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Muon step ms + achieved MFMA TFLOP/s on Qwen2.5-7B-shaped matrix set"
PEAK_MFMA_16BIT = 2500.0   # TFLOP/s, MI355X dense bf16 / fp16
PEAK_MFMA_F32 = 157.3      # TFLOP/s, MI355X dense fp32 matrix
PEAK_HBM = 8000.0          # GB/s, MI355X HBM3E
GEMM_CLASSES = ("syrk", "poly", "pqpg", "ph", "final", "xupd")
HBM_CLASSES = ("prep", "rownorm", "colsum", "colapply", "xcast", "wupd")
# steps per workload for the extra entries (the headline takes --steps)
EXTRA_STEPS = {1: 50, 2: 50, 3: 20, 4: 20, 5: 10}


def ns_flops(shapes, formulation: str = "auto", rr_products: int = 17) -> float:
    """Algorithmic flops of one step as this library evaluates it, symmetric
    products counted on the lower triangle.  Gram form: SYRK r^2 c +
    rr_products r x r products of r^3 (17 for N = 5: four per iteration,
    three in the first, two in the last) + final 2 r^2 c.  Direct form: per
    iteration SYRK r^2 c + A^2 r^3 + X update 2 r^2 c.  rr_products = 21 is
    the count of a recursion that also forms P^2 and G P^2 separately (three
    in the first iteration, five in the middle three, three in the last)."""
    tot = 0.0
    for m, n in shapes:
        r, c = min(m, n), max(m, n)
        if formulation == "direct" or (formulation == "auto" and 8 * c <= 9 * r):
            tot += 15.0 * r * r * c + 5.0 * r ** 3
        else:
            tot += 3.0 * r * r * c + rr_products * r ** 3
    return tot


def plan_flops_per_shape(plan, rr_products: int = 17) -> dict:
    """Algorithmic flops of one matrix of each planned shape (m, n), with the
    formulation the planner (or a tuning hint) chose for its bucket."""
    return {tuple(b["shape"]): ns_flops([b["shape"]], b["formulation"], rr_products)
            for b in plan.buckets()}


def blas_info():
    """(vendor, threads) of NumPy's BLAS."""
    try:
        from threadpoolctl import threadpool_info
        blas = [d for d in threadpool_info() if d.get("user_api") == "blas"]
        if blas:
            d = blas[0]
            return f"{d.get('internal_api')} {d.get('version') or ''}".strip(), d.get("num_threads")
    except Exception:  # pragma: no cover
        pass
    return "unknown", None


def cpu_baseline(w, flops_per_shape: dict, sample_shapes_max: int = 3):
    """Time the float64 oracle on one matrix per distinct shape (largest
    first, at most `sample_shapes_max` shapes, ~10-30 s of CPU work) and
    extrapolate to the whole matrix set by count."""
    import numpy as np
    from matrix_aware_optimizer_muon_amd import workloads as WL
    from oracle import muon_oracle as OR
    vendor, threads = blas_info()
    cores = len(os.sched_getaffinity(0))
    counts = {}
    for s in w.shapes:
        key = (min(s), max(s))
        counts[key] = counts.get(key, 0) + 1
    keys = sorted(counts, key=lambda k: -k[0] * k[0] * k[1])[:sample_shapes_max]
    per_shape = {}
    for r, c in keys:
        i = next(j for j, s in enumerate(w.shapes) if (min(s), max(s)) == (r, c))
        Wh = WL.host_weight(w, i)
        Gh = WL.host_grad(w, i, 0)
        Mh = np.zeros_like(Wh)
        t0 = time.perf_counter()
        OR.muon_step(Wh, Mh, Gh, w.lr, w.wd)
        per_shape[(r, c)] = time.perf_counter() - t0
    covered = sum(counts[k] for k in keys)
    total_s = sum(per_shape[k] * counts[k] for k in keys)
    covered_flops = sum(flops_per_shape[tuple(s)] for s in w.shapes if (min(s), max(s)) in per_shape)
    sample = ", ".join(f"{c}x{r} ({per_shape[(r, c)]:.1f} s)" for r, c in keys)
    return {
        "value": covered_flops / total_s / 1e12,
        "unit": "TFLOP/s",
        "cores": threads if threads else cores,
        "kind": "oracle",
        "sample": (f"float64 direct-form oracle, one matrix per shape [{sample}], "
                   f"extrapolated by count to {covered} of {len(w.shapes)} matrices; "
                   f"value = the GPU path's algorithmic flops / oracle seconds"),
        "blas": vendor,
        "blas_threads": threads,
        "ms_per_step_extrapolated": total_s * 1e3 * len(w.shapes) / covered,
        "host_cores_visible": cores,
    }


def cpu_baseline_whole(w, flops_per_shape: dict):
    """Time the float64 oracle on every matrix of a small workload (one step
    from zero momentum), for the workloads small enough to time whole."""
    import numpy as np
    from matrix_aware_optimizer_muon_amd import workloads as WL
    from oracle import muon_oracle as OR
    vendor, threads = blas_info()
    cores = len(os.sched_getaffinity(0))
    total_s = 0.0
    for i in range(len(w.shapes)):
        Wh = WL.host_weight(w, i)
        Gh = WL.host_grad(w, i, 0)
        Mh = np.zeros_like(Wh)
        t0 = time.perf_counter()
        OR.muon_step(Wh, Mh, Gh, w.lr, w.wd)
        total_s += time.perf_counter() - t0
    F = sum(flops_per_shape[tuple(s)] for s in w.shapes)
    return {
        "value": F / total_s / 1e12,
        "unit": "TFLOP/s",
        "cores": threads if threads else cores,
        "kind": "oracle",
        "sample": (f"float64 direct-form oracle on all {len(w.shapes)} matrices, one step "
                   f"(whole workload); value = the GPU path's algorithmic flops / oracle seconds"),
        "blas": vendor,
        "blas_threads": threads,
        "ms_per_step": total_s * 1e3,
        "host_cores_visible": cores,
    }


def roofline_of(ktimes: dict, ns_dtype: str, traffic: dict, classes=None):
    """Roofline entry of the class with the largest total time (among
    `classes` if given)."""
    cand = {k: v for k, v in ktimes.items() if classes is None or k in classes}
    if not cand:
        return None
    dom = max(cand, key=lambda k: cand[k]["ms"])
    v = cand[dom]
    total = sum(x["ms"] for x in ktimes.values())
    common = {"kernel": dom,
              "traffic": round(sum(traffic[dom]), 0) if dom in traffic else None,
              "ms_per_launch": round(v["ms"] / v["launches"], 5),
              "share_of_step": round(v["ms"] / total, 3),
              "algorithmic_bytes_per_launch": round(v["bytes"] / v["launches"], 0)}
    if dom in GEMM_CLASSES:
        peak = PEAK_MFMA_F32 if ns_dtype == "f32" else PEAK_MFMA_16BIT
        ach = v["flops"] / (v["ms"] * 1e-3) / 1e12
        out = {"bound": "mfma", "achieved": round(ach, 2), "peak": peak, "unit": "TFLOP/s",
               "frac": round(ach / peak, 4),
               "algorithmic_flops_per_launch": round(v["flops"] / v["launches"], 0)}
    else:
        ach = v["bytes"] / (v["ms"] * 1e-3) / 1e9
        out = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM, "unit": "GB/s",
               "frac": round(ach / PEAK_HBM, 4)}
    out.update(common)
    return out


def kernel_table(ktimes: dict) -> dict:
    kernels = {}
    for k, v in ktimes.items():
        e = {"ms_total": round(v["ms"], 4), "launches": v["launches"],
             "ms_per_launch": round(v["ms"] / v["launches"], 5)}
        if v["flops"] > 0:
            e["tflops"] = round(v["flops"] / (v["ms"] * 1e-3) / 1e12, 2)
        if v["bytes"] > 0:
            e["gbs"] = round(v["bytes"] / (v["ms"] * 1e-3) / 1e9, 1)
        kernels[k] = e
    return kernels


def run_workload(k: int, steps: int, warmup: int, form: str = "auto", hints=None,
                 max_ws: int = 0, profile: bool = True):
    """Plan, fill and time one workload.  Returns (result dict, plan, w)."""
    import torch
    import matrix_aware_optimizer_muon_amd as pkg
    from matrix_aware_optimizer_muon_amd import workloads as WL
    from matrix_aware_optimizer_muon_amd.profiling import read_traffic

    w = WL.config(k)
    dev = torch.device("cuda:0")
    if form == "auto" and w.ns_dtype != "bf16":
        form = "gram"
    W = [WL.device_weight(w, i, dev) for i in range(len(w.shapes))]
    M = [torch.zeros_like(x) for x in W]
    G = [WL.device_grad(w, i, 0, dev) for i in range(len(w.shapes))]
    plan = pkg.Plan(w.shapes, w.grad_dtype, w.ns_dtype, formulation=form, hints=hints,
                    max_workspace_bytes=max_ws)
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    ptr = lambda L: [x.data_ptr() for x in L]
    Wp, Mp, Gp = ptr(W), ptr(M), ptr(G)

    if w.prior_steps:
        # momentum from seeded prior gradients, accumulated by the library's
        # own momentum update (RowNorm step with lr = wd = 0 leaves W as is)
        for s in range(-w.prior_steps, 0):
            Gs = [WL.device_grad(w, i, s, dev) for i in range(len(w.shapes))]
            plan.rownorm_ptrs(Wp, Mp, ptr(Gs), 0.0, 0.0, ws.data_ptr(), ws.numel(), sp)
            del Gs
        torch.cuda.synchronize()

    K = w.refresh_period

    def one_step(t):
        if K and t % K != 0:
            plan.rownorm_ptrs(Wp, Mp, Gp, w.lr, w.wd, ws.data_ptr(), ws.numel(), sp)
            return "rownorm"
        plan.step_ptrs(Wp, Mp, Gp, w.lr, w.wd, ws.data_ptr(), ws.numel(), sp)
        return "refresh"

    def timed_pass(n, per_step):
        # per_step: an event pair around every step (each record is a marker
        # packet on the stream, a few us of idle per step); else one pair
        # around the whole pass
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n if per_step else 1)]
        kinds = []
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        if not per_step:
            evs[0][0].record(stream)
        for t in range(n):
            if per_step:
                evs[t][0].record(stream)
            kinds.append(one_step(t))
            if per_step:
                evs[t][1].record(stream)
        if not per_step:
            evs[0][1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return wall, [a.elapsed_time(b) for a, b in evs], kinds

    for t in range(warmup):
        one_step(t)
    # timed region: launch profiler off; per-step events only where the
    # refresh and RowNorm steps are reported apart
    wall, step_ms, kinds = timed_pass(steps, per_step=bool(K))
    if not K:
        # spread of single steps, from a separate pass with per-step events
        _, step_ms, _ = timed_pass(steps, per_step=True)
    ktimes = {}
    prof_wall = None
    if profile:
        # second pass, same steps, per-launch HIP events on the library's stream
        plan.set_profiling(True)
        prof_wall, _, _ = timed_pass(steps, per_step=False)
        ktimes = plan.kernel_times()
        plan.set_profiling(False)

    per_shape = plan_flops_per_shape(plan)
    per_shape21 = plan_flops_per_shape(plan, 21)
    F = sum(per_shape[tuple(s)] for s in w.shapes)
    F21 = sum(per_shape21[tuple(s)] for s in w.shapes)
    refresh_ms = [m for m, kd in zip(step_ms, kinds) if kd == "refresh"]
    rownorm_ms = [m for m, kd in zip(step_ms, kinds) if kd == "rownorm"]
    n_refresh = len(refresh_ms)
    traffic = read_traffic(w.name, ROOT)
    srt = sorted(step_ms)
    res = {
        "workload": w.name,
        "ms_per_step": round(wall * 1e3 / steps, 4),
        "step_ms_median": round(srt[len(srt) // 2], 4),
        "step_ms_p90": round(srt[min(len(srt) - 1, int(0.9 * len(srt)))], 4),
        "tflops": round(F * n_refresh / wall / 1e12, 3) if n_refresh else 0.0,
        "tflops_21r3_count": round(F21 * n_refresh / wall / 1e12, 3) if n_refresh else 0.0,
        "algorithmic_tflop_per_refresh": round(F / 1e12, 4),
        "steps": steps,
        "dtype": "bf16" if w.ns_dtype == "bf16" else "f32",
        "formulation": form,
    }
    if prof_wall is not None:
        res["ms_per_step_profiled"] = round(prof_wall * 1e3 / steps, 4)
        res["roofline"] = roofline_of(ktimes, w.ns_dtype, traffic)
        res["kernels"] = kernel_table(ktimes)
    if refresh_ms and rownorm_ms:
        res["refresh_ms"] = round(sum(refresh_ms) / len(refresh_ms), 4)
        res["rownorm_ms"] = round(sum(rownorm_ms) / len(rownorm_ms), 4)
        res["cycle_ms"] = round(res["refresh_ms"] + (K - 1) * res["rownorm_ms"], 4)
        if ktimes:
            rn = {c: v for c, v in ktimes.items() if c in ("rownorm", "colsum", "colapply")}
            res["rownorm_kernels_hbm"] = {
                c: {"gbs": round(v["bytes"] / (v["ms"] * 1e-3) / 1e9, 1),
                    "frac": round(v["bytes"] / (v["ms"] * 1e-3) / 1e9 / PEAK_HBM, 4)}
                for c, v in rn.items()}
    plan_desc = [{"shape": list(b["shape"]), "count": b["count"], "chunks": b["chunks"],
                  "tile": b["tile"], "formulation": b["formulation"]} for b in plan.buckets()]
    res["plan"] = plan_desc
    res["workspace_bytes"] = plan.workspace_bytes
    del W, M, G, ws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res, per_shape, w


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=4, help="workload 1..5 (4 = Qwen2.5-7B, 28 layers)")
    ap.add_argument("--formulation", choices=("auto", "gram", "direct"), default="auto",
                    help="Newton-Schulz evaluation (auto: direct for near-square, else gram)")
    ap.add_argument("--tuned", action="store_true",
                    help="per-shape tile / formulation from the tuning cache (shapes it lacks "
                         "are tuned first, on the device)")
    ap.add_argument("--tune-cache", default=None,
                    help="tuning cache file (default: the one shipped with the package)")
    ap.add_argument("--max-workspace-gib", type=float, default=0.0,
                    help="Newton-Schulz scratch cap passed to the planner (0: the library default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-profile", action="store_true", help="skip the profiled second pass")
    ap.add_argument("--no-extras", action="store_true", help="only the headline workload")
    ap.add_argument("--calibrate-copy-mb", type=int, default=0,
                    help="only run a plain device copy of this many MiB (HBM counter scale)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.calibrate_copy_mb:
        n = args.calibrate_copy_mb * (1 << 20) // 4
        a = torch.ones(n, device="cuda:0")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": n * 4, "bytes_written": n * 4}))
        return

    import matrix_aware_optimizer_muon_amd as pkg
    from matrix_aware_optimizer_muon_amd import workloads as WL

    lib_path = pkg.load()._name
    w = WL.config(args.config)
    form = args.formulation
    if form == "direct" and w.ns_dtype != "bf16":
        print("the direct form runs on the 16-bit path only", file=sys.stderr)
        sys.exit(2)
    hints = None
    if args.tuned:
        from matrix_aware_optimizer_muon_amd import tune as TU
        cache = TU.load_cache(args.tune_cache or TU.SHIPPED_CACHE)
        cache = TU.tune(w.shapes, w.grad_dtype, w.ns_dtype, cache,
                        log=lambda msg: print("tune: " + msg, file=sys.stderr, flush=True))
        hints = TU.hints_for(w.shapes, w.grad_dtype, w.ns_dtype, cache)
        torch.cuda.synchronize()
    max_ws = int(args.max_workspace_gib * (1 << 30))
    head, per_shape, w = run_workload(args.config, args.steps, args.warmup, form, hints, max_ws,
                                      profile=not args.no_profile)
    print(f"headline config {args.config}: {head['ms_per_step']} ms/step", file=sys.stderr, flush=True)

    out = {
        "metric": METRIC,
        "value": head["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic (seeded Gaussian W, G; random init, no checkpoints)",
        "config": {"workload": w.name, "formulation": head["formulation"], "tuned": bool(args.tuned),
                   "matrices": len(w.shapes), "params": w.numel(),
                   "grad_dtype": w.grad_dtype, "ns_dtype": w.ns_dtype,
                   "refresh_period": w.refresh_period,
                   "algorithmic_tflop_per_refresh": head["algorithmic_tflop_per_refresh"]},
        "value_21r3_count": head["tflops_21r3_count"],
        "step_ms_median": head["step_ms_median"],
        "step_ms_p90": head["step_ms_p90"],
        "roofline": head.get("roofline"),
        "ms_per_step_profiled": head.get("ms_per_step_profiled"),
        "kernels": head.get("kernels", {}),
        "library": os.path.relpath(lib_path, ROOT),
        "plan": head["plan"],
        "workspace_bytes": head["workspace_bytes"],
    }
    for key in ("refresh_ms", "rownorm_ms", "cycle_ms", "rownorm_kernels_hbm"):
        if key in head:
            out[key] = head[key]
    if not args.no_extras and not args.tuned and form == "auto" and not max_ws:
        extra = {}
        whole = {}  # small workloads whose oracle is timed whole: (w, flops per shape)
        for k in (1, 2, 3, 4, 5):
            if k == args.config:
                continue
            r, flops_k, w_k = run_workload(k, EXTRA_STEPS[k], 3, profile=not args.no_profile)
            if k <= 3:
                whole[k] = (w_k, flops_k)
            r.pop("plan", None)
            r.pop("kernels", None)
            extra[f"config{k}"] = r
            print(f"extra config {k}: {r['ms_per_step']} ms/step", file=sys.stderr, flush=True)
        if args.config == 4:
            # the same workload planned with the shipped tuning cache's
            # per-shape winners (no tuning at run time: shapes it lacks keep
            # the planner's rule)
            from matrix_aware_optimizer_muon_amd import tune as TU
            try:
                cache = TU.load_cache(TU.SHIPPED_CACHE)
                th = TU.hints_for(w.shapes, w.grad_dtype, w.ns_dtype, cache)
            except Exception as e:  # pragma: no cover
                th = None
                print(f"tuned extra skipped: {e}", file=sys.stderr)
            if th is not None:
                r, _, _ = run_workload(4, args.steps, args.warmup, hints=th, profile=False)
                r.pop("plan", None)
                r["hints"] = {f"{m}x{n}": h for (m, n), h in th.items()}
                extra["config4_tuned"] = r
                print(f"extra config 4 tuned: {r['ms_per_step']} ms/step", file=sys.stderr, flush=True)
        out["extra"] = extra
        if not args.no_cpu_baseline:
            for k, (w_k, fk) in whole.items():
                extra[f"config{k}"]["cpu_baseline"] = cpu_baseline_whole(w_k, fk)
                print(f"extra config {k}: oracle {extra[f'config{k}']['cpu_baseline']['ms_per_step']:.0f} ms "
                      f"whole", file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, per_shape)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
