"""Shape-adaptive choice of tile width and Newton-Schulz formulation.

"DMuon" 2.4 searches tile configurations per target and matrix shape and
caches the winners for reuse; 2.3 times every distinct matrix shape at
initialisation to obtain the per-shape costs that owner assignment balances.
This module does both for this library's kernels:

* ``candidates`` lists the settings the kernels provide for one shape
  (``muon_bucket_hint``: tile 64 / 128 / 256, Gram or direct form);
* ``time_bucket`` times one setting with a single-bucket plan of that shape
  and count on seeded synthetic device inputs (weights N(0, 0.02^2),
  gradients N(0, 1e-3^2) in the planned gradient dtype), median over a few
  steps after two warm-up steps (the first timed shape of a process runs
  ~15 % slow after a single one);
* ``tune`` times every candidate of every (shape, count) not yet in the
  cache, keeps the fastest, and stores all timings (the per-shape cost
  profile) in a JSON cache keyed by device, dtypes, shape and count;
* ``hints_for`` turns cached winners into ``Plan(hints=...)``.

The cache file is plain JSON: ``{"version": 1, "entries": {key: entry}}``
with ``entry = {"tile", "formulation", "ms", "default", "candidates":
[{"tile", "formulation", "ms"}...]}``.  Timing needs a GPU; the cache logic
does not.
"""
from __future__ import annotations

import json
import os
from collections import OrderedDict
from typing import Callable, Iterable, Optional, Sequence

CACHE_VERSION = 1
_HERE = os.path.dirname(os.path.abspath(__file__))
# Winners measured on the device this package targets, shipped with it.
SHIPPED_CACHE = os.path.join(_HERE, "tuned", "mi355x.json")


def default_cache_path() -> str:
    """MUON_TUNE_CACHE if set, else a per-user cache file."""
    env = os.environ.get("MUON_TUNE_CACHE")
    if env:
        return env
    base = os.environ.get("XDG_CACHE_HOME") or os.path.join(os.path.expanduser("~"), ".cache")
    return os.path.join(base, "matrix_aware_optimizer_muon_amd", "tune.json")


def shape_counts(shapes: Iterable[Sequence[int]]) -> "OrderedDict[tuple, int]":
    """Distinct (m, n) in order of first appearance, with their counts (the
    planner's buckets)."""
    out: "OrderedDict[tuple, int]" = OrderedDict()
    for m, n in shapes:
        k = (int(m), int(n))
        out[k] = out.get(k, 0) + 1
    return out


def cache_key(device: str, grad_dtype: str, ns_dtype: str, m: int, n: int, count: int) -> str:
    return f"{device}|g={grad_dtype}|ns={ns_dtype}|{m}x{n}x{count}"


def load_cache(path: str) -> dict:
    """The cache at `path`, or an empty one if the file is missing.  A file
    of another version is treated as empty."""
    try:
        with open(path) as f:
            data = json.load(f)
    except FileNotFoundError:
        return {"version": CACHE_VERSION, "entries": {}}
    if not isinstance(data, dict) or data.get("version") != CACHE_VERSION:
        return {"version": CACHE_VERSION, "entries": {}}
    data.setdefault("entries", {})
    return data


def save_cache(path: str, data: dict) -> None:
    """Write atomically (temporary file, then rename)."""
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    tmp = path + ".tmp"
    with open(tmp, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
        f.write("\n")
    os.replace(tmp, path)


def candidates(m: int, n: int, ns_dtype: str) -> list:
    """The settings the kernels provide for an m x n bucket.  fp32 path:
    Gram form with 64- or 128-wide tiles.  16-bit path: Gram form with 64-
    (r <= 1024), 128- or 256-wide tiles, and the direct form (256-wide)."""
    r = min(m, n)
    if ns_dtype == "f32":
        return [{"tile": 64, "formulation": "gram"}, {"tile": 128, "formulation": "gram"}]
    out = []
    if r <= 1024:
        out.append({"tile": 64, "formulation": "gram"})
    out.append({"tile": 128, "formulation": "gram"})
    out.append({"tile": 256, "formulation": "gram"})
    out.append({"tile": 256, "formulation": "direct"})
    return out


def device_name() -> str:
    import torch
    p = torch.cuda.get_device_properties(0)
    arch = getattr(p, "gcnArchName", "") or ""
    return f"{p.name} {arch.split(':')[0]}".strip()


def time_bucket(m: int, n: int, count: int, grad_dtype: str, ns_dtype: str, hint: Optional[dict],
                steps: int = 3, warmup: int = 2, seed: int = 0) -> float:
    """Median ms of one muon_step_batched call over `count` m x n matrices
    planned with `hint` (None: the planner's own rule)."""
    import torch
    from ._lib import Plan
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    plan = Plan([(m, n)] * count, grad_dtype, ns_dtype,
                hints={(m, n): hint} if hint else None)
    gdt = torch.bfloat16 if grad_dtype == "bf16" else torch.float32
    W = [torch.randn(m, n, device=dev, generator=gen) * 0.02 for _ in range(count)]
    M = [torch.zeros(m, n, device=dev) for _ in range(count)]
    G = [(torch.randn(m, n, device=dev, generator=gen) * 1e-3).to(gdt) for _ in range(count)]
    ws = torch.empty(max(plan.workspace_bytes, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    ptr = lambda L: [x.data_ptr() for x in L]
    Wp, Mp, Gp = ptr(W), ptr(M), ptr(G)
    times = []
    for i in range(warmup + steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        plan.step_ptrs(Wp, Mp, Gp, 0.02, 0.1, ws.data_ptr(), ws.numel(), stream.cuda_stream)
        b.record(stream)
        b.synchronize()
        if i >= warmup:
            times.append(a.elapsed_time(b))
    plan.close()
    del W, M, G, ws
    times.sort()
    return float(times[len(times) // 2])


def tune(shapes: Sequence[Sequence[int]], grad_dtype: str, ns_dtype: str,
         cache: Optional[dict] = None, device: Optional[str] = None, steps: int = 3,
         warmup: int = 2, timer: Optional[Callable] = None, log: Optional[Callable] = None) -> dict:
    """Time every candidate of each (shape, count) of `shapes` that `cache`
    does not hold yet and add the results.  `timer(m, n, count, hint)`
    replaces the device timing (tests).  Returns the (updated) cache."""
    if cache is None:
        cache = {"version": CACHE_VERSION, "entries": {}}
    if device is None:
        device = device_name()
    if timer is None:
        timer = lambda m, n, c, h: time_bucket(m, n, c, grad_dtype, ns_dtype, h, steps, warmup)
    for (m, n), count in shape_counts(shapes).items():
        key = cache_key(device, grad_dtype, ns_dtype, m, n, count)
        if key in cache["entries"]:
            continue
        default_ms = timer(m, n, count, None)
        rows = []
        for h in candidates(m, n, ns_dtype):
            ms = timer(m, n, count, h)
            rows.append({"tile": h["tile"], "formulation": h["formulation"], "ms": round(ms, 4)})
            if log:
                log(f"{m}x{n} x{count}: tile {h['tile']:3d} {h['formulation']:6s} {ms:9.3f} ms")
        best = min(rows, key=lambda e: e["ms"])
        cache["entries"][key] = {"tile": best["tile"], "formulation": best["formulation"],
                                 "ms": best["ms"], "default": round(default_ms, 4),
                                 "candidates": rows}
    return cache


def hints_for(shapes: Sequence[Sequence[int]], grad_dtype: str, ns_dtype: str, cache: dict,
              device: Optional[str] = None) -> dict:
    """Plan(hints=...) for the shapes whose (shape, count) the cache holds;
    shapes it does not hold keep the planner's rule."""
    if device is None:
        device = device_name()
    hints = {}
    for (m, n), count in shape_counts(shapes).items():
        e = cache.get("entries", {}).get(cache_key(device, grad_dtype, ns_dtype, m, n, count))
        if e:
            hints[(m, n)] = {"tile": int(e["tile"]), "formulation": e["formulation"]}
    return hints


def main(argv=None):
    """Tune the buckets of one of the package's workloads and merge the
    results into a cache file."""
    import argparse
    from . import workloads as WL
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", type=int, required=True)
    ap.add_argument("--cache", default=None, help="cache file (default: the per-user cache)")
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--retune", action="store_true", help="time again what the cache holds")
    a = ap.parse_args(argv)
    w = WL.config(a.config)
    path = a.cache or default_cache_path()
    cache = load_cache(path)
    dev = device_name()
    if a.retune:
        for (m, n), count in shape_counts(w.shapes).items():
            cache["entries"].pop(cache_key(dev, w.grad_dtype, w.ns_dtype, m, n, count), None)
    tune(w.shapes, w.grad_dtype, w.ns_dtype, cache, dev, steps=a.steps, log=print)
    save_cache(path, cache)
    for (m, n), count in shape_counts(w.shapes).items():
        e = cache["entries"][cache_key(dev, w.grad_dtype, w.ns_dtype, m, n, count)]
        print(f"{m}x{n} x{count}: best tile {e['tile']} {e['formulation']} {e['ms']:.3f} ms "
              f"(planner rule {e['default']:.3f} ms)")


if __name__ == "__main__":
    main()
