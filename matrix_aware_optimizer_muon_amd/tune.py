"""Shape-adaptive choice of tile width and Newton-Schulz formulation.

"DMuon" 2.4 searches tile configurations per target and matrix shape and
caches the winners for reuse; 2.3 times every distinct matrix shape at
initialisation to obtain the per-shape costs that owner assignment balances.
This module does both for this library's kernels:

* ``candidates`` lists the settings the kernels provide for one shape
  (``muon_bucket_hint``: tile 64 / 128 / 256, Gram or direct form), keeping
  only those the planner accepts for it (it refuses, for instance, the Gram
  form on near-square buckets of the 16-bit path);
* ``time_bucket`` times one setting with a single-bucket plan of that shape
  and count on seeded synthetic device inputs (weights N(0, 0.02^2),
  gradients N(0, 1e-3^2) in the planned gradient dtype), median over a few
  steps after two warm-up steps (the first timed shape of a process runs
  ~15 % slow after a single one), and returns the direction output of the
  bucket's first matrix from the first call;
* every candidate's direction is compared with the fp32 path's direction
  for the same input (a single-matrix plan on ``ns_dtype="f32"``, accurate
  to ~1e-5): a setting whose relative error exceeds ``ACCURACY_TOL`` is
  recorded but never chosen, so a fast but inaccurate setting cannot reach
  the cache's winners;
* ``tune`` times every candidate of every (shape, count) not yet in the
  cache, keeps the fastest accurate one, then, when that one runs on the
  256-wide kernels, searches their knobs one at a time from it (tile-order
  group height, XCD run length, four waves per workgroup for SYRK and the
  final product: ``KNOBS``), keeping a change only when it is faster by more
  than ``KNOB_GAIN``, and stores all timings (the per-shape cost profile) in
  a JSON cache keyed by device, dtypes, shape and count;
* ``hints_for`` turns cached winners into ``Plan(hints=...)``.

The cache file is plain JSON: ``{"version": 2, "entries": {key: entry}}``
with ``entry = {"tile", "formulation", "group", "xcd_chunk", "waves", "ms",
"default", "candidates": [{"tile", "formulation", ..., "ms", "err"}...]}``
(knob fields absent or 0: the planner's rule).  Timing needs a GPU; the
cache logic does not.
"""
from __future__ import annotations

import json
import os
from collections import OrderedDict
from typing import Callable, Iterable, Optional, Sequence

CACHE_VERSION = 2
# Largest relative Frobenius error of a candidate's direction against the
# fp32 path's that the tuner accepts: half the 16-bit path's 2e-2 bound (the
# sample is one matrix and one seed), and the fp32 path's own 1e-4 bound.
ACCURACY_TOL = {"bf16": 1e-2, "f32": 1e-4}
# Knobs of the 256-wide kernels (muon_bucket_hint) and the values tried for
# each, one knob at a time from the best tile / form: tile-order group height
# (rule: 8 rows for full grids, 4 for triangular ones), XCD run length (rule:
# 32; -1: one contiguous range per XCD), wave64s per workgroup of SYRK and
# the final product (rule: 8).
KNOBS = (("group", (2, 4, 16)), ("xcd_chunk", (-1, 16, 64, 256)), ("waves", (4,)))
KNOB_GAIN = 0.01   # a knob value must beat the current best by more than 1 %
HINT_FIELDS = ("tile", "formulation", "group", "xcd_chunk", "waves")
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
    Gram form with 64- or 128-wide tiles.  16-bit path: Gram and direct form
    with 64- and 128-wide (r <= 1024) and 256-wide tiles; settings the
    planner refuses for this shape are left out."""
    r = min(m, n)
    if ns_dtype == "f32":
        raw = [{"tile": 64, "formulation": "gram"}, {"tile": 128, "formulation": "gram"}]
    else:
        raw = []
        if r <= 1024:
            raw.append({"tile": 64, "formulation": "gram"})
        raw.append({"tile": 128, "formulation": "gram"})
        raw.append({"tile": 256, "formulation": "gram"})
        if r <= 1024:
            raw.append({"tile": 64, "formulation": "direct"})
            raw.append({"tile": 128, "formulation": "direct"})
        raw.append({"tile": 256, "formulation": "direct"})
    return [h for h in raw if _plannable(m, n, ns_dtype, h)]


def _plannable(m: int, n: int, ns_dtype: str, hint: dict) -> bool:
    from ._lib import MUON_ERR_UNSUPPORTED, MuonError, Plan
    try:
        Plan([(m, n)], "f32", ns_dtype, hints={(m, n): hint}).close()
    except MuonError as e:
        if e.status == MUON_ERR_UNSUPPORTED:
            return False
        raise
    return True


def device_name() -> str:
    import torch
    p = torch.cuda.get_device_properties(0)
    arch = getattr(p, "gcnArchName", "") or ""
    return f"{p.name} {arch.split(':')[0]}".strip()


def _inputs(m: int, n: int, count: int, grad_dtype: str, seed: int):
    """Seeded device inputs, matrix i drawn from its own generator, so the
    first matrix is the same for every count."""
    import torch
    dev = torch.device("cuda:0")
    gdt = torch.bfloat16 if grad_dtype == "bf16" else torch.float32
    W, M, G = [], [], []
    for i in range(count):
        gen = torch.Generator(device=dev)
        gen.manual_seed(seed * 1000003 + i)
        W.append(torch.randn(m, n, device=dev, generator=gen) * 0.02)
        M.append(torch.zeros(m, n, device=dev))
        G.append((torch.randn(m, n, device=dev, generator=gen) * 1e-3).to(gdt))
    return W, M, G


def time_bucket(m: int, n: int, count: int, grad_dtype: str, ns_dtype: str, hint: Optional[dict],
                steps: int = 3, warmup: int = 2, seed: int = 0):
    """Median ms of one muon_step_batched call over `count` m x n matrices
    planned with `hint` (None: the planner's own rule), and the direction
    output (fp32 m x n device tensor) of the first matrix from the first
    call."""
    import torch
    from ._lib import Plan
    dev = torch.device("cuda:0")
    plan = Plan([(m, n)] * count, grad_dtype, ns_dtype,
                hints={(m, n): hint} if hint else None)
    W, M, G = _inputs(m, n, count, grad_dtype, seed)
    O0 = torch.empty(m, n, device=dev)
    ws = torch.empty(max(plan.workspace_bytes, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    ptr = lambda L: [x.data_ptr() for x in L]
    Wp, Mp, Gp = ptr(W), ptr(M), ptr(G)
    Op = [O0.data_ptr()] + [0] * (count - 1)
    times = []
    for i in range(warmup + steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        plan.step_ptrs(Wp, Mp, Gp, 0.02, 0.1, ws.data_ptr(), ws.numel(), stream.cuda_stream,
                       Op if i == 0 else None)
        b.record(stream)
        b.synchronize()
        if i >= warmup:
            times.append(a.elapsed_time(b))
    plan.close()
    del W, M, G, ws
    times.sort()
    return float(times[len(times) // 2]), O0


def reference_direction(m: int, n: int, grad_dtype: str, seed: int = 0):
    """The fp32 path's direction for the first matrix of time_bucket's
    inputs (a single-matrix plan)."""
    import torch
    from ._lib import Plan
    plan = Plan([(m, n)], grad_dtype, "f32")
    W, M, G = _inputs(m, n, 1, grad_dtype, seed)
    O = torch.empty(m, n, device="cuda:0")
    ws = torch.empty(max(plan.workspace_bytes, 256), dtype=torch.uint8, device="cuda:0")
    plan.step_ptrs([W[0].data_ptr()], [M[0].data_ptr()], [G[0].data_ptr()], 0.02, 0.1,
                   ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream,
                   [O.data_ptr()])
    torch.cuda.synchronize()
    plan.close()
    return O


def _rel(a, b) -> float:
    nb = float(b.double().norm())
    return float((a.double() - b.double()).norm()) / nb if nb > 0 else float(a.double().norm())


def tune(shapes: Sequence[Sequence[int]], grad_dtype: str, ns_dtype: str,
         cache: Optional[dict] = None, device: Optional[str] = None, steps: int = 3,
         warmup: int = 2, timer: Optional[Callable] = None, log: Optional[Callable] = None) -> dict:
    """Time every candidate of each (shape, count) of `shapes` that `cache`
    does not hold yet, check its direction against the fp32 path's, and add
    the results.  `timer(m, n, count, hint)` replaces the device measurement
    (tests); it returns ms, or (ms, err) with err the candidate's relative
    error (None: not checked).  Returns the (updated) cache."""
    if cache is None:
        cache = {"version": CACHE_VERSION, "entries": {}}
    if device is None:
        device = device_name()
    tol = ACCURACY_TOL[ns_dtype]
    for (m, n), count in shape_counts(shapes).items():
        key = cache_key(device, grad_dtype, ns_dtype, m, n, count)
        if key in cache["entries"]:
            continue
        if timer is None:
            ref = reference_direction(m, n, grad_dtype)

            def measure(hint):
                ms, O0 = time_bucket(m, n, count, grad_dtype, ns_dtype, hint, steps, warmup)
                return ms, _rel(O0, ref)
        else:
            def measure(hint):
                out = timer(m, n, count, hint)
                return out if isinstance(out, tuple) else (out, None)
        default_ms, _ = measure(None)
        rows = []

        def trial(h):
            ms, err = measure(h)
            row = dict(h)
            row["ms"] = round(ms, 4)
            row["err"] = None if err is None else float(f"{err:.3e}")
            if err is not None and not err <= tol:
                row["rejected"] = True
            rows.append(row)
            if log:
                e = "-" if err is None else f"{err:.2e}"
                knobs = " ".join(f"{k}={h[k]}" for k, _ in KNOBS if h.get(k))
                log(f"{m}x{n} x{count}: tile {h['tile']:3d} {h['formulation']:6s} {knobs} "
                    f"{ms:9.3f} ms err {e}{' (rejected)' if row.get('rejected') else ''}")
            return row

        for h in candidates(m, n, ns_dtype):
            trial(h)
        ok = [e for e in rows if not e.get("rejected")]
        if not ok:
            raise RuntimeError(f"no setting of {m}x{n} x{count} meets the accuracy bound {tol}")
        best = min(ok, key=lambda e: e["ms"])
        if best["tile"] == 256:
            for knob, values in KNOBS:
                for v in values:
                    h = {k: best[k] for k in HINT_FIELDS if k in best}
                    h[knob] = v
                    if not _plannable(m, n, ns_dtype, h):
                        continue
                    row = trial(h)
                    if not row.get("rejected") and row["ms"] < best["ms"] * (1.0 - KNOB_GAIN):
                        best = row
        entry = {k: best[k] for k in HINT_FIELDS if k in best}
        entry.update({"ms": best["ms"], "default": round(default_ms, 4), "candidates": rows})
        cache["entries"][key] = entry
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
            hints[(m, n)] = {k: (e[k] if k == "formulation" else int(e[k]))
                             for k in HINT_FIELDS if k in e}
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
        knobs = " ".join(f"{k}={e[k]}" for k, _ in KNOBS if e.get(k))
        print(f"{m}x{n} x{count}: best tile {e['tile']} {e['formulation']} {knobs} {e['ms']:.3f} ms "
              f"(planner rule {e['default']:.3f} ms)")


if __name__ == "__main__":
    main()
