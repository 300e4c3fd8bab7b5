"""Host logic of the shape-adaptive tuner (tune.py): candidate lists, the
JSON cache, the choice of the fastest setting and the hints it yields.  The
device timing is replaced by a table here; the GPU tests time for real."""
import json

import pytest

from matrix_aware_optimizer_muon_amd import _lib as L
from matrix_aware_optimizer_muon_amd import tune as TU

DEV = "test-device gfx950"


def test_shape_counts_keep_first_appearance_order():
    sc = TU.shape_counts([(3, 5), (5, 3), (3, 5), (7, 7), (3, 5)])
    assert list(sc.items()) == [((3, 5), 3), ((5, 3), 1), ((7, 7), 1)]


def test_candidates_are_plannable():
    for ns in ("bf16", "f32"):
        for shape in [(64, 64), (300, 700), (1000, 1000), (3584, 18944), (18944, 3584)]:
            cands = TU.candidates(*shape, ns)
            assert cands and len({(c["tile"], c["formulation"]) for c in cands}) == len(cands)
            for c in cands:
                b = L.Plan([shape], "f32", ns, hints={shape: c}).buckets()[0]
                assert (b["tile"], b["formulation"]) == (c["tile"], c["formulation"])
    assert {c["formulation"] for c in TU.candidates(300, 700, "f32")} == {"gram"}
    # near-square buckets of the 16-bit path: the planner refuses the Gram form
    assert TU.candidates(3584, 3584, "bf16") == [{"tile": 256, "formulation": "direct"}]
    assert TU.candidates(64, 70, "bf16") == [{"tile": t, "formulation": "direct"} for t in (64, 128, 256)]
    assert {c["tile"] for c in TU.candidates(3584, 3584, "f32")} == {64, 128}
    assert 64 in {c["tile"] for c in TU.candidates(1024, 4096, "bf16")}


def test_tune_never_picks_an_inaccurate_setting():
    # the fastest candidate misses the accuracy bound: recorded, not chosen
    table = {(None, None): (10.0, 3e-3), (64, "gram"): (1.0, 5e-2), (128, "gram"): (7.5, 4e-3),
             (256, "gram"): (9.0, 4e-3), (256, "direct"): (8.0, 3e-3), (64, "direct"): (9.5, 3e-3),
             (128, "direct"): (9.9, 3e-3)}
    timer = lambda m, n, c, h: table[(None, None) if h is None else (h["tile"], h["formulation"])]
    cache = TU.tune([(512, 2048)], "bf16", "bf16", device=DEV, timer=timer)
    e = cache["entries"][TU.cache_key(DEV, "bf16", "bf16", 512, 2048, 1)]
    assert (e["tile"], e["formulation"], e["ms"]) == (128, "gram", 7.5)
    rej = [c for c in e["candidates"] if c.get("rejected")]
    assert [(c["tile"], c["formulation"], c["err"]) for c in rej] == [(64, "gram", 5e-2)]
    # no candidate within the bound: an error, not a silent choice
    bad = lambda m, n, c, h: (1.0, 1.0)
    with pytest.raises(RuntimeError):
        TU.tune([(512, 2048)], "bf16", "bf16", device=DEV, timer=bad)


def test_tune_picks_the_fastest_and_skips_cached_shapes():
    table = {(None, None): 10.0, (64, "gram"): 12.0, (128, "gram"): 7.5,
             (256, "gram"): 9.0, (256, "direct"): 8.0, (64, "direct"): 11.0, (128, "direct"): 11.5}
    calls = []

    def timer(m, n, count, hint):
        calls.append((m, n, count, None if hint is None else (hint["tile"], hint["formulation"])))
        key = (None, None) if hint is None else (hint["tile"], hint["formulation"])
        return table[key] * count

    shapes = [(512, 2048)] * 3 + [(2048, 512)]
    cache = TU.tune(shapes, "bf16", "bf16", device=DEV, timer=timer)
    e = cache["entries"][TU.cache_key(DEV, "bf16", "bf16", 512, 2048, 3)]
    assert (e["tile"], e["formulation"], e["ms"], e["default"]) == (128, "gram", 22.5, 30.0)
    assert len(e["candidates"]) == len(TU.candidates(512, 2048, "bf16"))
    assert TU.cache_key(DEV, "bf16", "bf16", 2048, 512, 1) in cache["entries"]
    n_calls = len(calls)
    TU.tune(shapes, "bf16", "bf16", cache, device=DEV, timer=timer)
    assert len(calls) == n_calls                       # everything cached
    hints = TU.hints_for(shapes + [(9, 9)], "bf16", "bf16", cache, device=DEV)
    assert hints == {(512, 2048): {"tile": 128, "formulation": "gram"},
                     (2048, 512): {"tile": 128, "formulation": "gram"}}
    # another count of the same shape is another bucket: not covered
    assert TU.hints_for([(512, 2048)], "bf16", "bf16", cache, device=DEV) == {}
    # other dtypes or devices do not match
    assert TU.hints_for(shapes, "f32", "bf16", cache, device=DEV) == {}
    assert TU.hints_for(shapes, "bf16", "bf16", cache, device="other") == {}
    # the hints plan
    L.Plan(shapes, "bf16", "bf16", hints=hints)


def test_cache_round_trip_and_versions(tmp_path):
    path = str(tmp_path / "sub" / "tune.json")
    assert TU.load_cache(path) == {"version": TU.CACHE_VERSION, "entries": {}}
    cache = TU.tune([(64, 256)], "f32", "f32", device=DEV, timer=lambda m, n, c, h: 1.0 if h is None else h["tile"] / 64)
    TU.save_cache(path, cache)
    again = TU.load_cache(path)
    assert again == json.loads(json.dumps(cache))
    assert again["entries"][TU.cache_key(DEV, "f32", "f32", 64, 256, 1)]["tile"] == 64
    with open(path, "w") as f:
        json.dump({"version": 999, "entries": {"x": 1}}, f)
    assert TU.load_cache(path)["entries"] == {}


def test_default_cache_path_honours_the_environment(monkeypatch, tmp_path):
    monkeypatch.setenv("MUON_TUNE_CACHE", str(tmp_path / "c.json"))
    assert TU.default_cache_path() == str(tmp_path / "c.json")
    monkeypatch.delenv("MUON_TUNE_CACHE")
    monkeypatch.setenv("XDG_CACHE_HOME", str(tmp_path))
    assert TU.default_cache_path().startswith(str(tmp_path))


def test_shipped_cache_entries_are_plannable():
    cache = TU.load_cache(TU.SHIPPED_CACHE)
    for key, e in cache["entries"].items():
        dev, g, ns, shape = key.split("|")
        m, n, count = (int(x) for x in shape.split("x"))
        b = L.Plan([(m, n)] * count, g[2:], ns[3:],
                   hints={(m, n): {"tile": e["tile"], "formulation": e["formulation"]}}).buckets()[0]
        assert (b["tile"], b["formulation"]) == (e["tile"], e["formulation"]), key
        assert e["ms"] == min(c["ms"] for c in e["candidates"] if not c.get("rejected")) or \
            any(c.get(k) for c in e["candidates"] for k, _ in TU.KNOBS), key


def test_knob_search_on_the_256_wide_kernels():
    # the fastest tile / form runs on the 256-wide kernels: each knob value is
    # tried from it, one knob at a time, and kept only when >1 % faster
    base = {(128, "gram"): 10.0, (256, "gram"): 8.0, (256, "direct"): 20.0}
    knob = {("group", 2): 8.5, ("group", 4): 7.0, ("group", 16): 7.95, ("xcd_chunk", -1): 6.0,
            ("xcd_chunk", 16): 6.99, ("xcd_chunk", 64): 6.5, ("xcd_chunk", 256): 7.5,
            ("waves", 4): 5.96}
    seen = []

    def timer(m, n, count, h):
        if h is None:
            return 9.0, 1e-3
        seen.append(dict(h))
        k = [(f, h[f]) for f, _ in TU.KNOBS if h.get(f)]
        if not k:
            return base[(h["tile"], h["formulation"])], 1e-3
        return knob[k[-1]], 1e-3

    cache = TU.tune([(3584, 18944)], "bf16", "bf16", device=DEV, timer=timer)
    e = cache["entries"][TU.cache_key(DEV, "bf16", "bf16", 3584, 18944, 1)]
    # group 4 (7.0) beats 8.0; xcd_chunk -1 (6.0) beats 7.0; waves 4 (5.96) is
    # within 1 % of 6.0 and is not taken
    assert (e["tile"], e["group"], e["xcd_chunk"], e.get("waves", 0), e["ms"]) == (256, 4, -1, 0, 6.0)
    hints = TU.hints_for([(3584, 18944)], "bf16", "bf16", cache, device=DEV)
    assert hints == {(3584, 18944): {"tile": 256, "formulation": "gram", "group": 4, "xcd_chunk": -1}}
    L.Plan([(3584, 18944)], "bf16", "bf16", hints=hints)
    # no knob is tried on a small-tile winner
    seen.clear()
    TU.tune([(128, 3584)], "bf16", "bf16", device=DEV,
            timer=lambda m, n, c, h: (1.0 if h and h["tile"] == 64 else 2.0, 1e-3))
