"""Host-side checks of bench.py (CPU, no kernel launch).

The algorithmic flop totals below were worked out by hand for each matrix
set from the step's operation counts (Gram form: the lower-triangle SYRK
r^2 c, 21 r x r products of r^3 for five quintic iterations when P^2 and
G P^2 are formed separately, the final product 2 r^2 c; direct form, five
times: SYRK r^2 c, A^2 r^3, X update 2 r^2 c), rounded as printed.  They pin
the flop model behind the reported TFLOP/s: a wrong exponent, a dropped
term or the wrong formulation rule moves at least one of them.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from matrix_aware_optimizer_muon_amd import workloads as WL  # noqa: E402

# (workload, AUTO total, all-Gram total) in flops, 21 r^3 count
HAND_TOTALS = [
    (1, 0.554e9, 0.554e9),      # 256x1024: 3*256^2*1024 + 21*256^3
    (2, 46.1e9, 50.4e9),        # 112 x 128x3584 (Gram) + 64 x 256^2 (direct: 20*256^3)
    (3, 6.943e12, 7.311e12),    # one Qwen2.5-7B layer, squares in the direct form
    (4, 194.4e12, 204.7e12),    # 28 layers
    (5, 401.3e12, 445.3e12),    # DiT refresh step: 160 x 4096^2, 40 + 40 x 16384x4096
]


@pytest.mark.parametrize("k,auto,gram", HAND_TOTALS)
def test_flop_model_matches_hand_totals(k, auto, gram):
    shapes = WL.config(k).shapes
    for form, want in (("auto", auto), ("gram", gram)):
        got = bench.ns_flops(shapes, form, rr_products=21)
        assert abs(got - want) <= 1e-3 * want, (k, form, got, want)


def test_seventeen_product_count_is_four_fewer_r3_per_matrix():
    # the library's recursion saves 4 r^3 per Gram-form matrix; the direct
    # form does not depend on the count
    for m, n in [(256, 1024), (3584, 18944), (18944, 3584), (512, 3584)]:
        r = min(m, n)
        d = bench.ns_flops([(m, n)], "gram", 21) - bench.ns_flops([(m, n)], "gram", 17)
        assert d == 4.0 * r ** 3
    assert bench.ns_flops([(3584, 3584)], "direct", 21) == bench.ns_flops([(3584, 3584)], "direct", 17)


def test_auto_takes_the_direct_form_up_to_nine_eighths():
    # c <= 1.125 r: direct; beyond: Gram (the planner's rule on the 16-bit path)
    r = 1024
    for m, n in [(r, 1152), (1152, r)]:
        assert bench.ns_flops([(m, n)], "auto") == bench.ns_flops([(m, n)], "direct")
    for m, n in [(r, 1153), (1153, r)]:
        assert bench.ns_flops([(m, n)], "auto") == bench.ns_flops([(m, n)], "gram")
    assert bench.ns_flops([(r, 1153)], "gram") != bench.ns_flops([(r, 1153)], "direct")


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr
    assert p.stdout == ""


def test_roofline_entry_arithmetic():
    # four launches of the final product: 1e14 flops in 100 ms -> 1000
    # TFLOP/s, 0.4 of the 2.5 PFLOP/s 16-bit peak; prep is the HBM class
    kt = {"final": {"ms": 100.0, "launches": 4, "flops": 1e14, "bytes": 8e10},
          "prep": {"ms": 20.0, "launches": 4, "flops": 0.0, "bytes": 1.2e11},
          "syrk": {"ms": 30.0, "launches": 2, "flops": 2e13, "bytes": 1e9}}
    r = bench.roofline_of(kt, "bf16", {"final": (3e10, 1e10)})
    assert (r["bound"], r["kernel"], r["unit"], r["peak"]) == ("mfma", "final", "TFLOP/s", 2500.0)
    assert r["achieved"] == 1000.0 and r["frac"] == 0.4
    assert r["ms_per_launch"] == 25.0 and r["share_of_step"] == round(100 / 150, 3)
    assert r["algorithmic_flops_per_launch"] == 2.5e13 and r["algorithmic_bytes_per_launch"] == 2e10
    assert r["traffic"] == 4e10
    # the fp32 path prices against the fp32 matrix peak
    r32 = bench.roofline_of(kt, "f32", {})
    assert r32["peak"] == 157.3 and r32["frac"] == round(1000.0 / 157.3, 4) and r32["traffic"] is None
    # restricted to the memory-bound classes: 1.2e11 B in 20 ms = 6000 GB/s
    h = bench.roofline_of(kt, "bf16", {}, classes=bench.HBM_CLASSES)
    assert (h["bound"], h["kernel"], h["unit"], h["peak"]) == ("hbm", "prep", "GB/s", 8000.0)
    assert h["achieved"] == 6000.0 and h["frac"] == 0.75
    assert bench.roofline_of(kt, "bf16", {}, classes=("rownorm",)) is None
