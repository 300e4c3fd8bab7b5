"""Buckets that are each too small to fill the GPU run concurrently on the
plan's internal streams, each with its own scratch region.  The kernels and
their inputs are the same as when every bucket is planned alone, so the
results must be bit-identical to running the buckets one plan at a time;
they are also held to the usual parity bars against the oracle."""
import numpy as np
import pytest

from tests.gpu_common import run
from tests.test_gpu_parity import LR, WD, check_ns, seeded

pytestmark = pytest.mark.gpu

SHAPES = [(640, 640)] * 2 + [(512, 1536)] * 2 + [(1536, 512)] + [(300, 700)] * 3 + [(96, 2000)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")
    import matrix_aware_optimizer_muon_amd as pkg
    pkg.load()


@pytest.mark.parametrize("grad_dtype", ["f32", "bf16"])
def test_concurrent_buckets_match_one_plan_per_bucket(grad_dtype):
    from matrix_aware_optimizer_muon_amd.workloads import bf16_round
    W, M, G = seeded(SHAPES, 91, mscale=1e-3)
    if grad_dtype == "bf16":
        G = [bf16_round(g) for g in G]
    (Wc, Mc, Oc), plan = run(SHAPES, W, M, G, LR, WD, grad_dtype, "bf16")
    assert len(plan.buckets()) == 5
    for shape in dict.fromkeys(SHAPES):
        idx = [i for i, s in enumerate(SHAPES) if s == shape]
        (Ws, Ms, Os), _ = run([shape] * len(idx), [W[i] for i in idx], [M[i] for i in idx],
                              [G[i] for i in idx], LR, WD, grad_dtype, "bf16")
        for k, i in enumerate(idx):
            assert np.array_equal(Wc[i], Ws[k]), (shape, i)
            assert np.array_equal(Mc[i], Ms[k]), (shape, i)
            assert np.array_equal(Oc[i], Os[k]), (shape, i)


def test_concurrent_buckets_parity_and_repeatability():
    W, M, G = seeded(SHAPES, 92, mscale=1e-3)
    check_ns(SHAPES, W, M, G, "bf16", label="concurrent buckets")
    (W1, _, O1), _ = run(SHAPES, W, M, G, LR, WD, "f32", "bf16")
    (W2, _, O2), _ = run(SHAPES, W, M, G, LR, WD, "f32", "bf16")
    for a, b in zip(O1 + W1, O2 + W2):
        assert np.array_equal(a, b)


def test_cap_fallback_matches_concurrent_run():
    from matrix_aware_optimizer_muon_amd import Plan
    each = max(Plan([s] * SHAPES.count(s)).workspace_bytes for s in dict.fromkeys(SHAPES))
    W, M, G = seeded(SHAPES, 93, mscale=1e-3)
    (Wc, Mc, Oc), pc = run(SHAPES, W, M, G, LR, WD, "f32", "bf16")
    (Ws, Ms, Os), ps = run(SHAPES, W, M, G, LR, WD, "f32", "bf16", max_ws=each)
    assert ps.workspace_bytes < pc.workspace_bytes
    for a, b in zip(Wc + Mc + Oc, Ws + Ms + Os):
        assert np.array_equal(a, b)
