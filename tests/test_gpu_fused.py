"""The fused r x r recursion (one launch per bucket, r_pad <= 128 on the
16-bit path) against the float64 oracle, for several iteration counts (the
last Q lands in either buffer of the pair), both orientations and both
padded sizes (64, 128), plus determinism (two runs are bit-identical)."""
import numpy as np
import pytest

from oracle import muon_oracle as OR
from tests.gpu_common import rel, run
from tests.test_gpu_parity import LR, WD, seeded

pytestmark = pytest.mark.gpu

# Clearly rectangular only: near-square buckets (c <= 1.125 r) take the
# direct form, and the planner refuses the Gram form there on the 16-bit path
# (on a small square it misses the 2e-2 bar: 64 x 64, N = 5, 2.5e-2).
SHAPES = [(100, 900), (900, 100), (128, 3584), (40, 300), (64, 200)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")
    import matrix_aware_optimizer_muon_amd as pkg
    pkg.load()


@pytest.mark.parametrize("steps", [1, 2, 3, 5])
def test_fused_recursion_iteration_counts(steps):
    from matrix_aware_optimizer_muon_amd import default_hparams
    hp = default_hparams()
    hp.ns_steps = steps
    W, M, G = seeded(SHAPES, 50 + steps, mscale=1e-3)
    (Wg, Mg, Og), plan = run(SHAPES, W, M, G, LR, WD, "f32", "bf16", hp=hp, formulation="gram")
    assert all(b["formulation"] == "gram" and b["tile"] < 256 for b in plan.buckets())
    ohp = OR.Hyper(ns_steps=steps)
    for i, (m, n) in enumerate(SHAPES):
        Wo, Mo, Oo = OR.muon_step(W[i], M[i], G[i], LR, WD, hp=ohp, form="direct")
        assert rel(Og[i], Oo) <= 2e-2, (steps, (m, n), rel(Og[i], Oo))
        assert rel(Mg[i], Mo) <= 1e-6


def test_fused_recursion_is_deterministic():
    W, M, G = seeded(SHAPES, 61, mscale=1e-3)
    (W1, M1, O1), _ = run(SHAPES, W, M, G, LR, WD, "f32", "bf16", formulation="gram")
    (W2, M2, O2), _ = run(SHAPES, W, M, G, LR, WD, "f32", "bf16", formulation="gram")
    for i in range(len(SHAPES)):
        assert np.array_equal(W1[i], W2[i]) and np.array_equal(O1[i], O2[i])
