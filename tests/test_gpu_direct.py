"""GPU parity of the direct formulation (MUON_FORM_DIRECT: eq. (2) of
"Infra Optimizers" iterated on X itself, N times A = X X^T, P~ = b A + c A^2,
X <- a X + P~ X) against the float64 oracle's direct routine, through the C
ABI, on every tile width.  Same bars as the Gram path on the bf16-MFMA path: NS output <= 2e-2
relative Frobenius, the update epilogue <= 1e-5 against the oracle's update
applied to the GPU's own output, momentum <= 1e-6."""
import numpy as np
import pytest

from matrix_aware_optimizer_muon_amd.workloads import bf16_round
from oracle import muon_oracle as OR
from tests.gpu_common import rel, run
from tests.test_gpu_parity import LR, WD, check_ns, seeded

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")
    import matrix_aware_optimizer_muon_amd as pkg
    pkg.load()


@pytest.mark.parametrize("shape", [(1, 1), (5, 3), (3, 5), (200, 200), (256, 256), (130, 70),
                                   (515, 129), (129, 515), (1024, 1024), (600, 1000), (1000, 600)])
def test_direct_shapes(shape):
    W, M, G = seeded([shape], 7 + shape[0] * 3 + shape[1], mscale=1e-3)
    check_ns([shape], W, M, G, "bf16", label=f"direct {shape}", formulation="direct")


# Every tile width of the direct form: 64 and 128 (the small-tile kernel,
# whose X' epilogue reads the a X term from the X buffers) and 256 (the
# direct-to-LDS kernel, which takes it from its operand ring), wide and tall
# (the tall ones end in the X' product plus the weight-update pass), ragged r
# and c, and N = 1, 2, 5 (the last X lands in either buffer of the pair).
@pytest.mark.parametrize("tile", [64, 128, 256])
@pytest.mark.parametrize("steps", [1, 2, 5])
def test_direct_tile_widths(tile, steps):
    from matrix_aware_optimizer_muon_amd import default_hparams
    hp = default_hparams()
    hp.ns_steps = steps
    shapes = [(256, 256)] * 3 + [(300, 700), (700, 300), (190, 200)]
    hints = {s: {"tile": tile, "formulation": "direct"} for s in set(shapes)}
    W, M, G = seeded(shapes, 90 + tile + steps, mscale=1e-3)
    (Wg, Mg, Og), plan = run(shapes, W, M, G, LR, WD, "f32", "bf16", hp=hp, hints=hints)
    assert all(b["tile"] == tile and b["formulation"] == "direct" for b in plan.buckets())
    ohp = OR.Hyper(ns_steps=steps)
    for i, (m, n) in enumerate(shapes):
        Wo, Mo, Oo = OR.muon_step(W[i], M[i], G[i], LR, WD, hp=ohp, form="direct")
        e = rel(Og[i], Oo)
        assert e <= 2e-2, (tile, steps, shapes[i], e)
        assert rel(Mg[i], Mo) <= 1e-6
        W_epi = OR.apply_update(W[i], Og[i], LR, WD, OR.update_scale(m, n))
        assert rel(Wg[i], W_epi) <= 1e-5, (tile, steps, shapes[i])


# The one-launch direct form (padded squares of 128 or 256 on small tiles):
# both sizes, ragged extents inside the padding, N = 1, 2, 5 (the iterations
# alternate the X buffer pair), the update epilogue and the O output.
@pytest.mark.parametrize("steps", [1, 2, 5])
def test_fused_direct_form(steps):
    from matrix_aware_optimizer_muon_amd import default_hparams
    hp = default_hparams()
    hp.ns_steps = steps
    shapes = [(256, 256)] * 3 + [(250, 256), (120, 128), (128, 128), (100, 110)]
    W, M, G = seeded(shapes, 140 + steps, mscale=1e-3)
    (Wg, Mg, Og), plan = run(shapes, W, M, G, LR, WD, "f32", "bf16", hp=hp)
    assert all(b["formulation"] == "direct" and b["fused"] for b in plan.buckets()), plan.buckets()
    ohp = OR.Hyper(ns_steps=steps)
    for i, (m, n) in enumerate(shapes):
        Wo, Mo, Oo = OR.muon_step(W[i], M[i], G[i], LR, WD, hp=ohp, form="direct")
        e = rel(Og[i], Oo)
        assert e <= 2e-2, (steps, shapes[i], e)
        assert rel(Mg[i], Mo) <= 1e-6
        W_epi = OR.apply_update(W[i], Og[i], LR, WD, OR.update_scale(m, n))
        assert rel(Wg[i], W_epi) <= 1e-5, (steps, shapes[i])


def test_fused_direct_is_deterministic_and_matches_the_launch_sequence():
    # same inputs twice: bit-identical; against the same products launched
    # one by one on 256-wide tiles (hint), close to the products' rounding
    shapes = [(256, 256)] * 4
    W, M, G = seeded(shapes, 151, mscale=1e-3)
    (W1, _, O1), p1 = run(shapes, W, M, G, LR, WD)
    (W2, _, O2), _ = run(shapes, W, M, G, LR, WD)
    (_, _, O3), p3 = run(shapes, W, M, G, LR, WD, hints={(256, 256): {"tile": 256}})
    assert p1.buckets()[0]["fused"] and not p3.buckets()[0]["fused"]
    for i in range(len(shapes)):
        assert np.array_equal(W1[i], W2[i]) and np.array_equal(O1[i], O2[i])
        assert rel(O1[i], O3[i]) <= 5e-3, rel(O1[i], O3[i])


def test_direct_small_tiles_match_large_tiles_closely():
    # the same iteration on the two kernels: both within the bar of the
    # oracle and close to each other (the a X term and A's b-term differ in
    # rounding only: fp32 A and X read back from fp16 here, fp16 A there)
    shapes = [(256, 256)] * 4
    W, M, G = seeded(shapes, 123, mscale=1e-3)
    outs = {}
    for tile in (64, 256):
        (_, _, O), _ = run(shapes, W, M, G, LR, WD, hints={(256, 256): {"tile": tile}})
        outs[tile] = O
    for i in range(len(shapes)):
        assert rel(outs[64][i], outs[256][i]) <= 1e-2


def test_direct_several_buckets_bf16_grads():
    shapes = [(256, 256)] * 5 + [(384, 1280), (1280, 384)] * 2 + [(1000, 1000)]
    W, M, G = seeded(shapes, 11, mscale=1e-3)
    G = [bf16_round(g) for g in G]
    check_ns(shapes, W, M, G, "bf16", grad_dtype="bf16", label="direct buckets",
             formulation="direct")


@pytest.mark.parametrize("steps", [1, 2, 5])
def test_direct_iteration_counts(steps):
    # odd and even N end in different X buffers of the double-buffered pair
    from matrix_aware_optimizer_muon_amd import default_hparams
    hp = default_hparams()
    hp.ns_steps = steps
    shapes = [(300, 700), (700, 300)]
    W, M, G = seeded(shapes, 20 + steps, mscale=1e-3)
    (Wg, Mg, Og), _ = run(shapes, W, M, G, LR, WD, "f32", "bf16", hp=hp, formulation="direct")
    ohp = OR.Hyper(ns_steps=steps)
    for i, (m, n) in enumerate(shapes):
        Wo, Mo, Oo = OR.muon_step(W[i], M[i], G[i], LR, WD, hp=ohp, form="direct")
        assert rel(Og[i], Oo) <= 2e-2, (steps, i, rel(Og[i], Oo))
        assert rel(Mg[i], Mo) <= 1e-6


def test_direct_is_deterministic_and_close_to_gram():
    # (the Gram form is refused on near-square buckets of the 16-bit path)
    shapes = [(512, 640), (768, 1536)]
    W, M, G = seeded(shapes, 31, mscale=1e-3)
    (W1, _, O1), _ = run(shapes, W, M, G, LR, WD, formulation="direct")
    (W2, _, O2), _ = run(shapes, W, M, G, LR, WD, formulation="direct")
    (_, _, Og), _ = run(shapes, W, M, G, LR, WD, formulation="gram")
    for i in range(len(shapes)):
        assert np.array_equal(W1[i], W2[i]) and np.array_equal(O1[i], O2[i])
        # both formulations are within 2e-2 of the same exact result
        assert rel(O1[i], Og[i]) <= 4e-2


def test_direct_full_size_square_pair():
    # two 3584^2 matrices (the q / o projections of the Qwen2.5-7B layer)
    shapes = [(3584, 3584)] * 2
    W, M, G = seeded(shapes, 41)
    check_ns(shapes, W, M, G, "bf16", label="direct 3584^2", formulation="direct")
