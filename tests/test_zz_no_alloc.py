"""The allocation-free entry point (muon_step_batched_noalloc) against the
workspace entry point (muon_step_batched), through the C ABI: two calls in a
row on the library's per-GPU scratch, the second with a smaller matrix set,
each compared element by element with the workspace call on the same
inputs; a plan too large for the scratch is refused before anything runs."""
import numpy as np
import pytest

from tests.gpu_common import rel, to_dev

pytestmark = pytest.mark.gpu

LR, WD = 0.02, 0.1


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")
    import matrix_aware_optimizer_muon_amd as pkg
    pkg.load()


def _inputs(shapes, seed):
    rng = np.random.default_rng(seed)
    W = [(rng.standard_normal(s) * 0.02).astype(np.float32) for s in shapes]
    M = [(rng.standard_normal(s) * 1e-3).astype(np.float32) for s in shapes]
    G = [(rng.standard_normal(s) * 1e-3).astype(np.float32) for s in shapes]
    return W, M, G


def _both(shapes, ns_dtype, seed, cap):
    import torch
    from matrix_aware_optimizer_muon_amd import Plan
    plan = Plan(shapes, "f32", ns_dtype, max_workspace_bytes=cap)
    W, M, G = _inputs(shapes, seed)
    st = torch.cuda.current_stream().cuda_stream
    ptr = lambda L: [x.data_ptr() for x in L]
    out = {}
    for mode in ("noalloc", "workspace"):
        Wd, Md, Gd = [to_dev(x) for x in W], [to_dev(x) for x in M], [to_dev(x) for x in G]
        Od = [torch.full_like(x, float("nan")) for x in Wd]
        if mode == "noalloc":
            plan.step_noalloc_ptrs(ptr(Wd), ptr(Md), ptr(Gd), LR, WD, st, ptr(Od))
        else:
            ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device="cuda")
            plan.step_ptrs(ptr(Wd), ptr(Md), ptr(Gd), LR, WD, ws.data_ptr(), ws.numel(), st, ptr(Od))
        torch.cuda.synchronize()
        out[mode] = [[x.cpu().numpy() for x in L] for L in (Wd, Md, Od)]
    a, b = out["noalloc"], out["workspace"]
    bitwise = all(np.array_equal(x, y) for La, Lb in zip(a, b) for x, y in zip(La, Lb))
    for i, s in enumerate(shapes):
        assert np.isfinite(a[2][i]).all(), s
        for k, name in enumerate(("W", "M", "O")):
            assert rel(a[k][i], b[k][i]) <= 1e-6, (name, s, rel(a[k][i], b[k][i]))
    print(f"noalloc {ns_dtype} {len(shapes)} matrices: bitwise {bitwise}", flush=True)
    return plan


@pytest.mark.parametrize("ns_dtype", ["bf16", "f32"])
def test_noalloc_matches_workspace_entry_two_calls(ns_dtype):
    # first call: several buckets (both orientations, a square taking the
    # direct form on the 16-bit path, a 3584-wide bucket chunked to fit);
    # second call: a smaller set on the same scratch
    big = [(256, 1024)] * 3 + [(1024, 256)] * 2 + [(300, 300)] + [(128, 3584)] * 24 + [(640, 1536)]
    small = [(64, 200)] * 2 + [(100, 100)]
    cap = 40 << 20
    p1 = _both(big, ns_dtype, 1, cap)
    assert p1.info()[1] > p1.info()[0]  # the cap split a bucket into chunks
    _both(small, ns_dtype, 2, cap)


def test_noalloc_refuses_a_plan_beyond_its_scratch():
    import torch
    from matrix_aware_optimizer_muon_amd import MuonError, Plan
    from matrix_aware_optimizer_muon_amd._lib import MUON_ERR_WORKSPACE_TOO_SMALL
    shapes = [(4096, 4096)]  # one matrix needs ~200 MB of scratch
    plan = Plan(shapes, "f32", "bf16")
    W = torch.randn(4096, 4096, device="cuda")
    W0 = W.clone()
    M = torch.zeros_like(W)
    G = torch.randn_like(W)
    with pytest.raises(MuonError) as e:
        plan.step_noalloc_ptrs([W.data_ptr()], [M.data_ptr()], [G.data_ptr()], LR, WD,
                               torch.cuda.current_stream().cuda_stream)
    assert e.value.status == MUON_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert torch.equal(W, W0) and torch.count_nonzero(M) == 0
