"""Helpers shared by the GPU parity tests: move seeded host inputs to the
device, call the C ABI through the binding, and compare with the oracle."""
from __future__ import annotations

import numpy as np

from matrix_aware_optimizer_muon_amd import Plan


def rel(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    if nb == 0.0:
        return float(np.linalg.norm(a))
    return float(np.linalg.norm(a - b) / nb)


def to_dev(x, dtype="f32"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def run(shapes, W, M, G, lr, wd, grad_dtype="f32", ns_dtype="bf16", hp=None, rownorm=False,
        max_ws=0, want_out=True, plan=None, steps_grads=None, formulation="auto", hints=None):
    """One call of muon_step_batched (or rownorm_step) on fresh device copies.
    Returns host arrays (W', M', O) and the plan."""
    import torch
    if plan is None:
        plan = Plan(shapes, grad_dtype, ns_dtype, hp, max_ws, formulation=formulation, hints=hints)
    Wd = [to_dev(w) for w in W]
    Md = [to_dev(m) for m in M]
    Gd = [to_dev(g, grad_dtype) for g in G]
    Od = [torch.full_like(w, float("nan")) for w in Wd] if want_out else None
    ws = torch.empty(max(plan.workspace_bytes, 256), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    fn = plan.rownorm_ptrs if rownorm else plan.step_ptrs
    fn([w.data_ptr() for w in Wd], [m.data_ptr() for m in Md], [g.data_ptr() for g in Gd], lr, wd,
       ws.data_ptr(), ws.numel(), stream, [o.data_ptr() for o in Od] if want_out else None)
    torch.cuda.synchronize()
    out = ([w.cpu().numpy() for w in Wd], [m.cpu().numpy() for m in Md],
           [o.cpu().numpy() for o in Od] if want_out else None)
    return out, plan
