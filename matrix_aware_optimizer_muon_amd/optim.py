"""Torch-facing wrapper over the C ABI: owns the plan, the momentum buffers
and the workspace, and passes tensor pointers and the current stream.

Periodic RowNorm Muon ("Scaling Muon for Diffusion Transformers", abstract):
with refresh_period K > 0, step t runs the Newton-Schulz refresh when
t mod K == 0 and the RowNorm step otherwise; K = 0 refreshes every step.
"""
from __future__ import annotations

from typing import List, Optional, Sequence

import torch

from ._lib import Hparams, Plan


class MuonMI355X:
    def __init__(self, params: Sequence[torch.Tensor], grad_dtype: str = "f32",
                 ns_dtype: str = "bf16", hp: Optional[Hparams] = None,
                 max_workspace_bytes: int = 0, refresh_period: int = 0):
        self.params = list(params)
        for p in self.params:
            if p.dim() != 2 or p.dtype != torch.float32 or not p.is_cuda or not p.is_contiguous():
                raise ValueError("parameters must be contiguous 2-D fp32 CUDA tensors")
        self.plan = Plan([tuple(p.shape) for p in self.params], grad_dtype, ns_dtype, hp,
                         max_workspace_bytes)
        dev = self.params[0].device
        self.momentum = [torch.zeros_like(p) for p in self.params]
        self.workspace = torch.empty(max(self.plan.workspace_bytes, 256), dtype=torch.uint8,
                                     device=dev)
        self.grad_dtype = torch.bfloat16 if grad_dtype == "bf16" else torch.float32
        self.refresh_period = int(refresh_period)
        self.t = 0

    def _check(self, grads):
        if len(grads) != len(self.params):
            raise ValueError("one gradient per parameter")
        for g, p in zip(grads, self.params):
            if g.shape != p.shape or g.dtype != self.grad_dtype or not g.is_contiguous():
                raise ValueError("gradient shape/dtype/layout does not match the plan")

    def step(self, grads: Sequence[torch.Tensor], lr: float, weight_decay: float,
             refresh: Optional[bool] = None, out: Optional[List[torch.Tensor]] = None):
        self._check(grads)
        if refresh is None:
            refresh = self.refresh_period <= 0 or self.t % self.refresh_period == 0
        stream = torch.cuda.current_stream(self.params[0].device).cuda_stream
        args = ([p.data_ptr() for p in self.params], [m.data_ptr() for m in self.momentum],
                [g.data_ptr() for g in grads], lr, weight_decay, self.workspace.data_ptr(),
                self.workspace.numel(), stream,
                [o.data_ptr() for o in out] if out is not None else None)
        if refresh:
            self.plan.step_ptrs(*args)
        else:
            self.plan.rownorm_ptrs(*args)
        self.t += 1
