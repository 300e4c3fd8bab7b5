"""Synthetic, seeded workloads shaped like the pages' models.

Shapes follow Qwen2.5-7B (hidden 3584, MLP 18944, 512-wide K/V projections,
per-KV-head 128 x 3584 splits) and a DiT with hidden 4096 and MLP 16384.
Values: weights N(0, 0.02^2), gradients N(0, 1e-3^2) (config 4 adds a
per-layer scale drawn log-uniform in [0.1, 10]), momentum zero unless a
config asks for prior steps.  No trained weights or datasets are involved:
an optimizer step's cost depends only on the shapes.

This module draws random numbers and casts them to their storage type; it
holds none of the optimizer's arithmetic.  Both the GPU path and the CPU
oracle consume what it produces.
"""
from __future__ import annotations

import dataclasses
from typing import List, Tuple

import numpy as np

HIDDEN_QWEN, MLP_QWEN, KV_QWEN = 3584, 18944, 512
HIDDEN_DIT, MLP_DIT = 4096, 16384

W_STD, G_STD = 0.02, 1e-3
KIND = {"W": 0, "G": 1, "M": 2, "scale": 3}


@dataclasses.dataclass
class Workload:
    name: str
    shapes: List[Tuple[int, int]]
    grad_dtype: str = "f32"           # storage type of G
    ns_dtype: str = "bf16"            # Newton-Schulz path
    lr: float = 0.02
    wd: float = 0.1
    seed: int = 0
    prior_steps: int = 0              # momentum built from this many seeded gradients
    layer_of: List[int] = dataclasses.field(default_factory=list)  # config 4 scale groups
    grad_layer_scale: bool = False
    refresh_period: int = 0           # periodic RowNorm: K (0 = every step refreshes)
    steps: int = 1

    def numel(self) -> int:
        return sum(m * n for m, n in self.shapes)


def qwen_layer() -> List[Tuple[int, int]]:
    h, f, kv = HIDDEN_QWEN, MLP_QWEN, KV_QWEN
    return [(h, h), (kv, h), (kv, h), (h, h), (f, h), (f, h), (h, f)]  # q k v o gate up down


def config(k: int) -> Workload:
    """The five configurations (1-based)."""
    if k == 1:
        return Workload("single-256x1024-fp32", [(256, 1024)], ns_dtype="f32", seed=0)
    if k == 2:
        shapes = [(128, HIDDEN_QWEN)] * 112 + [(256, 256)] * 64
        return Workload("batched-small-112x128x3584+64x256x256", shapes, seed=1, prior_steps=3)
    if k == 3:
        return Workload("qwen2.5-7b-one-layer", qwen_layer(), seed=2)
    if k == 4:
        shapes, layer_of = [], []
        for layer in range(28):
            for s in qwen_layer():
                shapes.append(s)
                layer_of.append(layer)
        return Workload("qwen2.5-7b-28-layers-bf16-grad", shapes, grad_dtype="bf16", seed=3,
                        layer_of=layer_of, grad_layer_scale=True, steps=20)
    if k == 5:
        d, f = HIDDEN_DIT, MLP_DIT
        shapes = []
        for _ in range(40):
            shapes += [(d, d)] * 4 + [(f, d), (d, f)]
        return Workload("dit-40-blocks-h4096-periodic-rownorm", shapes, seed=4, refresh_period=5,
                        steps=5)
    raise ValueError(k)


def _rng(seed: int, idx: int, kind: str, step: int) -> np.random.Generator:
    return np.random.default_rng([seed, idx, KIND[kind], step])


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bfloat16 (ties to even), returned as float32 values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32)


def layer_scale(w: Workload, layer: int) -> float:
    return float(10.0 ** _rng(w.seed, layer, "scale", 0).uniform(-1.0, 1.0))


def host_weight(w: Workload, i: int) -> np.ndarray:
    m, n = w.shapes[i]
    return (_rng(w.seed, i, "W", 0).standard_normal((m, n), dtype=np.float32) * W_STD).astype(np.float32)


def host_grad(w: Workload, i: int, step: int = 0) -> np.ndarray:
    """Gradient of matrix i at `step` (negative steps are the prior steps of
    a config that starts from accumulated momentum), in its storage values."""
    m, n = w.shapes[i]
    g = _rng(w.seed, i, "G", step + 1000).standard_normal((m, n), dtype=np.float32) * G_STD
    if w.grad_layer_scale:
        g = g * np.float32(layer_scale(w, w.layer_of[i]))
    g = g.astype(np.float32)
    return bf16_round(g) if w.grad_dtype == "bf16" else g


def device_weight(w: Workload, i: int, device):
    import torch
    m, n = w.shapes[i]
    gen = torch.Generator(device=device)
    gen.manual_seed(_torch_seed(w.seed, i, "W", 0))
    return torch.randn((m, n), generator=gen, device=device, dtype=torch.float32) * W_STD


def device_grad(w: Workload, i: int, step: int, device, out=None):
    """Device-side draw for the large configurations (torch Philox stream),
    cast to the storage type.  `out` (optional) is filled in place."""
    import torch
    m, n = w.shapes[i]
    gen = torch.Generator(device=device)
    gen.manual_seed(_torch_seed(w.seed, i, "G", step + 1000))
    scale = G_STD * (layer_scale(w, w.layer_of[i]) if w.grad_layer_scale else 1.0)
    g = torch.randn((m, n), generator=gen, device=device, dtype=torch.float32)
    g.mul_(scale)
    dt = torch.bfloat16 if w.grad_dtype == "bf16" else torch.float32
    if out is None:
        return g.to(dt)
    out.copy_(g)
    return out


def _torch_seed(seed: int, idx: int, kind: str, step: int) -> int:
    ss = np.random.SeedSequence([seed, idx, KIND[kind], step, 7])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))
