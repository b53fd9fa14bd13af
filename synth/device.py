"""Seeded weights generated on the GPU (for full-size runs).

Same recipe as synth.gen (N(0, 0.02), unit L2 norm along the d_model axis,
stored as bfloat16 bit patterns or float32, alpha = alpha_init) and the same
layouts, but drawn with torch's device generator: values differ from
synth.gen's numpy streams. Full-size benchmark weights (4.4e9 parameters for
the 36-layer shape) take seconds this way instead of a minute on the host.
Every tensor has its own generator seeded from (seed, tensor_id).
"""
from __future__ import annotations

from typing import Dict

import torch

from .configs import ModelConfig
from .gen import tensor_id, weight_shape


def _seed(cfg: ModelConfig, tid: int) -> int:
    return (cfg.seed * 1_000_003 + tid * 7_919 + 12_345) & 0x7FFF_FFFF_FFFF


def _draw(cfg: ModelConfig, layer: int, kind: str, device) -> torch.Tensor:
    shape, axis = weight_shape(cfg, kind)
    g = torch.Generator(device=device)
    g.manual_seed(_seed(cfg, tensor_id(layer, kind)))
    w = torch.randn(shape, generator=g, device=device, dtype=torch.float32) * cfg.init_std
    w = w / torch.linalg.vector_norm(w.double(), dim=axis, keepdim=True).float()
    if cfg.dtype == "bf16":
        return w.to(torch.bfloat16).view(torch.int16).contiguous()
    return w.contiguous()


def make_weights_device(cfg: ModelConfig, device="cuda") -> Dict[str, torch.Tensor]:
    w = {"embed": _draw(cfg, -1, "embed", device)}
    for l in range(cfg.n_layers):
        for kind in ("qkvg", "o", "ug", "down"):
            w[f"L{l}.{kind}"] = _draw(cfg, l, kind, device)
        w[f"L{l}.alpha_a"] = torch.full((cfg.d_model,), cfg.alpha_init, dtype=torch.float32, device=device)
        w[f"L{l}.alpha_m"] = torch.full((cfg.d_model,), cfg.alpha_init, dtype=torch.float32, device=device)
    return w
