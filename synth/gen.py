"""Seeded weight and token generators (numpy, host).

Every random tensor has its own PCG64 stream, SeedSequence([seed, tensor_id]),
so a tensor's values do not depend on which other tensors were drawn.
Token ids use SeedSequence([seed, 1_000_000 + seq_id]).

Weight layouts (row-major, the residual-stream axis is d = d_model):
  embed [vocab, d]        tied input embedding and LM head; rows unit-norm
  qkvg  [Nq+2Nkv+Ng, d]   rows are q | k | v | gate outputs; rows unit-norm
  o     [d, n_q*hd]       columns unit-norm (each column lives in R^d)
  ug    [2*d_ff, d]       rows 0..d_ff-1 are u ("up"), rows d_ff.. are v (SiLU input); rows unit-norm
  down  [d, d_ff]         columns unit-norm
  alpha_a, alpha_m [d]    float32, filled with alpha_init
Float32 models store float32 arrays; bfloat16 models store the bfloat16 bit
patterns as uint16 arrays.
"""
from __future__ import annotations

from typing import Dict, List, Tuple

import numpy as np

from .configs import ModelConfig

_KIND_ID = {"qkvg": 0, "o": 1, "ug": 2, "down": 3}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16, nearest-even, returning the 16-bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1
    return ((b + 0x7FFF + lsb) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def weight_names(cfg: ModelConfig) -> List[str]:
    names = ["embed"]
    for l in range(cfg.n_layers):
        names += [f"L{l}.qkvg", f"L{l}.o", f"L{l}.ug", f"L{l}.down", f"L{l}.alpha_a", f"L{l}.alpha_m"]
    return names


def weight_shape(cfg: ModelConfig, kind: str) -> Tuple[Tuple[int, int], int]:
    """(shape, axis along which the tensor is unit-normalised)."""
    d = cfg.d_model
    if kind == "embed":
        return (cfg.vocab, d), 1
    if kind == "qkvg":
        return (cfg.qkvg_dim, d), 1
    if kind == "o":
        return (d, cfg.q_dim), 0
    if kind == "ug":
        return (2 * cfg.d_ff, d), 1
    if kind == "down":
        return (d, cfg.d_ff), 0
    raise KeyError(kind)


def tensor_id(layer: int, kind: str) -> int:
    return 0 if kind == "embed" else 1 + 4 * layer + _KIND_ID[kind]


def _draw_unit(cfg: ModelConfig, layer: int, kind: str) -> np.ndarray:
    shape, axis = weight_shape(cfg, kind)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.seed, tensor_id(layer, kind)])))
    w = rng.standard_normal(shape, dtype=np.float32)
    w *= np.float32(cfg.init_std)
    w64 = w.astype(np.float64)
    w64 /= np.sqrt(np.sum(w64 * w64, axis=axis, keepdims=True))
    out = w64.astype(np.float32)
    if cfg.dtype == "bf16":
        return f32_to_bf16_bits(out)
    return out


def make_weights(cfg: ModelConfig) -> Dict[str, np.ndarray]:
    """All weights of `cfg`, keyed as in weight_names()."""
    w: Dict[str, np.ndarray] = {"embed": _draw_unit(cfg, -1, "embed")}
    for l in range(cfg.n_layers):
        for kind in ("qkvg", "o", "ug", "down"):
            w[f"L{l}.{kind}"] = _draw_unit(cfg, l, kind)
        w[f"L{l}.alpha_a"] = np.full(cfg.d_model, cfg.alpha_init, dtype=np.float32)
        w[f"L{l}.alpha_m"] = np.full(cfg.d_model, cfg.alpha_init, dtype=np.float32)
    return w


def make_tokens(cfg: ModelConfig, seq_id: int, shape) -> np.ndarray:
    """Uniform token ids in [0, vocab), int32."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.seed, 1_000_000 + seq_id])))
    return rng.integers(0, cfg.vocab, size=shape, dtype=np.int64).astype(np.int32)
