"""Model shapes and workloads of the looped normalized-GPT forward pass.

The architecture facts come from the pages on the Dory1.0-4B looped nGPT:
an input block run once, a shared recurrent block run k times and an output
block run once (ai.info summary, "Key Contributions" item 1; goremy.ai blog,
"What is Dory1.0-4B?"), a repeating pattern of three sliding-window layers and
one full-attention layer with grouped-query attention, sigmoid output gates
and two RoPE bases (ai.info summary, "Methodology in Plain English").
The pages disagree on the block split (16/40/16 vs 8/20/8), so the split is
a parameter and both shapes are defined below.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Tuple


@dataclasses.dataclass(frozen=True)
class ModelConfig:
    name: str
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    d_ff: int
    vocab: int
    n_in: int
    n_rec: int
    n_out: int
    window: int                      # sliding-window size in keys, self included
    layer_is_full: Tuple[bool, ...]  # per global layer index
    rope_base_swa: float = 1.0e4
    rope_base_full: float = 1.0e7
    dtype: str = "bf16"              # "f32" or "bf16": storage type of weights and activations
    attn_gate: int = 1               # 0 none, 1 elementwise, 2 one scalar per query head
    attn_scale: Optional[float] = None   # None -> sqrt(head_dim)
    logit_scale: Optional[float] = None  # None -> sqrt(d_model)
    combine_wh: float = 1.0          # loop re-injection: x_j = norm(wh*h_{j-1} + we*e)
    combine_we: float = 1.0
    alpha_init: float = 0.05
    init_std: float = 0.02
    seed: int = 0

    @property
    def n_layers(self) -> int:
        return self.n_in + self.n_rec + self.n_out

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def gate_dim(self) -> int:
        return {0: 0, 1: self.q_dim, 2: self.n_q_heads}[self.attn_gate]

    @property
    def qkvg_dim(self) -> int:
        return self.q_dim + 2 * self.kv_dim + self.gate_dim

    @property
    def scale_attn(self) -> float:
        return math.sqrt(self.head_dim) if self.attn_scale is None else float(self.attn_scale)

    @property
    def scale_logit(self) -> float:
        return math.sqrt(self.d_model) if self.logit_scale is None else float(self.logit_scale)

    def is_recurrent(self, layer: int) -> bool:
        return self.n_in <= layer < self.n_in + self.n_rec

    def layer_bytes(self) -> int:
        """Weight bytes of one layer (both projections of both sublayers)."""
        el = 4 if self.dtype == "f32" else 2
        d = self.d_model
        return el * (self.qkvg_dim * d + d * self.q_dim + 2 * self.d_ff * d + d * self.d_ff)

    def replace(self, **kw) -> "ModelConfig":
        return dataclasses.replace(self, **kw)


def pattern_every4(n_layers: int) -> Tuple[bool, ...]:
    """Three sliding-window layers then one full-attention layer, repeated."""
    return tuple(i % 4 == 3 for i in range(n_layers))


def pattern_alternating(n_layers: int) -> Tuple[bool, ...]:
    """Sliding-window first, then full, alternating."""
    return tuple(i % 2 == 1 for i in range(n_layers))


def _tiny() -> ModelConfig:
    return ModelConfig(
        name="tiny_d256_2-2-2", d_model=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
        d_ff=683, vocab=1024, n_in=2, n_rec=2, n_out=2, window=64,
        layer_is_full=pattern_alternating(6), rope_base_swa=1.0e4, rope_base_full=1.0e4,
        dtype="f32", seed=0)


def _c36() -> ModelConfig:
    return ModelConfig(
        name="4b_36L_8-20-8", d_model=3072, n_q_heads=24, n_kv_heads=8, head_dim=128,
        d_ff=8192, vocab=131072, n_in=8, n_rec=20, n_out=8, window=4096,
        layer_is_full=pattern_every4(36), dtype="bf16", seed=1)


def _c72() -> ModelConfig:
    return ModelConfig(
        name="4b_72L_16-40-16", d_model=2304, n_q_heads=18, n_kv_heads=6, head_dim=128,
        d_ff=6144, vocab=131072, n_in=16, n_rec=40, n_out=16, window=4096,
        layer_is_full=pattern_every4(72), dtype="bf16", seed=2)


# The five workloads. "model" is the shape; the rest describes the run.
CONFIGS = {
    "tiny": dict(model=_tiny(), batch=1, prompt=128, decode_steps=32, loops=(2,),
                 kv_modes=("per_loop", "last_loop"), chunk=128),
    "c36": dict(model=_c36(), batch=1, prompt=8192, decode_steps=256, loops=(1, 2, 4),
                kv_modes=("last_loop",), chunk=8192),
    "c72": dict(model=_c72(), batch=1, prompt=16384, decode_steps=256, loops=(1, 2, 3, 4),
                kv_modes=("per_loop", "last_loop"), chunk=8192),
    "c36_b64": dict(model=_c36().replace(seed=3), batch=64, prompt=32768, decode_steps=128,
                    loops=(4,), kv_modes=("per_loop", "last_loop"), chunk=8192),
    "c36_256k": dict(model=_c36().replace(seed=4), batch=1, prompt=262144, decode_steps=64,
                     loops=(2,), kv_modes=("last_loop",), chunk=8192),
}


def get_config(name: str) -> ModelConfig:
    return CONFIGS[name]["model"]


def scaled_config(base: ModelConfig, *, n_in: int, n_rec: int, n_out: int,
                  pattern: str = "every4", **kw) -> ModelConfig:
    """A shape of the same width with a different depth (for parity runs that
    the oracle must finish in seconds)."""
    n = n_in + n_rec + n_out
    pat = pattern_every4(n) if pattern == "every4" else pattern_alternating(n)
    return base.replace(n_in=n_in, n_rec=n_rec, n_out=n_out, layer_is_full=pat,
                        name=f"{base.name}_as_{n_in}-{n_rec}-{n_out}", **kw)
