"""KV-cache placement spec: which cache and which slot hold a key.

TEST INFRASTRUCTURE ONLY (see the package header).

Per-loop caching keeps a separate cache for every loop of a recurrent
attention layer, so memory grows with the loop count; last-loop caching keeps
one cache per recurrent attention layer that every loop overwrites, so the
footprint is the one-loop size at any loop count ("Dory 1.0 4B Benchmarks"
goremy.ai blog, How does looping work at inference time?; broadside review,
Key ideas). Input and output layers run once per token and own one cache each.

Placement (our reading, R10): a full-attention layer keeps every position
(slot = pos, max_ctx slots); a sliding-window layer of W keys keeps a ring of
min(W, max_ctx) slots with slot = pos mod W.

Buffer layout: caches are numbered layer by layer; a recurrent layer in
per-loop mode owns `kv_loops` consecutive ids (loop j -> base + j - 1).
Cache c occupies [K: batch x n_kv x slots_c x hd][V: batch x n_kv x
(vslots_c / 32) x hd x 32] in id order: values are kept in blocks of 32 slots
per head, each block holding the 32 values of one dimension contiguously
(vslots_c = slots_c rounded up to 32; the pad slots of the last block are
never written). Offsets below are in elements of the cache dtype.

Pinned by tests/test_oracle_kv.py: the footprint the oracle actually touches,
the pages' "independent of k" / "grows with k" statements, and closed forms.
"""
from __future__ import annotations

from typing import List

from synth.configs import ModelConfig

PER_LOOP = "per_loop"
LAST_LOOP = "last_loop"


def caches_of_layer(cfg: ModelConfig, kv_mode: str, kv_loops: int, layer: int) -> int:
    if cfg.is_recurrent(layer) and kv_mode == PER_LOOP:
        return kv_loops
    return 1


def slots(cfg: ModelConfig, max_ctx: int, layer: int) -> int:
    return max_ctx if cfg.layer_is_full[layer] else min(cfg.window, max_ctx)


VTILE = 32  # slots per value block


def vslots(cfg: ModelConfig, max_ctx: int, layer: int) -> int:
    return -(-slots(cfg, max_ctx, layer) // VTILE) * VTILE


def slot(cfg: ModelConfig, max_ctx: int, layer: int, pos: int) -> int:
    return pos if cfg.layer_is_full[layer] else pos % cfg.window


def cache_id(cfg: ModelConfig, kv_mode: str, kv_loops: int, layer: int, loop: int) -> int:
    """loop is 1-based for recurrent layers; ignored for the others."""
    base = sum(caches_of_layer(cfg, kv_mode, kv_loops, l) for l in range(layer))
    if cfg.is_recurrent(layer) and kv_mode == PER_LOOP:
        if not 1 <= loop <= kv_loops:
            raise ValueError("loop outside the allocated per-loop caches")
        return base + loop - 1
    return base


def cache_layers(cfg: ModelConfig, kv_mode: str, kv_loops: int) -> List[int]:
    """Layer of every cache id, in id order."""
    out: List[int] = []
    for l in range(cfg.n_layers):
        out += [l] * caches_of_layer(cfg, kv_mode, kv_loops, l)
    return out


def elem_bytes(cfg: ModelConfig) -> int:
    return 4 if cfg.dtype == "f32" else 2


def cache_elems(cfg: ModelConfig, max_ctx: int, batch: int, layer: int) -> int:
    """Elements of one cache (K rows, then the value blocks)."""
    return batch * cfg.n_kv_heads * cfg.head_dim * (slots(cfg, max_ctx, layer) + vslots(cfg, max_ctx, layer))


def kv_bytes(cfg: ModelConfig, kv_mode: str, kv_loops: int, max_ctx: int, batch: int) -> int:
    return elem_bytes(cfg) * sum(cache_elems(cfg, max_ctx, batch, l)
                                 for l in cache_layers(cfg, kv_mode, kv_loops))


def element_offset(cfg: ModelConfig, kv_mode: str, kv_loops: int, max_ctx: int, batch: int,
                   layer: int, loop: int, which: str, b: int, kvh: int, pos: int) -> int:
    """Offset (elements) of dimension 0 of K or V of (b, kvh, pos); dimension
    d is at + d * dim_stride(...)."""
    cid = cache_id(cfg, kv_mode, kv_loops, layer, loop)
    lays = cache_layers(cfg, kv_mode, kv_loops)
    start = sum(cache_elems(cfg, max_ctx, batch, l) for l in lays[:cid])
    ns = slots(cfg, max_ctx, layer)
    half = batch * cfg.n_kv_heads * ns * cfg.head_dim
    sl = slot(cfg, max_ctx, layer, pos)
    if which == "V":
        nv = vslots(cfg, max_ctx, layer)
        return start + half + ((b * cfg.n_kv_heads + kvh) * nv + sl // VTILE * VTILE) * cfg.head_dim + sl % VTILE
    return start + ((b * cfg.n_kv_heads + kvh) * ns + sl) * cfg.head_dim


def dim_stride(cfg: ModelConfig, max_ctx: int, layer: int, which: str) -> int:
    """Distance (elements) between consecutive dimensions of one K or V vector."""
    return VTILE if which == "V" else 1
