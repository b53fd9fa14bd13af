"""Pins of the KV-cache spec: last-loop bytes do not depend on k, per-loop
bytes grow linearly with k ("Dory 1.0 4B Benchmarks" goremy.ai blog, How does
looping work at inference time?; "Dory1.0-4B" summary, Key Contributions 4),
checked three ways: the caches the oracle actually touches, the spec's byte
count, and a closed form worked by hand for the 36-layer shape."""
import numpy as np
import pytest

from synth.configs import get_config, ModelConfig, pattern_alternating
from synth.gen import make_weights, make_tokens
from oracle import kvspec
from oracle.ngpt import LoopedNGPT, PER_LOOP, LAST_LOOP


def micro() -> ModelConfig:
    return ModelConfig(name="micro", d_model=16, n_q_heads=4, n_kv_heads=2, head_dim=8, d_ff=24,
                       vocab=64, n_in=1, n_rec=2, n_out=1, window=3,
                       layer_is_full=pattern_alternating(4), dtype="f32", seed=7)


def touched_bytes(o: LoopedNGPT, max_ctx: int) -> int:
    """Bytes of the caches the oracle created: keys for every slot, values in
    32-slot blocks (the last block padded)."""
    c = o.cfg
    total = 0
    for (l, _j) in o.cache:
        ns = kvspec.slots(c, max_ctx, l)
        total += (ns + -(-ns // 32) * 32) * c.n_kv_heads * c.head_dim * kvspec.elem_bytes(c) * o.batch
    return total


@pytest.mark.parametrize("mode", [PER_LOOP, LAST_LOOP])
def test_touched_caches_match_spec(mode):
    cfg = micro()
    w = make_weights(cfg)
    sizes = []
    for k in (1, 2, 3, 4):
        o = LoopedNGPT(cfg, w, max_ctx=16)
        o.generate(make_tokens(cfg, 0, (1, 5)), 2, k, mode)
        got = touched_bytes(o, 16)
        assert got == kvspec.kv_bytes(cfg, mode, k, 16, 1)
        sizes.append(got)
    if mode == LAST_LOOP:
        assert len(set(sizes)) == 1
    else:
        steps = np.diff(sizes)
        assert len(set(steps.tolist())) == 1 and steps[0] > 0


def test_closed_form_36_layer():
    cfg = get_config("c36")
    # 27 sliding layers keep 4096 slots, 9 full layers keep max_ctx = 8192 + 256
    # slots; one slot of one layer = K and V of 8 heads x 128 dims in bf16 = 4096 B.
    slot_b = 2 * 8 * 128 * 2
    assert slot_b == 4096
    last = (27 * 4096 + 9 * 8448) * slot_b
    assert last == 764_411_904
    for k in (1, 2, 3, 4):
        assert kvspec.kv_bytes(cfg, LAST_LOOP, k, 8448, 1) == last
    # the recurrent block (layers 8..27) holds 5 full and 15 sliding layers
    rec = (15 * 4096 + 5 * 8448) * slot_b
    for k in (1, 2, 4):
        assert kvspec.kv_bytes(cfg, PER_LOOP, k, 8448, 1) == last + (k - 1) * rec
    assert kvspec.kv_bytes(cfg, PER_LOOP, 4, 8448, 1) == 2_038_431_744


def test_slot_spec_ring_and_ids():
    cfg = micro()      # layers: 0 swa (in), 1 full (rec), 2 swa (rec), 3 full (out); W = 3
    assert [kvspec.slot(cfg, 16, 0, p) for p in range(7)] == [0, 1, 2, 0, 1, 2, 0]
    assert [kvspec.slot(cfg, 16, 1, p) for p in range(7)] == list(range(7))
    assert kvspec.slots(cfg, 2, 0) == 2             # window wider than the context
    ids = [kvspec.cache_id(cfg, PER_LOOP, 3, l, j) for l, j in
           [(0, 0), (1, 1), (1, 2), (1, 3), (2, 1), (2, 2), (2, 3), (3, 0)]]
    assert ids == list(range(8))
    ids = [kvspec.cache_id(cfg, LAST_LOOP, 3, l, j) for l, j in [(0, 0), (1, 1), (1, 3), (2, 2), (3, 0)]]
    assert ids == [0, 1, 1, 2, 3]
    with pytest.raises(ValueError):
        kvspec.cache_id(cfg, PER_LOOP, 2, 1, 3)


def test_element_offsets_tile_the_buffer():
    """Every element of every (cache, K/V, b, head, slot) vector has its own
    place inside kv_bytes; the only places left over are the pad slots of the
    last value block of each head; and the values of the 32 slots of one
    block (all dimensions) form one contiguous run."""
    cfg = micro()
    B, T, kl = 2, 40, 2      # full layers: 40 slots (one full block + 8); sliding: 3 slots
    seen = []
    pad = 0
    for l in range(cfg.n_layers):
        loops = range(1, kl + 1) if cfg.is_recurrent(l) else [0]
        ns = kvspec.slots(cfg, T, l)
        for j in loops:
            pad += B * cfg.n_kv_heads * cfg.head_dim * (-(-ns // 32) * 32 - ns)
            for which in "KV":
                st = kvspec.dim_stride(cfg, T, l, which)
                for b in range(B):
                    for h in range(cfg.n_kv_heads):
                        blocks = {}
                        for p in range(ns):
                            o = kvspec.element_offset(cfg, PER_LOOP, kl, T, B, l, j, which, b, h, p)
                            run = [o + d * st for d in range(cfg.head_dim)]
                            seen += run
                            if which == "V":
                                blocks.setdefault(p // 32, []).extend(run)
                        for blk, offs in blocks.items():
                            if len(offs) == 32 * cfg.head_dim:      # a full block is one contiguous run
                                assert sorted(offs) == list(range(min(offs), min(offs) + len(offs)))
    total = kvspec.kv_bytes(cfg, PER_LOOP, kl, T, B) // 4
    assert len(seen) == len(set(seen))
    assert min(seen) == 0 and max(seen) < total
    assert total - len(seen) == pad and pad > 0
