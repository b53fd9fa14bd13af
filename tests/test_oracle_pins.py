"""Pins of the oracle against what the pages and the mathematics fix.

Each test names the fact it pins. None of them re-runs the oracle's own
formula: they use closed forms, library routines (torch SDPA, torch's
bfloat16 cast), special cases with a known answer, an equivalent model built
from different weights (GQA vs MHA), and a scalar brute-force forward.
"""
import math

import numpy as np
import pytest
import torch

from synth.configs import ModelConfig, pattern_alternating, pattern_every4
from synth.gen import make_weights, make_tokens
from oracle.ngpt import (LoopedNGPT, OracleConfigError, attention, rope, round_bf16,
                         PER_LOOP, LAST_LOOP)
from bruteforce import Brute


def micro(**kw) -> ModelConfig:
    base = dict(name="micro", d_model=16, n_q_heads=4, n_kv_heads=2, head_dim=8, d_ff=24,
                vocab=64, n_in=1, n_rec=2, n_out=1, window=3,
                layer_is_full=pattern_alternating(4), rope_base_swa=1.0e4,
                rope_base_full=1.0e7, dtype="f32", alpha_init=0.3, seed=7)
    base.update(kw)
    if "layer_is_full" not in kw:
        n = base["n_in"] + base["n_rec"] + base["n_out"]
        base["layer_is_full"] = pattern_alternating(n)
    return ModelConfig(**base)


# ---------------------------------------------------------------------------
# depth: 32 + 40k for the 16/40/16 split, 16 + 20k for 8/20/8
# ("Dory1.0-4B: A Looped Normalized-GPT" summary, Key Contributions 1 and
#  Main Findings: 72 / 112 / 192 layer applications at k = 1 / 2 / 4)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("split,expected", [((16, 40, 16), {1: 72, 2: 112, 3: 152, 4: 192}),
                                            ((8, 20, 8), {1: 36, 2: 56, 3: 76, 4: 96})])
def test_effective_depth(split, expected):
    cfg = micro(d_model=8, n_q_heads=2, n_kv_heads=1, head_dim=4, d_ff=8, vocab=16,
                n_in=split[0], n_rec=split[1], n_out=split[2],
                layer_is_full=pattern_every4(sum(split)))
    w = make_weights(cfg)
    for k, apps in expected.items():
        o = LoopedNGPT(cfg, w, max_ctx=8)
        o.call(np.array([[1, 2]]), k, LAST_LOOP)
        assert o.layer_apps_per_token == [apps]
    # the figures the pages print (tests/golden/depth.json)
    if split == (16, 40, 16):
        import json, os
        gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "depth.json")))
        for k, apps in gold["split_16_40_16"].items():
            assert expected[int(k)] == apps
        assert all(expected[k] == 32 + 40 * k for k in expected)
    else:
        assert all(expected[k] == 16 + 20 * k for k in expected)


# ---------------------------------------------------------------------------
# hypersphere: every hidden state stays at unit norm
# ("Dory1.0-4B" summary, Methodology: everything is L2-normalised)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("mode", [PER_LOOP, LAST_LOOP])
def test_hypersphere(mode):
    cfg = micro()
    o = LoopedNGPT(cfg, make_weights(cfg), max_ctx=32)
    o.generate(make_tokens(cfg, 0, (1, 9)), steps=5, n_loops=3, kv_mode=mode)
    assert o.max_norm_dev <= 1e-4
    assert o.max_norm_dev <= 1e-12          # fp64: far inside the bound


# ---------------------------------------------------------------------------
# k = 1: per-loop and last-loop caching are the same thing
# ---------------------------------------------------------------------------
def test_k1_modes_identical():
    cfg = micro()
    w = make_weights(cfg)
    toks = make_tokens(cfg, 1, (1, 7))
    a = LoopedNGPT(cfg, w, max_ctx=32).generate(toks, 6, 1, PER_LOOP)
    b = LoopedNGPT(cfg, w, max_ctx=32).generate(toks, 6, 1, LAST_LOOP)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


# ---------------------------------------------------------------------------
# incremental decode == full recompute (per-loop any k; k=1 both modes);
# last-loop with k > 1 must NOT equal it (each loop overwrites the cache)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("k,mode,equal", [(1, PER_LOOP, True), (1, LAST_LOOP, True),
                                          (2, PER_LOOP, True), (3, PER_LOOP, True),
                                          (2, LAST_LOOP, False), (3, LAST_LOOP, False)])
def test_incremental_vs_full(k, mode, equal):
    cfg = micro()
    w = make_weights(cfg)
    toks = make_tokens(cfg, 2, (1, 8))
    full = LoopedNGPT(cfg, w, max_ctx=16).call(toks, k, mode, all_logits=True)[0]
    inc = LoopedNGPT(cfg, w, max_ctx=16)
    rows = [inc.call(toks[:, i:i + 1], k, mode)[0] for i in range(toks.shape[1])]
    inc_l = np.stack(rows)
    diff = np.max(np.abs(full - inc_l))
    if equal:
        assert diff <= 1e-9
    else:
        np.testing.assert_allclose(full[0], inc_l[0], atol=1e-12)   # first token has no past
        assert diff > 1e-6


def test_last_loop_cache_holds_final_loop():
    """After one k=3 call, the last-loop cache of a recurrent layer equals the
    per-loop cache of loop 3 and differs from loop 1's."""
    cfg = micro()
    w = make_weights(cfg)
    toks = make_tokens(cfg, 3, (1, 5))
    pl = LoopedNGPT(cfg, w, max_ctx=8)
    pl.call(toks, 3, PER_LOOP)
    ll = LoopedNGPT(cfg, w, max_ctx=8)
    ll.call(toks, 3, LAST_LOOP)
    for l in range(cfg.n_in, cfg.n_in + cfg.n_rec):
        np.testing.assert_allclose(ll.cache[(l, 0)]["K"][:, :, :5], pl.cache[(l, 3)]["K"][:, :, :5], atol=1e-14)
        np.testing.assert_allclose(ll.cache[(l, 0)]["V"][:, :, :5], pl.cache[(l, 3)]["V"][:, :, :5], atol=1e-14)
        assert np.max(np.abs(pl.cache[(l, 1)]["K"][:, :, :5] - pl.cache[(l, 3)]["K"][:, :, :5])) > 1e-6
    assert sorted(ll.cache) == [(l, 0) for l in range(cfg.n_layers)]


def test_call_validation():
    cfg = micro()
    w = make_weights(cfg)
    o = LoopedNGPT(cfg, w, max_ctx=8)
    o.call(np.array([[1, 2]]), 2, PER_LOOP)
    with pytest.raises(OracleConfigError):
        o.call(np.array([[3]]), 3, PER_LOOP)        # k change in per-loop mode
    with pytest.raises(OracleConfigError):
        o.call(np.array([[3]]), 2, LAST_LOOP)       # mode switch
    with pytest.raises(OracleConfigError):
        o.call(np.zeros((1, 7), dtype=np.int32), 2, PER_LOOP)   # overflow
    o2 = LoopedNGPT(cfg, w, max_ctx=8)
    o2.call(np.array([[1]]), 2, LAST_LOOP)
    o2.call(np.array([[2]]), 4, LAST_LOOP)          # elastic depth allowed in last-loop


# ---------------------------------------------------------------------------
# attention against the library: torch SDPA in float64
# ---------------------------------------------------------------------------
def _sdpa(q, k, v, scale, causal):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), is_causal=causal, scale=scale)[0, 0].numpy()


def test_attention_full_window_is_causal_sdpa():
    rng = np.random.default_rng(0)
    n, hd = 37, 16
    q, k, v = (rng.standard_normal((n, hd)) for _ in range(3))
    ours = attention(q, k, v, np.arange(n), window=None, scale=1.7)
    np.testing.assert_allclose(ours, _sdpa(q, k, v, 1.7, True), atol=1e-12)
    ours_w = attention(q, k, v, np.arange(n), window=n, scale=1.7)       # W >= T
    np.testing.assert_allclose(ours_w, ours, atol=0)


def test_attention_window_is_sdpa_on_the_window():
    rng = np.random.default_rng(1)
    n, hd, W = 29, 8, 5
    q, k, v = (rng.standard_normal((n, hd)) for _ in range(3))
    ours = attention(q, k, v, np.arange(n), window=W, scale=0.9)
    for t in range(n):
        lo = max(0, t - W + 1)
        ref = _sdpa(q[t:t + 1], k[lo:t + 1], v[lo:t + 1], 0.9, False)
        np.testing.assert_allclose(ours[t], ref[0], atol=1e-12)


def test_attention_offset_queries():
    """Queries at positions p0.. see keys 0..t (a later chunk of a sequence)."""
    rng = np.random.default_rng(2)
    T, hd, p0 = 20, 8, 12
    q = rng.standard_normal((T - p0, hd))
    k, v = rng.standard_normal((T, hd)), rng.standard_normal((T, hd))
    ours = attention(q, k, v, np.arange(p0, T), window=None, scale=1.0)
    for i, t in enumerate(range(p0, T)):
        ref = _sdpa(q[i:i + 1], k[:t + 1], v[:t + 1], 1.0, False)
        np.testing.assert_allclose(ours[i], ref[0], atol=1e-12)


# ---------------------------------------------------------------------------
# GQA == MHA with each KV head repeated for its query group
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("gate", [0, 1, 2])
def test_gqa_equals_repeated_mha(gate):
    cfg = micro(attn_gate=gate)
    w = make_weights(cfg)
    hd, nq, nkv = cfg.head_dim, cfg.n_q_heads, cfg.n_kv_heads
    mha = cfg.replace(n_kv_heads=nq)
    wm = dict(w)
    for l in range(cfg.n_layers):
        W = w[f"L{l}.qkvg"]
        q = W[:nq * hd]
        k = W[nq * hd:(nq + nkv) * hd].reshape(nkv, hd, -1)
        v = W[(nq + nkv) * hd:(nq + 2 * nkv) * hd].reshape(nkv, hd, -1)
        g = W[(nq + 2 * nkv) * hd:]
        grp = [hq * nkv // nq for hq in range(nq)]
        wm[f"L{l}.qkvg"] = np.concatenate([q, k[grp].reshape(nq * hd, -1), v[grp].reshape(nq * hd, -1), g])
    toks = make_tokens(cfg, 4, (1, 6))
    a = LoopedNGPT(cfg, w, max_ctx=16).generate(toks, 4, 2, PER_LOOP)
    b = LoopedNGPT(mha, wm, max_ctx=16).generate(toks, 4, 2, PER_LOOP)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_allclose(a[1], b[1], atol=1e-11)


# ---------------------------------------------------------------------------
# nGPT update special cases
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("k,mode", [(1, LAST_LOOP), (3, PER_LOOP), (4, LAST_LOOP)])
def test_alpha_zero_is_identity(k, mode):
    """With every alpha = 0 no layer moves h, and the combine of e with e is e,
    so the logits are s_z * <E[tok]/|E[tok]|, E[v]>: the input token wins with
    logit s_z * |E[tok]|."""
    cfg = micro(alpha_init=0.0)
    w = make_weights(cfg)
    toks = make_tokens(cfg, 5, (1, 6))
    o = LoopedNGPT(cfg, w, max_ctx=8)
    logits = o.call(toks, k, mode, all_logits=True)[0]
    assert np.all(np.argmax(logits, axis=-1) == toks[0])
    enorm = np.linalg.norm(w["embed"][toks[0]].astype(np.float64), axis=-1)   # 1 up to fp32 rounding
    np.testing.assert_allclose(logits[np.arange(6), toks[0]], cfg.scale_logit * enorm, rtol=1e-12)


def test_alpha_one_single_token_closed_form():
    """One layer, alpha_a = 1, alpha_m = 0, a single token: attention over one
    key returns that key's value, so h = norm(W_o norm(v * sigmoid(g)))."""
    cfg = micro(n_in=1, n_rec=0, n_out=0, layer_is_full=(False,), attn_gate=1)
    w = make_weights(cfg)
    w["L0.alpha_a"] = np.ones(cfg.d_model, np.float32)
    w["L0.alpha_m"] = np.zeros(cfg.d_model, np.float32)
    tok = 11
    o = LoopedNGPT(cfg, w, max_ctx=4)
    _, h = o.call(np.array([[tok]]), 1, LAST_LOOP, return_hidden=True)
    e = w["embed"][tok].astype(np.float64)
    x = e / np.linalg.norm(e)
    W = w["L0.qkvg"].astype(np.float64)
    hd, nq, nkv = cfg.head_dim, cfg.n_q_heads, cfg.n_kv_heads
    z = W @ x
    v = z[(nq + nkv) * hd:(nq + 2 * nkv) * hd].reshape(nkv, hd)
    g = z[(nq + 2 * nkv) * hd:].reshape(nq, hd)
    o_cat = np.concatenate([v[hq * nkv // nq] / (1 + np.exp(-g[hq])) for hq in range(nq)])
    o_cat /= np.linalg.norm(o_cat)
    y = w["L0.o"].astype(np.float64) @ o_cat
    np.testing.assert_allclose(h[0, 0], y / np.linalg.norm(y), atol=1e-12)


def test_update_closed_form_2d():
    from oracle.ngpt import ngpt_update
    h = np.array([1.0, 0.0])
    y = np.array([0.0, 3.0])              # norm(y) = e1
    out = ngpt_update(h, y, np.array([0.5, 0.5]))
    np.testing.assert_allclose(out, [1 / math.sqrt(2), 1 / math.sqrt(2)], atol=1e-15)
    out = ngpt_update(h, y, np.array([0.25, 0.25]))
    np.testing.assert_allclose(out, np.array([0.75, 0.25]) / math.hypot(0.75, 0.25), atol=1e-15)


# ---------------------------------------------------------------------------
# RoPE closed forms
# ---------------------------------------------------------------------------
def test_rope_closed_forms():
    hd, base = 8, 1.0e4
    pos = np.array([0, 1, 7, 262143])
    x = np.zeros((len(pos), 1, hd))
    x[:, 0, 0] = 1.0                      # e_0: theta_0 = 1
    r = rope(x, pos, base)
    np.testing.assert_allclose(r[:, 0, 0], np.cos(pos.astype(np.float64)), atol=1e-15)
    np.testing.assert_allclose(r[:, 0, hd // 2], np.sin(pos.astype(np.float64)), atol=1e-15)
    x = np.zeros((len(pos), 1, hd))
    x[:, 0, hd // 2 + 1] = 1.0            # e_{1+hd/2}: theta_1 = base^(-2/hd)
    r = rope(x, pos, base)
    th = base ** (-2.0 / hd)
    np.testing.assert_allclose(r[:, 0, 1], -np.sin(pos * th), atol=1e-12)
    np.testing.assert_allclose(r[:, 0, hd // 2 + 1], np.cos(pos * th), atol=1e-12)


def test_rope_identity_norm_relative():
    rng = np.random.default_rng(3)
    hd = 16
    q = rng.standard_normal((1, 1, hd))
    k = rng.standard_normal((1, 1, hd))
    np.testing.assert_array_equal(rope(q, np.array([0]), 1e4), q)
    for m in (3, 1000, 200000):
        rq = rope(q, np.array([m]), 1e7)
        np.testing.assert_allclose(np.linalg.norm(rq), np.linalg.norm(q), rtol=1e-14)
    d1 = np.sum(rope(q, np.array([10]), 1e4) * rope(k, np.array([4]), 1e4))
    d2 = np.sum(rope(q, np.array([1006]), 1e4) * rope(k, np.array([1000]), 1e4))
    np.testing.assert_allclose(d1, d2, rtol=1e-10)


# ---------------------------------------------------------------------------
# bfloat16 storage rounding against torch's cast (library routine)
# ---------------------------------------------------------------------------
def test_round_bf16_matches_torch():
    rng = np.random.default_rng(4)
    x = np.concatenate([rng.standard_normal(10000) * 10.0 ** rng.integers(-6, 6, 10000),
                        [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -0.0, 0.0, 65504.0, 1e-38]])
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(round_bf16(x), ref)
    assert round_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 1.0            # tie to even
    assert round_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6


# ---------------------------------------------------------------------------
# brute-force scalar forward on tiny shapes
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("gate,k,per_loop", [(1, 2, True), (1, 2, False), (2, 3, False),
                                             (0, 1, True), (1, 3, True)])
def test_bruteforce_tiny(gate, k, per_loop):
    cfg = micro(attn_gate=gate, d_model=12, d_ff=10, vocab=20, window=3, combine_wh=0.7,
                combine_we=1.3)
    w = make_weights(cfg)
    toks = make_tokens(cfg, 6, (1, 5))[0]
    mode = PER_LOOP if per_loop else LAST_LOOP
    o = LoopedNGPT(cfg, w, max_ctx=16)
    bf = Brute(cfg, w)
    got = o.call(toks[None, :4], k, mode)[0]
    ref = bf.call(list(toks[:4]), k, per_loop)
    np.testing.assert_allclose(got, ref, atol=1e-11)
    for t in [int(toks[4]), 3, 17]:                         # decode steps past the window
        got = o.call(np.array([[t]]), k, mode)[0]
        ref = bf.call([t], k, per_loop)
        np.testing.assert_allclose(got, ref, atol=1e-11)


def test_bf16_points_are_close_but_not_equal():
    cfg = micro(dtype="bf16")
    w = make_weights(cfg)
    toks = make_tokens(cfg, 7, (1, 6))
    a = LoopedNGPT(cfg, w, max_ctx=8).call(toks, 2, LAST_LOOP)
    b = LoopedNGPT(cfg, w, max_ctx=8, bf16_points=False).call(toks, 2, LAST_LOOP)
    d = np.max(np.abs(a - b))
    assert 0 < d < 0.05


def test_extra_norms_scale_invariant():
    """The L2 norms before the output and down projections change nothing
    after the update's own norm(y): scaling o or a by c > 0 is invisible.
    Checked on the update itself with W @ (c*x)."""
    from oracle.ngpt import ngpt_update, l2norm
    rng = np.random.default_rng(5)
    h = l2norm(rng.standard_normal(32))
    W = rng.standard_normal((32, 48))
    a = rng.standard_normal(48)
    al = np.full(32, 0.05)
    ref = ngpt_update(h, W @ l2norm(a), al)
    for c in (1e-3, 0.37, 250.0):
        np.testing.assert_allclose(ngpt_update(h, W @ (c * a), al), ref, atol=1e-15)
