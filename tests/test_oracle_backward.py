"""Pins of the depth-1 backward of oracle/backward.py (reading R21): central
finite differences of L = sum(G * h_out) for sampled entries of every
gradient, the training forward against LoopedNGPT's own layers, and the
alpha = 0 closed form."""
import numpy as np
import pytest

from oracle import backward as bw
from oracle.ngpt import LoopedNGPT
from synth.configs import ModelConfig
from synth.gen import make_weights


def _cfg(gate: int) -> ModelConfig:
    # 1 input, 2 recurrent (one sliding with a 5-key window, one full), 1 output layer
    return ModelConfig(name=f"bw_g{gate}", d_model=48, n_q_heads=4, n_kv_heads=2, head_dim=12, d_ff=40,
                       vocab=64, n_in=1, n_rec=2, n_out=1, window=5,
                       layer_is_full=(False, False, True, False), rope_base_swa=1.0e4, rope_base_full=1.0e6,
                       dtype="f32", attn_gate=gate, seed=5)


def _setup(gate: int, alpha: bool = True):
    cfg = _cfg(gate)
    w = {k: np.asarray(v, dtype=np.float64) for k, v in make_weights(cfg).items()}
    rng = np.random.default_rng(40 + gate)
    for l in range(cfg.n_layers):
        if alpha:                                    # per-channel alphas away from 0.05
            w[f"L{l}.alpha_a"] = rng.uniform(0.1, 0.6, cfg.d_model)
            w[f"L{l}.alpha_m"] = rng.uniform(0.1, 0.6, cfg.d_model)
        else:
            w[f"L{l}.alpha_a"] = np.zeros(cfg.d_model)
            w[f"L{l}.alpha_m"] = np.zeros(cfg.d_model)
    B, n = 2, 7
    x = rng.standard_normal((B, n, cfg.d_model))
    x /= np.linalg.norm(x, axis=-1, keepdims=True)
    G = rng.standard_normal((B, n, cfg.d_model))
    return cfg, w, x, G


@pytest.mark.parametrize("gate", [0, 1, 2])
def test_gradients_match_finite_differences(gate):
    cfg, w, x, G = _setup(gate)
    grads = bw.block_backward(cfg, w, x, G)
    rng = np.random.default_rng(7)
    eps = 1e-5
    checked = 0
    for name, ana in grads.items():
        if name == "x":
            continue
        base = w[name]
        flat = base.reshape(-1)
        if name.endswith(".qkvg"):   # entries in the q, k, v and gate row ranges
            K = base.shape[1]
            starts = [0, cfg.q_dim, cfg.q_dim + cfg.kv_dim, cfg.q_dim + 2 * cfg.kv_dim]
            rows = [s + int(rng.integers(0, max(1, e - s))) for s, e in
                    zip(starts, starts[1:] + [cfg.qkvg_dim]) if e > s]
            idx = [r * K + int(rng.integers(0, K)) for r in rows for _ in range(2)]
        else:
            idx = list(rng.choice(flat.size, size=6, replace=False))
        for i in idx:
            wp = dict(w)
            wm = dict(w)
            p = base.copy().reshape(-1)
            m = base.copy().reshape(-1)
            p[i] += eps
            m[i] -= eps
            wp[name] = p.reshape(base.shape)
            wm[name] = m.reshape(base.shape)
            num = (bw.loss(cfg, wp, x, G) - bw.loss(cfg, wm, x, G)) / (2 * eps)
            a = ana.reshape(-1)[i]
            assert abs(num - a) <= 1e-7 + 1e-6 * abs(a), (name, i, num, a)
            checked += 1
    # and the input
    dx = grads["x"].reshape(-1)
    for i in rng.choice(x.size, size=8, replace=False):
        xp = x.copy().reshape(-1)
        xm = x.copy().reshape(-1)
        xp[i] += eps
        xm[i] -= eps
        num = (bw.loss(cfg, w, xp.reshape(x.shape), G) - bw.loss(cfg, w, xm.reshape(x.shape), G)) / (2 * eps)
        assert abs(num - dx[i]) <= 1e-7 + 1e-6 * abs(dx[i]), ("x", i, num, dx[i])
        checked += 1
    assert checked > 40
    # every gradient of the block is non-trivial
    for l in range(cfg.n_in, cfg.n_in + cfg.n_rec):
        for p in ("qkvg", "o", "ug", "down", "alpha_a", "alpha_m"):
            assert np.max(np.abs(grads[f"L{l}.{p}"])) > 1e-4


def test_forward_equals_inference_layers():
    cfg, w, x, G = _setup(1)
    h_out, _ = bw.block_forward(cfg, w, x)
    ora = LoopedNGPT(cfg, w, compute="f64", bf16_points=False, max_ctx=16, batch=x.shape[0])
    ora.kv_mode = "per_loop"
    h = x.copy()
    pos = np.arange(x.shape[1])
    for l in range(cfg.n_in, cfg.n_in + cfg.n_rec):
        h = ora.layer(l, h, pos, (l, 1))
    h = h / np.linalg.norm(h, axis=-1, keepdims=True)
    np.testing.assert_allclose(h_out, h, rtol=0, atol=1e-12)


def test_alpha_zero_closed_form():
    """alpha = 0 makes every update the identity on unit rows: the block is
    norm(x), so dW = 0, dalpha is the only signal, and dx = G - x (x . G)."""
    cfg, w, x, G = _setup(1, alpha=False)
    grads = bw.block_backward(cfg, w, x, G)
    for l in range(cfg.n_in, cfg.n_in + cfg.n_rec):
        for p in ("qkvg", "o", "ug", "down"):
            np.testing.assert_allclose(grads[f"L{l}.{p}"], 0.0, atol=1e-14)
    expect = G - x * np.sum(x * G, axis=-1, keepdims=True)
    np.testing.assert_allclose(grads["x"], expect, atol=1e-12)
    # d/dalpha at 0: sum over rows of dz * (norm(y) - h), with dz the projected G
    assert np.max(np.abs(grads[f"L{cfg.n_in}.alpha_a"])) > 1e-3
