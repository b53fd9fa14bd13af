"""Depth-1 truncated backward of the last recurrent invocation.

TEST INFRASTRUCTURE ONLY (see the package header).

The pages say the looped stage is trained with backpropagation truncated to
depth one: only the final invocation of the recurrent block is trained
("Dory1.0-4B: A Looped Normalized-GPT", AI summary, Methodology in Plain
English). Reading taken (R21): for one training chunk of B sequences of n
positions starting at position 0,

    h_out = norm(R(x)),   R = the n_rec recurrent layers in order,

where x [B, n, d] is the last invocation's input (the re-injected
norm(w_h h + w_e e), taken as a constant: the truncation stops there) and
each layer is the forward of oracle/ngpt.py (attention sublayer and SwiGLU
sublayer, each closed by the nGPT update), with attention over the chunk's
own positions (causal, and t - s < W in sliding-window layers). Given a
synthetic upstream gradient G = dL/dh_out, the backward returns dL/dW for
the four projections and dL/d(alpha_A, alpha_M) of every recurrent layer and
dL/dx. Everything is float64 without the library's bfloat16 storage points:
this is the exact gradient of the exact forward.

Pinned by tests/test_oracle_backward.py: central finite differences of
L = sum(G * h_out) for sampled entries of every gradient (three gate modes,
a window shorter than the chunk, grouped-query heads), the forward against
LoopedNGPT's own layers, and the alpha = 0 closed form (R is then the
identity on unit rows: dW = 0, dx = G - x (x . G)).
"""
from __future__ import annotations

from typing import Dict, List, Optional

import numpy as np

from oracle.ngpt import rope_angles, sigmoid, silu
from synth.configs import ModelConfig
from synth.gen import bf16_bits_to_f32


def _w(weights: Dict[str, np.ndarray], name: str) -> np.ndarray:
    raw = weights[name]
    f = bf16_bits_to_f32(raw) if raw.dtype == np.uint16 else raw
    return np.asarray(f, dtype=np.float64)


def _norm_fwd(x: np.ndarray):
    """y = x / ||x|| along the last axis; returns (y, r)."""
    r = np.sqrt(np.maximum(np.sum(x * x, axis=-1, keepdims=True), 1e-30))
    return x / r, r


def _norm_bwd(y: np.ndarray, r: np.ndarray, dy: np.ndarray) -> np.ndarray:
    """d/dx of y = x / ||x||: (dy - y (y . dy)) / r."""
    return (dy - y * np.sum(y * dy, axis=-1, keepdims=True)) / r


def _rope(x: np.ndarray, pos: np.ndarray, base: float, sign: float = 1.0) -> np.ndarray:
    """Rotate-half RoPE of x [M, heads, hd] at positions pos [M]; sign -1 is
    the transpose (rotation by the negative angle)."""
    hd = x.shape[-1]
    half = hd // 2
    ang = rope_angles(pos, hd, base)
    c = np.cos(ang)[:, None, :]
    s = sign * np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def _mask(n: int, window: Optional[int]) -> np.ndarray:
    t = np.arange(n)[:, None]
    s = np.arange(n)[None, :]
    allowed = s <= t
    if window is not None:
        allowed &= (t - s) < window
    return allowed


def layer_forward(cfg: ModelConfig, weights, l: int, h: np.ndarray, B: int, n: int):
    """One layer on h [B*n, d] (rows of B sequences, positions 0..n-1 each).
    Returns (h_out, tape)."""
    c = cfg
    M, d = h.shape
    hd, nq, nkv = c.head_dim, c.n_q_heads, c.n_kv_heads
    full = c.layer_is_full[l]
    base = c.rope_base_full if full else c.rope_base_swa
    pos = np.tile(np.arange(n), B)
    T: Dict[str, np.ndarray] = {"h": h}

    P1 = h @ _w(weights, f"L{l}.qkvg").T
    q = P1[:, :c.q_dim].reshape(M, nq, hd)
    k = P1[:, c.q_dim:c.q_dim + c.kv_dim].reshape(M, nkv, hd)
    v = P1[:, c.q_dim + c.kv_dim:c.q_dim + 2 * c.kv_dim].reshape(M, nkv, hd)
    g = P1[:, c.q_dim + 2 * c.kv_dim:]
    qn, rq = _norm_fwd(_rope(q, pos, base))
    kn, rk = _norm_fwd(_rope(k, pos, base))
    T.update(qn=qn, rq=rq, kn=kn, rk=rk, v=v, g=g, pos=pos, base=np.float64(base))

    allowed = _mask(n, None if full else c.window)
    o = np.zeros((M, nq, hd))
    P = np.zeros((B, nq, n, n))
    for b in range(B):
        rows = slice(b * n, (b + 1) * n)
        for hq in range(nq):
            kvh = (hq * nkv) // nq
            S = c.scale_attn * (qn[rows, hq] @ kn[rows, kvh].T)
            S = np.where(allowed, S, -np.inf)
            p = np.exp(S - S.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            P[b, hq] = p
            o[rows, hq] = p @ v[rows, kvh]
    T.update(o=o, P=P)

    if c.attn_gate == 1:
        sg = sigmoid(g.reshape(M, nq, hd))
    elif c.attn_gate == 2:
        sg = sigmoid(g.reshape(M, nq, 1))
    else:
        sg = np.ones((M, nq, 1))
    cg = (o * sg).reshape(M, c.q_dim)
    oh, rc = _norm_fwd(cg)
    T.update(sg=sg, oh=oh, rc=rc)

    y = oh @ _w(weights, f"L{l}.o").T
    yh, ry = _norm_fwd(y)
    aA = _w(weights, f"L{l}.alpha_a")
    h1, rz = _norm_fwd(h + aA * (yh - h))
    T.update(yh=yh, ry=ry, rz=rz, h1=h1)

    P2 = h1 @ _w(weights, f"L{l}.ug").T
    u, vv = P2[:, :c.d_ff], P2[:, c.d_ff:]
    s = u * silu(vv)
    a, rs = _norm_fwd(s)
    T.update(u=u, vv=vv, a=a, rs=rs)

    y2 = a @ _w(weights, f"L{l}.down").T
    y2h, ry2 = _norm_fwd(y2)
    aM = _w(weights, f"L{l}.alpha_m")
    h2, rz2 = _norm_fwd(h1 + aM * (y2h - h1))
    T.update(y2h=y2h, ry2=ry2, rz2=rz2, h2=h2)
    return h2, T


def layer_backward(cfg: ModelConfig, weights, l: int, T, dh2: np.ndarray, B: int, n: int):
    """Gradients of one layer given dL/d(output). Returns (dL/d(input), grads)."""
    c = cfg
    M = dh2.shape[0]
    hd, nq, nkv = c.head_dim, c.n_q_heads, c.n_kv_heads
    G: Dict[str, np.ndarray] = {}
    h, h1 = T["h"], T["h1"]

    # MLP sublayer update: h2 = norm(h1 + aM (norm(y2) - h1))
    aM = _w(weights, f"L{l}.alpha_m")
    dz2 = _norm_bwd(T["h2"], T["rz2"], dh2)
    dh1 = dz2 * (1.0 - aM)
    G[f"L{l}.alpha_m"] = np.sum(dz2 * (T["y2h"] - h1), axis=0)
    dy2 = _norm_bwd(T["y2h"], T["ry2"], dz2 * aM)
    Wd = _w(weights, f"L{l}.down")
    G[f"L{l}.down"] = dy2.T @ T["a"]
    da = dy2 @ Wd
    ds = _norm_bwd(T["a"], T["rs"], da)
    u, vv = T["u"], T["vv"]
    sv = sigmoid(vv)
    du = ds * vv * sv                                   # d(u silu(v))/du = silu(v)
    dvv = ds * u * sv * (1.0 + vv * (1.0 - sv))         # silu'(v) = s(v) (1 + v (1 - s(v)))
    dP2 = np.concatenate([du, dvv], axis=1)
    Wug = _w(weights, f"L{l}.ug")
    G[f"L{l}.ug"] = dP2.T @ h1
    dh1 = dh1 + dP2 @ Wug

    # attention sublayer update: h1 = norm(h + aA (norm(y) - h))
    aA = _w(weights, f"L{l}.alpha_a")
    dz = _norm_bwd(h1, T["rz"], dh1)
    dh = dz * (1.0 - aA)
    G[f"L{l}.alpha_a"] = np.sum(dz * (T["yh"] - h), axis=0)
    dy = _norm_bwd(T["yh"], T["ry"], dz * aA)
    Wo = _w(weights, f"L{l}.o")
    G[f"L{l}.o"] = dy.T @ T["oh"]
    doh = dy @ Wo
    dcg = _norm_bwd(T["oh"], T["rc"], doh).reshape(M, nq, hd)
    o, sg = T["o"], T["sg"]
    do = dcg * sg
    if c.attn_gate == 1:
        dg = (dcg * o * sg * (1.0 - sg)).reshape(M, c.q_dim)
    elif c.attn_gate == 2:
        dg = np.sum(dcg * o, axis=-1) * (sg * (1.0 - sg))[..., 0]
    else:
        dg = np.zeros((M, 0))

    # attention: o = softmax(scale qn kn^T) v, per sequence and query head
    qn, kn, v, P = T["qn"], T["kn"], T["v"], T["P"]
    dqn = np.zeros_like(qn)
    dkn = np.zeros_like(kn)
    dv = np.zeros_like(v)
    for b in range(B):
        rows = slice(b * n, (b + 1) * n)
        for hq in range(nq):
            kvh = (hq * nkv) // nq
            p = P[b, hq]
            dv[rows, kvh] += p.T @ do[rows, hq]
            dp = do[rows, hq] @ v[rows, kvh].T
            dS = p * (dp - np.sum(dp * p, axis=1, keepdims=True))
            dqn[rows, hq] += c.scale_attn * (dS @ kn[rows, kvh])
            dkn[rows, kvh] += c.scale_attn * (dS.T @ qn[rows, hq])
    dq = _rope(_norm_bwd(qn, T["rq"], dqn), T["pos"], float(T["base"]), sign=-1.0)
    dk = _rope(_norm_bwd(kn, T["rk"], dkn), T["pos"], float(T["base"]), sign=-1.0)
    dP1 = np.concatenate([dq.reshape(M, c.q_dim), dk.reshape(M, c.kv_dim), dv.reshape(M, c.kv_dim), dg], axis=1)
    Wq = _w(weights, f"L{l}.qkvg")
    G[f"L{l}.qkvg"] = dP1.T @ h
    dh = dh + dP1 @ Wq
    return dh, G


def block_forward(cfg: ModelConfig, weights, x: np.ndarray):
    """x [B, n, d] -> (h_out [B, n, d], tapes) for the recurrent block."""
    B, n, d = x.shape
    h = np.asarray(x, dtype=np.float64).reshape(B * n, d)
    tapes: List = []
    for l in range(cfg.n_in, cfg.n_in + cfg.n_rec):
        h, T = layer_forward(cfg, weights, l, h, B, n)
        tapes.append(T)
    h_out, r = _norm_fwd(h)                                  # the block output on the sphere
    tapes.append({"h_out": h_out, "r": r})
    return h_out.reshape(B, n, d), tapes


def block_backward(cfg: ModelConfig, weights, x: np.ndarray, G_out: np.ndarray) -> Dict[str, np.ndarray]:
    """Depth-1 backward: gradients of L = sum(G_out * h_out) with respect to
    the recurrent layers' projections and alphas, and to x ("x")."""
    B, n, d = x.shape
    _, tapes = block_forward(cfg, weights, x)
    last = tapes[-1]
    dh = _norm_bwd(last["h_out"], last["r"], np.asarray(G_out, dtype=np.float64).reshape(B * n, d))
    grads: Dict[str, np.ndarray] = {}
    for i, l in reversed(list(enumerate(range(cfg.n_in, cfg.n_in + cfg.n_rec)))):
        dh, g = layer_backward(cfg, weights, l, tapes[i], dh, B, n)
        grads.update(g)
    grads["x"] = dh.reshape(B, n, d)
    return grads


def loss(cfg: ModelConfig, weights, x: np.ndarray, G_out: np.ndarray) -> float:
    h_out, _ = block_forward(cfg, weights, x)
    return float(np.sum(np.asarray(G_out, dtype=np.float64) * h_out))
