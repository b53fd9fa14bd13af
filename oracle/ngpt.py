"""Plain CPU forward pass of the looped normalized-GPT decoder (the oracle).

TEST INFRASTRUCTURE ONLY (see the package header). Numpy, float64 by default.

Sources. The pages describe one model, Dory1.0-4B:
  [S1] "Dory1.0-4B: A Looped Normalized-GPT", ai.info AI summary of the paper;
  [S4] "Dory 1.0 4B Benchmarks: How Do 1, 2 and 4 Loops Compare?", goremy.ai blog;
  [S5] "NVIDIA Nemotron Labs Dory 1.0 4B: a looped (latent-recurrent) LLM with
       elastic inference compute", broadside review of the model card.
What they fix:
  * input block once, shared recurrent block k times, output block once
    ([S1] Key Contributions 1; [S4] What is Dory1.0-4B?; [S5] One-sentence takeaway);
  * the recurrent block's output is L2-normalised and the input block's fixed
    output is re-injected before every pass ([S1] Methodology in Plain English);
  * nGPT residual updates that blend the normalised sublayer output with the
    normalised stream using learned per-channel weights, everything on the unit
    sphere; extra L2 norms of the concatenated gated attention output before the
    output projection and of the SwiGLU activation before the down projection
    ([S1] Methodology in Plain English);
  * sliding-window and full attention layers, grouped-query attention, RoPE
    with one base per layer type, input-dependent sigmoid output gates
    ([S1] Methodology in Plain English);
  * per-loop KV caching (one cache per loop) and last-loop caching (one cache
    per recurrent attention layer, each loop overwriting the previous loop's
    entries) ([S4] How does looping work at inference time?; [S5] Key ideas).

Readings where the pages are silent (each is a constructor argument or a
config field, so a different reading is one change away):
  R1  combine: x_1 = e, x_j = norm(wh*h_{j-1} + we*e) for j >= 2 (wh = we = 1),
      so k = 1 is the plain stack the model was pretrained as.
  R4  alpha is a per-channel vector (alpha_a, alpha_m per layer).
  R5  gate: sigmoid of a fourth slice of the fused projection, elementwise
      (attn_gate=1), one scalar per query head (2) or none (0).
  R7  nGPT eigen-scales s_qk = s_u = s_v = 1; attention logit scale sqrt(hd)
      (q and k are unit vectors); logit scale sqrt(d_model).
  R8  RoPE rotates the pairs (i, i + hd/2) by pos * base^(-2i/hd), angles in
      float64, absolute positions.
  R10 sliding window of W keys including the query itself: t-W < s <= t.
  R11 inside a call each loop writes its K/V for the call's positions, then
      attends; positions of earlier calls hold whatever the last write left.
  R14 per-loop mode needs one loop count for the whole sequence.
  R15 greedy argmax takes the lowest index on ties.
  R18 norm(x) = x / sqrt(max(sum x^2, 1e-30)).
bfloat16 storage points (bf16 models): the oracle computes in float64 and rounds
to bfloat16 (nearest-even) exactly where the stored tensor is bfloat16 - the
copies of h fed to the projections, the normalised q and k, v, the K/V cache,
the gated attention output and the SwiGLU activation. The residual stream h
stays in full precision.

Pinned by tests/test_oracle_pins.py (depth counts, hypersphere invariant,
mode equivalence at k=1, incremental == full recompute, attention == library
SDPA when the window covers the context, GQA == MHA with repeated heads,
alpha = 0 / 1 special cases, RoPE closed forms, weight orientation, brute-force
scalar forward on tiny shapes) and tests/test_oracle_kv.py (KV bytes).
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Tuple

import numpy as np

from synth.configs import ModelConfig
from synth.gen import bf16_bits_to_f32

PER_LOOP = "per_loop"
LAST_LOOP = "last_loop"


class OracleConfigError(ValueError):
    """A call that the readings above do not allow (R14, mode switch, overflow)."""


# ----------------------------------------------------------------------------
# elementary operations
# ----------------------------------------------------------------------------

def l2norm(x: np.ndarray, axis: int = -1) -> np.ndarray:
    """x / ||x||_2 along `axis` (R18 guard against a zero vector)."""
    ss = np.sum(x * x, axis=axis, keepdims=True)
    return x / np.sqrt(np.maximum(ss, 1e-30))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Value of x after storage as bfloat16 (via float32, nearest-even)."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(x.dtype)


def sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def silu(x: np.ndarray) -> np.ndarray:
    return x * sigmoid(x)


def rope_angles(positions: np.ndarray, head_dim: int, base: float) -> np.ndarray:
    """angle[p, i] = pos_p * base^(-2i/hd) for i < hd/2, in float64 (R8)."""
    half = head_dim // 2
    inv = base ** (-(2.0 * np.arange(half, dtype=np.float64)) / head_dim)
    return positions.astype(np.float64)[:, None] * inv[None, :]


def rope(x: np.ndarray, positions: np.ndarray, base: float) -> np.ndarray:
    """Rotate-half RoPE: pair (i, i+hd/2) rotated by the angle of position p.

    x: [..., n_pos, heads, hd] with the position axis third from the end.
    """
    hd = x.shape[-1]
    half = hd // 2
    ang = rope_angles(positions, hd, base)                 # [n, half]
    c = np.cos(ang)[:, None, :].astype(x.dtype)            # [n, 1, half]
    s = np.sin(ang)[:, None, :].astype(x.dtype)
    x1 = x[..., :half]
    x2 = x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def ngpt_update(h: np.ndarray, y: np.ndarray, alpha: np.ndarray) -> np.ndarray:
    """nGPT hypersphere step h <- norm(h + alpha * (norm(y) - h))."""
    return l2norm(h + alpha * (l2norm(y) - h))


def attention(q: np.ndarray, k_all: np.ndarray, v_all: np.ndarray, q_pos: np.ndarray,
              window: Optional[int], scale: float) -> np.ndarray:
    """Masked softmax attention for one sequence and one query head.

    q: [n, hd] at absolute positions q_pos; k_all, v_all: [T, hd] at positions
    0..T-1. Key s is allowed for query t iff s <= t and, for a sliding-window
    layer, t - s < window.
    """
    T = k_all.shape[0]
    s_pos = np.arange(T)
    allowed = s_pos[None, :] <= q_pos[:, None]
    if window is not None:
        allowed &= (q_pos[:, None] - s_pos[None, :]) < window
    scores = scale * (q @ k_all.T)
    scores = np.where(allowed, scores, -np.inf)
    m = np.max(scores, axis=1, keepdims=True)
    p = np.exp(scores - m)
    p /= np.sum(p, axis=1, keepdims=True)
    return p @ v_all


# ----------------------------------------------------------------------------
# the model
# ----------------------------------------------------------------------------

class LoopedNGPT:
    """Stateful oracle session: a KV cache plus a position counter.

    `call(tokens[B, n], n_loops, kv_mode)` processes n new positions of B
    sequences that share one position counter, exactly like one prefill chunk
    or one decode step of the library, and returns the logits of the last
    position (or of every position).
    """

    def __init__(self, cfg: ModelConfig, weights: Dict[str, np.ndarray], *,
                 compute: str = "f64", bf16_points: Optional[bool] = None,
                 max_ctx: int = 4096, batch: int = 1):
        self.cfg = cfg
        self.dt = {"f64": np.float64, "f32": np.float32}[compute]
        self.bf16 = (cfg.dtype == "bf16") if bf16_points is None else bool(bf16_points)
        self.max_ctx = max_ctx
        self.batch = batch
        self._w = weights
        self._wcache: Dict[str, np.ndarray] = {}
        self.reset()

    # weights are widened on first use (bfloat16 bit patterns widen exactly)
    def W(self, name: str) -> np.ndarray:
        if name not in self._wcache:
            raw = self._w[name]
            f = bf16_bits_to_f32(raw) if raw.dtype == np.uint16 else raw
            self._wcache[name] = np.ascontiguousarray(f, dtype=self.dt)
        return self._wcache[name]

    def reset(self) -> None:
        self.pos = 0
        self.kv_mode: Optional[str] = None
        self.seq_loops: Optional[int] = None
        self.cache: Dict[Tuple[int, int], Dict[str, np.ndarray]] = {}
        self.layer_apps_per_token: List[int] = []
        self.max_norm_dev = 0.0
        self.trace: Optional[Dict] = None

    # -- helpers ------------------------------------------------------------
    def _store(self, x: np.ndarray) -> np.ndarray:
        """Value after the library stores x in its activation dtype."""
        return round_bf16(x) if self.bf16 else x

    def _norm_check(self, h: np.ndarray) -> None:
        dev = float(np.max(np.abs(np.sqrt(np.sum(h.astype(np.float64) ** 2, axis=-1)) - 1.0)))
        self.max_norm_dev = max(self.max_norm_dev, dev)

    def cache_key(self, layer: int, loop: int) -> Tuple[int, int]:
        """Which cache a layer application uses: (layer, loop) for a recurrent
        layer in per-loop mode, (layer, 0) otherwise."""
        if self.cfg.is_recurrent(layer) and self.kv_mode == PER_LOOP:
            return (layer, loop)
        return (layer, 0)

    def _cache(self, key: Tuple[int, int]) -> Dict[str, np.ndarray]:
        if key not in self.cache:
            c = self.cfg
            shape = (self.batch, c.n_kv_heads, self.max_ctx, c.head_dim)
            self.cache[key] = {"K": np.full(shape, np.nan, dtype=self.dt),
                               "V": np.full(shape, np.nan, dtype=self.dt)}
        return self.cache[key]

    # -- one layer (attention sublayer + MLP sublayer) ---------------------
    def layer(self, l: int, h: np.ndarray, positions: np.ndarray, key: Tuple[int, int]) -> np.ndarray:
        c = self.cfg
        B, n, d = h.shape
        hd, nq, nkv = c.head_dim, c.n_q_heads, c.n_kv_heads
        full = c.layer_is_full[l]
        base = c.rope_base_full if full else c.rope_base_swa

        # fused projection [q | k | v | gate]
        qkvg = self._store(h) @ self.W(f"L{l}.qkvg").T
        q = qkvg[..., :c.q_dim].reshape(B, n, nq, hd)
        k = qkvg[..., c.q_dim:c.q_dim + c.kv_dim].reshape(B, n, nkv, hd)
        v = qkvg[..., c.q_dim + c.kv_dim:c.q_dim + 2 * c.kv_dim].reshape(B, n, nkv, hd)
        g = qkvg[..., c.q_dim + 2 * c.kv_dim:]

        # RoPE, then the per-head nGPT normalisation of q and k (s_qk = 1)
        q = self._store(l2norm(rope(q, positions, base)))
        k = self._store(l2norm(rope(k, positions, base)))
        v = self._store(v)

        # write this call's K/V (R11: write, then attend)
        cache = self._cache(key)
        p0, p1 = int(positions[0]), int(positions[-1]) + 1
        cache["K"][:, :, p0:p1, :] = np.transpose(k, (0, 2, 1, 3))
        cache["V"][:, :, p0:p1, :] = np.transpose(v, (0, 2, 1, 3))
        if self.trace is not None:
            self.trace.setdefault("kv_writes", []).append((l, key, p0, p1))

        window = None if full else c.window
        o = np.empty((B, n, nq, hd), dtype=self.dt)
        for b in range(B):
            for hq in range(nq):
                kvh = (hq * nkv) // nq
                o[b, :, hq, :] = attention(q[b, :, hq, :], cache["K"][b, kvh, :p1, :],
                                           cache["V"][b, kvh, :p1, :], positions, window,
                                           c.scale_attn)
        if c.attn_gate == 1:
            o = o * sigmoid(g.reshape(B, n, nq, hd))
        elif c.attn_gate == 2:
            o = o * sigmoid(g.reshape(B, n, nq, 1))
        o = l2norm(self._store(o.reshape(B, n, c.q_dim)))
        y = o @ self.W(f"L{l}.o").T
        h = ngpt_update(h, y, self.W(f"L{l}.alpha_a"))
        self._norm_check(h)

        uv = self._store(h) @ self.W(f"L{l}.ug").T
        a = uv[..., :c.d_ff] * silu(uv[..., c.d_ff:])
        a = l2norm(self._store(a))
        y = a @ self.W(f"L{l}.down").T
        h = ngpt_update(h, y, self.W(f"L{l}.alpha_m"))
        self._norm_check(h)
        return h

    # -- one call: n new positions ------------------------------------------
    def call(self, tokens: np.ndarray, n_loops: int, kv_mode: str, *,
             all_logits: bool = False, return_hidden: bool = False):
        c = self.cfg
        tokens = np.asarray(tokens)
        if tokens.ndim == 1:
            tokens = tokens[None, :]
        B, n = tokens.shape
        if B != self.batch:
            raise OracleConfigError("batch mismatch")
        if kv_mode not in (PER_LOOP, LAST_LOOP):
            raise OracleConfigError(f"unknown kv mode {kv_mode}")
        if n_loops < 1:
            raise OracleConfigError("n_loops must be >= 1")
        if self.kv_mode is not None and kv_mode != self.kv_mode:
            raise OracleConfigError("kv mode changed inside a sequence")
        if kv_mode == PER_LOOP and self.seq_loops is not None and n_loops != self.seq_loops:
            raise OracleConfigError("per-loop caching needs one loop count per sequence (R14)")
        if self.pos + n > self.max_ctx:
            raise OracleConfigError("context overflow")
        self.kv_mode = kv_mode
        if kv_mode == PER_LOOP:
            self.seq_loops = n_loops

        positions = np.arange(self.pos, self.pos + n)
        E = self.W("embed")
        h = l2norm(E[tokens])
        self._norm_check(h)
        apps = 0

        for l in range(c.n_in):                                   # input block, once
            h = self.layer(l, h, positions, self.cache_key(l, 0))
            apps += 1
        e = h                                                     # fixed re-injected input
        rec = range(c.n_in, c.n_in + c.n_rec)
        for j in range(1, n_loops + 1):                           # recurrent block, k times
            x = e if j == 1 else l2norm(c.combine_wh * h + c.combine_we * e)
            self._norm_check(x)
            for l in rec:
                x = self.layer(l, x, positions, self.cache_key(l, j))
                apps += 1
            h = l2norm(x)                                         # block output on the sphere
        for l in range(c.n_in + c.n_rec, c.n_layers):             # output block, once
            h = self.layer(l, h, positions, self.cache_key(l, 0))
            apps += 1

        self.layer_apps_per_token.append(apps)
        self.pos += n
        hs = h if all_logits else h[:, -1:, :]
        logits = c.scale_logit * (self._store(hs) @ E.T)
        out = logits if all_logits else logits[:, 0, :]
        if return_hidden:
            return out, h
        return out

    # -- greedy decoding ------------------------------------------------------
    @staticmethod
    def greedy(logits: np.ndarray) -> np.ndarray:
        """Index of the largest logit, lowest index on ties (R15)."""
        return np.argmax(logits, axis=-1).astype(np.int32)

    def generate(self, prompt: np.ndarray, steps: int, n_loops: int, kv_mode: str,
                 chunk: Optional[int] = None):
        """Prefill `prompt` [B, n] in chunks, then `steps` greedy decode calls.

        Returns (tokens [B, steps], logits [steps, B, V]) where logits[i] are
        the logits that chose tokens[:, i].
        """
        prompt = np.asarray(prompt)
        if prompt.ndim == 1:
            prompt = prompt[None, :]
        n = prompt.shape[1]
        chunk = n if chunk is None else chunk
        logits = None
        for s in range(0, n, chunk):
            logits = self.call(prompt[:, s:s + chunk], n_loops, kv_mode)
        toks, all_l = [], []
        for _ in range(steps):
            t = self.greedy(logits)
            toks.append(t)
            all_l.append(logits)
            logits = self.call(t[:, None], n_loops, kv_mode)
        return np.stack(toks, axis=1), np.stack(all_l, axis=0)

    def teacher_forced(self, prompt: np.ndarray, forced: np.ndarray, n_loops: int, kv_mode: str,
                       chunk: Optional[int] = None) -> np.ndarray:
        """Prefill, then decode feeding `forced` [B, steps]; returns logits
        [steps + 1, B, V] (after the prompt, then after each forced token)."""
        prompt = np.asarray(prompt)
        if prompt.ndim == 1:
            prompt = prompt[None, :]
        forced = np.asarray(forced)
        if forced.ndim == 1:
            forced = forced[None, :]
        n = prompt.shape[1]
        chunk = n if chunk is None else chunk
        for s in range(0, n, chunk):
            logits = self.call(prompt[:, s:s + chunk], n_loops, kv_mode)
        out = [logits]
        for i in range(forced.shape[1]):
            out.append(self.call(forced[:, i:i + 1], n_loops, kv_mode))
        return np.stack(out, axis=0)


def effective_depth(cfg: ModelConfig, n_loops: int) -> int:
    """Layer applications per token: n_in + n_out + k * n_rec."""
    return cfg.n_in + cfg.n_out + n_loops * cfg.n_rec
