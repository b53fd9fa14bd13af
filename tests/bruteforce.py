"""Scalar, loop-by-loop forward of the looped nGPT for tiny shapes.

An independent second reading of the same pages, used only to pin the
oracle: plain Python floats and `math`, one dot product at a time, a cache
keyed by (layer, loop-or-0, position), attention masks written as explicit
position tests. It shares no code with oracle/ (only the weights, as data).
"""
from __future__ import annotations

import math
from typing import Dict, List, Tuple


def _norm(x: List[float]) -> List[float]:
    s = math.sqrt(max(sum(t * t for t in x), 1e-30))
    return [t / s for t in x]


def _matvec(W: List[List[float]], x: List[float]) -> List[float]:
    # W is [out][in]
    return [sum(W[r][c] * x[c] for c in range(len(x))) for r in range(len(W))]


def _sig(x: float) -> float:
    return 1.0 / (1.0 + math.exp(-x))


class Brute:
    def __init__(self, cfg, weights):
        self.c = cfg
        tolist = lambda a: [[float(v) for v in row] for row in a]
        self.E = tolist(weights["embed"])
        self.L = []
        for l in range(cfg.n_layers):
            self.L.append(dict(
                qkvg=tolist(weights[f"L{l}.qkvg"]), o=tolist(weights[f"L{l}.o"]),
                ug=tolist(weights[f"L{l}.ug"]), down=tolist(weights[f"L{l}.down"]),
                aa=[float(v) for v in weights[f"L{l}.alpha_a"]],
                am=[float(v) for v in weights[f"L{l}.alpha_m"]]))
        self.cache: Dict[Tuple[int, int, int], Tuple[List[List[float]], List[List[float]]]] = {}
        self.pos = 0

    def _rope(self, x: List[float], p: int, base: float) -> List[float]:
        hd = len(x)
        half = hd // 2
        out = list(x)
        for i in range(half):
            ang = p * base ** (-2.0 * i / hd)
            c, s = math.cos(ang), math.sin(ang)
            out[i] = x[i] * c - x[i + half] * s
            out[i + half] = x[i + half] * c + x[i] * s
        return out

    def _layer(self, l: int, hs: List[List[float]], p0: int, loopkey: int) -> List[List[float]]:
        c, w = self.c, self.L[l]
        hd, nq, nkv = c.head_dim, c.n_q_heads, c.n_kv_heads
        base = c.rope_base_full if c.layer_is_full[l] else c.rope_base_swa
        n = len(hs)
        Qs, Gs = [], []
        for t in range(n):
            z = _matvec(w["qkvg"], hs[t])
            p = p0 + t
            q = [_norm(self._rope(z[hh * hd:(hh + 1) * hd], p, base)) for hh in range(nq)]
            off = nq * hd
            k = [_norm(self._rope(z[off + hh * hd: off + (hh + 1) * hd], p, base)) for hh in range(nkv)]
            off += nkv * hd
            v = [z[off + hh * hd: off + (hh + 1) * hd] for hh in range(nkv)]
            off += nkv * hd
            self.cache[(l, loopkey, p)] = (k, v)
            Qs.append(q)
            Gs.append(z[off:])
        out = []
        for t in range(n):
            p = p0 + t
            o_cat = []
            for hh in range(nq):
                kvh = hh // (nq // nkv)
                keys = []
                for s in range(0, p + 1):
                    if not c.layer_is_full[l] and p - s >= c.window:
                        continue
                    keys.append(s)
                sc = []
                for s in keys:
                    ks, _ = self.cache[(l, loopkey, s)]
                    sc.append(c.scale_attn * sum(Qs[t][hh][i] * ks[kvh][i] for i in range(hd)))
                m = max(sc)
                ex = [math.exp(x - m) for x in sc]
                z = sum(ex)
                o = [0.0] * hd
                for e_, s in zip(ex, keys):
                    _, vs = self.cache[(l, loopkey, s)]
                    for i in range(hd):
                        o[i] += e_ / z * vs[kvh][i]
                for i in range(hd):
                    if c.attn_gate == 1:
                        o[i] *= _sig(Gs[t][hh * hd + i])
                    elif c.attn_gate == 2:
                        o[i] *= _sig(Gs[t][hh])
                o_cat += o
            o_cat = _norm(o_cat)
            y = _norm(_matvec(w["o"], o_cat))
            h = hs[t]
            h = _norm([h[i] + w["aa"][i] * (y[i] - h[i]) for i in range(len(h))])
            uv = _matvec(w["ug"], h)
            ff = c.d_ff
            a = _norm([uv[i] * (uv[ff + i] * _sig(uv[ff + i])) for i in range(ff)])
            y = _norm(_matvec(w["down"], a))
            h = _norm([h[i] + w["am"][i] * (y[i] - h[i]) for i in range(len(h))])
            out.append(h)
        return out

    def call(self, tokens: List[int], k: int, per_loop: bool) -> List[float]:
        c = self.c
        p0 = self.pos
        hs = [_norm(list(self.E[t])) for t in tokens]
        for l in range(c.n_in):
            hs = self._layer(l, hs, p0, 0)
        e = hs
        h = None
        for j in range(1, k + 1):
            if j == 1:
                x = [list(r) for r in e]
            else:
                x = [_norm([c.combine_wh * h[t][i] + c.combine_we * e[t][i] for i in range(c.d_model)])
                     for t in range(len(tokens))]
            for l in range(c.n_in, c.n_in + c.n_rec):
                x = self._layer(l, x, p0, j if per_loop else 0)
            h = [_norm(r) for r in x]
        for l in range(c.n_in + c.n_rec, c.n_layers):
            h = self._layer(l, h, p0, 0)
        self.pos += len(tokens)
        last = h[-1]
        return [c.scale_logit * sum(last[i] * row[i] for i in range(c.d_model)) for row in self.E]
