"""NVFP4-style 4-bit weights with a dynamic MSE choice of each block's scale.

TEST INFRASTRUCTURE ONLY (see the package header).

The pages name NVFP4 checkpoints of the model and say that their block scales
are chosen dynamically by minimum squared error over the 126 positive E4M3
values ("Dory1.0-4B: A Looped Normalized-GPT", AI summary, Methodology in
Plain English: post-training; Key Contributions 4). They do not define the
format. Reading taken (R20), the published NVFP4 layout:

- a block is 16 consecutive weights of one output row along the contraction
  dimension K;
- each element is an E2M1 code (1 sign bit, 2 exponent bits with bias 1, 1
  mantissa bit): magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; two codes per byte,
  the even element in the low nibble;
- each block has one E4M3 scale byte (a positive finite E4M3 value, codes
  1..126), and each tensor one float32 scale g; element code q of block scale
  s stands for e2m1(q) * e4m3(s) * g;
- g = float32(amax / 2688) with amax = max |w| over the tensor (2688 = 6 * 448:
  a block scale of 448 then reaches the tensor's largest magnitude); an
  all-zero tensor takes g = 1;
- for each block, every one of the 126 candidate scales s is tried: with
  S = e4m3(s) * g, each |w| is rounded to the nearest E2M1 magnitude of |w| / S
  (ties to the even code, saturating at 6) by exact comparison of |w| with
  S times the midpoints 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5 (products exact in
  float64), and the block's error is accumulated in float64 in element order
  as err = ((e_0^2 + e_1^2) + e_2^2) + ..., e_i = |w_i| - m_i * S; the
  candidate of least error is kept, the smallest code on equal errors (so an
  all-zero block stores code 1);
- the element's sign bit is the sign bit of w (-0.0 -> code 8).

Where floating point decides the integer codes, the decision is taken in
float64 with this exact order of operations on both sides.

Pinned by tests/test_oracle_nvfp4.py: E2M1 values from the bit fields, the
element rounding at every midpoint and between them, the scale choice against
exact rational squared errors (fractions) on small blocks, blocks that a
known scale represents exactly (zero error, smallest such code), the tensor
scale, that the choice is never worse than the amax/6 scale rounded to E4M3,
bfloat16 exactness of e2m1 * e4m3, and the packing order; the C search
(choose_scales_c, oracle/c/nvfp4_search.c) against this numpy search.
"""
from __future__ import annotations

import numpy as np

from oracle import mxfp8

BLOCK = 16
E2M1_MAX = 6.0
TENSOR_DIV = 2688.0          # 6 * 448
_MIDS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


def e2m1_value(code: int) -> float:
    """Value of an E2M1 code from its bit fields."""
    s = -1.0 if code & 0x8 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        return s * 0.5 * m                      # subnormal: m * 2^(1-1) * 0.5
    return s * (1.0 + 0.5 * m) * 2.0 ** (e - 1)


_E2M1 = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
_MAG = _E2M1[:8]                                # 0, .5, 1, 1.5, 2, 3, 4, 6
_E4M3_POS = np.array([mxfp8.e4m3_value(c) for c in range(1, 127)], dtype=np.float64)


def magnitude_index(a: np.ndarray, S) -> np.ndarray:
    """Index 0..7 of the E2M1 magnitude nearest to a / S (a >= 0, S > 0),
    ties to the even index, saturating at 7 (6.0). Exact: compares a with the
    products S * midpoint, which float64 holds exactly."""
    a = np.asarray(a, dtype=np.float64)
    T = np.asarray(S, dtype=np.float64)[..., None] * _MIDS       # thresholds between index j and j+1
    idx = np.zeros((), dtype=np.int64)
    for j in range(7):
        t = T[..., j]
        if t.ndim < a.ndim:
            t = t[..., None]
        idx = idx + (a > t).astype(np.int64)
        if j % 2 == 1:                         # a tie between j (odd) and j+1 (even) goes up
            idx = idx + (a == t).astype(np.int64)
    return idx


def tensor_scale(w: np.ndarray) -> np.float32:
    amax = np.float32(np.max(np.abs(np.asarray(w, dtype=np.float32)))) if np.size(w) else np.float32(0)
    if amax == 0:
        return np.float32(1.0)
    return np.float32(amax / np.float32(TENSOR_DIV))             # float32 division, correctly rounded


def block_error(a: np.ndarray, S) -> np.ndarray:
    """Squared error of blocks a [..., 16] (magnitudes) at scales S [...],
    float64, summed in element order."""
    S = np.asarray(S, dtype=np.float64)
    idx = magnitude_index(a, S)
    e = a - _MAG[idx] * S[..., None]
    err = np.zeros(a.shape[:-1], dtype=np.float64)
    for i in range(a.shape[-1]):
        err = err + e[..., i] * e[..., i]
    return err


def choose_scales(a: np.ndarray, g) -> np.ndarray:
    """E4M3 code (1..126) of least block_error for each block of a [nb, 16]:
    all 126 candidates at once for 64 blocks at a time; argmin takes the first
    (smallest) code among equal errors."""
    S = (_E4M3_POS * float(g))[:, None]                          # [126, 1], exact products
    best = np.zeros(a.shape[0], dtype=np.int64)
    for i0 in range(0, a.shape[0], 64):
        part = a[None, i0:i0 + 64]                             # [1, nb', 16]
        err = block_error(part, np.broadcast_to(S, (126, part.shape[1])))   # [126, nb']
        best[i0:i0 + 64] = np.argmin(err, axis=0) + 1
    return best


def choose_scales_c(a: np.ndarray, g) -> np.ndarray:
    """choose_scales by the plain C loops of oracle/c/nvfp4_search.c (the
    same definition; for tensors too large for numpy to finish in seconds)."""
    from oracle import native
    a = np.ascontiguousarray(a, dtype=np.float64)
    out = np.zeros(a.shape[0], dtype=np.int32)
    native.lib().nvfp4_choose_scales(a.ctypes.data, a.shape[0], float(g), out.ctypes.data)
    return out.astype(np.int64)


def quantize(w: np.ndarray, g=None, use_c: bool = False):
    """w [N, K] (K % 16 == 0) -> (codes uint8 [N, K/2], scale codes uint8
    [N, K/16], tensor scale float32). g: the tensor scale to use (default:
    from w; given when only some rows of a tensor are quantised). use_c: the
    scale search in C (choose_scales_c)."""
    w = np.asarray(w, dtype=np.float64)
    N, K = w.shape
    if K % BLOCK:
        raise ValueError("K must be a multiple of 16")
    if g is None:
        g = tensor_scale(w)
    blocks = w.reshape(N * K // BLOCK, BLOCK)
    a = np.abs(blocks)
    sc = choose_scales_c(a, g) if use_c else choose_scales(a, g)
    S = _E4M3_POS[sc - 1] * float(g)
    idx = magnitude_index(a, S)
    q = (idx | (np.signbit(blocks).astype(np.int64) << 3)).reshape(N, K)
    packed = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    return packed, sc.reshape(N, K // BLOCK).astype(np.uint8), np.float32(g)


def unpack(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    q = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    q[:, 0::2] = p & 0xF
    q[:, 1::2] = p >> 4
    return q


def dequantize(packed: np.ndarray, scales: np.ndarray, g, with_tensor_scale: bool = True) -> np.ndarray:
    """Values the stored weights stand for (float64, exact): e2m1 * e4m3 * g,
    or e2m1 * e4m3 alone (with_tensor_scale=False)."""
    q = unpack(packed)
    N, K = q.shape
    s = mxfp8.e4m3_decode(scales).astype(np.float64)
    v = _E2M1[q].reshape(N, K // BLOCK, BLOCK) * s[..., None]
    if with_tensor_scale:
        v = v * float(g)
    return v.reshape(N, K)
