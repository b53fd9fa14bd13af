"""MXFP8 weights: blocks of 32 values with one shared power-of-two scale.

TEST INFRASTRUCTURE ONLY (see the package header).

The pages name MXFP8 checkpoints of the model ("Dory1.0-4B: A Looped
Normalized-GPT", AI summary, Key Contributions 4; "NVIDIA Nemotron Labs Dory
1.0 4B" review, Key ideas) but do not define the format. Reading taken (R19):
the OCP Microscaling (MX) v1.0 definition of MXFP8 with E4M3 elements:

- a block is 32 consecutive weights of one output row along the contraction
  dimension K (K a multiple of 32);
- the block's shared scale is X = floor(log2(max |w|)) - 8, where 8 is the
  exponent of the largest E4M3 normal (448 = 1.75 * 2^8), kept in [-127, 127]
  and stored as the E8M0 byte X + 127; an all-zero block stores byte 0;
- each element is w / 2^X rounded to the nearest E4M3 value (ties to the even
  code), magnitudes beyond 448 saturating to 448; E4M3 = 1 sign bit, 4
  exponent bits (bias 7), 3 mantissa bits, subnormals below 2^-6, no
  infinities, S.1111.111 = NaN (never produced);
- the stored weight stands for e4m3(q) * 2^X.

Pinned by tests/test_oracle_mxfp8.py: code values from the bit fields, the
encoder against torch's float8_e4m3fn cast on every tie and subnormal within
the finite range, saturation, scale exponents of exact powers of two, zero
blocks, the round-trip error bound, and exact representability of every
dequantised weight in bfloat16.
"""
from __future__ import annotations

import numpy as np

BLOCK = 32
E4M3_MAX = 448.0
EMAX_ELEM = 8


def e4m3_value(code: int) -> float:
    """Value of an E4M3 code from its bit fields (NaN for S.1111.111)."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * (m / 8.0) * 2.0 ** -6
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
_POS = _TABLE[:127]          # codes 0x00..0x7E: 0 .. 448, strictly increasing


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Round to the nearest E4M3 code, ties to the even code, saturating at
    448; the sign bit is the sign of x (so -0.0 and tiny negatives give 0x80)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_POS, a, side="left")          # first code with value >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _POS[lo]
    dhi = _POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(_POS[hi] == a, hi, code)             # exact values
    sign = np.signbit(x).astype(np.uint8) << 7
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def block_scale_exponent(amax: np.ndarray) -> np.ndarray:
    """X = floor(log2(amax)) - 8 (exact, via frexp), clamped to [-127, 127];
    -127 for an all-zero block."""
    amax = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(amax)                 # amax = f * 2^e, f in [0.5, 1)
    X = (e - 1) - EMAX_ELEM
    X = np.where(amax > 0, X, -127)
    return np.clip(X, -127, 127).astype(np.int64)


def quantize(w: np.ndarray):
    """w [N, K] (K % 32 == 0) -> (codes uint8 [N, K], scale bytes uint8 [N, K/32])."""
    w = np.asarray(w, dtype=np.float64)
    N, K = w.shape
    if K % BLOCK:
        raise ValueError("K must be a multiple of 32")
    blocks = w.reshape(N, K // BLOCK, BLOCK)
    X = block_scale_exponent(np.max(np.abs(blocks), axis=-1))
    q = e4m3_encode(blocks / np.ldexp(1.0, X)[..., None])
    return q.reshape(N, K), (X + 127).astype(np.uint8)


def dequantize(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Values the stored weights stand for (float64)."""
    q = np.asarray(q, dtype=np.uint8)
    N, K = q.shape
    X = s.astype(np.int64) - 127
    v = e4m3_decode(q).reshape(N, K // BLOCK, BLOCK) * np.ldexp(1.0, X)[..., None]
    return v.reshape(N, K)
