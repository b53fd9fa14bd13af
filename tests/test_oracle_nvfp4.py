"""Pins of the NVFP4-style weight format of oracle/nvfp4.py (reading R20):
E2M1 values from the OCP bit fields, element rounding at and between every
midpoint, the MSE scale choice against exact rational arithmetic, blocks that
a known scale represents exactly, the tensor scale, the comparison with the
plain amax/6 scale, bfloat16 exactness of the stored products, packing."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import mxfp8, nvfp4
from synth.gen import f32_to_bf16_bits, bf16_bits_to_f32

GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
E4M3 = [Fraction(mxfp8.e4m3_value(c)) for c in range(1, 127)]


def test_e2m1_values():
    assert [nvfp4.e2m1_value(c) for c in range(8)] == GRID
    assert [nvfp4.e2m1_value(c) for c in range(8, 16)] == [-v for v in GRID]
    assert np.signbit(nvfp4.e2m1_value(8))


@pytest.mark.parametrize("S", [1.0, 0.3, 2.0 ** -20 * 1.375, 12345.678])
def test_magnitude_index_midpoints(S):
    S = float(S)
    for j in range(8):
        assert nvfp4.magnitude_index(np.array([GRID[j] * S]), S)[0] == j          # grid points
    for j in range(7):
        mid = (GRID[j] + GRID[j + 1]) / 2
        even = j if j % 2 == 0 else j + 1
        assert nvfp4.magnitude_index(np.array([mid * S]), S)[0] == even            # exact ties
        lo, hi = np.nextafter(mid * S, 0.0), np.nextafter(mid * S, np.inf)
        assert nvfp4.magnitude_index(np.array([lo]), S)[0] == j
        assert nvfp4.magnitude_index(np.array([hi]), S)[0] == j + 1
    assert nvfp4.magnitude_index(np.array([7.0 * S, 1e300]), S).tolist() == [7, 7]  # saturation


def _nearest_exact(a: Fraction, S: Fraction) -> Fraction:
    """E2M1 magnitude nearest to a / S, exact rationals, ties to the even code."""
    x = a / S
    best = None
    for j, m in enumerate(GRID):
        d = abs(x - Fraction(m))
        if best is None or d < best[0] or (d == best[0] and j % 2 == 0):
            best = (d, j, m)
    return Fraction(best[2])


def test_scale_choice_is_least_exact_squared_error():
    rng = np.random.default_rng(5)
    g = np.float32(0.0123)
    blocks = rng.standard_normal((12, 16)) * np.exp(rng.uniform(-3, 3, (12, 1)))
    blocks = bf16_bits_to_f32(f32_to_bf16_bits(blocks.astype(np.float32))).astype(np.float64)
    chosen = nvfp4.choose_scales(np.abs(blocks), g)
    for b in range(blocks.shape[0]):
        a = [Fraction(abs(float(v))) for v in blocks[b]]
        errs = []
        for s in E4M3:
            S = s * Fraction(float(g))
            errs.append(sum((ai - _nearest_exact(ai, S) * S) ** 2 for ai in a))
        best = min(errs)
        got = errs[chosen[b] - 1]
        assert got <= best * (1 + Fraction(1, 10 ** 12))
        if sorted(errs)[1] > best * (1 + Fraction(1, 10 ** 9)):      # a clear winner: the same code
            assert chosen[b] - 1 == errs.index(best)


def test_blocks_a_scale_represents_exactly():
    s0 = mxfp8.e4m3_value(0x38)                       # 1.0, code 56
    half = mxfp8.e4m3_value(0x30)                     # 0.5, code 48
    g = np.float32(1.0)
    w = np.zeros((3, 32))
    w[0, :16] = s0 * np.array([6, 4, 3, 2, 1.5, 1, 0.5, 0, -6, -4, -3, -2, -1.5, -1, -0.5, -0.0])
    w[1, :16] = 0.0
    w[1, 0], w[1, 1] = 6 * s0, 3 * s0                 # also exact at 1.5*s0 and 2*s0: smallest code wins
    w[2, :16] = 3 * s0                                # exact at s0/2 (6), s0 (3), 2*s0 (1.5), 3/4*s0 (4) ...
    w[0, 16:] = w[0, :16] * 2.0 ** -7                 # exact at s0 * 2^-7
    q, sc, gg = nvfp4.quantize(w, g)
    assert gg == 1.0
    assert sc[0, 0] == 56 and sc[1, 0] == 56
    # 3*s0 = 6 * 0.5 = 4 * 0.75 = 3 * 1: the smallest code with zero error is 0.5 (code 48)
    assert sc[2, 0] == 48 and half == 0.5
    assert sc[0, 1] == 4 and mxfp8.e4m3_value(4) == 2.0 ** -7   # 2^-7 is the subnormal 4/8 * 2^-6
    assert sc[1, 1] == 1 and sc[2, 1] == 1            # all-zero blocks: code 1
    d = nvfp4.dequantize(q, sc, gg)
    np.testing.assert_array_equal(d, w)
    np.testing.assert_array_equal(np.signbit(d[0, :16]), np.signbit(w[0, :16]))


def test_packing_order_and_signs():
    w = np.zeros((1, 16))
    w[0, 0], w[0, 1], w[0, 2], w[0, 3] = 0.5, -6.0, -0.0, 1.5
    w[0, 4:] = 6.0
    q, sc, g = nvfp4.quantize(w, np.float32(1.0))
    assert sc[0, 0] == 0x38                           # 1.0
    # element 0 (0.5: code 1) in the low nibble, element 1 (-6: code 15) in the high one
    assert q[0, 0] == (1 | (15 << 4))
    assert q[0, 1] == (8 | (3 << 4))                  # -0.0 -> sign-only code 8; 1.5 -> code 3
    assert np.all(q[0, 2:] == (7 | (7 << 4)))


def test_tensor_scale():
    assert nvfp4.tensor_scale(np.array([[2688.0, -1.0]])) == np.float32(1.0)
    assert nvfp4.tensor_scale(np.array([[0.0, -0.0]])) == np.float32(1.0)
    v = nvfp4.tensor_scale(np.array([[-3.0, 1.0]]))
    assert v == np.float32(3.0) / np.float32(2688.0) and v.dtype == np.float32
    # the largest block can take scale 448 exactly when amax / 2688 is exact
    w = np.zeros((1, 32))
    w[0, 0] = 2688.0 * 0.25
    q, sc, g = nvfp4.quantize(w)
    assert g == np.float32(0.25) and sc[0, 0] == 126 and nvfp4.dequantize(q, sc, g)[0, 0] == w[0, 0]


def test_never_worse_than_amax_over_6():
    """The plain choice s = e4m3(amax_b / (6 g)) is one of the candidates, so
    the searched error can only be smaller or equal."""
    rng = np.random.default_rng(9)
    w = rng.standard_normal((32, 64)) * np.exp(rng.uniform(-4, 1, (32, 1)))
    q, sc, g = nvfp4.quantize(w)
    a = np.abs(w).reshape(-1, 16)
    amax = a.max(axis=1)
    plain = mxfp8.e4m3_encode(np.minimum(amax / (6.0 * float(g)), 448.0))
    plain = np.maximum(plain, 1)
    S_plain = mxfp8.e4m3_decode(plain) * float(g)
    e_plain = nvfp4.block_error(a, S_plain)
    S_mse = mxfp8.e4m3_decode(sc.reshape(-1)) * float(g)
    e_mse = nvfp4.block_error(a, S_mse)
    assert np.all(e_mse <= e_plain)
    assert np.mean(e_mse < e_plain) > 0.3            # and strictly better on many blocks


def test_stored_products_are_bfloat16_values():
    prods = np.array([m * float(s) for m in GRID for s in E4M3])
    back = bf16_bits_to_f32(f32_to_bf16_bits(prods.astype(np.float32))).astype(np.float64)
    np.testing.assert_array_equal(back, prods)


def test_round_trip_error_bound():
    """Every element lands within half a grid step (relative to its block
    scale) or saturates; zero-error blocks come back exactly."""
    rng = np.random.default_rng(11)
    w = rng.standard_normal((16, 128)) * np.exp(rng.uniform(-6, 2, (16, 1)))
    q, sc, g = nvfp4.quantize(w)
    d = nvfp4.dequantize(q, sc, g)
    S = (mxfp8.e4m3_decode(sc).astype(np.float64) * float(g)).repeat(16, axis=1)
    x = np.abs(w) / S
    step = np.where(x < 2, 0.5, np.where(x < 4, 1.0, 2.0))
    sat = x > 6
    assert np.all((np.abs(np.abs(d) - np.abs(w)) <= step * S / 2 * (1 + 1e-12)) | sat)
    assert np.all(np.sign(d) * np.sign(w) >= 0)


def test_c_search_equals_numpy_search():
    """The C loops (oracle/c/nvfp4_search.c) choose the same codes as the numpy
    definition: random blocks over many binades, exact ties for several
    candidates, zero and single-element blocks."""
    rng = np.random.default_rng(13)
    w = rng.standard_normal((64, 256)) * np.exp(rng.uniform(-8, 3, (64, 1)))
    w = bf16_bits_to_f32(f32_to_bf16_bits(w.astype(np.float32))).astype(np.float64)
    w[0, :16] = 0.0
    w[1, :16] = 0.0
    w[1, 5] = -3.0
    for r, s in zip(range(2, 10), (0x38, 0x30, 0x3C, 0x20, 0x04, 0x41, 0x7E, 0x01)):
        w[r, :16] = np.array(GRID * 2)[:16] * mxfp8.e4m3_value(s)        # exact for scale s
        w[r, 16:23] = nvfp4._MIDS * mxfp8.e4m3_value(s)                   # ties for scale s
    for g in (nvfp4.tensor_scale(w), np.float32(1.0), np.float32(3e-3)):
        a = np.abs(w).reshape(-1, 16)
        np.testing.assert_array_equal(nvfp4.choose_scales_c(a, g), nvfp4.choose_scales(a, g))
    q1, s1, g1 = nvfp4.quantize(w)
    q2, s2, g2 = nvfp4.quantize(w, use_c=True)
    np.testing.assert_array_equal(q1, q2)
    np.testing.assert_array_equal(s1, s2)
    assert g1 == g2
