"""Pins of the MXFP8 weight format of oracle/mxfp8.py (OCP MX v1.0 reading):
code values from the bit fields, the element encoder against torch's own
float8_e4m3fn cast, saturation, block scales of exact powers of two, zero
blocks, the round-trip error bound and bfloat16 representability."""
import numpy as np
import pytest

from oracle import mxfp8
from synth.gen import f32_to_bf16_bits, bf16_bits_to_f32

torch = pytest.importorskip("torch")


def test_code_values_from_bit_fields():
    assert mxfp8.e4m3_value(0x38) == 1.0
    assert mxfp8.e4m3_value(0x7E) == 448.0            # largest normal: 1.75 * 2^8
    assert mxfp8.e4m3_value(0x08) == 2.0 ** -6        # smallest normal
    assert mxfp8.e4m3_value(0x01) == 2.0 ** -9        # smallest subnormal
    assert mxfp8.e4m3_value(0x07) == 7 * 2.0 ** -9    # largest subnormal
    assert mxfp8.e4m3_value(0xB8) == -1.0
    assert np.isnan(mxfp8.e4m3_value(0x7F)) and np.isnan(mxfp8.e4m3_value(0xFF))
    assert mxfp8.e4m3_value(0x80) == 0.0 and np.signbit(mxfp8.e4m3_value(0x80))
    # the decode table agrees with torch's float8_e4m3fn on every code
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    np.testing.assert_array_equal(mxfp8.e4m3_decode(np.arange(256)), t)


def test_encoder_matches_torch_cast_within_range():
    """Every code value, every midpoint between neighbours (the ties), points a
    quarter of the way in, and random values, both signs, |x| <= 448."""
    pos = mxfp8.e4m3_decode(np.arange(127))
    mids = (pos[:-1] + pos[1:]) / 2
    quarter = pos[:-1] + (pos[1:] - pos[:-1]) / 4
    rnd = np.random.default_rng(0).uniform(0, 448, 20000).astype(np.float32).astype(np.float64)
    x = np.concatenate([pos, mids, quarter, rnd, [2.0 ** -11, 2.0 ** -10, 3 * 2.0 ** -10]])
    x = np.concatenate([x, -x])
    ours = mxfp8.e4m3_encode(x)
    theirs = torch.from_numpy(x).float().to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # x is exactly representable in float32 (all the points above are), so the
    # float32 detour of the reference does not move any tie
    assert np.all(x.astype(np.float32).astype(np.float64) == x)
    np.testing.assert_array_equal(ours, theirs)


def test_saturation_and_sign():
    assert mxfp8.e4m3_encode(np.array([448.0, 449.0, 464.0, 500.0, 1e30])).tolist() == [0x7E] * 5
    assert mxfp8.e4m3_encode(np.array([-1e9])).tolist() == [0xFE]
    assert mxfp8.e4m3_encode(np.array([-0.0, -1e-30, 0.0])).tolist() == [0x80, 0x80, 0x00]


def test_block_scales_and_zero_blocks():
    w = np.zeros((2, 64))
    w[0, :32] = np.linspace(-1.0, 1.0, 32)     # amax 1.0 = 2^0 -> X = -8
    w[0, 32] = 448.0                            # amax 448: floor(log2) = 8 -> X = 0
    w[1, :32] = 1.5                             # amax 1.5 -> X = -8; 1.5 * 256 = 384 is a code value
    q, s = mxfp8.quantize(w)
    assert s.tolist() == [[119, 127], [119, 0]]     # second block of row 1 is all zero
    assert q[0, 32] == 0x7E and q[0, 0] == mxfp8.e4m3_encode(np.array([-256.0]))[0]
    assert np.all(q[1, 32:] == 0)
    d = mxfp8.dequantize(q, s)
    assert d[1, 0] == 1.5 and d[0, 32] == 448.0 and d[0, 0] == -1.0 and d[0, 31] == 1.0
    assert np.all(d[1, 32:] == 0)


def test_round_trip_bound_and_bf16_exactness():
    rng = np.random.default_rng(3)
    w = rng.standard_normal((64, 256)) * np.exp(rng.uniform(-6, 2, (64, 1)))
    w[5, 40:72] = 0.0
    w[7, 0] = 1e-12                             # far below its block's scale: rounds to zero
    q, s = mxfp8.quantize(w)
    d = mxfp8.dequantize(q, s)
    X = (s.astype(np.int64) - 127).repeat(32, axis=1)
    # error <= half a step: the subnormal step 2^(X-9) below 2^(X-6), else a step of at most
    # |w| * 2^-3 (3 mantissa bits); elements above 448 * 2^X saturate (checked below)
    step = np.where(np.abs(d) < np.ldexp(1.0, X - 6), np.ldexp(1.0, X - 9), np.abs(w) * 2.0 ** -3)
    sat = np.abs(w) > 448.0 * np.ldexp(1.0, X)
    assert np.all((np.abs(d - w) <= step / 2 + 1e-300) | sat)
    # every stored weight is exactly a bfloat16 value
    assert np.all(bf16_bits_to_f32(f32_to_bf16_bits(d.astype(np.float32))).astype(np.float64) == d)
    # blocks whose max exceeds 448 * 2^X saturate (1.75 <= max / 2^(floor(log2 max)) < 2)
    wsat = np.zeros((1, 32))
    wsat[0, 0] = 1.9375                             # X = -8 -> 496 -> 448
    qs, ss = mxfp8.quantize(wsat)
    assert qs[0, 0] == 0x7E and mxfp8.dequantize(qs, ss)[0, 0] == 1.75
