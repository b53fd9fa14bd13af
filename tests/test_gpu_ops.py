"""Single-kernel GPU checks through the C ABI: the linear kernels (matrix-
vector, the two MFMA GEMMs and the simple tiled path, both epilogues) against a float64 numpy
product of the same stored values, and the greedy argmax bit for bit against
numpy.argmax (lowest index on ties)."""
import math

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import looped_ngpt_amd as dory  # noqa: E402
from synth.gen import f32_to_bf16_bits, bf16_bits_to_f32  # noqa: E402


def _dev(a: np.ndarray):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda()
    return torch.from_numpy(a).cuda()


CASES = [
    # dtype, M, N, K, epilogue, algo
    ("f32", 1, 683, 256, 0, 1), ("f32", 3, 1024, 683, 0, 1), ("f32", 8, 2048, 256, 0, 1),
    ("f32", 2, 2 * 683, 256, 1, 1), ("f32", 130, 683, 256, 0, 2), ("f32", 70, 2 * 683, 256, 1, 2),
    ("bf16", 1, 8192, 3072, 0, 1), ("bf16", 1, 3072, 8192, 0, 1), ("bf16", 4, 1000, 3072, 0, 1),
    ("bf16", 1, 2 * 8192, 3072, 1, 1), ("bf16", 5, 2 * 1000, 2304, 1, 1), ("bf16", 1, 3072, 2304, 0, 1),
    # batch 1, long rows: each output's K range on two waves (8 or 6 chunks), a ragged last workgroup
    ("bf16", 1, 2304, 6144, 0, 1), ("bf16", 1, 1001, 8192, 0, 1), ("bf16", 1, 7, 5640, 0, 1),
    ("bf16", 130, 1000, 3072, 0, 2), ("bf16", 256, 8192, 3072, 0, 2), ("bf16", 200, 2 * 1000, 3072, 1, 2),
    ("bf16", 64, 3072, 8192, 0, 2), ("bf16", 33, 2304, 2304, 0, 2), ("bf16", 97, 2 * 6144, 2304, 1, 2),
    # 9..64 rows: the weight-streaming GEMM (eight waves below 512 workgroups, four from there; the
    # SwiGLU epilogue; a K range of one 128-deep batch per wave; ragged M and N)
    ("bf16", 64, 2 * 8192, 3072, 1, 2), ("bf16", 40, 8192, 3072, 0, 2), ("bf16", 9, 2 * 1000, 3072, 1, 2),
    ("bf16", 17, 1000, 1024, 0, 2), ("bf16", 64, 3072, 3072, 0, 2),
    # M >= 1024: the 256x256-tile kernel (ragged M and N tiles, both epilogues, K multiple of 32)
    ("bf16", 1100, 1000, 3072, 0, 2), ("bf16", 1030, 2 * 1000, 2304, 1, 2), ("bf16", 2048, 3072, 1088, 0, 2),
    ("bf16", 1024, 2 * 384, 3072, 1, 2),
    # more tiles than CUs: each persistent workgroup walks several tiles of its XCD's run, ragged
    # last M and N tiles among them (561 tiles of 256 x 256; 297 SwiGLU tiles)
    ("bf16", 4200, 8200, 1088, 0, 2), ("bf16", 2100, 2 * 4100, 640, 1, 2),
]


@pytest.mark.parametrize("dt,M,N,K,epi,algo", CASES)
def test_linear(dt, M, N, K, epi, algo):
    rng = np.random.default_rng(M * 7919 + N * 31 + K)
    x = rng.standard_normal((M, K)).astype(np.float32)
    W = (rng.standard_normal((N, K)) / math.sqrt(K)).astype(np.float32)
    if dt == "bf16":
        xs, Ws = f32_to_bf16_bits(x), f32_to_bf16_bits(W)
        x64, W64 = bf16_bits_to_f32(xs).astype(np.float64), bf16_bits_to_f32(Ws).astype(np.float64)
        code = dory.DORY_BF16
    else:
        xs, Ws, x64, W64 = x, W, x.astype(np.float64), W.astype(np.float64)
        code = dory.DORY_F32
    scale = 1.7 if epi == 0 else 1.0
    ref = (x64 @ W64.T) * scale
    if epi == 1:
        F = N // 2
        u, v = ref[:, :F], ref[:, F:]
        ref = u * v / (1.0 + np.exp(-v))
        ydt = torch.int16 if dt == "bf16" else torch.float32
        y = torch.zeros((M, F), dtype=ydt, device="cuda")
    else:
        y = torch.zeros((M, N), dtype=torch.float32, device="cuda")
    print(f"linear {dt} M={M} N={N} K={K} epi={epi} algo={algo}", flush=True)
    dory.op_linear(code, _dev(xs), _dev(Ws), y, M, N, K, epilogue=epi, scale=scale, algo=algo)
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    if got.dtype == np.int16:
        got = bf16_bits_to_f32(got.view(np.uint16)).astype(np.float64)
        tol = np.abs(ref) * 2.0 ** -8 + 1e-4
    else:
        tol = 2e-5 * math.sqrt(K) * max(1.0, scale)
    err = np.abs(got - ref)
    assert np.all(err <= tol), f"max err {err.max()}"


def test_argmax_ties_and_specials():
    V = 131072 + 77
    B = 6
    rng = np.random.default_rng(11)
    L = rng.standard_normal((B, V)).astype(np.float32)
    L[1] = 0.0
    L[1, [5, 70000, 7]] = 3.0                      # ties: lowest index wins
    L[2] = -np.inf
    L[2, 10], L[2, 3] = -0.0, 0.0                  # -0 == +0: index 3
    L[3, [100, 200]] = np.inf
    L[4] = -np.inf                                 # every logit -inf: index 0
    L[5, V - 1] = 50.0                             # the ragged tail
    out = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    scratch = torch.empty(dory.argmax_scratch_bytes(B, V), dtype=torch.uint8, device="cuda")
    dory.op_argmax(_dev(L), out, scratch)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), np.argmax(L, axis=1))


# ---------------------------------------------------------------------------
# MXFP8 weights: the device quantiser byte for byte against the oracle's
# (OCP MX reading), and the decode GEMV against a float64 product with the
# oracle's dequantised weights
# ---------------------------------------------------------------------------
def test_quant_mxfp8_bit_exact():
    from oracle import mxfp8
    rng = np.random.default_rng(21)
    N, K = 96, 256
    w = (rng.standard_normal((N, K)) * np.exp(rng.uniform(-9, 4, (N, 1)))).astype(np.float32)
    w[3, 32:64] = 0.0                                           # zero block
    w[4, :32] = -0.0                                            # negative zeros
    w[5, :32] = 0.0
    w[5, 0], w[5, 1] = 1e-30, -3e-31                            # tiny block scale
    w[6, :32] = (1.0 + 1.0 / 16 + np.arange(32) % 7 / 8.0) / 256.0  # E4M3 ties after the 2^8 scaling
    w[6, 31] = 1.0                                              # amax 1.0 -> X = -8
    w[7, :32] = 0.01
    w[7, 0] = 1.9375                                            # 496 after scaling: saturates
    w[8, :32] = 0.0
    w[8, 0] = 2.0 ** -130                                       # subnormal block max: X clamped to -127
    wb = f32_to_bf16_bits(w)
    q_ref, s_ref = mxfp8.quantize(bf16_bits_to_f32(wb).astype(np.float64))
    q = torch.zeros((N, K), dtype=torch.uint8, device="cuda")
    sc = torch.zeros((N, K // 32), dtype=torch.uint8, device="cuda")
    dory.op_quant_mxfp8(_dev(wb), N, K, q, sc)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(sc.cpu().numpy(), s_ref)
    np.testing.assert_array_equal(q.cpu().numpy(), q_ref)


MX_CASES = [(1, 8192, 3072, 0), (1, 2 * 8192, 3072, 1), (3, 1000, 2304, 0), (5, 2 * 1000, 2304, 1),
            (1, 3072, 8192, 0), (8, 704, 256, 0), (2, 2 * 704, 256, 1)]


@pytest.mark.parametrize("M,N,K,epi", MX_CASES)
def test_linear_mx(M, N, K, epi):
    from oracle import mxfp8
    rng = np.random.default_rng(M * 131 + N + K)
    x = rng.standard_normal((M, K)).astype(np.float32)
    W = (rng.standard_normal((N, K)) / math.sqrt(K)).astype(np.float32)
    xs = f32_to_bf16_bits(x)
    x64 = bf16_bits_to_f32(xs).astype(np.float64)
    q, sc = mxfp8.quantize(bf16_bits_to_f32(f32_to_bf16_bits(W)).astype(np.float64))
    W64 = mxfp8.dequantize(q, sc)
    scale = 1.7 if epi == 0 else 1.0
    ref = (x64 @ W64.T) * scale
    if epi == 1:
        F = N // 2
        ref = ref[:, :F] * ref[:, F:] / (1.0 + np.exp(-ref[:, F:]))
        y = torch.zeros((M, F), dtype=torch.int16, device="cuda")
    else:
        y = torch.zeros((M, N), dtype=torch.float32, device="cuda")
    print(f"linear mx M={M} N={N} K={K} epi={epi}", flush=True)
    dory.op_linear_mx(_dev(xs), _dev(q), _dev(sc), y, M, N, K, epilogue=epi, scale=scale)
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    if epi == 1:
        got = bf16_bits_to_f32(got.view(np.uint16)).astype(np.float64)
        tol = np.abs(ref) * 2.0 ** -8 + 1e-4
    else:
        tol = 2e-5 * math.sqrt(K) * scale
    err = np.abs(got - ref)
    assert np.all(err <= tol), f"max err {err.max()}"



# ---------------------------------------------------------------------------
# NVFP4-style weights: the device quantiser code for code against the oracle,
# at moderate and at full size (sampled blocks), and the decode GEMV on
# arbitrary codes against a float64 product with the oracle's dequantisation
# ---------------------------------------------------------------------------
def _quant_fp4_gpu(wb, N, K):
    q = torch.zeros((N, K // 2), dtype=torch.uint8, device="cuda")
    sc = torch.zeros((N, K // 16), dtype=torch.uint8, device="cuda")
    g = torch.zeros(1, dtype=torch.float32, device="cuda")
    dory.op_quant_nvfp4(_dev(wb), N, K, q, sc, g)
    torch.cuda.synchronize()
    return q.cpu().numpy(), sc.cpu().numpy(), g.cpu().numpy()[0]


def test_quant_nvfp4_bit_exact():
    from oracle import mxfp8, nvfp4
    rng = np.random.default_rng(31)
    N, K = 64, 512
    w = (rng.standard_normal((N, K)) * np.exp(rng.uniform(-7, -1.5, (N, 1)))).astype(np.float32)
    w = np.clip(w, -2.5, 2.5)
    w[0, 0] = 2688.0 * 2.0 ** -10                       # amax: g = 2^-10 exactly
    S = 2.0 ** -10
    w[1, :16] = 0.0                                     # zero block
    w[1, 16:32] = -0.0                                  # negative zeros
    for r, s in zip(range(2, 8), (0x38, 0x30, 0x28, 0x3C, 0x44, 0x10)):
        e = mxfp8.e4m3_value(s) * S
        w[r, :16] = np.array([0, .5, 1, 1.5, 2, 3, 4, 6] * 2) * e             # exact at scale s
        w[r, 16:23] = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]) * e  # ties at scale s
        w[r, 23:32] = -w[r, 16:25]
    wb = f32_to_bf16_bits(w)
    w64 = bf16_bits_to_f32(wb).astype(np.float64)
    q_ref, s_ref, g_ref = nvfp4.quantize(w64)
    q, sc, g = _quant_fp4_gpu(wb, N, K)
    assert g == g_ref == np.float32(2.0 ** -10)
    np.testing.assert_array_equal(sc, s_ref)
    np.testing.assert_array_equal(q, q_ref)
    # an all-zero matrix: g = 1, every block scale code 1, codes 0 / 8 (sign of -0)
    z = np.zeros((4, 64), dtype=np.uint16)
    z[1] = 0x8000
    q, sc, g = _quant_fp4_gpu(z, 4, 64)
    assert g == 1.0 and np.all(sc == 1) and np.all(q[0] == 0) and np.all(q[1] == 0x88)


def test_quant_nvfp4_full_size_sampled():
    """16384 x 3072 (the 36-layer up/gate shape): the tensor scale exactly,
    2048 random blocks code for code."""
    from oracle import nvfp4
    rng = np.random.default_rng(32)
    N, K = 16384, 3072
    w = (rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02))
    w[123, 456] = 0.5
    wb = f32_to_bf16_bits(w)
    q, sc, g = _quant_fp4_gpu(wb, N, K)
    g_ref = nvfp4.tensor_scale(bf16_bits_to_f32(wb))
    assert g == g_ref
    idx = rng.choice(N * K // 16, size=2048, replace=False)
    blocks = bf16_bits_to_f32(wb.reshape(-1, 16)[idx]).astype(np.float64)
    qb, sb, _ = nvfp4.quantize(blocks, g_ref)
    np.testing.assert_array_equal(sc.reshape(-1)[idx], sb.reshape(-1))
    np.testing.assert_array_equal(q.reshape(-1, 8)[idx], qb)


FP4_CASES = [(1, 8192, 3072, 0), (1, 2 * 8192, 3072, 1), (3, 1000, 2304, 0), (5, 2 * 1000, 2304, 1),
             (1, 3072, 8192, 0), (8, 704, 256, 0), (2, 2 * 704, 256, 1), (4, 512, 8192, 0), (1, 64, 16384, 0),
             (2, 2 * 96, 6144, 1)]


@pytest.mark.parametrize("M,N,K,epi", FP4_CASES)
def test_linear_fp4(M, N, K, epi):
    """Arbitrary codes (every E2M1 code, -0 included) and block scales over a
    wide range; scale = g times an extra factor."""
    from oracle import nvfp4
    rng = np.random.default_rng(M * 977 + N + K)
    x = rng.standard_normal((M, K)).astype(np.float32)
    xs = f32_to_bf16_bits(x)
    x64 = bf16_bits_to_f32(xs).astype(np.float64)
    q = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    sc = rng.integers(20, 100, size=(N, K // 16), dtype=np.uint8)
    g = np.float32(0.37 / math.sqrt(K))
    W64 = nvfp4.dequantize(q, sc, g)
    extra = 1.3 if epi == 0 else 1.0
    ref = (x64 @ W64.T) * extra
    absref = (np.abs(x64) @ np.abs(W64).T) * extra
    if epi == 1:
        F = N // 2
        ref = ref[:, :F] * ref[:, F:] / (1.0 + np.exp(-ref[:, F:]))
        y = torch.zeros((M, F), dtype=torch.int16, device="cuda")
    else:
        y = torch.zeros((M, N), dtype=torch.float32, device="cuda")
    print(f"linear fp4 M={M} N={N} K={K} epi={epi}", flush=True)
    dory.op_linear_fp4(_dev(xs), _dev(q), _dev(sc), y, M, N, K, epilogue=epi, scale=float(g) * extra)
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    if epi == 1:
        got = bf16_bits_to_f32(got.view(np.uint16)).astype(np.float64)
        tol = np.abs(ref) * 2.0 ** -8 + 1e-4 * (1 + np.abs(ref))
    else:
        tol = 2e-5 * absref + 1e-7
    err = np.abs(got - ref)
    assert np.all(err <= tol), f"max err {err.max()} (tol at argmax {tol.reshape(-1)[np.argmax(err)]})"
