"""Depth-1 truncated backward of the last recurrent invocation on the GPU
(dory_backward_last_loop) against the float64 oracle (oracle/backward.py):
every gradient of every recurrent layer and the gradient of the input.

Every tensor is compared element by element: max |g - g_ref| <= bar x
max |g_ref|. float32 models: bar 2e-4 (float32 arithmetic against float64).
bfloat16 models: bar 3e-2 — the products take bfloat16 operands (activations
and gradients rounded once per GEMM, about 2^-9 relative each, a few such
roundings on every path) against the oracle's exact float64; the relative
Frobenius error is printed beside it."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import looped_ngpt_amd as dory  # noqa: E402
from oracle import backward as bw  # noqa: E402
from synth.configs import ModelConfig, get_config, scaled_config  # noqa: E402
from synth.gen import make_weights  # noqa: E402


def _small(gate: int, dtype: str) -> ModelConfig:
    # 1 input, 2 recurrent (one sliding with a 5-key window, one full), 1 output layer; hd 64
    return ModelConfig(name=f"bwg_{dtype}_{gate}", d_model=128, n_q_heads=4, n_kv_heads=2, head_dim=64, d_ff=96,
                       vocab=256, n_in=1, n_rec=2, n_out=1, window=5,
                       layer_is_full=(False, False, True, False), rope_base_swa=1.0e4, rope_base_full=1.0e6,
                       dtype=dtype, attn_gate=gate, seed=11 + gate)


def _alphas(cfg, w, seed):
    rng = np.random.default_rng(seed)
    for l in range(cfg.n_layers):
        w[f"L{l}.alpha_a"] = rng.uniform(0.1, 0.6, cfg.d_model).astype(np.float32)
        w[f"L{l}.alpha_m"] = rng.uniform(0.1, 0.6, cfg.d_model).astype(np.float32)
    return w


def _inputs(cfg, B, n, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, n, cfg.d_model))
    x /= np.linalg.norm(x, axis=-1, keepdims=True)
    G = rng.standard_normal((B, n, cfg.d_model))
    return x.astype(np.float32), G.astype(np.float32)


def _run(cfg, w, x, G):
    dw = dory.upload_weights(cfg, w)
    s = dory.Session(cfg, dw, max_batch=1, max_ctx=max(64, x.shape[1]), max_chunk=8, kv_mode="last_loop")
    xt = torch.from_numpy(x).cuda()
    gt = torch.from_numpy(G).cuda()
    print(f"backward {cfg.name} B={x.shape[0]} n={x.shape[1]}", flush=True)
    out = s.backward_last_loop(xt, gt)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy().astype(np.float64) for k, v in out.items()}


def _compare(cfg, got, ref, x_shape, bar):
    worst, worst_fro = 0.0, 0.0
    for l in range(cfg.n_in, cfg.n_in + cfg.n_rec):
        for p in ("qkvg", "o", "ug", "down", "alpha_a", "alpha_m"):
            key = f"L{l}.{p}"
            assert got[key].shape == ref[key].shape, key
            e, f = _err(key, got[key], ref[key], bar)
            worst, worst_fro = max(worst, e), max(worst_fro, f)
    e, f = _err("x", got["x"].reshape(x_shape), ref["x"], bar)
    worst, worst_fro = max(worst, e), max(worst_fro, f)
    print(f"{cfg.name}: worst max|diff|/max|ref| {worst:.3e} (relative Frobenius {worst_fro:.3e})", flush=True)


def _err(key, g, r, bar):
    e = np.max(np.abs(g - r)) / max(np.max(np.abs(r)), 1e-30)
    f = np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30)
    assert e <= bar, f"{key}: element error {e:.3e} of the largest entry > {bar}"
    return e, f


@pytest.mark.parametrize("gate", [0, 1, 2])
def test_backward_f32_small(gate):
    cfg = _small(gate, "f32")
    w = _alphas(cfg, make_weights(cfg), 70 + gate)
    x, G = _inputs(cfg, 2, 24, 80 + gate)
    ref = bw.block_backward(cfg, w, x.astype(np.float64), G.astype(np.float64))
    got = _run(cfg, w, x, G)
    _compare(cfg, got, ref, x.shape, 2e-4)


@pytest.mark.parametrize("n", [40, 23])
def test_backward_bf16_small(n):
    """n 40: the one-wave-per-row softmax kernels; 23 (not a multiple of 4): the per-row-workgroup ones."""
    cfg = _small(1, "bf16")
    w = _alphas(cfg, make_weights(cfg), 90)
    x, G = _inputs(cfg, 2, n, 91)
    ref = bw.block_backward(cfg, w, x.astype(np.float64), G.astype(np.float64))
    got = _run(cfg, w, x, G)
    _compare(cfg, got, ref, x.shape, 3e-2)


def test_backward_bf16_36layer_widths():
    """d 3072, 24 / 8 heads of 128, d_ff 8192: 1 input, 2 recurrent (one sliding with a 100-key window, one
    full), 1 output layer; 300 positions: 300 rows take the library GEMMs for the projections and their
    gradients, and the softmax rows hold two float4 groups per lane."""
    cfg = scaled_config(get_config("c36"), n_in=1, n_rec=2, n_out=1).replace(vocab=512, name="c36w_bw")
    cfg = cfg.replace(layer_is_full=(False, False, True, False), window=100)
    w = _alphas(cfg, make_weights(cfg), 92)
    x, G = _inputs(cfg, 1, 300, 93)
    ref = bw.block_backward(cfg, w, x.astype(np.float64), G.astype(np.float64))
    got = _run(cfg, w, x, G)
    _compare(cfg, got, ref, x.shape, 3e-2)


def test_backward_bf16_split_contraction():
    """d 256, d_ff 2048, 2 x 520 positions (1040 rows, a ragged last row tile): the output projections of
    the MLP (contraction 2048) and the input gradient through up/gate (contraction 4096) have too few
    output tiles to fill the chip, so each runs the two halves of its contraction side by side and adds
    the partial sums afterwards."""
    cfg = ModelConfig(name="bw_split", d_model=256, n_q_heads=4, n_kv_heads=2, head_dim=64, d_ff=2048,
                      vocab=256, n_in=1, n_rec=2, n_out=1, window=37,
                      layer_is_full=(False, False, True, False), rope_base_swa=1.0e4, rope_base_full=1.0e6,
                      dtype="bf16", attn_gate=1, seed=17)
    w = _alphas(cfg, make_weights(cfg), 94)
    x, G = _inputs(cfg, 2, 520, 95)
    ref = bw.block_backward(cfg, w, x.astype(np.float64), G.astype(np.float64))
    got = _run(cfg, w, x, G)
    _compare(cfg, got, ref, x.shape, 3e-2)


def test_backward_bf16_long_rows():
    """d 4352 and d_ff 8448: rows longer than the register-held row kernels take (4096 for the updates,
    8192 for SwiGLU), so the streaming versions of those kernels run."""
    cfg = ModelConfig(name="bw_long_rows", d_model=4352, n_q_heads=4, n_kv_heads=2, head_dim=64, d_ff=8448,
                      vocab=256, n_in=1, n_rec=2, n_out=1, window=5,
                      layer_is_full=(False, False, True, False), rope_base_swa=1.0e4, rope_base_full=1.0e6,
                      dtype="bf16", attn_gate=1, seed=19)
    w = _alphas(cfg, make_weights(cfg), 96)
    x, G = _inputs(cfg, 1, 24, 97)
    ref = bw.block_backward(cfg, w, x.astype(np.float64), G.astype(np.float64))
    got = _run(cfg, w, x, G)
    _compare(cfg, got, ref, x.shape, 3e-2)


def test_backward_argument_errors():
    cfg = _small(1, "f32")
    w = make_weights(cfg)
    dw = dory.upload_weights(cfg, w)
    s = dory.Session(cfg, dw, max_batch=1, max_ctx=32, max_chunk=8, kv_mode="last_loop")
    x = torch.zeros((1, 40, cfg.d_model), dtype=torch.float32, device="cuda")
    with pytest.raises(dory.DoryError):
        s.backward_last_loop(x, x)            # n > max_ctx


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_kept_forward_equals_recompute(dtype):
    """The full workspace keeps every layer's forward values; the minimum one
    recomputes each layer's forward during the backward: the same kernels on
    the same inputs, so the gradients agree bit for bit."""
    cfg = _small(2, dtype)
    w = _alphas(cfg, make_weights(cfg), 95)
    x, G = _inputs(cfg, 2, 32, 96)
    dw = dory.upload_weights(cfg, w)
    s = dory.Session(cfg, dw, max_batch=1, max_ctx=64, max_chunk=8, kv_mode="last_loop")
    xt, gt = torch.from_numpy(x).cuda(), torch.from_numpy(G).cuda()
    print(f"backward kept vs recomputed forward, {dtype}", flush=True)
    kept = {k: v.cpu().numpy() for k, v in s.backward_last_loop(xt, gt).items()}
    again = {k: v.cpu().numpy() for k, v in s.backward_last_loop(xt, gt, recompute=True).items()}
    assert kept.keys() == again.keys()
    for k in kept:
        np.testing.assert_array_equal(kept[k], again[k], err_msg=k)
