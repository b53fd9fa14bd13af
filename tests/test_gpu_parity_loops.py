"""Parity of the batch-1 bfloat16 decode path that the benchmark times (the
fused decode: GEMVs with the nGPT update in their prologue, matrix-core
split-K attention summed into fixed-point accumulators, the output GEMV
staged from them) against the oracle, at every loop count the metric names
and in both KV modes; bfloat16 KV placement; and the attention sums when every
score sits far below the bound.

Loop counts and the two cache modes: "Dory 1.0 4B Benchmarks" (goremy.ai
blog), How does looping work at inference time?; "Dory1.0-4B: A Looped
Normalized-GPT" (ai.info summary), Key Contributions 1.

Bars: max |logit difference| <= 3e-2 against the float64 oracle that rounds
to bfloat16 where the library stores bfloat16, 100% greedy agreement; KV
placement exact (every slot the spec does not name still holds its sentinel).
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import looped_ngpt_amd as dory  # noqa: E402
from gpu_run import generate, session  # noqa: E402
from oracle import kvspec  # noqa: E402
from oracle.ngpt import LoopedNGPT  # noqa: E402
from synth.configs import get_config, scaled_config  # noqa: E402
from synth.gen import f32_to_bf16_bits, make_tokens, make_weights  # noqa: E402

BF16_TOL = 3e-2

_cache = {}


def _model(name):
    if name not in _cache:
        if name == "c36w":            # the 36-layer model's widths, 2/2/2 layers (layer 3 full)
            m = scaled_config(get_config("c36"), n_in=2, n_rec=2, n_out=2)
        elif name == "tiny_bf16":     # d 256, hd 64, 64-key rings
            m = get_config("tiny").replace(dtype="bf16", d_ff=688, name="tiny_bf16")
        elif name == "tiny_bf16_s30":  # softmax scale 30: too large for the fixed-point bins
            m = get_config("tiny").replace(dtype="bf16", d_ff=688, attn_scale=30.0, name="tiny_bf16_s30")
        elif name == "tiny_bf16_w40":  # hd 64, a 40-key ring: a multiple of 8 but not of 32
            m = get_config("tiny").replace(dtype="bf16", d_ff=688, window=40, name="tiny_bf16_w40")
        elif name == "c36w_w40":       # the c36w weights (hd 128) with 40-key rings
            m0, w, dw = _model("c36w")
            _cache[name] = (m0.replace(window=40, name="c36w_w40"), w, dw)
            return _cache[name]
        else:
            raise KeyError(name)
        w = make_weights(m)
        _cache[name] = (m, w, dory.upload_weights(m, w))
    return _cache[name]


def _report(tag, gl, ol):
    d = np.abs(gl - ol)
    print(f"{tag}: max|dlogit| {d.max():.3e} mean {d.mean():.3e}", flush=True)
    return d.max()


# ---------------------------------------------------------------------------
# the fused decode at k = 1, 3, 4 (k = 2 is in test_gpu_parity.py), both modes,
# at the 36-layer widths (d 3072, 24 / 8 heads of 128, d_ff 8192, vocab 131072)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("k,mode", [(1, "per_loop"), (1, "last_loop"), (4, "per_loop"), (4, "last_loop"),
                                    (3, "last_loop")])
def test_c36w_fused_decode_loop_counts(k, mode):
    m, w, dw = _model("c36w")
    n, steps, ctx = 48, 10, 64
    prompt = make_tokens(m, 80 + k, (1, n))
    print(f"c36w k={k} {mode}: oracle", flush=True)
    ora = LoopedNGPT(m, w, max_ctx=ctx)
    o_tok, o_log = ora.generate(prompt, steps, k, mode)
    margins = np.sort(o_log, axis=-1)
    print(f"c36w k={k} {mode}: min top1-top2 margin {np.min(margins[..., -1] - margins[..., -2]):.3e}", flush=True)
    s = session(m, dw, batch=1, max_ctx=ctx, chunk=n, kv_mode=mode, k=k)
    g_tok, g_log, lib_next = generate(s, prompt, steps, k)
    assert _report(f"c36w fused decode {mode} k={k}", g_log, o_log) <= BF16_TOL
    np.testing.assert_array_equal(g_tok, o_tok)
    np.testing.assert_array_equal(lib_next, g_tok[:, 1:])


# ---------------------------------------------------------------------------
# bfloat16 KV placement: after a chunked prefill (the prefill KV writer) and
# greedy decode steps (the decode attention kernel's store of the new key and
# value), every live position's K and V sit at the spec's offsets and nothing
# else was written
# ---------------------------------------------------------------------------
SENTINEL = 0x7FC1   # a bfloat16 NaN that no computation produces


@pytest.mark.parametrize("name,k,mode,n,chunk,steps,ctx", [
    ("tiny_bf16", 2, "per_loop", 90, 64, 6, 128),    # 64-key rings wrap; two prefill chunks
    ("tiny_bf16", 3, "last_loop", 90, 64, 6, 128),   # last-loop: the final loop's K/V
    ("c36w", 2, "per_loop", 40, 32, 6, 64),           # hd 128, 8 kv heads
    ("c36w", 4, "last_loop", 40, 32, 6, 64),
])
def test_bf16_kv_placement_exact(name, k, mode, n, chunk, steps, ctx):
    m, w, dw = _model(name)
    prompt = make_tokens(m, 90 + k, (1, n))
    ora = LoopedNGPT(m, w, max_ctx=ctx)
    o_tok, _ = ora.generate(prompt, steps, k, mode, chunk=chunk)
    s = session(m, dw, batch=1, max_ctx=ctx, chunk=chunk, kv_mode=mode, k=k)
    s.kv.view(torch.int16).fill_(SENTINEL)
    g_tok, _, _ = generate(s, prompt, steps, k)
    np.testing.assert_array_equal(g_tok, o_tok)
    raw = s.kv.view(torch.int16).cpu().numpy().view(np.uint16)
    kv = (raw.astype(np.uint32) << 16).view(np.float32)
    kv_loops = k if mode == "per_loop" else 1
    ctxw = n + steps - 1                                      # positions written
    hd, nkv = m.head_dim, m.n_kv_heads
    written = np.zeros(raw.shape, dtype=bool)
    worst = 0.0
    for l in range(m.n_layers):
        rec = m.is_recurrent(l)
        loops = range(1, k + 1) if (rec and mode == "per_loop") else [k if rec else 0]
        for j in loops:
            key = (l, j) if (rec and mode == "per_loop") else (l, 0)
            live = range(ctxw) if m.layer_is_full[l] else range(max(0, ctxw - m.window), ctxw)
            for which in "KV":
                st = kvspec.dim_stride(m, ctx, l, which)
                for h in range(nkv):
                    offs = np.array([kvspec.element_offset(m, mode, kv_loops, ctx, 1, l, j, which, 0, h, p)
                                     for p in live])
                    idx = offs[:, None] + st * np.arange(hd)[None, :]
                    got = kv[idx]
                    ref = ora.cache[key][which][0, h, list(live)]
                    # bfloat16 storage of nearly equal float values: a few units in
                    # the last place; keys of two positions differ by far more
                    err = np.abs(got - ref)
                    worst = max(worst, float(err.max()))
                    np.testing.assert_allclose(got, ref, rtol=2 ** -6, atol=2e-3,
                                               err_msg=f"L{l} loop{j} {which} h{h}")
                    written[idx] = True
    print(f"{name} {mode} k={k}: largest |K/V - oracle| {worst:.2e}", flush=True)
    assert np.all(raw[~written] == SENTINEL), "a slot outside the spec was written"
    # the spec's slots are bijective with the live positions: no two share one
    assert int(written.sum()) == sum(
        (len(range(ctxw)) if m.layer_is_full[l] else min(ctxw, m.window)) * 2 * nkv * hd *
        (k if (m.is_recurrent(l) and mode == "per_loop") else 1) for l in range(m.n_layers))


# ---------------------------------------------------------------------------
# every score near -scale: one layer whose q is the negated key direction on
# the slowest RoPE pair, all positions the same token. The decode sums sit
# 2^-32.6 (hd 128) below the bound per key; the accumulators must keep the
# softmax output exact to bfloat16
# ---------------------------------------------------------------------------
def _far_below_bound_model(full: bool):
    """d 256, 2 q heads / 1 kv head of 128, one recurrent layer (k = 1). The
    key rows are zero except dims 63 and 127 (the pair RoPE turns slowest),
    which copy the embedding of token 5, so every position's key is the same
    unit vector up to a rotation of < 1e-3 rad; the query rows are the key
    rows negated: q.k ~ -1 for every key. alpha_a = 1 makes the layer output
    norm(W_o o), alpha_m = 0 leaves it unchanged, so the logits see the
    attention output directly."""
    base = get_config("tiny").replace(
        name="far_below_bound", dtype="bf16", d_model=256, n_q_heads=2, n_kv_heads=1, head_dim=128,
        d_ff=64, vocab=512, n_in=0, n_rec=1, n_out=0, window=8192, layer_is_full=(full,),
        rope_base_swa=1.0e7, rope_base_full=1.0e7, seed=7)
    w = make_weights(base)
    emb = (w["embed"].astype(np.uint32) << 16).view(np.float32)
    tok = 5
    qkvg = (w["L0.qkvg"].astype(np.uint32) << 16).view(np.float32).copy()
    hd = 128
    kr = np.zeros((hd, base.d_model), np.float32)
    kr[63] = emb[tok] * 0.6
    kr[127] = emb[tok] * 0.8
    q0, k0 = 0, base.q_dim
    for hq in range(base.n_q_heads):
        qkvg[q0 + hq * hd:q0 + (hq + 1) * hd] = -kr
    qkvg[k0:k0 + hd] = kr
    w["L0.qkvg"] = f32_to_bf16_bits(qkvg)
    w["L0.alpha_a"] = np.ones(base.d_model, np.float32)
    w["L0.alpha_m"] = np.zeros(base.d_model, np.float32)
    return base, w, tok


@pytest.mark.parametrize("full", [True, False])
@pytest.mark.parametrize("n", [1, 4096])
def test_decode_sums_far_below_score_bound(full, n):
    m, w, tok = _far_below_bound_model(full)
    dw = dory.upload_weights(m, w)
    steps = 4
    ctx = (n + steps + 7) // 8 * 8 + 8   # a multiple of 8: the matrix-core decode attention
    ora = LoopedNGPT(m, w, max_ctx=ctx)
    prompt = np.full((1, n), tok, np.int32)
    ol = [ora.call(prompt, 1, "last_loop")]
    for _ in range(steps):
        ol.append(ora.call(np.array([[tok]], np.int32), 1, "last_loop"))
    s = session(m, dw, batch=1, max_ctx=ctx, chunk=min(n, 4096), kv_mode="last_loop", k=1)
    s.prefill(torch.from_numpy(prompt).cuda(), 1)
    gl = [s.logits().clone()]
    for _ in range(steps):
        s.decode(torch.tensor([tok], dtype=torch.int32, device="cuda"), 1)
        gl.append(s.logits().clone())
    torch.cuda.synchronize()
    gl = torch.stack(gl).cpu().numpy()
    ol = np.stack(ol)
    assert np.all(np.isfinite(gl))
    assert _report(f"scores near -scale, {'full' if full else 'sliding'}, {n} cached keys", gl, ol) <= BF16_TOL
    np.testing.assert_array_equal(np.argmax(gl, axis=-1), np.argmax(ol, axis=-1))


def test_large_softmax_scale_takes_float_merge():
    """attn_scale 30 (scale log2 e = 43.3): more binary orders of magnitude
    than the fixed-point bins cover, so decode sums go through the float
    split + merge path; still within the bar."""
    m, w, dw = _model("tiny_bf16_s30")
    n, steps, ctx, k = 70, 10, 96, 2
    prompt = make_tokens(m, 95, (1, n))
    ora = LoopedNGPT(m, w, max_ctx=ctx)
    o_tok, o_log = ora.generate(prompt, steps, k, "last_loop")
    s = session(m, dw, batch=1, max_ctx=ctx, chunk=n, kv_mode="last_loop", k=k)
    g_tok, g_log, _ = generate(s, prompt, steps, k)
    assert np.all(np.isfinite(g_log))
    assert _report("tiny bf16 attn_scale 30", g_log, o_log) <= BF16_TOL
    np.testing.assert_array_equal(g_tok, o_tok)


# ---------------------------------------------------------------------------
# ring layers whose window is a multiple of 8 but not of 32: the ring's last
# 32-slot tile runs past the ring; decode from before the ring fills (every
# slot above t unwritten) through several wraps
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name,k,mode", [("tiny_bf16_w40", 2, "last_loop"), ("c36w_w40", 2, "per_loop")])
def test_decode_ring_window_not_multiple_of_32(name, k, mode):
    m, w, dw = _model(name)
    n, steps, ctx = 24, 64, 96
    prompt = make_tokens(m, 90, (1, n))
    print(f"{name} k={k} {mode}: oracle", flush=True)
    ora = LoopedNGPT(m, w, max_ctx=ctx)
    o_tok, o_log = ora.generate(prompt, steps, k, mode)
    s = session(m, dw, batch=1, max_ctx=ctx, chunk=n, kv_mode=mode, k=k)
    g_tok, g_log, _ = generate(s, prompt, steps, k)
    assert _report(f"{name} ring decode {mode} k={k}", g_log, o_log) <= BF16_TOL
    np.testing.assert_array_equal(g_tok, o_tok)
