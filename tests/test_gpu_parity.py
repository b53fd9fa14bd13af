"""End-to-end parity of the HIP library with the oracle, through the C ABI.

float32 model: max |logit difference| <= 1e-3 against the float64 oracle.
bfloat16 models: max |logit difference| <= 3e-2 against the float64 oracle
that rounds to bfloat16 where the library stores bfloat16, and 100% greedy
agreement over the decode horizon. KV placement and argmax are bit-exact;
per-loop and last-loop caching are bit-identical at k = 1; reruns are
bit-identical.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import looped_ngpt_amd as dory  # noqa: E402
from gpu_run import generate, session, teacher_forced  # noqa: E402
from oracle import kvspec  # noqa: E402
from oracle.ngpt import LoopedNGPT  # noqa: E402
from synth.configs import get_config, scaled_config  # noqa: E402
from synth.gen import make_tokens, make_weights  # noqa: E402

F32_TOL = 1e-3
BF16_TOL = 3e-2

_cache = {}


def model_and_weights(name):
    if name not in _cache:
        if name == "tiny":
            m = get_config("tiny")
        elif name == "c36w":          # the 36-layer model's widths, 2/2/2 layers (layer 3 full)
            m = scaled_config(get_config("c36"), n_in=2, n_rec=2, n_out=2)
        elif name == "c72w":          # the 72-layer model's widths, 1/3/1 layers (layer 3 full)
            m = scaled_config(get_config("c72"), n_in=1, n_rec=3, n_out=1)
        elif name == "tiny_bf16":     # the tiny shape in bfloat16 (64-key window, matrix-core decode)
            m = get_config("tiny").replace(dtype="bf16", d_ff=688, name="tiny_bf16")
        elif name == "tiny_bf16_w60":  # a window that is not a multiple of 8 (per-key value gathers)
            m = get_config("tiny").replace(dtype="bf16", d_ff=688, window=60, name="tiny_bf16_w60")
        elif name == "tiny_mx":       # the tiny shape in bfloat16 with MXFP8-compatible widths (multiples of 32)
            m = get_config("tiny").replace(dtype="bf16", d_ff=704, name="tiny_mx")
        elif name == "wide_fp4":      # the 36-layer model's d_model (3072) with one head and a narrow MLP, 1/1/1
            m = scaled_config(get_config("c36"), n_in=1, n_rec=1, n_out=1).replace(
                n_q_heads=1, n_kv_heads=1, d_ff=64, vocab=2048, window=64, name="wide_fp4")
        elif name == "c36w_w192":     # the c36w weights with 192-key rings that wrap
            m0, w, dw = model_and_weights("c36w")
            _cache[name] = (m0.replace(window=192, name="c36w_w192"), w, dw)
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
# float32 tiny model (d 256, 2/2/2, SWA 64 / full alternating), prompt 128,
# 32 greedy steps at k = 2, both cache modes
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("mode", ["per_loop", "last_loop"])
def test_tiny_f32_generate(mode):
    m, w, dw = model_and_weights("tiny")
    k, steps = 2, 32
    prompt = make_tokens(m, 0, (1, 128))
    ora = LoopedNGPT(m, w, max_ctx=256)
    o_tok, o_log = ora.generate(prompt, steps, k, mode)
    print(f"tiny {mode}: oracle tokens {o_tok[0, :8]}...", flush=True)
    s = session(m, dw, batch=1, max_ctx=256, chunk=128, kv_mode=mode, k=k)
    g_tok, g_log, lib_next = generate(s, prompt, steps, k)
    assert _report(f"tiny {mode} free-running", g_log, o_log) <= F32_TOL
    np.testing.assert_array_equal(g_tok, o_tok)
    np.testing.assert_array_equal(lib_next, g_tok[:, 1:])          # library argmax == numpy argmax
    np.testing.assert_array_equal(np.argmax(g_log, axis=-1).T, g_tok)
    assert ora.max_norm_dev <= 1e-4


def test_tiny_f32_batched_chunked_long():
    """B = 3 sequences, a 600-token prompt in 128-position chunks (the 64-slot
    rings wrap inside and across chunks, many attention splits), 12 steps at
    k = 3 in last-loop mode (chunk-schedule dependent: same schedule on both)."""
    m, w, dw = model_and_weights("tiny")
    B, n, k, steps, chunk = 3, 600, 3, 12, 128
    prompt = make_tokens(m, 1, (B, n))
    ora = LoopedNGPT(m, w, max_ctx=640, batch=B)
    o_tok, o_log = ora.generate(prompt, steps, k, "last_loop", chunk=chunk)
    s = session(m, dw, batch=B, max_ctx=640, chunk=chunk, kv_mode="last_loop", k=k)
    g_tok, g_log, _ = generate(s, prompt, steps, k)
    assert _report("tiny batched chunked", g_log, o_log) <= F32_TOL
    np.testing.assert_array_equal(g_tok, o_tok)


def test_tiny_elastic_depth_last_loop():
    """Last-loop mode accepts a different k on every call (1, 4, 2, 3)."""
    m, w, dw = model_and_weights("tiny")
    prompt = make_tokens(m, 2, (1, 40))
    ks = [1, 4, 2, 3]
    ora = LoopedNGPT(m, w, max_ctx=64)
    ol = [ora.call(prompt, ks[0], "last_loop")]
    s = session(m, dw, batch=1, max_ctx=64, chunk=64, kv_mode="last_loop", k=1)
    s.prefill(torch.from_numpy(prompt).cuda(), ks[0])
    gl = [s.logits().cpu().numpy()]
    toks = [5, 900, 17]
    for t, k in zip(toks, ks[1:]):
        ol.append(ora.call(np.array([[t]]), k, "last_loop"))
        s.decode(torch.tensor([t], dtype=torch.int32, device="cuda"), k)
        gl.append(s.logits().cpu().numpy())
    assert _report("tiny elastic", np.stack(gl), np.stack(ol)) <= F32_TOL


def test_tiny_kv_placement_bit_exact():
    """After prefill + decode in per-loop mode at k = 2 the KV buffer holds,
    at exactly the spec's offsets, the oracle's K/V of the live positions, and
    every other slot still holds the sentinel the buffer was filled with."""
    m, w, dw = model_and_weights("tiny")
    k, n, steps, T = 2, 90, 6, 128
    prompt = make_tokens(m, 3, (1, n))
    ora = LoopedNGPT(m, w, max_ctx=T)
    o_tok, _ = ora.generate(prompt, steps, k, "per_loop")
    s = session(m, dw, batch=1, max_ctx=T, chunk=64, kv_mode="per_loop", k=k)
    s.kv.view(torch.int32).fill_(0x7FC00001)                   # NaN sentinel
    generate(s, prompt, steps, k)
    kv = s.kv.view(torch.float32).cpu().numpy()
    ctx = n + steps - 1                                         # positions written
    hd, nkv = m.head_dim, m.n_kv_heads
    written = np.zeros(kv.shape, dtype=bool)
    for l in range(m.n_layers):
        loops = range(1, k + 1) if m.is_recurrent(l) else [0]
        for j in loops:
            key = (l, j if m.is_recurrent(l) else 0)
            live = range(ctx) if m.layer_is_full[l] else range(max(0, ctx - m.window), ctx)
            for p in live:
                for which in "KV":
                    st = kvspec.dim_stride(m, T, l, which)
                    for h in range(nkv):
                        off = kvspec.element_offset(m, "per_loop", k, T, 1, l, j, which, 0, h, p)
                        idx = off + st * np.arange(hd)
                        got = kv[idx]
                        ref = ora.cache[key][which][0, h, p]
                        np.testing.assert_allclose(got, ref, atol=2e-5, err_msg=f"L{l} loop{j} {which} pos{p}")
                        written[idx] = True
    # everything else (the full layers' slots >= ctx; the rings are all live
    # since ctx > W) still holds the sentinel
    assert np.all(kv[~written].view(np.uint32) == 0x7FC00001)
    for l in range(m.n_layers):
        if not m.layer_is_full[l]:
            continue
        loops = range(1, k + 1) if m.is_recurrent(l) else [0]
        for j in loops:
            off = kvspec.element_offset(m, "per_loop", k, T, 1, l, j, "K", 0, 0, ctx)
            assert np.all(kv[off:off + hd].view(np.uint32) == 0x7FC00001)


def test_tiny_k1_modes_bit_identical_and_deterministic():
    m, w, dw = model_and_weights("tiny")
    prompt = make_tokens(m, 4, (1, 70))
    runs = []
    for mode in ("per_loop", "last_loop", "last_loop"):
        s = session(m, dw, batch=1, max_ctx=128, chunk=32, kv_mode=mode, k=1)
        runs.append(generate(s, prompt, 8, 1)[1])
    np.testing.assert_array_equal(runs[0], runs[1])
    np.testing.assert_array_equal(runs[1], runs[2])


def test_state_errors_on_gpu():
    m, w, dw = model_and_weights("tiny")
    s = session(m, dw, batch=1, max_ctx=64, chunk=64, kv_mode="per_loop", k=2)
    s.prefill(torch.from_numpy(make_tokens(m, 5, (1, 8))).cuda(), 2)
    with pytest.raises(dory.DoryError) as e:
        s.decode(None, 1)                                   # k change in per-loop mode
    assert e.value.status == dory.DORY_E_LOOPS
    with pytest.raises(dory.DoryError) as e:
        s.decode(None, 2, kv_mode="last_loop")              # other mode
    assert e.value.status == dory.DORY_E_KV_MODE
    s.decode(None, 2)
    s.reset()
    s.prefill(torch.from_numpy(make_tokens(m, 5, (1, 8))).cuda(), 2)


# ---------------------------------------------------------------------------
# bfloat16 at the 4B-shaped widths (fewer layers so the oracle finishes)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name,k,mode,n,steps,ctx", [("c36w", 2, "last_loop", 64, 12, 96),
                                                     ("c36w", 2, "per_loop", 40, 8, 77),
                                                     ("c72w", 3, "per_loop", 33, 8, 64),
                                                     ("tiny_bf16", 2, "last_loop", 150, 24, 192),
                                                     ("tiny_bf16", 3, "per_loop", 97, 20, 160)])
def test_bf16_widths(name, k, mode, n, steps, ctx):
    """ctx = max_ctx: multiples of 8 take the matrix-core decode attention,
    77 the vector fallback; the tiny shape's 64-key rings wrap."""
    m, w, dw = model_and_weights(name)
    prompt = make_tokens(m, 6, (1, n))
    ora = LoopedNGPT(m, w, max_ctx=ctx)
    o_tok, o_log = ora.generate(prompt, steps, k, mode)
    margins = np.sort(o_log, axis=-1)
    print(f"{name}: min top1-top2 margin {np.min(margins[..., -1] - margins[..., -2]):.3e}", flush=True)
    s = session(m, dw, batch=1, max_ctx=ctx, chunk=n, kv_mode=mode, k=k)
    g_tok, g_log, lib_next = generate(s, prompt, steps, k)
    assert _report(f"{name} {mode} k={k}", g_log, o_log) <= BF16_TOL
    np.testing.assert_array_equal(g_tok, o_tok)
    np.testing.assert_array_equal(lib_next, g_tok[:, 1:])


# ---------------------------------------------------------------------------
# chunked bfloat16 prefill (matrix-core prefill attention): keys from the
# cache and from the call, ring wrap inside and across chunks, chunk starts
# that are not multiples of 8 (per-key value gathers), ragged last chunks
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name,B,n,chunk,k,mode,ctx,steps", [
    ("tiny_bf16", 2, 300, 100, 2, "last_loop", 320, 8),     # p0 = 100 (gathers), 200; 64-key rings
    ("tiny_bf16_w60", 1, 257, 64, 3, "per_loop", 272, 6),   # 60-key rings; last chunk is 1 position
    ("c36w_w192", 1, 520, 256, 2, "last_loop", 544, 6),     # hd 128, 3 q heads per kv head
])
def test_bf16_prefill_chunked(name, B, n, chunk, k, mode, ctx, steps):
    m, w, dw = model_and_weights(name)
    prompt = make_tokens(m, 21, (B, n))
    ora = LoopedNGPT(m, w, max_ctx=ctx, batch=B)
    o_tok, o_log = ora.generate(prompt, steps, k, mode, chunk=chunk)
    print(f"{name}: oracle done", flush=True)
    s = session(m, dw, batch=B, max_ctx=ctx, chunk=chunk, kv_mode=mode, k=k)
    g_tok, g_log, lib_next = generate(s, prompt, steps, k)
    assert _report(f"{name} chunked prefill {mode} k={k}", g_log, o_log) <= BF16_TOL
    np.testing.assert_array_equal(g_tok, o_tok)
    np.testing.assert_array_equal(lib_next, g_tok[:, 1:])


@pytest.mark.parametrize("nq,nkv,hd,n,chunk", [
    (4, 4, 64, 77, 40),     # 1 query head per kv head; second chunk starts at 40 (gathers)
    (8, 2, 64, 90, 90),     # 4 per kv head: 12 work items of 32 queries, the second workgroup half empty
    (6, 1, 128, 70, 64),    # 6 per kv head, hd 128: the 6-position last chunk leaves two waves idle
    (8, 1, 64, 100, 100),   # 8 per kv head: each workgroup spans one 32-query block of all heads
])
def test_bf16_prefill_query_group_sizes(nq, nkv, hd, n, chunk):
    """The prefill attention groups the query heads of a kv head into one
    workgroup; group sizes other than the named shapes' 2 and 3, ragged
    prompt lengths and chunk boundaries inside a 64-key ring."""
    name = f"tiny_bf16_g{nq}x{nkv}_hd{hd}"
    if name not in _cache:
        m = get_config("tiny").replace(dtype="bf16", d_ff=688, n_q_heads=nq, n_kv_heads=nkv, head_dim=hd,
                                       name=name)
        w = make_weights(m)
        _cache[name] = (m, w, dory.upload_weights(m, w))
    m, w, dw = _cache[name]
    k, mode, steps, ctx = 2, "last_loop", 6, 128
    prompt = make_tokens(m, 23, (1, n))
    ora = LoopedNGPT(m, w, max_ctx=ctx)
    o_tok, o_log = ora.generate(prompt, steps, k, mode, chunk=chunk)
    print(f"{name}: oracle done", flush=True)
    s = session(m, dw, batch=1, max_ctx=ctx, chunk=chunk, kv_mode=mode, k=k)
    g_tok, g_log, _ = generate(s, prompt, steps, k)
    assert _report(f"{name} n={n} chunk={chunk}", g_log, o_log) <= BF16_TOL
    np.testing.assert_array_equal(g_tok, o_tok)


# ---------------------------------------------------------------------------
# per-sequence loop counts in one batched call (last-loop caching): each
# sequence must get what it gets alone with its own counts — the reference is
# one single-sequence oracle per row
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name,tol", [("tiny", F32_TOL), ("tiny_bf16", BF16_TOL)])
def test_mixed_loop_counts_match_separate_sequences(name, tol):
    m, w, dw = model_and_weights(name)
    B, n, chunk, ctx = 3, 70, 64, 128
    prompt = make_tokens(m, 40, (B, n))
    pre_k = [1, 3, 2]
    sched = [[1, 3, 2], [2, 2, 4], [1, 1, 1], [3, 1, 2], [4, 2, 1]]
    forced = np.random.default_rng(5).integers(0, m.vocab, size=(len(sched), B)).astype(np.int32)
    ref = np.zeros((len(sched) + 1, B, m.vocab))
    for b in range(B):
        o = LoopedNGPT(m, w, max_ctx=ctx, batch=1)
        for s0 in range(0, n, chunk):
            lg = o.call(prompt[b:b + 1, s0:s0 + chunk], pre_k[b], "last_loop")
        ref[0, b] = lg[0]
        for i, ks in enumerate(sched):
            ref[i + 1, b] = o.call(forced[i:i + 1, b:b + 1], ks[b], "last_loop")[0]
    s = session(m, dw, batch=B, max_ctx=ctx, chunk=chunk, kv_mode="last_loop", k=4)
    s.prefill_mixed(torch.from_numpy(prompt).cuda(), pre_k)
    got = [s.logits().cpu().numpy()]
    for i, ks in enumerate(sched):
        s.decode_mixed(torch.from_numpy(forced[i]).cuda(), ks)
        got.append(s.logits().cpu().numpy())
    assert _report(f"{name} mixed loop counts", np.stack(got), ref) <= tol


# ---------------------------------------------------------------------------
# MXFP8 layer projections: the oracle runs on its own quantise-dequantise of
# the weights (exactly bfloat16 values); the library quantises on the device
# and decodes with the MXFP8 GEMVs (prefill expands each projection to
# bfloat16 and takes the GEMM)
# ---------------------------------------------------------------------------
def _mx_oracle_weights(m, w):
    from oracle import mxfp8
    from synth.gen import bf16_bits_to_f32, f32_to_bf16_bits
    out = dict(w)
    for l in range(m.n_layers):
        for p in ("qkvg", "o", "ug", "down"):
            q, sc = mxfp8.quantize(bf16_bits_to_f32(w[f"L{l}.{p}"]).astype(np.float64))
            out[f"L{l}.{p}"] = f32_to_bf16_bits(mxfp8.dequantize(q, sc).astype(np.float32))
    return out


@pytest.mark.parametrize("name,k,mode,n,steps,ctx", [("tiny_mx", 2, "last_loop", 100, 16, 160),
                                                     ("tiny_mx", 3, "per_loop", 70, 8, 96),
                                                     ("c36w", 2, "last_loop", 64, 8, 96)])
def test_mxfp8_weights_generate(name, k, mode, n, steps, ctx):
    m, w, dw = model_and_weights(name)
    prompt = make_tokens(m, 50, (1, n))
    ora = LoopedNGPT(m, _mx_oracle_weights(m, w), max_ctx=ctx)
    o_tok, o_log = ora.generate(prompt, steps, k, mode)
    dq = dory.quantize_weights_mxfp8(m, dw)
    s = dory.Session(m, dq, max_batch=1, max_ctx=ctx, max_chunk=n, max_loops=8, kv_mode=mode,
                     kv_loops=k if mode == "per_loop" else 1, weight_format=dory.WEIGHTS_MXFP8)
    g_tok, g_log, lib_next = generate(s, prompt, steps, k)
    assert _report(f"{name} MXFP8 {mode} k={k}", g_log, o_log) <= BF16_TOL
    np.testing.assert_array_equal(g_tok, o_tok)
    np.testing.assert_array_equal(lib_next, g_tok[:, 1:])


# ---------------------------------------------------------------------------
# NVFP4-style layer projections: the oracle runs on its own quantisation (the
# least-error block scales, dequantised exactly in float64); the library
# quantises on the device and decodes with the 4-bit GEMVs (prefill expands
# e2m1 * e4m3 to bfloat16 and applies the tensor scale in the GEMM)
# ---------------------------------------------------------------------------
_fp4_cache = {}


def _fp4_oracle_weights(name, m, w):
    from oracle import nvfp4
    from synth.gen import bf16_bits_to_f32
    if name not in _fp4_cache:
        out = dict(w)
        for l in range(m.n_layers):
            for p in ("qkvg", "o", "ug", "down"):
                q, sc, g = nvfp4.quantize(bf16_bits_to_f32(w[f"L{l}.{p}"]).astype(np.float64), use_c=True)
                out[f"L{l}.{p}"] = nvfp4.dequantize(q, sc, g)
        _fp4_cache[name] = out
    return _fp4_cache[name]


@pytest.mark.parametrize("name,k,mode,n,steps,ctx", [("tiny_mx", 2, "last_loop", 100, 16, 160),
                                                     ("tiny_mx", 3, "per_loop", 70, 8, 96),
                                                     ("wide_fp4", 2, "last_loop", 96, 8, 128)])
def test_nvfp4_weights_generate(name, k, mode, n, steps, ctx):
    m, w, dw = model_and_weights(name)
    prompt = make_tokens(m, 60, (1, n))
    ora = LoopedNGPT(m, _fp4_oracle_weights(name, m, w), max_ctx=ctx)
    o_tok, o_log = ora.generate(prompt, steps, k, mode)
    dq = dory.quantize_weights_nvfp4(m, dw)
    s = dory.Session(m, dq, max_batch=1, max_ctx=ctx, max_chunk=n, max_loops=8, kv_mode=mode,
                     kv_loops=k if mode == "per_loop" else 1, weight_format=dory.WEIGHTS_NVFP4)
    g_tok, g_log, lib_next = generate(s, prompt, steps, k)
    assert _report(f"{name} NVFP4 {mode} k={k}", g_log, o_log) <= BF16_TOL
    np.testing.assert_array_equal(g_tok, o_tok)
    np.testing.assert_array_equal(lib_next, g_tok[:, 1:])


# ---------------------------------------------------------------------------
# batched decode across the row-count boundaries of the decode kernels: up to
# 8 rows take the GEMVs (sums by atomics into the output GEMV), more rows the
# split merge and the tiled GEMMs (low-bit weights expanded to bfloat16)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name,fmt,B", [("tiny_bf16", "bf16", 10), ("tiny_bf16", "bf16", 7),
                                        # 36-layer widths: the output (K 3072) and down (K 8192)
                                        # projections split their contraction in two at 9..64 rows
                                        ("c36w", "bf16", 12), ("c36w", "bf16", 36),
                                        ("tiny_mx", "mxfp8", 10), ("tiny_mx", "mxfp8", 5),
                                        ("tiny_mx", "nvfp4", 3), ("tiny_mx", "nvfp4", 9)])
def test_batched_decode_row_paths(name, fmt, B):
    m, w, dw = model_and_weights(name)
    k, n, steps, ctx = (2, 40, 6, 64) if name != "c36w" else (2, 16, 4, 64)
    prompt = make_tokens(m, 70 + B, (B, n))
    if fmt == "bf16":
        ow, gw, wf = w, dw, dory.WEIGHTS_DTYPE
    elif fmt == "mxfp8":
        ow, gw, wf = _mx_oracle_weights(m, w), dory.quantize_weights_mxfp8(m, dw), dory.WEIGHTS_MXFP8
    else:
        ow, gw, wf = _fp4_oracle_weights(name, m, w), dory.quantize_weights_nvfp4(m, dw), dory.WEIGHTS_NVFP4
    ora = LoopedNGPT(m, ow, max_ctx=ctx, batch=B)
    o_tok, o_log = ora.generate(prompt, steps, k, "last_loop")
    s = dory.Session(m, gw, max_batch=B, max_ctx=ctx, max_chunk=n, max_loops=8, kv_mode="last_loop",
                     weight_format=wf)
    g_tok, g_log, lib_next = generate(s, prompt, steps, k)
    assert _report(f"{name} {fmt} batch {B}", g_log, o_log) <= BF16_TOL
    np.testing.assert_array_equal(g_tok, o_tok)
    np.testing.assert_array_equal(lib_next, g_tok[:, 1:])


# ---------------------------------------------------------------------------
# resuming from a caller-filled KV buffer: a copy of one context's cache,
# resumed in a second context, decodes exactly like the first
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name,mode", [("tiny_bf16", "last_loop"), ("tiny_bf16", "per_loop"), ("tiny", "last_loop")])
def test_resume_from_copied_cache_bit_identical(name, mode):
    m, w, dw = model_and_weights(name)
    B, n, k, ctx = 2, 77, 2, 128
    prompt = torch.from_numpy(make_tokens(m, 30, (B, n))).cuda()
    a = session(m, dw, batch=B, max_ctx=ctx, chunk=64, kv_mode=mode, k=k)
    b = session(m, dw, batch=B, max_ctx=ctx, chunk=64, kv_mode=mode, k=k)
    a.prefill(prompt, k)
    first = torch.argmax(a.logits(), dim=-1).to(torch.int32)
    torch.cuda.synchronize()
    b.kv.copy_(a.kv)
    b.resume(B, n, k)
    toks = [first] + [torch.tensor([(7 * i + 3) % m.vocab] * B, dtype=torch.int32, device="cuda") for i in range(4)]
    for i, t in enumerate(toks):
        a.decode(t.contiguous(), k)
        b.decode(t.contiguous(), k)
        la, lb = a.logits().cpu().numpy(), b.logits().cpu().numpy()
        np.testing.assert_array_equal(la, lb, err_msg=f"step {i}")
    # greedy continuation also works after the explicit first token
    b.decode(None, k)
    a.decode(None, k)
    np.testing.assert_array_equal(a.logits().cpu().numpy(), b.logits().cpu().numpy())


# ---------------------------------------------------------------------------
# recorded decode steps: continued greedy decoding of a bfloat16 model is
# recorded once per (loop count, batch) and replayed; each replay must equal
# the same step launched kernel by kernel
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("mode", ["last_loop", "per_loop"])
def test_bf16_decode_graph_replays_match_eager(mode):
    """Bit-identical logits and tokens at every replay, with eager torch work
    and synchronisations between replays, loop counts switching between
    recordings (last-loop mode), and a second sequence after a reset that
    reuses the recordings (its position comes from the device counter)."""
    m, w, dw = model_and_weights("tiny_bf16")
    B, ctx = 2, 192
    sched = [2, 2, 3, 1, 3, 2, 2, 1, 3, 3] if mode == "last_loop" else [3] * 10
    runs = []
    for graphs in (False, True):
        s = session(m, dw, batch=B, max_ctx=ctx, chunk=64, kv_mode=mode, k=3)
        s.set_graphs(graphs)
        out = []
        for seq in range(2):
            k0 = 2 if mode == "last_loop" else 3
            prompt = torch.from_numpy(make_tokens(m, 10 + seq, (B, 70 + 9 * seq))).cuda()
            print(f"graphs={graphs} {mode} seq {seq}", flush=True)
            s.prefill(prompt, k0)
            for k in sched:
                nxt = torch.empty(B, dtype=torch.int32, device="cuda")
                s.decode(None, k, next_tokens=nxt)
                lg = s.logits()
                junk = torch.randn(4096, device="cuda").sum()      # unrelated eager work between replays
                torch.cuda.synchronize()
                assert torch.isfinite(junk)
                out.append((lg.cpu().numpy(), nxt.cpu().numpy()))
            s.reset()
        runs.append(out)
    for i, ((la, ta), (lb, tb)) in enumerate(zip(*runs)):
        np.testing.assert_array_equal(ta, tb, err_msg=f"step {i}")
        np.testing.assert_array_equal(la, lb, err_msg=f"step {i}")
    # the greedy tokens are the argmax of the logits they follow
    for (la, ta) in runs[1]:
        np.testing.assert_array_equal(np.argmax(la, axis=-1), ta)


# ---------------------------------------------------------------------------
# a decode step captured into the caller's own graph: the library sees the
# capture and has the decode attention read the position from the device
# counter (on eager calls it passes the position by value), so every replay
# continues the sequence
# ---------------------------------------------------------------------------
def test_bf16_decode_captured_by_caller_replays_match_eager():
    m, w, dw = model_and_weights("tiny_bf16")
    B, ctx, k, steps = 2, 192, 2, 6
    prompt = torch.from_numpy(make_tokens(m, 31, (B, 50))).cuda()
    stream = torch.cuda.Stream()
    ref = []
    s = dory.Session(m, dw, max_batch=B, max_ctx=ctx, max_chunk=64, kv_mode="last_loop", stream=stream)
    with torch.cuda.stream(stream):
        s.prefill(prompt, k)
        for _ in range(steps):
            s.decode(None, k)
            ref.append(s.logits().clone())
    torch.cuda.synchronize()
    s2 = dory.Session(m, dw, max_batch=B, max_ctx=ctx, max_chunk=64, kv_mode="last_loop", stream=stream)
    with torch.cuda.stream(stream):
        s2.prefill(prompt, k)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    print("capturing one decode step", flush=True)
    with torch.cuda.graph(g, stream=stream):
        s2.decode(None, k)           # recorded, not run: replays advance the device position
    got = []
    for i in range(steps):
        with torch.cuda.stream(stream):                     # the replay and the copy on the session's stream
            g.replay()
            got.append(s2.logits().clone())
        junk = torch.randn(4096, device="cuda").sum()      # unrelated eager work between replays
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
    for i, (a, b) in enumerate(zip(ref, got)):
        np.testing.assert_array_equal(a.cpu().numpy(), b.cpu().numpy(), err_msg=f"replay {i}")


def test_markers_leave_results_unchanged():
    """roctx ranges around calls and layer applications are host-side only."""
    m, w, dw = model_and_weights("tiny_bf16")
    prompt = make_tokens(m, 32, (1, 40))
    outs = []
    for markers in (False, True):
        s = session(m, dw, batch=1, max_ctx=128, chunk=64, kv_mode="per_loop", k=2)
        try:
            s.set_markers(markers)
        except dory.DoryError:
            pytest.skip("no ROCm marker library on this machine")
        toks, logits, _ = generate(s, prompt, 5, 2)
        outs.append((toks, logits))
    np.testing.assert_array_equal(outs[0][0], outs[1][0])
    np.testing.assert_array_equal(outs[0][1], outs[1][1])
