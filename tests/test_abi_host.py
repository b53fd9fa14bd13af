"""Host-side checks of the C ABI (no GPU): the library loads, exports every
function include/dory.h declares, its KV layout equals the oracle's spec
bit for bit, and argument validation returns the documented codes without
touching HIP."""
import ctypes
import os
import re
import subprocess

import pytest

import looped_ngpt_amd as dory
from looped_ngpt_amd import binding
from oracle import kvspec
from synth.configs import ModelConfig, get_config, pattern_alternating, pattern_every4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "dory.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dory_[a-z0-9_]+)\s*\(", text)))


def test_exports_match_header():
    decl = declared_functions()
    assert sorted(binding.EXPORTS) == decl
    nm = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (dory_\w+)", nm))
    for f in decl:
        assert f in exported, f
        assert hasattr(dory.lib(), f)


def small(**kw):
    base = dict(name="t", d_model=64, n_q_heads=4, n_kv_heads=2, head_dim=64, d_ff=96, vocab=128,
                n_in=2, n_rec=3, n_out=1, window=5, layer_is_full=pattern_alternating(6), dtype="bf16")
    base.update(kw)
    return ModelConfig(**base)


@pytest.mark.parametrize("model,max_ctx,batch", [(small(), 11, 1), (small(dtype="f32", window=64), 40, 3),
                                                 (get_config("c36"), 8448, 1), (get_config("c72"), 16640, 1),
                                                 (get_config("c36"), 32896, 64)])
def test_kv_bytes_match_spec(model, max_ctx, batch):
    c, _keep = dory.make_config(model, max_batch=batch, max_ctx=max_ctx, max_chunk=min(max_ctx, 64))
    for mode, code in dory.KV_MODES.items():
        for loops in (1, 2, 3, 4, 8):
            assert dory.kv_bytes(c, code, loops) == kvspec.kv_bytes(model, mode, loops, max_ctx, batch)


def test_last_loop_bytes_flat_per_loop_linear():
    c, _k = dory.make_config(get_config("c72"), max_batch=1, max_ctx=16640, max_chunk=8192)
    last = [dory.kv_bytes(c, dory.DORY_KV_LAST_LOOP, k) for k in (1, 2, 3, 4)]
    per = [dory.kv_bytes(c, dory.DORY_KV_PER_LOOP, k) for k in (1, 2, 3, 4)]
    assert len(set(last)) == 1 and per[0] == last[0]
    assert len({per[i + 1] - per[i] for i in range(3)}) == 1


@pytest.mark.parametrize("mode", ["per_loop", "last_loop"])
def test_kv_slot_bit_exact(mode):
    model = small(n_rec=2, layer_is_full=pattern_every4(5), n_in=2, n_out=1)
    B, T, loops = 2, 13, 3
    c, _k = dory.make_config(model, max_batch=B, max_ctx=T, max_chunk=T)
    code = dory.KV_MODES[mode]
    for l in range(model.n_layers):
        js = range(1, loops + 1) if model.is_recurrent(l) else [0]
        for j in js:
            for p in range(T):
                cid, slot, ko, vo = dory.kv_slot(c, code, loops, l, j, p)
                assert cid == kvspec.cache_id(model, mode, loops, l, j)
                assert slot == kvspec.slot(model, T, l, p)
                assert ko == kvspec.element_offset(model, mode, loops, T, B, l, j, "K", 0, 0, p)
                assert vo == kvspec.element_offset(model, mode, loops, T, B, l, j, "V", 0, 0, p)


@pytest.mark.parametrize("bad", [dict(head_dim=96), dict(n_q_heads=5, n_kv_heads=1), dict(window=0),
                                 dict(d_ff=100), dict(attn_gate=3), dict(rope_base_swa=1.0),
                                 dict(n_in=0, n_rec=0, n_out=0, layer_is_full=())])
def test_invalid_configs(bad):
    m = small(**bad)
    c, _k = dory.make_config(m, max_batch=1, max_ctx=16, max_chunk=16)
    assert dory.validate_config(c) == dory.DORY_E_ARG
    assert dory.kv_bytes(c, 0, 1) == 0 and dory.workspace_bytes(c) == 0


def test_capacity_configs():
    m = small()
    c, _k = dory.make_config(m, max_batch=1, max_ctx=16, max_chunk=32)    # chunk > ctx
    assert dory.validate_config(c) == dory.DORY_E_ARG
    c, _k = dory.make_config(m, max_batch=1, max_ctx=16, max_chunk=16, max_loops=2)
    assert dory.validate_config(c) == dory.DORY_OK
    assert dory.kv_bytes(c, dory.DORY_KV_PER_LOOP, 3) == 0                 # more caches than max_loops


def test_weight_format_configs():
    """MXFP8 projections need a bfloat16 model whose contraction widths are
    multiples of 32; the workspace grows by one expanded projection."""
    m = small(dtype="bf16", d_ff=704)
    base, _k1 = dory.make_config(m, max_batch=1, max_ctx=16, max_chunk=16)
    mx, _k2 = dory.make_config(m, max_batch=1, max_ctx=16, max_chunk=16, weight_format=dory.WEIGHTS_MXFP8)
    assert dory.validate_config(base) == dory.DORY_OK and dory.validate_config(mx) == dory.DORY_OK
    qkvg_dim = 2 * m.q_dim + 2 * m.kv_dim
    biggest = max(qkvg_dim * m.d_model, m.d_model * m.q_dim, 2 * m.d_ff * m.d_model) * 2
    assert biggest <= dory.workspace_bytes(mx) - dory.workspace_bytes(base) < biggest + 512
    for bad in (small(dtype="bf16", d_ff=688), small(dtype="f32", d_ff=704)):
        c, _k = dory.make_config(bad, max_batch=1, max_ctx=16, max_chunk=16, weight_format=dory.WEIGHTS_MXFP8)
        assert dory.validate_config(c) == dory.DORY_E_ARG
    fp4, _k3 = dory.make_config(m, max_batch=1, max_ctx=16, max_chunk=16, weight_format=dory.WEIGHTS_NVFP4)
    assert dory.validate_config(fp4) == dory.DORY_OK
    assert dory.workspace_bytes(fp4) == dory.workspace_bytes(mx)
    for bad in (small(dtype="bf16", d_ff=688), small(dtype="f32", d_ff=704)):
        c, _k = dory.make_config(bad, max_batch=1, max_ctx=16, max_chunk=16, weight_format=dory.WEIGHTS_NVFP4)
        assert dory.validate_config(c) == dory.DORY_E_ARG
    c, _k = dory.make_config(m, max_batch=1, max_ctx=16, max_chunk=16, weight_format=3)
    assert dory.validate_config(c) == dory.DORY_E_ARG


class FakeCtx:
    """A context bound to fake, aligned device addresses: only the validation
    paths (which return before any HIP call) may be exercised with it."""

    def __init__(self, model, *, kv_mode="last_loop", kv_loops=1, max_batch=2, max_ctx=16, max_loops=4,
                 kv_bytes=None, ws_bytes=None, kv_addr=1 << 20, ws_addr=1 << 30, weight_format=0,
                 scales=False, tscales=None):
        L = model.n_layers
        self.c, self._k = dory.make_config(model, max_batch=max_batch, max_ctx=max_ctx, max_chunk=8,
                                           max_loops=max_loops, weight_format=weight_format)
        arrs = [(ctypes.c_void_p * L)(*[(1 << 16) * (l + 1) for l in range(L)]) for _ in range(6)]
        self._arrs = arrs
        vp = lambda a: ctypes.cast(a, ctypes.POINTER(ctypes.c_void_p))
        self.w = binding.DoryWeights(embed=1 << 12, qkvg=vp(arrs[0]), o=vp(arrs[1]), ug=vp(arrs[2]),
                                     down=vp(arrs[3]), alpha_attn=vp(arrs[4]), alpha_mlp=vp(arrs[5]))
        if scales:   # fake block-scale arrays (even addresses)
            sarrs = [(ctypes.c_void_p * L)(*[(1 << 24) + 64 * (l + 1) for l in range(L)]) for _ in range(4)]
            self._arrs += sarrs
            self.w.qkvg_scale, self.w.o_scale, self.w.ug_scale, self.w.down_scale = [vp(a) for a in sarrs]
        if tscales is not None:
            tarr = (ctypes.c_float * L)(*tscales)
            self._arrs.append(tarr)
            fp = ctypes.cast(tarr, ctypes.POINTER(ctypes.c_float))
            self.w.qkvg_tscale = self.w.o_tscale = self.w.ug_tscale = self.w.down_tscale = fp
        code = dory.KV_MODES[kv_mode]
        kvb = dory.kv_bytes(self.c, code, kv_loops) if kv_bytes is None else kv_bytes
        wsb = dory.workspace_bytes(self.c) if ws_bytes is None else ws_bytes
        h = ctypes.c_void_p()
        self.status = dory.lib().dory_create(ctypes.byref(self.c), ctypes.byref(self.w), kv_addr, kvb, code,
                                             kv_loops, ws_addr, wsb, None, ctypes.byref(h))
        self.h = h

    def __del__(self):
        if self.h:
            dory.lib().dory_destroy(self.h)


def test_create_validation():
    m = small()
    assert FakeCtx(m).status == dory.DORY_OK
    # MXFP8 projections without their scale arrays
    mb = small(dtype="bf16", d_ff=704)
    assert FakeCtx(mb, weight_format=dory.WEIGHTS_MXFP8).status == dory.DORY_E_ARG
    assert FakeCtx(mb, weight_format=dory.WEIGHTS_MXFP8, scales=True).status == dory.DORY_OK
    # NVFP4 projections need block scales and positive finite tensor scales
    L = mb.n_layers
    assert FakeCtx(mb, weight_format=dory.WEIGHTS_NVFP4, scales=True).status == dory.DORY_E_ARG
    assert FakeCtx(mb, weight_format=dory.WEIGHTS_NVFP4, tscales=[0.01] * L).status == dory.DORY_E_ARG
    assert FakeCtx(mb, weight_format=dory.WEIGHTS_NVFP4, scales=True, tscales=[0.01] * L).status == dory.DORY_OK
    for badg in (0.0, -1.0, float("inf"), float("nan")):
        t = [0.01] * L
        t[L - 1] = badg
        assert FakeCtx(mb, weight_format=dory.WEIGHTS_NVFP4, scales=True, tscales=t).status == dory.DORY_E_ARG
    assert FakeCtx(m, kv_bytes=100).status == dory.DORY_E_ARG
    assert FakeCtx(m, ws_bytes=100).status == dory.DORY_E_ARG
    assert FakeCtx(m, kv_addr=(1 << 20) + 8).status == dory.DORY_E_ARG
    assert FakeCtx(m, kv_mode="per_loop", kv_loops=5).status == dory.DORY_E_LOOPS


def test_call_validation_codes():
    m = small()
    L = dory.lib()
    f = FakeCtx(m, kv_mode="per_loop", kv_loops=2)
    assert f.status == dory.DORY_OK
    h = f.h
    tok = 1 << 14
    PL, LL = dory.DORY_KV_PER_LOOP, dory.DORY_KV_LAST_LOOP
    assert L.dory_decode_step(h, tok, 2, PL, None) == dory.DORY_E_STATE
    assert L.dory_logits(h, 1 << 14) == dory.DORY_E_STATE
    assert L.dory_prefill(h, None, 1, 4, 2, PL) == dory.DORY_E_ARG
    assert L.dory_prefill(h, tok, 1, 4, 0, PL) == dory.DORY_E_LOOPS
    assert L.dory_prefill(h, tok, 1, 4, 5, PL) == dory.DORY_E_LOOPS          # > max_loops
    assert L.dory_prefill(h, tok, 1, 4, 3, PL) == dory.DORY_E_LOOPS          # > per-loop caches
    assert L.dory_prefill(h, tok, 1, 4, 2, LL) == dory.DORY_E_KV_MODE
    assert L.dory_prefill(h, tok, 3, 4, 2, PL) == dory.DORY_E_CAPACITY       # batch
    assert L.dory_prefill(h, tok, 1, 17, 2, PL) == dory.DORY_E_CAPACITY      # context
    assert L.dory_prefill(h, tok, 1, 0, 2, PL) == dory.DORY_OK               # empty: no-op
    assert L.dory_decode_step(h, tok, 2, PL, None) == dory.DORY_E_STATE      # still nothing prefilled
    assert L.dory_set_trace(h, 1 << 14, 0) == dory.DORY_E_ARG
    assert L.dory_set_trace(h, 1 << 14, 3) == dory.DORY_OK
    assert L.dory_prefill(h, tok, 1, 4, 2, PL) == dory.DORY_E_CAPACITY       # 2+1+2*3 apps > 3
    assert L.dory_set_trace(h, None, 0) == dory.DORY_OK
    assert b"capacity" in L.dory_status_string(dory.DORY_E_CAPACITY)
    assert L.dory_reset(h) == dory.DORY_OK
    assert L.dory_reset(None) == dory.DORY_E_ARG
    # resuming from a caller-filled cache: every bad argument is caught before any device work
    assert L.dory_resume(h, 0, 4, 2, PL) == dory.DORY_E_CAPACITY             # batch
    assert L.dory_resume(h, 3, 4, 2, PL) == dory.DORY_E_CAPACITY
    assert L.dory_resume(h, 1, 0, 2, PL) == dory.DORY_E_CAPACITY             # pos
    assert L.dory_resume(h, 1, 16, 2, PL) == dory.DORY_E_CAPACITY            # pos = max_ctx
    assert L.dory_resume(h, 1, 4, 2, LL) == dory.DORY_E_KV_MODE
    assert L.dory_resume(h, 1, 4, 3, PL) == dory.DORY_E_LOOPS                # > per-loop caches
    assert L.dory_resume(h, 1, 4, 0, PL) == dory.DORY_E_LOOPS
    assert L.dory_resume(None, 1, 4, 2, PL) == dory.DORY_E_ARG


def test_mixed_loop_validation_codes():
    m = small()
    L = dory.lib()
    LL, PL = dory.DORY_KV_LAST_LOOP, dory.DORY_KV_PER_LOOP
    tok = 1 << 14
    arr = lambda *v: ctypes.cast((ctypes.c_int32 * len(v))(*v), ctypes.c_void_p)
    f = FakeCtx(m, kv_mode="last_loop")
    assert f.status == dory.DORY_OK
    h = f.h
    ok2 = arr(1, 3)
    assert L.dory_prefill_mixed(h, tok, 2, 4, None, LL) == dory.DORY_E_ARG
    assert L.dory_prefill_mixed(h, None, 2, 4, ok2, LL) == dory.DORY_E_ARG
    assert L.dory_prefill_mixed(h, tok, 2, 4, ok2, PL) == dory.DORY_E_KV_MODE
    assert L.dory_prefill_mixed(h, tok, 2, 4, arr(1, 5), LL) == dory.DORY_E_LOOPS   # > max_loops
    assert L.dory_prefill_mixed(h, tok, 2, 4, arr(0, 1), LL) == dory.DORY_E_LOOPS
    assert L.dory_prefill_mixed(h, tok, 3, 4, arr(1, 1, 1), LL) == dory.DORY_E_CAPACITY  # batch
    assert L.dory_prefill_mixed(h, tok, 2, 17, ok2, LL) == dory.DORY_E_CAPACITY          # context
    assert L.dory_prefill_mixed(h, tok, 2, 0, ok2, LL) == dory.DORY_OK                   # empty: no-op
    assert L.dory_decode_step_mixed(h, tok, ok2, LL, None) == dory.DORY_E_STATE          # nothing prefilled
    g = FakeCtx(m, kv_mode="per_loop", kv_loops=2)
    assert L.dory_prefill_mixed(g.h, tok, 2, 4, ok2, PL) == dory.DORY_E_KV_MODE         # per-loop caches


def test_op_validation():
    L = dory.lib()
    assert L.dory_op_linear(2, 1 << 12, 8, 1 << 12, 1 << 12, 1, 8, 8, 0, 1.0, 0, None) == dory.DORY_E_ARG
    assert L.dory_op_linear(1, 1 << 12, 4, 1 << 12, 1 << 12, 1, 8, 8, 0, 1.0, 0, None) == dory.DORY_E_ARG  # ldx < K
    assert L.dory_op_linear(1, 1 << 12, 8, 1 << 12, 1 << 12, 1, 7, 8, 1, 1.0, 0, None) == dory.DORY_E_ARG  # odd SwiGLU N
    assert L.dory_op_argmax(None, 1, 8, 1 << 12, 1 << 12, None) == dory.DORY_E_ARG
    assert dory.argmax_scratch_bytes(2, 3000) == 2 * 3 * 8


def test_backward_workspace_and_validation():
    """dory_backward_workspace_bytes grows with the rows; dory_backward_last_loop
    rejects bad arguments on the host, before anything is enqueued."""
    m = small(dtype="bf16", d_ff=704)
    c, _k = dory.make_config(m, max_batch=1, max_ctx=16, max_chunk=16)
    a = dory.backward_workspace_min_bytes(c, 1, 8)
    b = dory.backward_workspace_min_bytes(c, 2, 8)
    assert 0 < a < b and dory.backward_workspace_min_bytes(c, 0, 8) == 0
    # the checkpointed layer inputs alone: (n_rec + 1) * rows * d float32
    assert a >= (m.n_rec + 1) * 8 * m.d_model * 4
    # keeping every recurrent layer's forward values: one more group per layer
    s1, s2 = dory.backward_workspace_bytes(c, 1, 8), dory.backward_workspace_bytes(c, 2, 8)
    assert a < s1 < s2 and dory.backward_workspace_bytes(c, 1, 0) == 0
    assert m.n_rec == 1 or (s1 - a) % (m.n_rec - 1) == 0
    lib = dory.lib()
    L = m.n_rec
    fake = (ctypes.c_void_p * L)(*[(1 << 20) * (i + 1) for i in range(L)])
    vp = ctypes.cast(fake, ctypes.POINTER(ctypes.c_void_p))
    g = binding.DoryGrads(qkvg=vp, o=vp, ug=vp, down=vp, alpha_attn=vp, alpha_mlp=vp)
    ctx = FakeCtx(m, max_ctx=16)
    assert ctx.status == dory.DORY_OK
    ws = 1 << 30
    call = lambda n, grads, wsb, x=1 << 12: lib.dory_backward_last_loop(ctx.h, x, 1 << 12, 1, n,
                                                                       ctypes.byref(grads) if grads else None,
                                                                       None, ws, wsb)
    assert call(17, g, 1 << 40) == dory.DORY_E_ARG          # n > max_ctx
    assert call(8, None, 1 << 40) == dory.DORY_E_ARG        # no gradient arrays
    assert call(8, g, 100) == dory.DORY_E_ARG               # workspace too small
    assert call(8, g, 1 << 40, x=0) == dory.DORY_E_ARG      # no input
    zero = (ctypes.c_void_p * L)(*([0] * L))
    g0 = binding.DoryGrads(qkvg=vp, o=vp, ug=vp, down=vp, alpha_attn=ctypes.cast(zero, ctypes.POINTER(ctypes.c_void_p)),
                           alpha_mlp=vp)
    assert call(8, g0, 1 << 40) == dory.DORY_E_ARG          # a null gradient pointer
    mx = FakeCtx(m, weight_format=dory.WEIGHTS_MXFP8, scales=True, max_ctx=16)
    assert mx.status == dory.DORY_OK
    assert lib.dory_backward_last_loop(mx.h, 1 << 12, 1 << 12, 1, 8, ctypes.byref(g), None, ws,
                                       1 << 40) == dory.DORY_E_ARG   # low-bit weights
