"""ctypes binding of libdory.so (the C ABI in include/dory.h).

Argument marshalling only: every step of the forward pass runs in the HIP
library. PyTorch provides device memory and the stream. If the library is
missing this module raises at import time; there is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Dict, Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libdory.so")

# PyTorch ships its own HIP runtime with the same soname (libamdhip64.so.7).
# Loading torch first makes the loader bind libdory.so to that runtime, so
# one process never holds two HIP runtimes (the second finds no device).
try:
    import torch as _torch  # noqa: F401
except ImportError:  # host-only use (sizes, layout, validation) needs no torch
    _torch = None

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m looped_ngpt_amd.build` "
                      "(the HIP library is the only implementation; there is no fallback)")
_lib = ctypes.CDLL(LIB_PATH)

DORY_OK, DORY_E_ARG, DORY_E_CAPACITY, DORY_E_LOOPS, DORY_E_KV_MODE, DORY_E_STATE, DORY_E_HIP = 0, -1, -2, -3, -4, -5, -6
DORY_F32, DORY_BF16 = 0, 1
DORY_KV_PER_LOOP, DORY_KV_LAST_LOOP = 0, 1
KV_MODES = {"per_loop": DORY_KV_PER_LOOP, "last_loop": DORY_KV_LAST_LOOP}

# every function dory.h declares, for the export check
EXPORTS = ["dory_validate_config", "dory_kv_bytes", "dory_workspace_bytes", "dory_kv_slot",
           "dory_status_string", "dory_create", "dory_destroy", "dory_reset", "dory_prefill",
           "dory_decode_step", "dory_resume", "dory_prefill_mixed", "dory_decode_step_mixed", "dory_op_quant_mxfp8",
           "dory_op_linear_mx", "dory_op_quant_nvfp4", "dory_op_linear_fp4", "dory_logits", "dory_last_error", "dory_set_trace", "dory_set_graphs", "dory_set_markers",
           "dory_set_kernel_timing",
           "dory_kernel_time", "dory_op_linear",
           "dory_argmax_scratch_bytes", "dory_op_argmax", "dory_op_argmax_noalloc", "dory_backward_workspace_bytes", "dory_backward_workspace_min_bytes",
           "dory_backward_last_loop"]


class DoryConfig(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("n_in", ctypes.c_int32), ("n_rec", ctypes.c_int32), ("n_out", ctypes.c_int32),
                ("window", ctypes.c_int32), ("layer_is_full", ctypes.POINTER(ctypes.c_uint8)),
                ("rope_base_swa", ctypes.c_double), ("rope_base_full", ctypes.c_double),
                ("dtype", ctypes.c_int32), ("attn_gate", ctypes.c_int32),
                ("attn_scale", ctypes.c_float), ("logit_scale", ctypes.c_float),
                ("combine_wh", ctypes.c_float), ("combine_we", ctypes.c_float),
                ("max_batch", ctypes.c_int32), ("max_ctx", ctypes.c_int32), ("max_chunk", ctypes.c_int32),
                ("max_loops", ctypes.c_int32), ("weight_format", ctypes.c_int32)]


class DoryWeights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("qkvg", ctypes.POINTER(ctypes.c_void_p)),
                ("o", ctypes.POINTER(ctypes.c_void_p)), ("ug", ctypes.POINTER(ctypes.c_void_p)),
                ("down", ctypes.POINTER(ctypes.c_void_p)), ("alpha_attn", ctypes.POINTER(ctypes.c_void_p)),
                ("alpha_mlp", ctypes.POINTER(ctypes.c_void_p)),
                ("qkvg_scale", ctypes.POINTER(ctypes.c_void_p)), ("o_scale", ctypes.POINTER(ctypes.c_void_p)),
                ("ug_scale", ctypes.POINTER(ctypes.c_void_p)), ("down_scale", ctypes.POINTER(ctypes.c_void_p)),
                ("qkvg_tscale", ctypes.POINTER(ctypes.c_float)), ("o_tscale", ctypes.POINTER(ctypes.c_float)),
                ("ug_tscale", ctypes.POINTER(ctypes.c_float)), ("down_tscale", ctypes.POINTER(ctypes.c_float))]


class DoryGrads(ctypes.Structure):
    _fields_ = [(k, ctypes.POINTER(ctypes.c_void_p)) for k in ("qkvg", "o", "ug", "down", "alpha_attn", "alpha_mlp")]


_P = ctypes.c_void_p
_I = ctypes.c_int32
_C = ctypes.POINTER(DoryConfig)
_sig = {
    "dory_validate_config": (_I, [_C]),
    "dory_kv_bytes": (ctypes.c_size_t, [_C, _I, _I]),
    "dory_workspace_bytes": (ctypes.c_size_t, [_C]),
    "dory_kv_slot": (_I, [_C, _I, _I, _I, _I, _I, ctypes.POINTER(_I), ctypes.POINTER(_I),
                          ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)]),
    "dory_status_string": (ctypes.c_char_p, [_I]),
    "dory_create": (_I, [_C, ctypes.POINTER(DoryWeights), _P, ctypes.c_size_t, _I, _I, _P, ctypes.c_size_t, _P,
                         ctypes.POINTER(_P)]),
    "dory_destroy": (None, [_P]),
    "dory_reset": (_I, [_P]),
    "dory_prefill": (_I, [_P, _P, _I, _I, _I, _I]),
    "dory_decode_step": (_I, [_P, _P, _I, _I, _P]),
    "dory_logits": (_I, [_P, _P]),
    "dory_last_error": (ctypes.c_char_p, [_P]),
    "dory_set_trace": (_I, [_P, _P, _I]),
    "dory_set_graphs": (_I, [_P, _I]),
    "dory_set_markers": (_I, [_P, _I]),
    "dory_resume": (_I, [_P, _I, _I, _I, _I]),
    "dory_prefill_mixed": (_I, [_P, _P, _I, _I, _P, _I]),
    "dory_decode_step_mixed": (_I, [_P, _P, _P, _I, _P]),
    "dory_op_quant_mxfp8": (_I, [_P, _I, _I, _P, _P, _P]),
    "dory_op_linear_mx": (_I, [_P, ctypes.c_int64, _P, _P, _P, _I, _I, _I, _I, ctypes.c_float, _P]),
    "dory_op_quant_nvfp4": (_I, [_P, _I, _I, _P, _P, _P, _P]),
    "dory_op_linear_fp4": (_I, [_P, ctypes.c_int64, _P, _P, _P, _I, _I, _I, _I, ctypes.c_float, _P]),
    "dory_set_kernel_timing": (_I, [_P, _I, _I]),
    "dory_kernel_time": (_I, [_P, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_I)]),
    "dory_op_linear": (_I, [_I, _P, ctypes.c_int64, _P, _P, _I, _I, _I, _I, ctypes.c_float, _I, _P]),
    "dory_argmax_scratch_bytes": (ctypes.c_size_t, [_I, _I]),
    "dory_op_argmax": (_I, [_P, _I, _I, _P, _P, _P]),
    "dory_op_argmax_noalloc": (_I, [_P, _I, _I, _P, _P]),
    "dory_backward_workspace_bytes": (ctypes.c_size_t, [_C, _I, _I]),
    "dory_backward_workspace_min_bytes": (ctypes.c_size_t, [_C, _I, _I]),
    "dory_backward_last_loop": (_I, [_P, _P, _P, _I, _I, ctypes.POINTER(DoryGrads), _P, _P, ctypes.c_size_t]),
}
for _name, (_res, _args) in _sig.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args


class DoryError(RuntimeError):
    def __init__(self, status: int, msg: str = ""):
        self.status = status
        text = _lib.dory_status_string(status).decode()
        super().__init__(f"{text} ({status}){': ' + msg if msg else ''}")


def lib():
    return _lib


WEIGHTS_DTYPE, WEIGHTS_MXFP8, WEIGHTS_NVFP4 = 0, 1, 2
PROJECTIONS = ("qkvg", "o", "ug", "down")


def make_config(model, *, max_batch: int, max_ctx: int, max_chunk: int, max_loops: int = 8,
                weight_format: int = 0):
    """dory_config for a synth.ModelConfig. Returns (struct, keepalive)."""
    full = (ctypes.c_uint8 * model.n_layers)(*[1 if f else 0 for f in model.layer_is_full])
    c = DoryConfig(
        d_model=model.d_model, n_q_heads=model.n_q_heads, n_kv_heads=model.n_kv_heads, head_dim=model.head_dim,
        d_ff=model.d_ff, vocab=model.vocab, n_in=model.n_in, n_rec=model.n_rec, n_out=model.n_out,
        window=model.window, layer_is_full=ctypes.cast(full, ctypes.POINTER(ctypes.c_uint8)),
        rope_base_swa=model.rope_base_swa, rope_base_full=model.rope_base_full,
        dtype=DORY_F32 if model.dtype == "f32" else DORY_BF16, attn_gate=model.attn_gate,
        attn_scale=float(model.attn_scale or 0.0), logit_scale=float(model.logit_scale or 0.0),
        combine_wh=model.combine_wh, combine_we=model.combine_we,
        max_batch=max_batch, max_ctx=max_ctx, max_chunk=max_chunk, max_loops=max_loops,
        weight_format=weight_format)
    return c, full


def validate_config(c: DoryConfig) -> int:
    return _lib.dory_validate_config(ctypes.byref(c))


def kv_bytes(c: DoryConfig, kv_mode: int, kv_loops: int) -> int:
    return _lib.dory_kv_bytes(ctypes.byref(c), kv_mode, kv_loops)


def workspace_bytes(c: DoryConfig) -> int:
    return _lib.dory_workspace_bytes(ctypes.byref(c))


def backward_workspace_bytes(c: DoryConfig, batch: int, n: int) -> int:
    """workspace that keeps every recurrent layer's forward values"""
    return _lib.dory_backward_workspace_bytes(ctypes.byref(c), batch, n)


def backward_workspace_min_bytes(c: DoryConfig, batch: int, n: int) -> int:
    """workspace of the backward that recomputes each layer's forward"""
    return _lib.dory_backward_workspace_min_bytes(ctypes.byref(c), batch, n)


def kv_slot(c: DoryConfig, kv_mode: int, kv_loops: int, layer: int, loop: int, pos: int):
    cid, slot = _I(), _I()
    ko, vo = ctypes.c_int64(), ctypes.c_int64()
    s = _lib.dory_kv_slot(ctypes.byref(c), kv_mode, kv_loops, layer, loop, pos, ctypes.byref(cid),
                          ctypes.byref(slot), ctypes.byref(ko), ctypes.byref(vo))
    if s != DORY_OK:
        raise DoryError(s)
    return cid.value, slot.value, ko.value, vo.value


# ---------------------------------------------------------------------------
# device side (needs torch + a GPU)
# ---------------------------------------------------------------------------

def _ptr(t) -> int:
    return t.data_ptr()


def _stream_handle(stream) -> int:
    return 0 if stream is None else int(stream.cuda_stream)


def upload_weights(model, weights: Dict, device="cuda") -> Dict:
    """numpy weights from synth.make_weights -> device tensors (raw bytes kept)."""
    import numpy as np
    import torch
    out = {}
    for k, v in weights.items():
        a = np.ascontiguousarray(v)
        if a.dtype == np.uint16:
            t = torch.from_numpy(a.view(np.int16)).to(device)
        else:
            t = torch.from_numpy(a).to(device)
        out[k] = t
    return out


def quantize_weights_mxfp8(model, dev_weights: Dict, stream=None) -> Dict:
    """bfloat16 device weights -> a dict whose layer projections are MXFP8 codes
    (uint8 [N, K]) with scales under "<name>_scale" (uint8 [N, K/32]); the rest is shared."""
    import torch
    out = dict(dev_weights)
    for l in range(model.n_layers):
        for p in PROJECTIONS:
            w = dev_weights[f"L{l}.{p}"]
            N, K = w.shape
            q = torch.empty((N, K), dtype=torch.uint8, device=w.device)
            s = torch.empty((N, K // 32), dtype=torch.uint8, device=w.device)
            op_quant_mxfp8(w, N, K, q, s, stream=stream)
            out[f"L{l}.{p}"] = q
            out[f"L{l}.{p}_scale"] = s
    return out


def quantize_weights_nvfp4(model, dev_weights: Dict, stream=None) -> Dict:
    """bfloat16 device weights -> a dict whose layer projections are NVFP4
    codes (uint8 [N, K/2]) with block scales under "<name>_scale" (uint8
    [N, K/16]) and the tensor scale under "<name>_tscale" (a Python float, read
    back from the device); the rest is shared."""
    import torch
    out = dict(dev_weights)
    for l in range(model.n_layers):
        for p in PROJECTIONS:
            w = dev_weights[f"L{l}.{p}"]
            N, K = w.shape
            q = torch.empty((N, K // 2), dtype=torch.uint8, device=w.device)
            s = torch.empty((N, K // 16), dtype=torch.uint8, device=w.device)
            g = torch.empty(1, dtype=torch.float32, device=w.device)
            op_quant_nvfp4(w, N, K, q, s, g, stream=stream)
            out[f"L{l}.{p}"] = q
            out[f"L{l}.{p}_scale"] = s
            out[f"L{l}.{p}_tscale"] = g
    torch.cuda.synchronize()
    for key in [k for k in out if k.endswith("_tscale")]:
        out[key] = float(out[key].item())
    return out


class Session:
    """One dory_ctx with its KV buffer and workspace (torch-allocated)."""

    def __init__(self, model, dev_weights: Dict, *, max_batch: int = 1, max_ctx: int = 1024,
                 max_chunk: Optional[int] = None, max_loops: int = 8, kv_mode: str = "last_loop",
                 kv_loops: int = 1, stream=None, device="cuda", weight_format: int = 0):
        import torch
        self.model = model
        self.device = torch.device(device)
        self.cfg, self._keep = make_config(model, max_batch=max_batch, max_ctx=max_ctx,
                                           max_chunk=max_chunk or max_ctx, max_loops=max_loops,
                                           weight_format=weight_format)
        s = validate_config(self.cfg)
        if s != DORY_OK:
            raise DoryError(s, "invalid config")
        self.kv_mode = KV_MODES[kv_mode]
        self.kv_loops = kv_loops
        kvb = kv_bytes(self.cfg, self.kv_mode, kv_loops)
        wsb = workspace_bytes(self.cfg)
        if kvb == 0 or wsb == 0:
            raise DoryError(DORY_E_ARG, "zero-sized buffers")
        self.kv = torch.empty(kvb, dtype=torch.uint8, device=self.device)
        self.ws = torch.empty(wsb, dtype=torch.uint8, device=self.device)
        self.weights = dev_weights
        L = model.n_layers
        arr = lambda kind: (ctypes.c_void_p * L)(*[_ptr(dev_weights[f"L{l}.{kind}"]) for l in range(L)])
        self._arrays = {k: arr(k) for k in ("qkvg", "o", "ug", "down", "alpha_a", "alpha_m")}
        vp = lambda a: ctypes.cast(a, ctypes.POINTER(ctypes.c_void_p))
        lowbit = weight_format in (WEIGHTS_MXFP8, WEIGHTS_NVFP4)
        if lowbit:
            for k in PROJECTIONS:
                self._arrays[k + "_scale"] = arr(k + "_scale")
        if weight_format == WEIGHTS_NVFP4:
            for k in PROJECTIONS:
                self._arrays[k + "_tscale"] = (ctypes.c_float * L)(
                    *[float(dev_weights[f"L{l}.{k}_tscale"]) for l in range(L)])
        sc = (lambda k: vp(self._arrays[k + "_scale"])) if lowbit else (lambda k: None)
        ts = ((lambda k: ctypes.cast(self._arrays[k + "_tscale"], ctypes.POINTER(ctypes.c_float)))
              if weight_format == WEIGHTS_NVFP4 else (lambda k: None))
        self.wstruct = DoryWeights(embed=_ptr(dev_weights["embed"]), qkvg=vp(self._arrays["qkvg"]),
                                   o=vp(self._arrays["o"]), ug=vp(self._arrays["ug"]),
                                   down=vp(self._arrays["down"]), alpha_attn=vp(self._arrays["alpha_a"]),
                                   alpha_mlp=vp(self._arrays["alpha_m"]), qkvg_scale=sc("qkvg"), o_scale=sc("o"),
                                   ug_scale=sc("ug"), down_scale=sc("down"), qkvg_tscale=ts("qkvg"),
                                   o_tscale=ts("o"), ug_tscale=ts("ug"), down_tscale=ts("down"))
        self.stream = stream if stream is not None else torch.cuda.current_stream(self.device)
        h = ctypes.c_void_p()
        s = _lib.dory_create(ctypes.byref(self.cfg), ctypes.byref(self.wstruct), _ptr(self.kv), kvb, self.kv_mode,
                             kv_loops, _ptr(self.ws), wsb, _stream_handle(self.stream), ctypes.byref(h))
        if s != DORY_OK:
            raise DoryError(s, "dory_create")
        self.h = h
        self.batch = None
        self._trace = None

    def _check(self, s: int):
        if s != DORY_OK:
            raise DoryError(s, _lib.dory_last_error(self.h).decode())

    def __del__(self):
        h = getattr(self, "h", None)
        if h and _lib is not None:  # at interpreter exit the module globals may be gone
            _lib.dory_destroy(h)
            self.h = None

    def prefill(self, tokens, n_loops: int, kv_mode: Optional[str] = None) -> None:
        import torch
        assert tokens.dtype == torch.int32 and tokens.is_contiguous() and tokens.dim() == 2
        mode = self.kv_mode if kv_mode is None else KV_MODES[kv_mode]
        self._check(_lib.dory_prefill(self.h, _ptr(tokens), tokens.shape[0], tokens.shape[1], n_loops, mode))
        self.batch = tokens.shape[0]

    def decode(self, tokens=None, n_loops: int = 2, kv_mode: Optional[str] = None, next_tokens=None) -> None:
        mode = self.kv_mode if kv_mode is None else KV_MODES[kv_mode]
        self._check(_lib.dory_decode_step(self.h, _ptr(tokens) if tokens is not None else None, n_loops, mode,
                                          _ptr(next_tokens) if next_tokens is not None else None))

    def logits(self, out=None):
        import torch
        if out is None:
            out = torch.empty((self.batch, self.model.vocab), dtype=torch.float32, device=self.device)
        self._check(_lib.dory_logits(self.h, _ptr(out)))
        return out

    def reset(self) -> None:
        self._check(_lib.dory_reset(self.h))
        self.batch = None

    def prefill_mixed(self, tokens, loops) -> None:
        """Prefill with a loop count per sequence (last-loop caching)."""
        import torch
        assert tokens.dtype == torch.int32 and tokens.is_contiguous() and tokens.dim() == 2
        arr = (ctypes.c_int32 * len(loops))(*[int(k) for k in loops])
        self._check(_lib.dory_prefill_mixed(self.h, _ptr(tokens), tokens.shape[0], tokens.shape[1],
                                            ctypes.cast(arr, ctypes.c_void_p), KV_MODES["last_loop"]))
        self.batch = tokens.shape[0]

    def decode_mixed(self, tokens, loops, next_tokens=None) -> None:
        """One decode position with a loop count per sequence (last-loop caching)."""
        arr = (ctypes.c_int32 * len(loops))(*[int(k) for k in loops])
        self._check(_lib.dory_decode_step_mixed(self.h, _ptr(tokens) if tokens is not None else None,
                                                ctypes.cast(arr, ctypes.c_void_p), KV_MODES["last_loop"],
                                                _ptr(next_tokens) if next_tokens is not None else None))

    def resume(self, batch: int, pos: int, n_loops: int, kv_mode: Optional[str] = None) -> None:
        """Take positions [0, pos) of `batch` sequences as already in the KV buffer."""
        mode = self.kv_mode if kv_mode is None else KV_MODES[kv_mode]
        self._check(_lib.dory_resume(self.h, batch, pos, n_loops, mode))
        self.batch = batch

    def backward_last_loop(self, x, grad_out, *, ws=None, grads=None, stream_sync: bool = False,
                           recompute: bool = False):
        """Depth-1 backward of the last recurrent invocation (dory_backward_last_loop).
        x, grad_out: float32 [B, n, d] device tensors. Returns a dict of float32
        gradients keyed like the weights ("L{l}.qkvg", ..., "L{l}.alpha_a",
        "L{l}.alpha_m" for the recurrent layers) plus "x". recompute: pass the
        smaller workspace, with which each layer's forward runs again."""
        import torch
        m = self.model
        B, n, d = x.shape
        wsb = (backward_workspace_min_bytes if recompute else backward_workspace_bytes)(self.cfg, B, n)
        if wsb == 0:
            raise DoryError(DORY_E_ARG, "backward workspace size")
        if ws is None or ws.numel() < wsb:
            ws = torch.empty(wsb, dtype=torch.uint8, device=self.device)
        rec = list(range(m.n_in, m.n_in + m.n_rec))
        if grads is None:
            grads = {}
            for l in rec:
                for key in ("qkvg", "o", "ug", "down"):
                    grads[f"L{l}.{key}"] = torch.empty(tuple(self.weights[f"L{l}.{key}"].shape), dtype=torch.float32,
                                                       device=self.device)
                grads[f"L{l}.alpha_a"] = torch.empty(d, dtype=torch.float32, device=self.device)
                grads[f"L{l}.alpha_m"] = torch.empty(d, dtype=torch.float32, device=self.device)
            grads["x"] = torch.empty((B, n, d), dtype=torch.float32, device=self.device)
        arr = lambda key: (ctypes.c_void_p * len(rec))(*[_ptr(grads[f"L{l}.{key}"]) for l in rec])
        keep = {k: arr(k) for k in ("qkvg", "o", "ug", "down", "alpha_a", "alpha_m")}
        vp = lambda a: ctypes.cast(a, ctypes.POINTER(ctypes.c_void_p))
        g = DoryGrads(qkvg=vp(keep["qkvg"]), o=vp(keep["o"]), ug=vp(keep["ug"]), down=vp(keep["down"]),
                      alpha_attn=vp(keep["alpha_a"]), alpha_mlp=vp(keep["alpha_m"]))
        self._check(_lib.dory_backward_last_loop(self.h, _ptr(x), _ptr(grad_out), B, n, ctypes.byref(g),
                                                 _ptr(grads["x"]) if "x" in grads else None, _ptr(ws), wsb))
        if stream_sync:
            torch.cuda.synchronize(self.device)
        return grads

    def set_graphs(self, enable: bool) -> None:
        self._check(_lib.dory_set_graphs(self.h, 1 if enable else 0))

    def set_markers(self, enable: bool) -> None:
        """roctx ranges around calls and layer applications (rocprofv3 --marker-trace)."""
        self._check(_lib.dory_set_markers(self.h, 1 if enable else 0))

    TIME_KINDS = {"ug": 1, "qkvg": 2, "down": 3, "o": 4, "attn": 5}

    def set_kernel_timing(self, kind: Optional[str], max_launches: int = 0) -> None:
        self._check(_lib.dory_set_kernel_timing(self.h, self.TIME_KINDS[kind] if kind else 0, max_launches))

    def kernel_time(self):
        """(summed milliseconds, launches) recorded since the last read."""
        ms, n = ctypes.c_double(), _I()
        self._check(_lib.dory_kernel_time(self.h, ctypes.byref(ms), ctypes.byref(n)))
        return ms.value, n.value

    def set_trace(self, buf, max_apps: int) -> None:
        self._trace = buf
        self._check(_lib.dory_set_trace(self.h, _ptr(buf) if buf is not None else None, max_apps))


def op_linear(dtype: int, x, W, y, M: int, N: int, K: int, *, ldx: Optional[int] = None, epilogue: int = 0,
              scale: float = 1.0, algo: int = 0, stream=None) -> None:
    s = _lib.dory_op_linear(dtype, _ptr(x), ldx if ldx is not None else K, _ptr(W), _ptr(y), M, N, K, epilogue,
                            scale, algo, _stream_handle(stream))
    if s != DORY_OK:
        raise DoryError(s, "dory_op_linear")


def op_quant_mxfp8(w, N: int, K: int, codes, scales, stream=None) -> None:
    s = _lib.dory_op_quant_mxfp8(_ptr(w), N, K, _ptr(codes), _ptr(scales), _stream_handle(stream))
    if s != DORY_OK:
        raise DoryError(s, "dory_op_quant_mxfp8")


def op_quant_nvfp4(w, N: int, K: int, codes, scales, tscale, stream=None) -> None:
    s = _lib.dory_op_quant_nvfp4(_ptr(w), N, K, _ptr(codes), _ptr(scales), _ptr(tscale), _stream_handle(stream))
    if s != DORY_OK:
        raise DoryError(s, "dory_op_quant_nvfp4")


def op_linear_fp4(x, codes, scales, y, M: int, N: int, K: int, *, ldx: Optional[int] = None, epilogue: int = 0,
                  scale: float = 1.0, stream=None) -> None:
    s = _lib.dory_op_linear_fp4(_ptr(x), ldx if ldx is not None else K, _ptr(codes), _ptr(scales), _ptr(y), M, N,
                                K, epilogue, scale, _stream_handle(stream))
    if s != DORY_OK:
        raise DoryError(s, "dory_op_linear_fp4")


def op_linear_mx(x, codes, scales, y, M: int, N: int, K: int, *, ldx: Optional[int] = None, epilogue: int = 0,
                 scale: float = 1.0, stream=None) -> None:
    s = _lib.dory_op_linear_mx(_ptr(x), ldx if ldx is not None else K, _ptr(codes), _ptr(scales), _ptr(y), M, N, K,
                               epilogue, scale, _stream_handle(stream))
    if s != DORY_OK:
        raise DoryError(s, "dory_op_linear_mx")


def op_argmax(logits, out, scratch, stream=None) -> None:
    B, V = logits.shape
    s = _lib.dory_op_argmax(_ptr(logits), B, V, _ptr(out), _ptr(scratch), _stream_handle(stream))
    if s != DORY_OK:
        raise DoryError(s, "dory_op_argmax")


def op_argmax_noalloc(logits, out, stream=None) -> None:
    """op_argmax with the library's own partials (no scratch argument)."""
    B, V = logits.shape
    s = _lib.dory_op_argmax_noalloc(_ptr(logits), B, V, _ptr(out), _stream_handle(stream))
    if s != DORY_OK:
        raise DoryError(s, "dory_op_argmax_noalloc")


def argmax_scratch_bytes(B: int, V: int) -> int:
    return _lib.dory_argmax_scratch_bytes(B, V)
