"""Drives the HIP library (through the binding) the way the oracle's
generate/teacher_forced do, so the two can be compared call for call."""
from __future__ import annotations

import numpy as np
import torch

import looped_ngpt_amd as dory


def session(model, dev_w, *, batch, max_ctx, chunk, kv_mode, k, max_loops=8):
    kv_loops = k if kv_mode == "per_loop" else 1
    return dory.Session(model, dev_w, max_batch=batch, max_ctx=max_ctx, max_chunk=chunk, max_loops=max_loops,
                        kv_mode=kv_mode, kv_loops=kv_loops)


def _greedy_of(sess, logits):
    B, V = logits.shape
    out = torch.empty(B, dtype=torch.int32, device="cuda")
    scratch = torch.empty(dory.argmax_scratch_bytes(B, V), dtype=torch.uint8, device="cuda")
    dory.op_argmax(logits, out, scratch, stream=sess.stream)
    return out


def generate(sess, prompt: np.ndarray, steps: int, k: int):
    """Free-running greedy decode on the GPU. Returns (tokens [B, steps],
    logits [steps, B, V]) where logits[i] chose tokens[:, i], plus the
    library's own greedy choices for steps 1.. (to check argmax exactness)."""
    p = torch.from_numpy(np.ascontiguousarray(prompt, dtype=np.int32)).cuda()
    sess.prefill(p, k)
    logits = [sess.logits().clone()]
    toks = [_greedy_of(sess, logits[0])]
    lib_next = []
    for i in range(steps - 1):
        nxt = torch.empty(p.shape[0], dtype=torch.int32, device="cuda")
        sess.decode(None, k, next_tokens=nxt)
        logits.append(sess.logits().clone())
        toks.append(_greedy_of(sess, logits[-1]))
        lib_next.append(nxt)
    torch.cuda.synchronize()
    T = torch.stack(toks, 1).cpu().numpy()
    L = torch.stack(logits, 0).cpu().numpy()
    N = torch.stack(lib_next, 1).cpu().numpy() if lib_next else np.zeros((p.shape[0], 0), np.int32)
    return T, L, N


def teacher_forced(sess, prompt: np.ndarray, forced: np.ndarray, k: int):
    """Prefill, then decode feeding `forced` [B, steps]; logits [steps+1, B, V]."""
    p = torch.from_numpy(np.ascontiguousarray(prompt, dtype=np.int32)).cuda()
    f = torch.from_numpy(np.ascontiguousarray(forced, dtype=np.int32)).cuda()
    sess.prefill(p, k)
    out = [sess.logits().clone()]
    for i in range(f.shape[1]):
        sess.decode(f[:, i].contiguous(), k)
        out.append(sess.logits().clone())
    torch.cuda.synchronize()
    return torch.stack(out, 0).cpu().numpy()
