"""Decode throughput of the looped nGPT on one MI355X.

Workload: the 36-layer ~4B shape (8 input / 20 recurrent / 8 output layers,
d 3072, 24/8 heads, hd 128, d_ff 8192, vocab 131072, 3 sliding-window(4096)
layers then 1 full layer, bf16, seeded random weights drawn on the GPU),
batch 1, an 8192-token random prompt prefilled in one chunk, then greedy
decode in last-loop KV mode. A step is one decode position through the whole
path: embedding, input block, k passes of the recurrent block with input
re-injection, output block, tied LM head and argmax (the next step consumes
the argmax on the device). The headline value is decode tokens/s at k = 2
(the pages' recommended default); k = 1 and k = 4 are reported beside it.

Prints ONE JSON line. --gpus must be 1: this build runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # B/s, MI355X HBM3E
MFMA_PEAK = 2.5e15         # FLOP/s, MI355X dense bf16 matrix cores
METRIC = "decode tokens/s @ k=1,2,4 (last-loop KV) + % of HBM roofline, 1×MI355X"


# bytes per projection weight of each storage format: bfloat16; MXFP8 (one
# E4M3 byte + one scale byte per 32); NVFP4 (half a byte + one scale byte per 16)
WEIGHT_BYTES = {"bf16": 2.0, "mxfp8": 1.0 + 1.0 / 32, "nvfp4": 0.5 + 1.0 / 16}


def decode_bytes(m, k, ctx_mean, B=1, fmt="bf16"):
    """Algorithmic HBM bytes of one decode step: every weight once (the
    recurrent block k times), the tied LM head, each layer application's K/V
    reads over its window and its one-position K/V write, per sequence.
    fmt: storage of the layer projections (WEIGHT_BYTES); the LM head stays
    bfloat16."""
    el = 2
    apps_full, apps_swa = 0, 0
    for l in range(m.n_layers):
        reps = k if m.is_recurrent(l) else 1
        if m.layer_is_full[l]:
            apps_full += reps
        else:
            apps_swa += reps
    per_key = 2 * m.n_kv_heads * m.head_dim * el
    layer = int(m.layer_bytes() // 2 * WEIGHT_BYTES[fmt])
    weights = (m.n_in + m.n_out + k * m.n_rec) * layer + m.vocab * m.d_model * el
    kv_read = B * per_key * (apps_full * ctx_mean + apps_swa * min(ctx_mean, m.window))
    kv_write = B * per_key * (apps_full + apps_swa)
    return weights + kv_read + kv_write


# HBM bytes per launch of the decode up/gate GEMV from two rocprofv3 --pmc
# passes over bench.py (FETCH_SIZE and WRITE_SIZE, KiB per dispatch, medians
# over 1008 launches), each scaled by what the same counter reads for a 1 GiB
# device copy (FETCH_SIZE: 0.5 GiB, factor 2; WRITE_SIZE: 1 GiB, factor 1).
# They hold for the GEMV source they were taken on, identified by a
# fingerprint of that source; after any change the bench reports null.
UG_TRAFFIC = {"fetch_kib": 49349.0, "fetch_factor": 2.0, "write_kib": 28.03, "write_factor": 1.0,
              "sources": ("looped_ngpt_amd/csrc/k_linear.hip", "looped_ngpt_amd/csrc/common.h",
                          "looped_ngpt_amd/csrc/linear_common.h"),
              "sha256_16": "6866375d5b610beb"}


def ug_traffic():
    import hashlib
    h = hashlib.sha256()
    for f in UG_TRAFFIC["sources"]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest()[:16] != UG_TRAFFIC["sha256_16"]:
        return None
    return int(round((UG_TRAFFIC["fetch_kib"] * UG_TRAFFIC["fetch_factor"]
                      + UG_TRAFFIC["write_kib"] * UG_TRAFFIC["write_factor"]) * 1024))


def ug_bytes(m, B=1, fmt="bf16"):
    """Algorithmic bytes of one SwiGLU up/gate projection launch (B rows): the
    two weight matrices (WEIGHT_BYTES per weight: bfloat16, or codes plus
    block-scale bytes), the prologue's inputs (sublayer output y, residual h,
    alpha; float32) and outputs (new residual, float32; activation, bf16)."""
    wb = int(2 * m.d_ff * m.d_model * WEIGHT_BYTES[fmt])
    return wb + B * m.d_model * 4 * 3 + B * m.d_model * 4 + B * m.d_ff * 2


def attn_flops(m, k, n):
    """Attention FLOPs of prefilling n positions from an empty cache:
    4*n_q*hd per allowed (query, key) pair (QK^T and PV) per layer application."""
    pairs_full = n * (n + 1) // 2
    W = m.window
    pairs_swa = W * (W + 1) // 2 + (n - W) * W if n > W else pairs_full
    flops = 0
    for l in range(m.n_layers):
        reps = k if m.is_recurrent(l) else 1
        flops += reps * 4 * m.q_dim * (pairs_full if m.layer_is_full[l] else pairs_swa)
    return flops


def prefill_flops(m, k, n):
    """Dense FLOPs of prefilling n positions from an empty cache: 2 per
    weight per position for every layer application, the attention pairs,
    and the LM head on the last position."""
    apps = m.n_in + m.n_out + k * m.n_rec
    return apps * 2 * n * (m.layer_bytes() // 2) + attn_flops(m, k, n) + 2 * m.vocab * m.d_model


def _host_info():
    """CPU model and the BLAS library numpy calls (threadpoolctl), for the report."""
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas, threads = "unknown", len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            blas = ", ".join(f"{i.get('internal_api')} {i.get('version')}" for i in libs)
            threads = max(int(i.get("num_threads", 1)) for i in libs)
    except Exception:  # pragma: no cover
        pass
    return cpu, blas, threads


def cpu_baseline(model, dev_w, k_head: int, ctx: int = 8192, budget_s: float = 15.0):
    """The oracle (numpy, float32 compute, bfloat16 storage points) on the
    host, on the full 36-layer model with the benchmark's weights, decoding
    at the benchmark's context: its KV caches are filled for positions
    0..ctx-1 with synthetic bfloat16 keys (unit vectors per head) and values
    (N(0, 1/d) entries, the scale of a unit row times unit weight rows), as
    the GPU run's caches hold prefilled keys, and greedy decode calls at
    k = k_head are timed over as many calls as fit in about budget_s (at
    least 3). The sample therefore includes the attention over ctx cached
    positions (full layers) and the 4096-key windows (sliding layers)."""
    import numpy as np
    from oracle.ngpt import LoopedNGPT, round_bf16
    cpu_model, blas, threads = _host_info()
    t_start = time.perf_counter()
    w = {}
    for name, t in dev_w.items():
        a = t.cpu().numpy()
        w[name] = a.view(np.uint16) if a.dtype == np.int16 else a
    o = LoopedNGPT(model, w, compute="f32", bf16_points=True, max_ctx=ctx + 64)
    rng = np.random.default_rng(12345)
    hd, nkv = model.head_dim, model.n_kv_heads
    kk = rng.standard_normal((1, nkv, ctx, hd), dtype=np.float32)
    kk /= np.linalg.norm(kk, axis=-1, keepdims=True)
    vv = rng.standard_normal((1, nkv, ctx, hd), dtype=np.float32) / np.float32(np.sqrt(model.d_model))
    kk, vv = round_bf16(kk), round_bf16(vv)
    o.kv_mode = "last_loop"
    for l in range(model.n_layers):
        c = o._cache(o.cache_key(l, 0))
        c["K"][:, :, :ctx, :] = kk
        c["V"][:, :, :ctx, :] = vv
    o.pos = ctx
    tok = 17
    logits = o.call(np.array([[tok]], dtype=np.int32), k_head, "last_loop")  # also widens every weight once
    t_setup = time.perf_counter() - t_start
    tok = int(np.argmax(logits[0]))
    calls, t0 = 0, time.perf_counter()
    while calls < 3 or (time.perf_counter() - t0 < budget_s and calls < 50):
        logits = o.call(np.array([[tok]], dtype=np.int32), k_head, "last_loop")
        tok = int(np.argmax(logits[0]))
        calls += 1
    sec = (time.perf_counter() - t0) / calls
    return {"value": round(1.0 / sec, 4), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": cpu_model, "blas": blas,
            "sample": (f"numpy oracle (float32 compute, bfloat16 storage points), full {model.n_layers}-layer model, "
                       f"{calls} greedy decode calls at k={k_head} at context {ctx + 1}..{ctx + calls + 1} "
                       f"(KV caches filled with synthetic bf16 keys/values for positions 0..{ctx - 1}, so the "
                       f"attention over the {ctx}-position context is included; {sec * 1e3:.0f} ms/token; "
                       f"weight widening and cache fill, {t_setup:.0f} s, excluded)"),
            "wall_s": round(time.perf_counter() - t_start, 1)}


def _timed_decode(sess, B, k, steps, warmup, first_tokens=None):
    """warmup + steps decode calls; returns ms per step (HIP events on the session's stream)."""
    import torch
    st = sess.stream
    if first_tokens is not None:
        sess.decode(first_tokens, k)
        warmup -= 1
    for _ in range(max(warmup, 0)):
        sess.decode(None, k)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(steps):
        sess.decode(None, k)
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def _line(workload, value, ms, B, steps, warmup, n, k, mode, extra):
    res = {
        "metric": METRIC, "value": round(value, 2), "unit": "tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded random-init weights, uniform random token ids)",
        "config": {"workload": workload, "global_batch": B, "seq_len": n, "n_loops": k, "kv_mode": mode,
                   "parallelism": "none (1 GPU)"},
        "roofline": None, "cpu_baseline": None,
    }
    res.update(extra)
    print(json.dumps(res))


def run_other(args, dev):
    """The scope table's other measurement workloads (one JSON line each)."""
    import torch
    import looped_ngpt_amd as dory
    from synth.configs import CONFIGS
    from synth.device import make_weights_device
    stream = torch.cuda.current_stream(dev)
    log = lambda msg: print(f"[bench:{args.workload}] {msg}", file=sys.stderr, flush=True)
    K, Wm = args.steps, args.warmup

    if args.workload == "c72":
        model = CONFIGS["c72"]["model"]
        n = 16384
        w = make_weights_device(model, dev)
        g = torch.Generator(device="cpu")
        g.manual_seed(model.seed * 7 + 1)
        prompt = torch.randint(0, model.vocab, (1, n), generator=g, dtype=torch.int32).to(dev)
        max_ctx = (n + Wm + K + 2 + 255) // 256 * 256
        table = {}
        for mode in ("last_loop", "per_loop"):
            for k in (1, 2, 3, 4):
                sess = dory.Session(model, w, max_batch=1, max_ctx=max_ctx, max_chunk=8192, kv_mode=mode,
                                    kv_loops=k if mode == "per_loop" else 1, stream=stream, device=dev)
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                sess.prefill(prompt, k)
                e1.record(stream)
                torch.cuda.synchronize()
                pms = e0.elapsed_time(e1)
                ms = _timed_decode(sess, 1, k, K, Wm)
                step_bytes = decode_bytes(model, k, n + Wm + (K - 1) / 2.0)
                table[f"{mode}/k={k}"] = {"tokens_per_s": round(1e3 / ms, 2), "ms_per_step": round(ms, 4),
                                         "hbm_frac": round(step_bytes / (ms / 1e3) / HBM_PEAK, 4),
                                         "kv_bytes": int(sess.kv.numel()), "prefill_ms": round(pms, 1),
                                         "prefill_tokens_per_s": round(n / (pms / 1e3), 1)}
                log(f"{mode} k={k}: {1e3 / ms:.1f} tok/s, KV {sess.kv.numel() / 1e9:.3f} GB, prefill {pms:.0f} ms")
                del sess
                torch.cuda.empty_cache()
        hk = table["last_loop/k=2"]
        _line(f"{model.name} bf16, batch 1, {n}-token random prompt (2 chunks of 8192), greedy decode, "
              "k=1..4 in both KV modes (headline value: k=2, last-loop)",
              hk["tokens_per_s"], hk["ms_per_step"], 1, K, Wm, n, 2, "last_loop", {"by_mode_k": table})
        return

    if args.workload == "long":
        model = CONFIGS["c36_256k"]["model"]
        n, k = 262144, 2
        w = make_weights_device(model, dev)
        g = torch.Generator(device="cpu")
        g.manual_seed(model.seed * 7 + 1)
        prompt = torch.randint(0, model.vocab, (1, n), generator=g, dtype=torch.int32).to(dev)
        max_ctx = (n + Wm + K + 2 + 255) // 256 * 256
        sess = dory.Session(model, w, max_batch=1, max_ctx=max_ctx, max_chunk=8192, kv_mode="last_loop",
                            stream=stream, device=dev)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for c0 in range(0, n, 8192):   # one chunk per call, so the run reports progress
            sess.prefill(prompt[:, c0:c0 + 8192].contiguous(), k)
            if c0 % (8 * 8192) == 0:
                torch.cuda.synchronize()
                log(f"prefill {c0 + 8192} / {n}")
        e1.record(stream)
        torch.cuda.synchronize()
        pms = e0.elapsed_time(e1)
        ms = _timed_decode(sess, 1, k, K, Wm)
        step_bytes = decode_bytes(model, k, n + Wm + (K - 1) / 2.0)
        fl = prefill_flops(model, k, n)
        log(f"prefill {pms / 1e3:.2f} s ({n / (pms / 1e3):.0f} tok/s), decode {1e3 / ms:.1f} tok/s")
        _line(f"{model.name} bf16, batch 1, {n}-token random prompt in 8192-token chunks, greedy decode at k=2, "
              "last-loop KV", 1e3 / ms, ms, 1, K, Wm, n, k, "last_loop",
              {"hbm_frac_step": round(step_bytes / (ms / 1e3) / HBM_PEAK, 4), "kv_bytes": int(sess.kv.numel()),
               "prefill": {"ms": round(pms, 1), "tokens_per_s": round(n / (pms / 1e3), 1),
                           "mfma_frac_whole": round(fl / (pms / 1e3) / MFMA_PEAK, 4)}})
        return

    if args.workload in ("mxfp8", "nvfp4"):
        fmt = args.workload
        model = CONFIGS["c36"]["model"]
        n = args.prompt
        w = make_weights_device(model, dev)
        torch.cuda.synchronize()
        tq = time.perf_counter()
        if fmt == "mxfp8":
            wq = dory.quantize_weights_mxfp8(model, w, stream=stream)
        else:
            wq = dory.quantize_weights_nvfp4(model, w, stream=stream)
        torch.cuda.synchronize()
        log(f"quantised {4 * model.n_layers} projections in {time.perf_counter() - tq:.2f} s")
        for key in [x for x in w if x.split(".")[-1] in dory.PROJECTIONS]:
            del w[key]                       # the bfloat16 projections are not used from here on
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        g = torch.Generator(device="cpu")
        g.manual_seed(model.seed * 7 + 1)
        prompt = torch.randint(0, model.vocab, (1, n), generator=g, dtype=torch.int32).to(dev)
        max_ctx = (n + Wm + K + args.kernel_steps + 2 + 255) // 256 * 256
        sess = dory.Session(model, wq, max_batch=1, max_ctx=max_ctx, max_chunk=n, kv_mode="last_loop",
                            stream=stream, device=dev,
                            weight_format=dory.WEIGHTS_MXFP8 if fmt == "mxfp8" else dory.WEIGHTS_NVFP4)
        table, roof = {}, None
        for k in (1, 2, 4):
            sess.reset()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            sess.prefill(prompt, k)
            e1.record(stream)
            torch.cuda.synchronize()
            pms = e0.elapsed_time(e1)
            ms = _timed_decode(sess, 1, k, K, Wm)
            step_bytes = decode_bytes(model, k, n + Wm + (K - 1) / 2.0, fmt=fmt)
            table[f"k={k}"] = {"tokens_per_s": round(1e3 / ms, 2), "ms_per_step": round(ms, 4),
                               "hbm_frac": round(step_bytes / (ms / 1e3) / HBM_PEAK, 4),
                               "bytes_per_step": step_bytes, "prefill_ms": round(pms, 1)}
            log(f"k={k}: {1e3 / ms:.1f} tok/s, HBM {100 * table[f'k={k}']['hbm_frac']:.1f}%, prefill {pms:.0f} ms")
            if k == 2 and args.kernel_steps > 0:
                apps = model.n_in + model.n_out + k * model.n_rec
                sess.set_kernel_timing("ug", args.kernel_steps * apps)
                for _ in range(args.kernel_steps):
                    sess.decode(None, k)
                tot, cnt = sess.kernel_time()
                sess.set_kernel_timing(None)
                ug_ms = tot / max(cnt, 1)
                ach = ug_bytes(model, fmt=fmt) / (ug_ms / 1e3)
                kname = ("k_gemv_pro_lb<MXFP8,1,3,SwiGLU>" if fmt == "mxfp8" else "k_gemv_pro1_lb<NVFP4,2,SwiGLU>")
                roof = {"bound": "hbm", "achieved": round(ach / 1e9, 1), "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                        "frac": round(ach / HBM_PEAK, 4), "traffic": None,
                        "kernel": f"{kname} ({fmt.upper()} up/gate projection with the nGPT update prologue, "
                                  "M=1, N=2x8192, K=3072)",
                        "bytes_per_launch": ug_bytes(model, fmt=fmt), "avg_launch_us": round(ug_ms * 1e3, 2)}
                log(f"{fmt} up/gate GEMV: {cnt} launches, {ug_ms * 1e3:.1f} us avg, {100 * roof['frac']:.1f}% HBM")
        hk = table["k=2"]
        desc = ("MXFP8 layer projections (E4M3, 32-element blocks, E8M0 scales)" if fmt == "mxfp8" else
                "NVFP4-style layer projections (E2M1, 16-element blocks, least-error E4M3 scales, float32 "
                "tensor scale)")
        _line(f"{model.name} with {desc}, batch 1, {n}-token random prompt, greedy decode at k=1,2,4, last-loop "
              "KV (headline value: k=2)", hk["tokens_per_s"], hk["ms_per_step"], 1, K, Wm, n, 2, "last_loop",
              {"by_k": table, "roofline": roof, "dtype": f"bf16 activations, {fmt.upper()} weights"})
        return

    if args.workload == "backward":
        # depth-1 truncated backward of the last recurrent invocation: the
        # 20 recurrent layers of the 36-layer shape on one training chunk
        model = CONFIGS["c36"]["model"]
        B, n = 1, args.bw_tokens
        K = min(K, 10)                                       # a call takes a good fraction of a second
        w = make_weights_device(model, dev)
        sess = dory.Session(model, w, max_batch=1, max_ctx=max(n, 256), max_chunk=256, kv_mode="last_loop",
                            stream=stream, device=dev)
        g = torch.Generator(device=dev)
        g.manual_seed(model.seed * 7 + 5)
        x = torch.randn((B, n, model.d_model), generator=g, device=dev, dtype=torch.float32)
        x /= x.norm(dim=-1, keepdim=True)
        G = torch.randn((B, n, model.d_model), generator=g, device=dev, dtype=torch.float32)
        wsb = dory.backward_workspace_bytes(sess.cfg, B, n)
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
        grads = sess.backward_last_loop(x, G, ws=ws)       # allocates the gradients once
        torch.cuda.synchronize()
        for _ in range(max(Wm - 1, 0)):
            sess.backward_last_loop(x, G, ws=ws, grads=grads)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(K):
            sess.backward_last_loop(x, G, ws=ws, grads=grads)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / K
        M = B * n
        params = model.layer_bytes() // 2
        pairs_full = n * (n + 1) // 2
        Wn = model.window
        pairs_swa = Wn * (Wn + 1) // 2 + (n - Wn) * Wn if n > Wn else pairs_full
        attn_fwd = sum(4 * model.q_dim * (pairs_full if model.layer_is_full[l] else pairs_swa)
                       for l in range(model.n_in, model.n_in + model.n_rec))
        # training FLOPs of the block: forward 2 M P + backward 4 M P per layer, attention forward + 2x backward
        flops = model.n_rec * 6 * M * params + 3 * attn_fwd
        log(f"backward of {model.n_rec} layers on {M} positions: {ms:.2f} ms, "
            f"{M / (ms / 1e3):.0f} tokens/s, {flops / (ms / 1e3) / 1e12:.0f} TFLOP/s, workspace {wsb / 1e9:.2f} GB")
        res = {
            "metric": "depth-1 truncated backward of the last recurrent invocation, tokens/s, 1xMI355X",
            "value": round(M / (ms / 1e3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": Wm,
            "ms_per_step": round(ms, 3), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16", "data": "synthetic (seeded random-init weights, random unit inputs and gradients)",
            "config": {"workload": f"{model.name}: backward through the {model.n_rec} recurrent layers, batch {B}, "
                                   f"{n} positions (causal, window {model.window})", "global_batch": B,
                       "seq_len": n, "parallelism": "none (1 GPU)"},
            "roofline": {"bound": "mfma", "achieved": round(flops / (ms / 1e3) / 1e12, 1), "peak": MFMA_PEAK / 1e12,
                         "unit": "TFLOP/s", "frac": round(flops / (ms / 1e3) / MFMA_PEAK, 4), "traffic": None,
                         "kernel": "whole call (gradient GEMMs, attention, row kernels)", "flops": flops},
            "workspace_bytes": wsb, "cpu_baseline": None,
        }
        print(json.dumps(res))
        return

    # b64: 64 sequences whose 32768 cached positions are synthetic: random
    # bfloat16 values written straight into the caller-owned KV buffer, then
    # dory_resume (decode throughput does not depend on cache contents)
    model = CONFIGS["c36_b64"]["model"]
    B, ctx, k = 64, 32768, 4
    w = make_weights_device(model, dev)
    max_ctx = (ctx + Wm + K + 2 + 255) // 256 * 256
    g = torch.Generator(device=dev)
    g.manual_seed(model.seed * 7 + 3)
    results = {}
    for mode in ("last_loop", "per_loop"):
        kv_loops = k if mode == "per_loop" else 1
        probe = dory.Session(model, w, max_batch=1, max_ctx=max_ctx, max_chunk=1, kv_mode=mode, kv_loops=kv_loops,
                             stream=stream, device=dev)
        per_seq = probe.kv.numel()
        del probe
        torch.cuda.empty_cache()
        free = torch.cuda.mem_get_info(dev)[0]
        fit = int((free - (4 << 30)) // per_seq)     # leave 4 GiB for the workspace and the allocator
        Bm = min(B, fit)
        entry = {"kv_bytes_at_batch_64": per_seq * B, "free_bytes": int(free)}
        if Bm < 1:
            entry["oom"] = True
            results[mode] = entry
            continue
        if Bm < B:
            entry["oom_at_batch_64"] = True
            log(f"{mode}: KV for 64 sequences is {per_seq * B / 1e9:.1f} GB, {free / 1e9:.1f} GB free: "
                f"largest batch that fits is {Bm}")
        sess = dory.Session(model, w, max_batch=Bm, max_ctx=max_ctx, max_chunk=1, kv_mode=mode, kv_loops=kv_loops,
                            stream=stream, device=dev)
        kvv = sess.kv.view(torch.bfloat16)
        step = 1 << 29
        for i in range(0, kvv.numel(), step):
            m = min(step, kvv.numel() - i)
            kvv[i:i + m].normal_(0.0, 0.05, generator=g)
            if (i // step) % 32 == 31:
                torch.cuda.synchronize()
                log(f"{mode}: filled {2 * (i + m) / 1e9:.0f} / {2 * kvv.numel() / 1e9:.0f} GB of synthetic cache")
        torch.cuda.synchronize()
        sess.resume(Bm, ctx, k)
        first = torch.randint(0, model.vocab, (Bm,), generator=g, device=dev, dtype=torch.int32)
        ms = _timed_decode(sess, Bm, k, K, Wm, first_tokens=first)
        step_bytes = decode_bytes(model, k, ctx + Wm + (K - 1) / 2.0, B=Bm)
        entry.update({"batch": Bm, "tokens_per_s": round(Bm * 1e3 / ms, 1), "ms_per_step": round(ms, 3),
                      "hbm_frac": round(step_bytes / (ms / 1e3) / HBM_PEAK, 4), "kv_bytes": int(sess.kv.numel()),
                      "bytes_per_step": step_bytes})
        results[mode] = entry
        log(f"{mode} batch {Bm}: {Bm * 1e3 / ms:.1f} tok/s ({ms:.2f} ms/step), HBM {100 * entry['hbm_frac']:.1f}%")
        del sess, kvv
        torch.cuda.empty_cache()
    ll = results["last_loop"]
    _line(f"{model.name} bf16, batch 64, 32768 cached positions per sequence (synthetic caches, resumed), "
          "greedy decode at k=4, both KV modes (headline value: last-loop)", ll["tokens_per_s"], ll["ms_per_step"],
          ll["batch"], K, Wm, ctx, k, "last_loop", {"by_mode": results})


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--prompt", type=int, default=8192)
    ap.add_argument("--ks", type=str, default="1,2,4")
    ap.add_argument("--headline-k", type=int, default=2)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--kernel-steps", type=int, default=16, help="decode steps of the kernel-timing pass")
    ap.add_argument("--graphs", action="store_true", help="replay decode steps as recorded HIP graphs")
    ap.add_argument("--markers", action="store_true",
                    help="roctx ranges around calls and layer applications (rocprofv3 --marker-trace)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first copy 1 GiB on the device 3 times (reference for the HBM byte counters)")
    ap.add_argument("--no-prefill-taps", action="store_true", help="skip the prefill kernel-timing passes")
    ap.add_argument("--no-per-loop", action="store_true", help="skip the per-loop KV decode timings")
    ap.add_argument("--bw-tokens", type=int, default=2048, help="positions of the backward workload")
    ap.add_argument("--workload", choices=["c36", "c72", "b64", "long", "mxfp8", "nvfp4", "backward"],
                    default="c36",
                    help="c36: the headline (default). c72: the 72-layer shape, 16384-token prompt, k=1..4 in "
                         "both KV modes. b64: 64 sequences at 32768 cached positions (synthetic caches), k=4, "
                         "both KV modes. long: a 262144-token prompt in 8192-token chunks, k=2. mxfp8 / nvfp4: the c36 shape "
                         "with MXFP8 / NVFP4-style layer projections, decode at k=1,2,4. backward: the depth-1 "
                         "truncated backward of the c36 recurrent block on --bw-tokens positions")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path (sequences are "
              "independent, so batches would split across GPUs with no exchange).", file=sys.stderr)
        sys.exit(2)

    import torch
    import looped_ngpt_amd as dory
    from synth.configs import get_config
    from synth.device import make_weights_device

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.workload != "c36":
        return run_other(args, dev)
    model = get_config("c36")
    ks = [int(x) for x in args.ks.split(",")]
    if args.headline_k not in ks:
        ks.append(args.headline_k)
    n, K, Wm = args.prompt, args.steps, args.warmup
    # positions needed, rounded to 256 (a multiple of 8 keeps the cached
    # values' 8-position runs aligned for the matrix-core decode attention)
    max_ctx = (n + Wm + K + args.kernel_steps + 2 + 255) // 256 * 256

    if args.copy_calibration:
        src = torch.ones(1 << 29, dtype=torch.int16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] calibration: 3 device copies of {src.numel() * 2} B", file=sys.stderr, flush=True)
        del src, dst
    t0 = time.perf_counter()
    w = make_weights_device(model, dev)
    torch.cuda.synchronize()
    print(f"[bench] weights {sum(t.numel() * t.element_size() for t in w.values()) / 1e9:.2f} GB "
          f"generated in {time.perf_counter() - t0:.1f}s", file=sys.stderr, flush=True)
    g = torch.Generator(device="cpu")
    g.manual_seed(model.seed * 7 + 1)
    prompt = torch.randint(0, model.vocab, (1, n), generator=g, dtype=torch.int32).to(dev)
    stream = torch.cuda.current_stream(dev)

    by_k, prefill, pre_taps = {}, {}, {}
    ug_ms = None
    sess = dory.Session(model, w, max_batch=1, max_ctx=max_ctx, max_chunk=n, kv_mode="last_loop",
                        stream=stream, device=dev)
    sess.set_graphs(args.graphs)
    if args.markers:
        sess.set_markers(True)
    # warm-up prefill (untimed) at the timed shapes: first-use costs of the
    # code objects and of the GEMM library (its per-shape algorithm choice)
    sess.prefill(prompt, ks[0])
    torch.cuda.synchronize()
    for k in ks:
        sess.reset()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        sess.prefill(prompt, k)
        e1.record(stream)
        torch.cuda.synchronize()
        pms = e0.elapsed_time(e1)
        prefill[k] = {"tokens_per_s": n / (pms / 1e3), "ms": pms,
                      "mfma_frac_whole": prefill_flops(model, k, n) / (pms / 1e3) / MFMA_PEAK}
        print(f"[bench] k={k} prefill {n} tokens: {pms:.1f} ms", file=sys.stderr, flush=True)
        for _ in range(Wm):
            sess.decode(None, k)
        torch.cuda.synchronize()
        e0.record(stream)
        th = time.perf_counter()
        for _ in range(K):
            sess.decode(None, k)
        host_ms = (time.perf_counter() - th) * 1e3  # enqueue time: host-bound if close to ms
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        print(f"[bench] k={k} host enqueue {host_ms / K:.3f} ms/step", file=sys.stderr, flush=True)
        ctx_mean = n + Wm + (K - 1) / 2.0
        step_bytes = decode_bytes(model, k, ctx_mean)
        by_k[k] = {"tokens_per_s": K / (ms / 1e3), "ms_per_step": ms / K,
                   "hbm_frac": step_bytes / (ms / 1e3 / K) / HBM_PEAK, "bytes_per_step": step_bytes,
                   "kv_bytes": int(sess.kv.numel())}
        print(f"[bench] k={k} decode: {ms / K:.3f} ms/step, {K / (ms / 1e3):.1f} tok/s, "
              f"HBM {100 * by_k[k]['hbm_frac']:.1f}%", file=sys.stderr, flush=True)
        if k == args.headline_k and args.kernel_steps > 0:
            # kernel-timing pass: HIP events around every SwiGLU up/gate projection
            apps = model.n_in + model.n_out + k * model.n_rec
            sess.set_kernel_timing("ug", args.kernel_steps * apps)
            for _ in range(args.kernel_steps):
                sess.decode(None, k)
            tot, cnt = sess.kernel_time()
            sess.set_kernel_timing(None)
            ug_ms = tot / max(cnt, 1)
            print(f"[bench] SwiGLU up/gate projection: {cnt} launches, {ug_ms * 1e3:.1f} us avg",
                  file=sys.stderr, flush=True)
        if k == args.headline_k and not args.no_prefill_taps:
            # prefill kernel-timing passes: the up/gate GEMM and the attention
            apps = model.n_in + model.n_out + k * model.n_rec
            d, qd = model.d_model, model.q_dim
            shapes = {"qkvg": (model.qkvg_dim, d, "q|k|v|gate projection"),
                      "o": (d, qd, "output projection"),
                      "ug": (2 * model.d_ff, d, "up/gate projection with the SwiGLU epilogue"),
                      "down": (d, model.d_ff, "down projection")}
            for kind in ("qkvg", "o", "ug", "down", "attn"):
                sess.reset()
                sess.set_kernel_timing(kind, apps)
                sess.prefill(prompt, k)
                tot, cnt = sess.kernel_time()
                sess.set_kernel_timing(None)
                if cnt == 0 or tot <= 0:
                    continue
                if kind in shapes:
                    N_, K_, what = shapes[kind]
                    fl = 2.0 * n * N_ * K_ * cnt
                    name = "k_gemm_big %s (M=%d, N=%d, K=%d)" % (what, n, N_, K_)
                else:
                    fl = float(attn_flops(model, k, n))
                    name = "attention (flash, causal + window %d)" % model.window
                pre_taps[kind] = {"kernel": name, "launches": cnt, "total_ms": round(tot, 3),
                                  "avg_us": round(tot * 1e3 / max(cnt, 1), 2),
                                  "tflops": round(fl / (tot / 1e3) / 1e12, 1),
                                  "mfma_frac": round(fl / (tot / 1e3) / MFMA_PEAK, 4)}
                print(f"[bench] prefill {name}: {cnt} launches, {tot:.2f} ms, "
                      f"{pre_taps[kind]['tflops']} TFLOP/s", file=sys.stderr, flush=True)

    # per-loop KV mode at the same loop counts: one cache per loop of every
    # recurrent layer (KV bytes grow with k), same prompt, same timed steps
    per_loop = {}
    if not args.no_per_loop:
        del sess
        torch.cuda.empty_cache()
        for k in ks:
            sp = dory.Session(model, w, max_batch=1, max_ctx=max_ctx, max_chunk=n, kv_mode="per_loop", kv_loops=k,
                              stream=stream, device=dev)
            sp.prefill(prompt, k)
            ms = _timed_decode(sp, 1, k, K, Wm)
            step_bytes = decode_bytes(model, k, n + Wm + (K - 1) / 2.0)
            per_loop[str(k)] = {"tokens_per_s": round(1e3 / ms, 2), "ms_per_step": round(ms, 4),
                                "hbm_frac": round(step_bytes / (ms / 1e3) / HBM_PEAK, 4),
                                "kv_bytes": int(sp.kv.numel())}
            print(f"[bench] per-loop k={k} decode: {ms:.3f} ms/step, {1e3 / ms:.1f} tok/s, "
                  f"KV {sp.kv.numel() / 1e9:.3f} GB", file=sys.stderr, flush=True)
            del sp
            torch.cuda.empty_cache()

    hk = args.headline_k
    roof = None
    if ug_ms:
        ach = ug_bytes(model) / (ug_ms / 1e3)
        roof = {"bound": "hbm", "achieved": round(ach / 1e9, 1), "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK, 4), "traffic": ug_traffic(),
                "kernel": "k_gemv_pro<1,6,SwiGLU> (up/gate projection with the nGPT update prologue, M=1, N=2x8192, K=3072, bf16)",
                "bytes_per_launch": ug_bytes(model), "avg_launch_us": round(ug_ms * 1e3, 2)}
    cpu = None
    if not args.no_cpu:
        try:
            cpu = cpu_baseline(model, w, hk)
        except Exception as ex:  # report, never hide
            cpu = {"error": repr(ex)}
    res = {
        "metric": METRIC, "value": round(by_k[hk]["tokens_per_s"], 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": K, "warmup": Wm, "ms_per_step": round(by_k[hk]["ms_per_step"], 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded random-init weights, uniform random token ids)",
        "config": {"workload": f"4b_36L_8-20-8 bf16, batch 1, {n}-token random prompt, greedy decode at "
                               f"k={hk}, last-loop KV", "global_batch": 1, "seq_len": n, "n_loops": hk,
                   "kv_mode": "last_loop", "parallelism": "none (1 GPU)"},
        "hbm_frac_step": round(by_k[hk]["hbm_frac"], 4),
        "by_k": {str(k): {kk: (round(v, 4) if isinstance(v, float) else v) for kk, v in d.items()}
                 for k, d in by_k.items()},
        "per_loop": per_loop or None,
        "prefill": {str(k): {kk: round(v, 4) for kk, v in d.items()} for k, d in prefill.items()},
        "prefill_kernels": pre_taps or None,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res))


if __name__ == "__main__":
    main()
