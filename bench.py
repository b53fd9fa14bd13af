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
METRIC = "decode tokens/s @ k=1,2,4 (last-loop KV) + % of HBM roofline, 1×MI355X"


def decode_bytes(m, k, ctx_mean, B=1):
    """Algorithmic HBM bytes of one decode step: every weight once (the
    recurrent block k times), the tied LM head, each layer application's K/V
    reads over its window and its one-position K/V write, per sequence."""
    el = 2
    apps_full, apps_swa = 0, 0
    for l in range(m.n_layers):
        reps = k if m.is_recurrent(l) else 1
        if m.layer_is_full[l]:
            apps_full += reps
        else:
            apps_swa += reps
    per_key = 2 * m.n_kv_heads * m.head_dim * el
    weights = (m.n_in + m.n_out + k * m.n_rec) * m.layer_bytes() + m.vocab * m.d_model * el
    kv_read = B * per_key * (apps_full * ctx_mean + apps_swa * min(ctx_mean, m.window))
    kv_write = B * per_key * (apps_full + apps_swa)
    return weights + kv_read + kv_write


def ug_bytes(m, B=1):
    """Algorithmic bytes of one SwiGLU up/gate projection launch (B rows): the
    two weight matrices, the prologue's inputs (sublayer output y, residual h,
    alpha; float32) and outputs (new residual, float32; activation, bf16)."""
    return 2 * m.d_ff * m.d_model * 2 + B * m.d_model * 4 * 3 + B * m.d_model * 4 + B * m.d_ff * 2


def prefill_flops(m, k, n):
    """Dense FLOPs of prefilling n positions from an empty cache: 2 per
    weight per position for every layer application, 4*n_q*hd per allowed
    (query, key) pair (QK^T and PV), and the LM head on the last position."""
    flops = 0
    pairs_full = n * (n + 1) // 2
    W = m.window
    pairs_swa = sum(min(t + 1, W) for t in range(n)) if n <= 65536 else None
    per_app_w = m.layer_bytes() // 2
    for l in range(m.n_layers):
        reps = k if m.is_recurrent(l) else 1
        pairs = pairs_full if m.layer_is_full[l] else pairs_swa
        flops += reps * (2 * n * per_app_w + 4 * m.q_dim * pairs)
    return flops + 2 * m.vocab * m.d_model


def cpu_baseline(model, dev_w, k_head: int, budget_s: float = 20.0):
    """The oracle (numpy, float32 compute, bfloat16 storage points) on the
    host: decode calls of a 1/2/1-layer model at the benchmark's widths over a
    short context, timed at k = 1 and k = 2; the per-layer-application and
    per-token fixed costs are solved from the two and scaled to the 36-layer
    shape at k = k_head."""
    import numpy as np
    import torch
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    from oracle.ngpt import LoopedNGPT
    from synth.configs import scaled_config
    small = scaled_config(model, n_in=1, n_rec=2, n_out=1)
    w = {"embed": dev_w["embed"].cpu().numpy().view(np.uint16)}
    # layers 0..3 of the sample take the weights of layers 0, 8, 9, 28 (one of each block)
    src = [0, model.n_in, model.n_in + 1, model.n_in + model.n_rec]
    for i, l in enumerate(src):
        for kind in ("qkvg", "o", "ug", "down"):
            w[f"L{i}.{kind}"] = dev_w[f"L{l}.{kind}"].cpu().numpy().view(np.uint16)
        w[f"L{i}.alpha_a"] = dev_w[f"L{l}.alpha_a"].cpu().numpy()
        w[f"L{i}.alpha_m"] = dev_w[f"L{l}.alpha_m"].cpu().numpy()
    prompt = np.arange(8, dtype=np.int32)[None, :] * 997 % model.vocab
    times = {}
    t_start = time.perf_counter()
    for k in (1, 2):
        o = LoopedNGPT(small, w, compute="f32", bf16_points=True, max_ctx=64)
        o.call(prompt, k, "last_loop")            # widen weights, warm caches
        reps = 0
        t0 = time.perf_counter()
        while True:
            o.call(np.array([[reps % model.vocab]], dtype=np.int32), k, "last_loop")
            reps += 1
            if reps >= 3 and (time.perf_counter() - t0 > budget_s / 4 or reps >= 20):
                break
        times[k] = (time.perf_counter() - t0) / reps
    t_app = (times[2] - times[1]) / small.n_rec
    t_fixed = times[1] - (small.n_in + small.n_out + small.n_rec) * t_app
    apps = model.n_in + model.n_out + k_head * model.n_rec
    sec_per_tok = apps * t_app + max(t_fixed, 0.0)
    return {"value": 1.0 / sec_per_tok, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"numpy oracle (f32 compute, bf16 storage points) decoding 1 token per call at the "
                       f"36-layer model's widths with a 1/2/1-layer stack over an 8-token context, timed at "
                       f"k=1 ({times[1]*1e3:.1f} ms/call) and k=2 ({times[2]*1e3:.1f} ms/call); per layer "
                       f"application {t_app*1e3:.1f} ms and fixed {t_fixed*1e3:.1f} ms/token scaled to "
                       f"{apps} layer applications (k={k_head}); excludes attention over an 8K context"),
            "wall_s": round(time.perf_counter() - t_start, 1)}


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
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(the sharding design is described in DESIGN.md).", file=sys.stderr)
        sys.exit(2)

    import torch
    import looped_ngpt_amd as dory
    from synth.configs import get_config
    from synth.device import make_weights_device

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    model = get_config("c36")
    ks = [int(x) for x in args.ks.split(",")]
    if args.headline_k not in ks:
        ks.append(args.headline_k)
    n, K, Wm = args.prompt, args.steps, args.warmup
    # positions needed, rounded to 256 (a multiple of 4 keeps the cached
    # values' 4-position runs aligned for the matrix-core decode attention)
    max_ctx = (n + Wm + K + args.kernel_steps + 2 + 255) // 256 * 256

    t0 = time.perf_counter()
    w = make_weights_device(model, dev)
    torch.cuda.synchronize()
    print(f"[bench] weights {sum(t.numel() * t.element_size() for t in w.values()) / 1e9:.2f} GB "
          f"generated in {time.perf_counter() - t0:.1f}s", file=sys.stderr, flush=True)
    g = torch.Generator(device="cpu")
    g.manual_seed(model.seed * 7 + 1)
    prompt = torch.randint(0, model.vocab, (1, n), generator=g, dtype=torch.int32).to(dev)
    stream = torch.cuda.current_stream(dev)

    by_k, prefill = {}, {}
    ug_ms = None
    sess = dory.Session(model, w, max_batch=1, max_ctx=max_ctx, max_chunk=n, kv_mode="last_loop",
                        stream=stream, device=dev)
    sess.set_graphs(args.graphs)
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
                      "mfma_frac_whole": prefill_flops(model, k, n) / (pms / 1e3) / 2.5e15}
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
                   "hbm_frac": step_bytes / (ms / 1e3 / K) / HBM_PEAK, "bytes_per_step": step_bytes}
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

    hk = args.headline_k
    roof = None
    if ug_ms:
        ach = ug_bytes(model) / (ug_ms / 1e3)
        roof = {"bound": "hbm", "achieved": round(ach / 1e9, 1), "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK, 4), "traffic": None,
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
        "prefill": {str(k): {kk: round(v, 4) for kk, v in d.items()} for k, d in prefill.items()},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res))


if __name__ == "__main__":
    main()
