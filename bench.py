#!/usr/bin/env python3
"""Training-step throughput on one MI355X.

One step = slt_forward_loss + slt_backward + slt_adamw_step over one batch of
synthetic tokens for the Llama-style decoder d=384, 8 layers, 8 heads,
T=256, B=64, V=4096, SwiGLU 1024 (bf16 activations, fp32 master weights and
moments), inputs resident in HBM.  Prints one JSON line: tokens/s, the
roofline position of the dominant kernel (timed live with HIP events on the
stream it runs on) and the CPU oracle timed on a bounded sample of the same
workload.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {"bf16_tflops": 2500.0, "f32_tflops": 157.3, "hbm_gbs": 8000.0}


def step_flops(w) -> float:
    """Algorithmic FLOPs of one step: 6 per matmul parameter per token
    (forward, dX, dW) plus causal attention 6 L C (T+1) per token."""
    d = w.C // w.H
    qkv = (w.H + 2 * w.Hkv) * d
    if w.block == "llama":
        per_layer = w.C * qkv + w.C * w.H * d + 3 * w.C * w.F
    else:
        per_layer = w.C * qkv + w.C * w.F + w.C * (w.H * d + w.F)
    mat = w.L * per_layer + w.V * w.C
    return w.N * (6.0 * mat + 6.0 * w.L * w.C * (w.T + 1))


def time_launches(fn, reps: int, torch) -> float:
    """Average duration (s) of fn() over reps launches, HIP events on the
    current stream (the one the library launches on)."""
    s = torch.cuda.current_stream()
    fn()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(s)
    for _ in range(reps):
        fn()
    b.record(s)
    b.synchronize()
    return a.elapsed_time(b) / 1e3 / reps


def dominant_kernel(w, ts, torch, reps):
    """The step's most expensive launch class is its largest GEMM family; time
    the [W1;W3] projection (M=N_tok, N=2F, K=C, bf16 in/out) exactly as the
    forward launches it, on the step's own buffers."""
    from scratch_llama_transformer_amd import binding as B
    dt = B.BF16 if w.act == "bf16" else B.F32
    es = 2 if dt == B.BF16 else 4
    M, N, K = w.N, 2 * w.F, w.C
    layout = {t["name"]: t for t in ts.layout}
    wptr = ts.compute_params.data_ptr() + layout["h0.w1"]["offset"] * es
    x = torch.empty((M, K), dtype=torch.bfloat16 if dt == B.BF16 else torch.float32, device="cuda").normal_()
    y = torch.empty((M, N), dtype=x.dtype, device="cuda")

    def fn():
        B.slt_gemm(M, N, K, x, K, 1, wptr, K, 1, y, N, None, 0, dt, dt)

    sec = time_launches(fn, reps, torch)
    flops = 2.0 * M * N * K
    peak = PEAK["bf16_tflops"] if dt == B.BF16 else PEAK["f32_tflops"]
    ach = flops / sec / 1e12
    return {"kernel": f"gemm_k NT {M}x{N}x{K} ([W1;W3] forward projection)", "bound": "mfma",
            "achieved": round(ach, 2), "peak": peak, "unit": "TFLOP/s", "frac": round(ach / peak, 4),
            "traffic": None, "avg_launch_us": round(sec * 1e6, 2)}


def cpu_baseline(w, seconds_hint=20.0):
    """The oracle (numpy float64) on a bounded sample of the same workload:
    one full step (forward, backward, AdamW) on B_s sequences of the batch."""
    import numpy as np
    import oracle as O
    import slt_workloads as W
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    Bs = 8
    ws = w.with_(B=Bs)
    params = W.make_params(ws, 1003)
    tokens = W.make_tokens(ws, 1003)
    t0 = time.perf_counter()
    O.train_step(ws, params, tokens)
    dt = time.perf_counter() - t0
    return {"value": round(Bs * w.T / dt, 1), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"one full step (forward, backward, AdamW on all {W.n_params(ws)} parameters) "
                      f"on {Bs} of the {w.B} sequences ({Bs * w.T} tokens), float64 numpy; {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3, help="workload index (3 = the headline shape)")
    ap.add_argument("--kernel-reps", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(the data-parallel design is described, not built).", file=sys.stderr)
        sys.exit(2)

    import torch
    import slt_workloads as W
    from scratch_llama_transformer_amd.trainer import TrainStep

    w = W.get_config(args.config)
    ts = TrainStep(w, seed=1000 + args.config)
    tok = torch.from_numpy(W.make_tokens(w, 1000 + args.config)).cuda()
    for _ in range(args.warmup):
        ts.step(tok)
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(args.steps):
        ts.step(tok)
    e1.record(s)
    e1.synchronize()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    loss = float(ts.loss.item())
    tps = w.N / (ms / 1e3)
    flops = step_flops(w)
    peak = PEAK["bf16_tflops"] if w.act == "bf16" else PEAK["f32_tflops"]
    roof = dominant_kernel(w, ts, torch, args.kernel_reps)
    out = {
        "metric": "train tokens/s (fwd+bwd+AdamW) d=384 8L T=256 B=64",
        "value": round(tps, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.act == "bf16" else "f32",
        "data": "synthetic (seeded Zipf(1.1) token ids, device-initialised N(0, 0.02) weights)",
        "config": {"workload": f"{w.name}: Llama-style decoder V={w.V} C={w.C} H={w.H} L={w.L} "
                               f"T={w.T} B={w.B} F={w.F}, RoPE, SwiGLU, untied head",
                   "global_batch": w.B, "seq_len": w.T, "tokens_per_step": w.N},
        "mfma_util_pct": round(100.0 * flops / (ms / 1e3) / 1e12 / peak, 2),
        "step_tflops": round(flops / (ms / 1e3) / 1e12, 2),
        "loss_after_steps": round(loss, 5),
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
