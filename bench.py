#!/usr/bin/env python3
"""Training-step throughput on one MI355X.

One step = slt_forward_loss + slt_backward + slt_adamw_step over one batch of
synthetic tokens for the Llama-style decoder d=384, 8 layers, 8 heads,
T=256, B=64, V=4096, SwiGLU 1024 (bf16 activations, fp32 master weights and
moments), inputs resident in HBM.  Prints one JSON line with tokens/s, a
per-class kernel breakdown (each class re-launched through the C ABI with the
step's shapes and timed with HIP events on the current stream, the one the
library launches on), the roofline position of the dominant class, and the CPU
oracle timed on a bounded sample of the same workload.

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

PEAK = {"bf16": 2500.0, "f32": 157.3, "hbm": 8000.0}  # TFLOP/s, TFLOP/s, GB/s (vendor figures)


def shapes(w):
    """The step's GEMM launches as (M, N, K, residual) per class: forward
    projections (k-major operands), activation gradients dX = dY W and
    weight gradients dW = dY^T X."""
    d = w.C // w.H
    qd, kd = w.H * d, w.Hkv * d
    qkv = qd + 2 * kd
    N, C, F, V = w.N, w.C, w.F, w.V
    fwd, dx, dw = [], [], []
    for _ in range(w.L):
        if w.block == "llama":
            fwd += [(N, qkv, C, 0), (N, C, qd, 1), (N, 2 * F, C, 0), (N, C, F, 1)]
            dx += [(N, F, C, 0), (N, C, 2 * F, 0), (N, qd, C, 0), (N, C, qkv, 0)]
            dw += [(C, F, N, 0), (2 * F, C, N, 0), (C, qd, N, 0), (qkv, C, N, 0)]
        else:
            iw, ow = qkv + F, qd + F
            fwd += [(N, iw, C, 0), (N, C, ow, 1)]
            dx += [(N, ow, C, 0), (N, C, iw, 0)]
            dw += [(C, ow, N, 0), (iw, C, N, 0)]
    fwd.append((N, V, C, 0))
    dx.append((N, C, V, 0))
    dw.append((V, C, N, 0))
    return {"gemm_fwd": fwd, "gemm_dx": dx, "gemm_dw": dw}


def attn_flops(w):
    """Algorithmic causal attention FLOPs (forward, backward) of one step: per
    (b, h) the forward has two products over the T(T+1)/2 causal pairs (S and
    P V), the backward four (dP, dV, dK, dQ); recomputing S is not counted."""
    f = 4.0 * w.B * w.H * (w.T * (w.T + 1) / 2) * (w.C // w.H) * w.L
    return f, 2.0 * f


def step_flops(w):
    """Algorithmic FLOPs of one step: 6 per matmul parameter per token plus
    causal attention (3x its forward products)."""
    g = sum(2.0 * M * N * K for cls in shapes(w).values() for (M, N, K, _) in cls)
    fa, ba = attn_flops(w)
    return g + fa + ba


def describe(w):
    if w.block == "llama":
        heads = f"H={w.H}" + (f"/Hkv={w.Hkv} (GQA)" if w.Hkv != w.H else "")
        return (f"{w.name}: Llama-style decoder V={w.V} C={w.C} {heads} L={w.L} T={w.T} B={w.B} F={w.F}, "
                f"RMSNorm, rotate-half RoPE, SwiGLU, untied head")
    return (f"{w.name}: parallel-block (GPT-J style) decoder V={w.V} C={w.C} H={w.H} L={w.L} T={w.T} B={w.B} "
            f"F={w.F}, LayerNorm, even-odd RoPE on {w.R} of {w.C // w.H} dims, GELU MLP, untied head")


def time_block(fn, reps, torch):
    """Average seconds of fn() (which enqueues on the current stream), HIP
    events on that stream."""
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


def kernel_classes(w, ts, torch, reps, only=None):
    """Per-class time of one step, each class re-run through the C ABI with
    the step's shapes on fresh buffers (``only``: just that GEMM class)."""
    from scratch_llama_transformer_amd import binding as B
    dt = B.BF16 if w.act == "bf16" else B.F32
    tdt = torch.bfloat16 if dt == B.BF16 else torch.float32
    peak = PEAK["bf16"] if dt == B.BF16 else PEAK["f32"]
    es = 2 if dt == B.BF16 else 4
    out = {}
    ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    for cls, launches in shapes(w).items():
        if only is not None and cls != only:
            continue
        bufs = []
        for (M, N, K, res) in launches:
            if cls == "gemm_fwd":
                A = torch.empty((M, K), dtype=tdt, device="cuda").normal_()
                Bm = torch.empty((N, K), dtype=tdt, device="cuda").normal_()
                Cm = torch.empty((M, N), dtype=tdt, device="cuda")
                R = torch.empty((M, N), dtype=tdt, device="cuda").normal_() if res else None
                bufs.append((M, N, K, A, K, 1, Bm, K, 1, Cm, N, R, N, dt, dt, None, 0))
            elif cls == "gemm_dx":
                A = torch.empty((M, K), dtype=tdt, device="cuda").normal_()
                Bm = torch.empty((K, N), dtype=tdt, device="cuda").normal_()
                Cm = torch.empty((M, N), dtype=tdt, device="cuda")
                bufs.append((M, N, K, A, K, 1, Bm, N, 0, Cm, N, None, 0, dt, dt, None, 0))
            else:
                A = torch.empty((K, M), dtype=tdt, device="cuda").normal_()
                Bm = torch.empty((K, N), dtype=tdt, device="cuda").normal_()
                Cm = torch.empty((M, N), dtype=torch.float32, device="cuda")
                bufs.append((M, N, K, A, M, 0, Bm, N, 0, Cm, N, None, 0, dt, B.F32, ws, ws.numel()))

        if cls == "gemm_dw" and dt == B.BF16:
            # as the step runs them: one grouped launch per layer (the head's
            # product joins the last layer's group)
            per = 4 if w.block == "llama" else 2
            items = [(a[0], a[1], a[3], a[4], a[6], a[7], a[9], a[10], 1.0, 0) for a in bufs]
            groups = [items[i:i + per] for i in range(0, len(items) - 1, per)]
            groups[-1] = groups[-1] + [items[-1]]

            def run(groups=groups, K=launches[0][2]):
                for grp in groups:
                    B.slt_gemm_dw_group(grp, K, ws, ws.numel())
        else:
            def run(bufs=bufs):
                for args in bufs:
                    B.slt_gemm(*args)

        sec = time_block(run, reps, torch)
        flops = sum(2.0 * M * N * K for (M, N, K, _) in launches)
        out[cls] = {"ms_per_step": sec * 1e3, "launches": len(launches), "tflops": flops / sec / 1e12,
                    "frac_of_peak": flops / sec / 1e12 / peak, "flops": flops, "avg_launch_us": sec * 1e6 / len(launches),
                    "bound": "mfma", "peak": peak}
        del bufs
    if only is not None:
        return out
    # attention: forward, and backward (dQ then dK/dV) on the step's strides
    d = w.C // w.H
    qd, kd = w.H * d, w.Hkv * d
    ld = qd + 2 * kd + (w.F if w.block != "llama" else 0)
    qkv = torch.empty((w.N, ld), dtype=tdt, device="cuda").normal_()
    o = torch.empty((w.N, qd), dtype=tdt, device="cuda")
    ores = torch.empty((w.N, qd), dtype=tdt, device="cuda") if dt == B.BF16 else None
    lse = torch.empty((w.B, w.H, w.T), device="cuda")
    cs = torch.empty((w.T, max(w.R, 2)), device="cuda")
    B.slt_rope_table(w.T, w.R, w.base, cs)
    g = torch.empty((w.N, qd), dtype=tdt, device="cuda").normal_()
    dqkv = torch.empty_like(qkv)
    aws = torch.empty(B.slt_attention_bwd_workspace(w.B, w.T, w.H, w.Hkv, d, dt), dtype=torch.uint8, device="cuda")
    fws = B.slt_attention_fwd_workspace(w.B, w.T, w.H, w.Hkv, d, dt)
    fw = torch.empty(fws, dtype=torch.uint8, device="cuda") if fws else None
    p, dp = qkv.data_ptr(), dqkv.data_ptr()
    mode = B.ROPE_HALF if w.rope_mode == "half" else B.ROPE_PAIRS

    def fwd():
        for _ in range(w.L):
            B.slt_attention_fwd(p, p + qd * es, p + (qd + kd) * es, o, lse, ores, ld, ld, ld, qd,
                                w.B, w.T, w.H, w.Hkv, d, w.R, mode, cs, dt, fw)

    def bwd():
        for _ in range(w.L):
            B.slt_attention_bwd(p, p + qd * es, p + (qd + kd) * es, o, ores, g, lse, dp, dp + qd * es,
                                dp + (qd + kd) * es, ld, ld, ld, qd, qd, ld, ld, ld, w.B, w.T, w.H, w.Hkv, d, w.R,
                                mode, cs, dt, aws)

    fa, ba = attn_flops(w)
    for name, fn, fl, nl in [("attention_fwd", fwd, fa, w.L), ("attention_bwd", bwd, ba, 2 * w.L)]:
        sec = time_block(fn, reps, torch)
        out[name] = {"ms_per_step": sec * 1e3, "launches": nl, "tflops": fl / sec / 1e12,
                     "frac_of_peak": fl / sec / 1e12 / peak, "flops": fl, "avg_launch_us": sec * 1e6 / nl,
                     "bound": "mfma", "peak": peak}
    del qkv, o, ores, g, dqkv, aws
    # HBM-bound optimizer-side kernels over the flat parameter buffer: AdamW
    # (theta, g, m, v read; theta, m, v written; the bf16 copy written) and
    # the global gradient norm used for clipping (g read once)
    _, n = B.slt_param_layout(B.make_config(w))
    th = torch.empty(n, device="cuda").normal_(0, 0.02)
    gr = torch.empty(n, device="cuda").normal_(0, 1e-3)
    m = torch.zeros(n, device="cuda")
    v = torch.zeros(n, device="cuda")
    sh = torch.empty(n, dtype=torch.int16, device="cuda") if dt == B.BF16 else None
    cws = torch.empty(B.slt_clip_workspace_bytes(), dtype=torch.uint8, device="cuda")
    nrm = torch.empty(2, device="cuda")
    byt_adamw = n * (30 if sh is not None else 28)
    hbm = PEAK["hbm"]
    for name, fn, byt, nl in [
        ("adamw", lambda: B.slt_adamw_step(n, th, sh, gr, m, v, 1, 1e-3, 0.9, 0.999, 1e-8, 0.1), byt_adamw, 1),
        ("grad_norm", lambda: B.slt_clip_grad_norm(n, gr, B.NORM_L2, 1.0, nrm, nrm.data_ptr() + 4, cws), 4 * n, 1),
    ]:
        sec = time_block(fn, reps, torch)
        gbs = byt / sec / 1e9
        out[name] = {"ms_per_step": sec * 1e3, "launches": nl, "gbps": gbs, "frac_of_peak": gbs / hbm,
                     "bytes": byt, "avg_launch_us": sec * 1e6 / nl, "bound": "hbm", "peak": hbm}
    return out


def measured_traffic(w):
    """HBM bytes per launch of the forward-projection GEMM from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary, scaled by a plain copy's
    counts; None when that summary is for another workload or for a GEMM
    source other than the one built now."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "gemm_fwd_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
        with open(os.path.join(ROOT, "scratch_llama_transformer_amd", "csrc", "gemm.hip"), "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except OSError:
        return None
    if rec.get("gemm_hip_sha256") != sha or rec.get("workload") != w.name:
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(w):
    """The oracle (numpy float64) on a bounded sample of the same workload:
    one full step (forward, backward, AdamW) on up to 64 of the batch's
    sequences (all of them for the d=384 workload, about 10-30 s of CPU)."""
    import oracle as O
    import slt_workloads as W
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    Bs = min(w.B, 64)
    ws = w.with_(B=Bs)
    params = W.make_params(ws, 1003)
    tokens = W.make_tokens(ws, 1003)
    t0 = time.perf_counter()
    O.train_step(ws, params, tokens)
    dt = time.perf_counter() - t0
    return {"value": round(Bs * w.T / dt, 1), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"one full step (forward, backward, AdamW on all {W.n_params(ws)} parameters) on {Bs} of "
                      f"the {w.B} sequences ({Bs * w.T} tokens), float64 numpy; {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3, help="workload index (3 = the headline shape)")
    ap.add_argument("--kernel-reps", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-breakdown", action="store_true")
    ap.add_argument("--only-class", choices=["gemm_fwd", "gemm_dx", "gemm_dw"], default=None,
                    help="only time one GEMM class of the breakdown (for hardware-counter runs) and exit")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB device-to-device 5 times (for scaling HBM byte counters) and exit")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(the data-parallel design is described, not built).", file=sys.stderr)
        sys.exit(2)

    import torch
    import slt_workloads as W
    from scratch_llama_transformer_amd.trainer import TrainStep

    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}), flush=True)
        return

    w = W.get_config(args.config)
    if args.only_class:
        cl = kernel_classes(w, None, torch, args.kernel_reps, only=args.only_class)[args.only_class]
        print(json.dumps({"workload": w.name, "class": args.only_class, "launches": cl["launches"],
                          "avg_launch_us": round(cl["avg_launch_us"], 2), "tflops": round(cl["tflops"], 2)}),
              flush=True)
        return
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
    peak = PEAK["bf16"] if w.act == "bf16" else PEAK["f32"]
    out = {
        "metric": "train tokens/s (fwd+bwd+AdamW) d=384 8L T=256 B=64; MFMA util %, HBM GB/s",
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
        "data": f"synthetic (seeded {'Zipf(1.1)' if w.tokens == 'zipf' else 'uniform'} token ids, "
                "device-initialised N(0, 0.02) weights)",
        "config": {"workload": describe(w),
                   "global_batch": w.B, "seq_len": w.T, "tokens_per_step": w.N},
        "mfma_util_pct": round(100.0 * flops / (ms / 1e3) / 1e12 / peak, 2),
        "step_tflops": round(flops / (ms / 1e3) / 1e12, 2),
        "loss_after_steps": round(loss, 5),
    }
    del ts
    torch.cuda.empty_cache()
    if not args.no_breakdown:
        cl = kernel_classes(w, None, torch, args.kernel_reps)
        out["kernels"] = {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()
                              if kk in ("ms_per_step", "launches", "tflops", "gbps", "frac_of_peak", "avg_launch_us")}
                          for k, v in cl.items()}
        # the dominant kernel class of the step (largest time in the
        # breakdown): the forward-projection GEMMs, both operands k-major
        # (bf16: gemm_d64_k for 384 to 1152 output columns, gemm_w8_k's
        # 256 x 256 tiles for the wide ones; fp32: gemm_k on the fp32 matrix
        # instructions)
        c = cl["gemm_fwd"]
        kern = "gemm_k, fp32" if w.act == "f32" else "gemm_d64_k, gemm_w8_k"
        out["roofline"] = {"kernel": f"forward-projection GEMMs ({kern}; k-major x k-major)",
                           "bound": c["bound"],
                           "achieved": round(c["tflops"], 2), "peak": c["peak"], "unit": "TFLOP/s",
                           "frac": round(c["tflops"] / c["peak"], 4), "traffic": measured_traffic(w),
                           "avg_launch_us": round(c["avg_launch_us"], 2), "launches_per_step": c["launches"]}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
