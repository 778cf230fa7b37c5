#!/usr/bin/env python3
"""Training-step throughput on one MI355X.

One step = slt_forward_loss + slt_backward_adamw (the backward with each
layer's AdamW update folded in) over one batch of synthetic tokens for the
Llama-style decoder d=384, 8 layers, 8 heads, T=256, B=64, V=4096, SwiGLU 1024
(bf16 activations, fp32 master weights and moments), inputs resident in HBM.
Prints one JSON line with tokens/s, a per-class kernel breakdown of the step
(the library's HIP event brackets around each class's launches, on the stream
each runs on, over a few steps after the timed ones), the same classes
re-launched alone through the C ABI for comparison, every HBM-bound kernel in
GB/s, the roofline position of the dominant class, and the CPU oracle timed on
a bounded sample of the same workload.

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
        oes = 4 if cls == "gemm_dw" else es  # weight gradients are written in fp32
        byt = sum((M * K + N * K) * es + M * N * oes * (2 if r else 1) for (M, N, K, r) in launches)
        out[cls] = {"ms_per_step": sec * 1e3, "launches": len(launches), "tflops": flops / sec / 1e12,
                    "frac_of_peak": flops / sec / 1e12 / peak, "flops": flops, "bytes": byt,
                    "avg_launch_us": sec * 1e6 / len(launches), "bound": "mfma", "peak": peak}
        del bufs
    if only is not None and only.startswith("gemm"):
        return out
    # attention: forward, and backward (dQ then dK/dV) on the step's strides,
    # with q and k taken as already rotated (R = 0), as the step's projection
    # epilogue leaves them (the per-op calls would otherwise rotate them into
    # their workspace first)
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
                                w.B, w.T, w.H, w.Hkv, d, 0, mode, cs, dt, fw)

    def bwd():
        for _ in range(w.L):
            B.slt_attention_bwd(p, p + qd * es, p + (qd + kd) * es, o, ores, g, lse, dp, dp + qd * es,
                                dp + (qd + kd) * es, ld, ld, ld, qd, qd, ld, ld, ld, w.B, w.T, w.H, w.Hkv, d, 0,
                                mode, cs, dt, aws)

    fa, ba = attn_flops(w)
    # algorithmic bytes per layer: forward reads q, k, v and writes o and the
    # log-sum-exp; backward reads q, k, v, o, dO and the log-sum-exp and
    # writes dQ, dK, dV
    qb, kb = w.N * qd * es, w.N * kd * es
    ab = {"attention_fwd": 2 * qb + 2 * kb + 4 * w.B * w.H * w.T,
          "attention_bwd": 5 * qb + 4 * kb + 4 * w.B * w.H * w.T}
    fwd()  # lse for the backward
    for name, fn, fl, nl in [("attention_fwd", fwd, fa, w.L), ("attention_bwd", bwd, ba, 2 * w.L)]:
        if only is not None and name != only:
            continue
        sec = time_block(fn, reps, torch)
        out[name] = {"ms_per_step": sec * 1e3, "launches": nl, "tflops": fl / sec / 1e12,
                     "frac_of_peak": fl / sec / 1e12 / peak, "flops": fl, "bytes": ab[name] * w.L,
                     "avg_launch_us": sec * 1e6 / nl, "bound": "mfma", "peak": peak}
    del qkv, o, ores, g, dqkv, aws
    return out


TRAIN_BYTES = 1 << 30  # footprint of one timed train of an HBM-bound kernel
PROF_STEPS = 3  # steps run with the library's per-class launch timing on


def time_train(fns, reps, torch):
    """Median and best seconds per launch of a train of launches fns[0],
    fns[1], ... (each on its own buffers) timed as one with HIP events on
    the current stream.  With the buffers' total footprint at 1 GiB or more,
    the 256 MB Infinity Cache holds none of a launch's inputs when it starts,
    and lines written by one launch are written back to HBM during the
    following ones: the train runs at the sustained HBM rate, not the cache's."""
    s = torch.cuda.current_stream()
    for f in fns:
        f()
    times = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(s)
        for f in fns:
            f()
        b.record(s)
        b.synchronize()
        times.append(a.elapsed_time(b) / 1e3 / len(fns))
    times.sort()
    return times[len(times) // 2], times[0]


def machine_bounds(torch):
    """The library's own streaming copy over 2 x 2 GiB (read + write GB/s,
    best of its launch shapes) and its MFMA loop (bf16 TFLOP/s, best of 6):
    the measured bounds the kernels are also reported against."""
    from scratch_llama_transformer_amd import binding as B
    n = 2 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    s = torch.cuda.current_stream()
    best, best_v = None, 0
    for v in range(5):
        for _ in range(4):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(s)
            B.slt_stream_copy(src, dst, n, v)
            b.record(s)
            b.synchronize()
            t = a.elapsed_time(b) / 1e3
            if best is None or t < best:
                best, best_v = t, v
    del src, dst
    blocks, iters = 256 * 8, 4096
    out = torch.empty(blocks * 256, device="cuda")
    rates = {}
    for var in range(3):
        bestm = None
        for _ in range(4):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(s)
            B.slt_mfma_loop(blocks, iters, out, var)
            b.record(s)
            b.synchronize()
            t = a.elapsed_time(b) / 1e3
            bestm = t if bestm is None else min(bestm, t)
        rates[var] = B.slt_mfma_loop_flops(blocks, iters, var) / bestm / 1e12
    return {"copy_gbps": round(2.0 * n / best / 1e9, 1), "copy_bytes": 2 * n,
            "mfma_bf16_tflops": round(max(rates.values()), 1),
            "mfma_loop_tflops": {"16x16x32 x8": round(rates[0], 1), "32x32x16 x8": round(rates[1], 1),
                                 "16x16x32 x16": round(rates[2], 1)},
            "copy_kernel": f"slt_stream_copy variant {best_v} (16-byte loads and stores, 2 GiB each way; best of "
                           "5 launch shapes x 4)",
            "mfma_kernel": "slt_mfma_loop (independent MFMA chains per wave, 32 waves per CU; best variant)"}


HBM_CLASSES = ["rmsnorm_fwd", "rmsnorm_bwd", "swiglu_fwd", "swiglu_bwd", "layernorm_fwd", "layernorm_bwd", "gelu_fwd",
               "gelu_bwd", "softmax_xent", "embedding_fwd", "embedding_bwd", "adamw", "grad_norm"]


def hbm_classes(w, torch, reps, machine, only=None):
    """Every HBM-bound kernel of the step at the step's sizes and strides:
    norm forward and backward, SwiGLU or GELU forward and backward, softmax
    cross-entropy, embedding forward and backward, AdamW and the gradient
    norm.  Each is timed in trains of launches over as many copies of its
    operands as make 1 GiB (time_train).  Bytes are the algorithmic ones
    (each operand read or written once)."""
    from scratch_llama_transformer_amd import binding as B
    import slt_workloads as W
    dt = B.BF16 if w.act == "bf16" else B.F32
    tdt = torch.bfloat16 if dt == B.BF16 else torch.float32
    e = 2 if dt == B.BF16 else 4
    N, C, F, V = w.N, w.C, w.F, w.V
    rnd = lambda *shape: torch.empty(*shape, dtype=tdt, device="cuda").normal_()
    emp = lambda *shape, dtype=tdt: torch.empty(*shape, dtype=dtype, device="cuda")
    out = {}

    def add(name, factory, byt):
        if only is not None and name != only:
            return
        k = max(1, min(64, -(-TRAIN_BYTES // int(byt))))
        fns = [factory() for _ in range(k)]
        med, best = time_train(fns, reps, torch)
        del fns
        gbs = byt / med / 1e9
        out[name] = {"us_per_launch": round(med * 1e6, 2), "best_us": round(best * 1e6, 2), "bytes": int(byt),
                     "gbps": round(gbs, 1), "frac_of_peak": round(gbs / PEAK["hbm"], 4),
                     "frac_of_copy": round(gbs / machine["copy_gbps"], 4), "bound": "hbm", "train": k}

    g, bta = torch.ones(C, dtype=tdt, device="cuda"), torch.zeros(C, dtype=tdt, device="cuda")
    if w.block == "llama":
        def rms_fwd():
            x, y, r = rnd(N, C), emp(N, C), emp(N, dtype=torch.float32)
            return lambda: B.slt_rmsnorm_fwd(x, g, y, r, N, C, w.eps, dt)

        def rms_bwd():
            x, dy, dres, dx = rnd(N, C), rnd(N, C), rnd(N, C), emp(N, C)
            r, dg = emp(N, dtype=torch.float32), emp(C, dtype=torch.float32)
            nws = emp(B.slt_norm_bwd_workspace(N, C), dtype=torch.uint8)
            B.slt_rmsnorm_fwd(x, g, dx, r, N, C, w.eps, dt)
            return lambda: B.slt_rmsnorm_bwd(x, g, r, dy, dres, dx, dg, N, C, dt, nws)

        def swi_fwd():
            ab, h = rnd(N, 2 * F), emp(N, F)
            pa = ab.data_ptr()
            return lambda ab=ab: B.slt_swiglu_fwd(pa, pa + F * e, h, N, F, 2 * F, 2 * F, F, dt)

        def swi_bwd():
            ab, dh, dab = rnd(N, 2 * F), rnd(N, F), emp(N, 2 * F)
            pa, pd = ab.data_ptr(), dab.data_ptr()
            return lambda ab=ab, dab=dab: B.slt_swiglu_bwd(pa, pa + F * e, dh, pd, pd + F * e, N, F, 2 * F, 2 * F, F,
                                                           2 * F, 2 * F, dt)

        add("rmsnorm_fwd", rms_fwd, N * (2 * C * e + 4) + C * e)
        add("rmsnorm_bwd", rms_bwd, N * (4 * C * e + 4) + C * (e + 4))
        add("swiglu_fwd", swi_fwd, 3 * N * F * e)
        add("swiglu_bwd", swi_bwd, 5 * N * F * e)
    else:
        def ln_fwd():
            x, y = rnd(N, C), emp(N, C)
            mu, r = emp(N, dtype=torch.float32), emp(N, dtype=torch.float32)
            return lambda: B.slt_layernorm_fwd(x, g, bta, y, mu, r, N, C, w.eps, dt)

        def ln_bwd():
            x, dy, dres, dx = rnd(N, C), rnd(N, C), rnd(N, C), emp(N, C)
            mu, r = emp(N, dtype=torch.float32), emp(N, dtype=torch.float32)
            dg, db = emp(C, dtype=torch.float32), emp(C, dtype=torch.float32)
            nws = emp(B.slt_norm_bwd_workspace(N, C), dtype=torch.uint8)
            B.slt_layernorm_fwd(x, g, bta, dx, mu, r, N, C, w.eps, dt)
            return lambda: B.slt_layernorm_bwd(x, g, mu, r, dy, dres, dx, dg, db, N, C, dt, nws)

        def gelu_fwd():
            a, u = rnd(N, F), emp(N, F)
            return lambda: B.slt_gelu_fwd(a, u, N, F, F, F, dt)

        def gelu_bwd():
            a, du, da = rnd(N, F), rnd(N, F), emp(N, F)
            return lambda: B.slt_gelu_bwd(a, du, da, N, F, F, F, F, dt)

        add("layernorm_fwd", ln_fwd, N * (2 * C * e + 8) + 2 * C * e)
        add("layernorm_bwd", ln_bwd, N * (4 * C * e + 8) + C * (e + 8))
        add("gelu_fwd", gelu_fwd, 2 * N * F * e)
        add("gelu_bwd", gelu_bwd, 3 * N * F * e)
    tok = torch.from_numpy(W.make_tokens(w, 1000)).cuda()

    def xent():
        z, loss, rl = rnd(N, V), emp(1, dtype=torch.float32), emp(4 * N, dtype=torch.uint8)
        return lambda: B.slt_softmax_xent(z, V, tok, w.B, w.T, w.T + 1, V, loss, None, dt, rl)

    def emb_fwd():
        wte, xe = rnd(V, C), emp(N, C)
        return lambda: B.slt_embedding_fwd(tok, w.B, w.T, w.T + 1, wte, xe, V, C, dt)

    def emb_bwd():
        dxe, dwte = rnd(N, C), emp(V, C, dtype=torch.float32)
        ews = emp(B.slt_embedding_bwd_workspace(N, V), dtype=torch.uint8)
        return lambda: B.slt_embedding_bwd(tok, w.B, w.T, w.T + 1, dxe, dwte, V, C, dt, ews)

    add("softmax_xent", xent, 2 * N * V * e + 4 * N)
    add("embedding_fwd", emb_fwd, N * (2 * C * e + 4))
    add("embedding_bwd", emb_bwd, N * (C * e + 4) + V * C * 4)
    _, n = B.slt_param_layout(B.make_config(w))
    bf = dt == B.BF16

    def adamw():
        th, gr = torch.empty(n, device="cuda").normal_(0, 0.02), torch.empty(n, device="cuda").normal_(0, 1e-3)
        m, v = torch.zeros(n, device="cuda"), torch.zeros(n, device="cuda")
        sh = emp(n, dtype=torch.int16) if bf else None
        return lambda: B.slt_adamw_step(n, th, sh, gr, m, v, 1, 1e-3, 0.9, 0.999, 1e-8, 0.1)

    def gnorm():
        gr = torch.empty(n, device="cuda").normal_(0, 1e-3)
        cws, nrm = emp(B.slt_clip_workspace_bytes(), dtype=torch.uint8), emp(2, dtype=torch.float32)
        return lambda: B.slt_clip_grad_norm(n, gr, B.NORM_L2, 1.0, nrm, nrm.data_ptr() + 4, cws)

    add("adamw", adamw, n * (30 if bf else 28))
    add("grad_norm", gnorm, 4 * n)
    return out


def measured_traffic(w, cls):
    """HBM bytes per launch of a kernel class from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary (profiles/<class>_traffic.json), scaled by
    a plain copy's counts; None when that summary is for another workload or
    for kernel sources other than the ones built now."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{cls}_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
        sha = hashlib.sha256()
        for src in rec.get("sources", ["gemm.hip"]):
            with open(os.path.join(ROOT, "scratch_llama_transformer_amd", "csrc", src), "rb") as f:
                sha.update(f.read())
    except OSError:
        return None
    if rec.get("sources_sha256") != sha.hexdigest() or rec.get("workload") != w.name:
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
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(Bs * w.T / dt, 1), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": model,
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
    ap.add_argument("--only-class", choices=["gemm_fwd", "gemm_dx", "gemm_dw", "attention_fwd", "attention_bwd"]
                    + HBM_CLASSES, default=None,
                    help="only time one kernel class of the breakdown (for hardware-counter runs) and exit")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB 5 times with slt_stream_copy (for scaling HBM byte counters) and exit")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(the data-parallel design is described, not built).", file=sys.stderr)
        sys.exit(2)

    import torch
    import slt_workloads as W
    from scratch_llama_transformer_amd import binding as B
    from scratch_llama_transformer_amd.trainer import TrainStep

    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            B.slt_stream_copy(src, dst, n, 2)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}), flush=True)
        return

    w = W.get_config(args.config)
    if args.only_class in HBM_CLASSES:
        r = hbm_classes(w, torch, max(args.kernel_reps, 1), {"copy_gbps": float("nan")}, only=args.only_class)
        r = r[args.only_class]
        print(json.dumps({"workload": w.name, "class": args.only_class, "us_per_launch": r["us_per_launch"],
                          "gbps": r["gbps"], "train": r["train"]}), flush=True)
        return
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
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    ev[0].record(s)
    for i in range(args.steps):
        ts.step(tok)
        ev[i + 1].record(s)
    ev[-1].synchronize()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[-1]) / args.steps
    per_step = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
    loss = float(ts.loss.item())
    # the step's own launches by class: PROF_STEPS more steps with the
    # library's event brackets on (kept out of the timed steps above: the
    # events add gaps between launches)
    in_step = None
    if not args.no_breakdown:
        B.slt_timing(True)
        t0 = time.perf_counter()
        for _ in range(PROF_STEPS):
            ts.step(tok)
        torch.cuda.synchronize()
        prof_ms = (time.perf_counter() - t0) * 1e3 / PROF_STEPS  # host clock, enqueue to completion
        B.slt_timing(False)
        in_step = B.slt_timing_read()
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
        "ms_per_step_median": round(per_step[len(per_step) // 2], 4),
        "ms_per_step_best": round(per_step[0], 4),
        "tokens_per_s_median": round(w.N / (per_step[len(per_step) // 2] / 1e3), 1),
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
        machine = machine_bounds(torch)
        out["machine"] = machine
        sa = kernel_classes(w, None, torch, args.kernel_reps)
        mpeak = machine["mfma_bf16_tflops"] if w.act == "bf16" else None
        # in the step: each class's bracketed launches over the profiling
        # steps, with the same algorithmic FLOPs and bytes per step
        cl = {}
        for k, v in sa.items():
            ms_tot, n = in_step[k]
            if n == 0 or ms_tot <= 0:  # no bracketed launch of the class: keep the standalone figures
                cl[k] = dict(v)
                continue
            msps = ms_tot / PROF_STEPS
            cl[k] = dict(v, ms_per_step=msps, launches=n // PROF_STEPS, avg_launch_us=ms_tot * 1e3 / max(n, 1),
                         tflops=v["flops"] / (msps / 1e3) / 1e12,
                         frac_of_peak=v["flops"] / (msps / 1e3) / 1e12 / v["peak"])
        keep = ("ms_per_step", "launches", "tflops", "frac_of_peak", "frac_of_measured", "avg_launch_us", "bytes")
        for d_ in (cl, sa):
            for v in d_.values():
                if mpeak:
                    v["frac_of_measured"] = v["tflops"] / mpeak
        out["kernels"] = {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()
                              if kk in keep} for k, v in cl.items()}
        out["kernels_from"] = (f"library event brackets around each class's launches over {PROF_STEPS} steps after "
                               f"the timed ones ({prof_ms:.4f} ms per step with the brackets on)")
        out["kernels_standalone"] = {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv)
                                         for kk, vv in v.items() if kk in keep} for k, v in sa.items()}
        out["hbm_kernels"] = hbm_classes(w, torch, max(args.kernel_reps, 5), machine)
        # the dominant kernel class of the step: the largest time per step in
        # the breakdown (MFMA classes; the HBM-bound kernels above each take
        # a smaller share)
        name = max(cl, key=lambda k: cl[k]["ms_per_step"])
        c = cl[name]
        # the roof that bounds it: HBM when its arithmetic intensity (FLOPs
        # per algorithmic byte) is below the ridge point peak FLOP/s / peak
        # HBM bytes/s, the matrix cores otherwise
        ai = c["flops"] / c["bytes"]
        ridge = c["peak"] * 1e12 / (PEAK["hbm"] * 1e9)
        kern = {"gemm_fwd": "forward-projection GEMMs (k-major x k-major)",
                "gemm_dx": "activation-gradient GEMMs dX = dY W",
                "gemm_dw": "grouped weight-gradient GEMMs dW = dY^T X",
                "attention_fwd": "causal attention forward (fl_fwd_k)",
                "attention_bwd": "causal attention backward (fl_dq_k + fl_dkdv2_k)"}[name]
        if ai >= ridge:
            ach, pk, unit, mp = c["tflops"], c["peak"], "TFLOP/s", mpeak
        else:
            ach, pk, unit, mp = c["bytes"] / (c["ms_per_step"] / 1e3) / 1e9, PEAK["hbm"], "GB/s", machine["copy_gbps"]
        out["roofline"] = {"kernel": kern, "class": name, "bound": "mfma" if ai >= ridge else "hbm",
                           "achieved": round(ach, 2), "peak": pk, "unit": unit, "frac": round(ach / pk, 4),
                           "frac_of_measured": round(ach / mp, 4) if mp else None,
                           "traffic": measured_traffic(w, name),
                           "algorithmic_bytes_per_launch": int(c["bytes"] / c["launches"]),
                           "flops_per_launch": int(c["flops"] / c["launches"]),
                           "arithmetic_intensity": round(ai, 1), "ridge": round(ridge, 1),
                           "tflops": round(c["tflops"], 2),
                           "avg_launch_us": round(c["avg_launch_us"], 2), "launches_per_step": c["launches"]}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
