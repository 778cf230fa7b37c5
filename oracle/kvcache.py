"""Plain float64 CPU oracle for the key/value-cache forward (prefill and
single-token decode).

TEST INFRASTRUCTURE: imported only by tests, the smoke check and the
benchmark's CPU-baseline leg.  It shares no code with the GPU library.

Sources (page title, section):
  * randyGPT, "Features": a true KV cache -- the prompt is run once (prefill)
    and every further token costs one single-token forward.
  * Transformer in Rust, "CodeGen Inference Pipeline": prefill populates the
    cache; each generated token runs a single-token forward and appends its
    keys and values to the cache.  "Key Features": the KV cache serves
    autoregressive generation without recomputation.
  * strata, model table: KV-cache parity with pre-rotated keys for the modern
    (RoPE, RMSNorm, SwiGLU, GQA) decoder; "rules": the KV-cache decoder must
    equal the full forward pass (to about 1e-9 at float64).

Readings (the pages give no more than the above):
  * The cache holds, per layer, the keys after RoPE at their absolute
    positions ("pre-rotated keys") and the values, [B, Hkv, Tmax, d].
  * A call takes the next Tq tokens of every sequence (the same count for all
    sequences) at positions pos0 .. pos0 + Tq - 1, pos0 being the number of
    positions already cached.  Prefill is pos0 = 0; decode is Tq = 1.
  * Query i of the call attends to cached positions 0 .. pos0 + i, its own
    included, exactly as row pos0 + i of the causal full forward does.
  * Precision: for bf16 models the cache is an activation stored in memory, so
    the rotated keys are rounded to bf16 when written (the values already are,
    being part of the rounded projection).  Everything else follows the full
    forward's storage rounding.
"""
from __future__ import annotations

import math

import numpy as np

from .model import (store_fn, embedding_fwd, rmsnorm_fwd, layernorm_fwd, rope_tables, rope_apply,
                    swiglu_fwd, gelu_fwd, _expand_kv)

__all__ = ["kv_cache_new", "forward_cached"]


def kv_cache_new(cfg, B, Tmax):
    """An empty cache for B sequences of up to Tmax positions."""
    d = cfg.C // cfg.H
    return {"len": 0, "Tmax": Tmax, "B": B,
            "k": [np.zeros((B, cfg.Hkv, Tmax, d)) for _ in range(cfg.L)],
            "v": [np.zeros((B, cfg.Hkv, Tmax, d)) for _ in range(cfg.L)]}


def _cached_attention(q, kc, vc, pos0):
    """q [B, H, Tq, d] (rotated) against cached keys and values
    [B, Hkv, L, d], L = pos0 + Tq: query i sees positions j <= pos0 + i.
    Stable softmax (row maximum subtracted), scale 1/sqrt(d)."""
    B, H, Tq, d = q.shape
    L = kc.shape[2]
    s = np.matmul(q, np.swapaxes(_expand_kv(kc, H), -1, -2)) / math.sqrt(d)
    allowed = np.arange(L)[None, :] <= (pos0 + np.arange(Tq))[:, None]
    s = np.where(allowed, s, -np.inf)
    e = np.exp(s - np.max(s, axis=-1, keepdims=True))
    p = e / np.sum(e, axis=-1, keepdims=True)
    return np.matmul(p, _expand_kv(vc, H))


def forward_cached(cfg, params, cache, ids, jitter=0.0, seed=0):
    """Run the next Tq tokens of each sequence through the model.

    ids: int [B, Tq].  Their positions are cache["len"] .. cache["len"]+Tq-1.
    Each layer rotates q and k at those absolute positions, writes the rotated
    keys and the values into the cache, and attends over every cached
    position up to the query's own.  Returns the logits [B, Tq, V] (rounded
    like the full forward's) and advances cache["len"] by Tq.

    jitter/seed: as for the full forward (see store_fn), applied to the stored
    activations only; the bf16 copy of the weights is the plain rounding.
    With jitter = 2^-24 this is another valid bf16 computation of the same
    call, whose distance from the plain one measures the spread that
    storage-rounding flips cause."""
    S = store_fn(cfg.act, jitter, seed)
    W = {k: store_fn(cfg.act)(np.asarray(v, np.float64)) for k, v in params.items()}
    ids = np.asarray(ids)
    B, Tq = ids.shape
    pos0 = cache["len"]
    L = pos0 + Tq
    if B != cache["B"] or L > cache["Tmax"]:
        raise ValueError("batch or length does not fit the cache")
    C, H, Hkv, d, R = cfg.C, cfg.H, cfg.Hkv, cfg.C // cfg.H, cfg.R
    qd, kd = H * d, Hkv * d
    cos, sin = rope_tables(L, R, cfg.base)
    cos, sin = cos[pos0:], sin[pos0:]          # angles of the new positions

    def heads(x2d, nh):
        return x2d.reshape(B, Tq, nh, d).transpose(0, 2, 1, 3)

    x = embedding_fwd(W["wte"], ids.reshape(-1))
    for l in range(cfg.L):
        p = f"h{l}."
        if cfg.block == "llama":
            n1 = S(rmsnorm_fwd(x, W[p + "attn_norm"], cfg.eps)[0])
        else:
            n1 = S(layernorm_fwd(x, W[p + "ln_g"], W[p + "ln_b"], cfg.eps)[0])
        qkv = S(n1 @ W[p + "qkvw"].T)
        q = rope_apply(heads(qkv[:, :qd], H), cos, sin, R, cfg.rope_mode)
        k = rope_apply(heads(qkv[:, qd:qd + kd], Hkv), cos, sin, R, cfg.rope_mode)
        v = heads(qkv[:, qd + kd:], Hkv)
        cache["k"][l][:, :, pos0:L] = S(k)
        cache["v"][l][:, :, pos0:L] = S(v)
        o4 = _cached_attention(q, cache["k"][l][:, :, :L], cache["v"][l][:, :, :L], pos0)
        o = S(o4.transpose(0, 2, 1, 3).reshape(B * Tq, qd))
        if cfg.block == "llama":
            x = S(x + o @ W[p + "w_o"].T)
            n2 = S(rmsnorm_fwd(x, W[p + "mlp_norm"], cfg.eps)[0])
            h = S(swiglu_fwd(S(n2 @ W[p + "w1"].T), S(n2 @ W[p + "w3"].T)))
            x = S(x + h @ W[p + "w2"].T)
        else:
            u = S(gelu_fwd(S(n1 @ W[p + "fc_in"].T)))
            x = S(x + np.concatenate([o, u], axis=1) @ W[p + "w_out"].T)
    if cfg.block == "llama":
        nf = S(rmsnorm_fwd(x, W["norm_f"], cfg.eps)[0])
    else:
        nf = S(layernorm_fwd(x, W["lnf_g"], W["lnf_b"], cfg.eps)[0])
    z = S(nf @ W["lm_head"].T)
    cache["len"] = L
    return z.reshape(B, Tq, cfg.V)
