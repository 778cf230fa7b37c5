"""Workload definitions and seeded synthetic inputs for one training step.

This module holds the five model configurations, the list of parameter tensors
each configuration has (names, shapes, how they are initialised) and seeded
generators for token ids and initial weights.  It holds none of the step's
arithmetic: both the CPU oracle and the GPU library receive what it produces.

Model family (Hephaistos, "Architecture at a glance"; strata, the GPT-2 to
modern table; Transformer in Rust, "CodeGen: Parallel Sub-Block Design"):
a bias-free decoder with token embedding, per-block norm/attention/MLP, a final
norm and an untied lm_head.
"""
from __future__ import annotations

import dataclasses
import numpy as np

__all__ = ["Config", "CONFIGS", "get_config", "param_specs", "n_params",
           "make_tokens", "make_params", "uniform_tokens", "zipf_tokens"]


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    V: int            # vocabulary
    C: int            # n_embd
    H: int            # query heads
    Hkv: int          # key/value heads (GQA when Hkv < H)
    L: int            # layers
    T: int            # sequence length
    B: int            # batch
    F: int            # MLP hidden width
    R: int            # rotary dims per head (R <= d)
    rope_mode: str    # "half" (rotate-half pairs j, j+R/2) | "pairs" (even-odd 2j, 2j+1)
    block: str        # "llama" (RMSNorm, SwiGLU, sequential) | "parallel" (LayerNorm, GELU, GPT-J style)
    act: str          # storage type of activations and compute weights: "f32" | "bf16"
    tokens: str       # "uniform" | "zipf"
    scale_out: bool   # scale output projections by 1/sqrt(2L) at init
    eps: float = 1e-5
    base: float = 10000.0
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    adam_eps: float = 1e-8
    wd: float = 0.1
    init_std: float = 0.02
    dropout: float = 0.0      # inverted-dropout probability (training forward only); 0 = off
    dropout_seed: int = 0     # key of the counter-based generator that draws the masks

    @property
    def d(self) -> int:
        return self.C // self.H

    @property
    def N(self) -> int:
        return self.B * self.T

    def with_(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


CONFIGS = [
    Config("cfg1_tiny_f32", V=27, C=16, H=4, Hkv=4, L=1, T=16, B=1, F=42, R=4,
           rope_mode="half", block="llama", act="f32", tokens="uniform", scale_out=False),
    Config("cfg2_llama_f32", V=500, C=256, H=8, Hkv=8, L=6, T=256, B=64, F=682, R=32,
           rope_mode="half", block="llama", act="f32", tokens="uniform", scale_out=True),
    Config("cfg3_llama_bf16", V=4096, C=384, H=8, Hkv=8, L=8, T=256, B=64, F=1024, R=48,
           rope_mode="half", block="llama", act="bf16", tokens="zipf", scale_out=False),
    Config("cfg4_gqa_bf16", V=32000, C=1024, H=16, Hkv=4, L=16, T=1024, B=16, F=2816, R=64,
           rope_mode="half", block="llama", act="bf16", tokens="uniform", scale_out=False),
    Config("cfg5_parallel_bf16", V=51200, C=1024, H=16, Hkv=16, L=20, T=2048, B=8, F=4096, R=32,
           rope_mode="pairs", block="parallel", act="bf16", tokens="uniform", scale_out=False),
]


def get_config(i: int) -> Config:
    """1-based index into CONFIGS."""
    return CONFIGS[i - 1]


def param_specs(cfg: Config):
    """Ordered parameter tensors: list of (name, shape, init) with init in
    {"normal", "normal_out", "ones", "zeros"}.  Matrices are stored [out, in].

    Llama block: attn_norm, qkvw, w_o, mlp_norm, w1, w3, w2 (w1 and w3 adjacent,
    so [w1; w3] is one [2F, C] matrix in the flat buffer).
    Parallel block: ln_g, ln_b, qkvw, fc_in (adjacent: one [3C+F, C] matrix),
    w_out = [W_o | W_fc2] as one [C, C+F] matrix.
    """
    C, F, d = cfg.C, cfg.F, cfg.d
    qkv_rows = (cfg.H + 2 * cfg.Hkv) * d
    specs = [("wte", (cfg.V, C), "normal")]
    for l in range(cfg.L):
        p = f"h{l}."
        if cfg.block == "llama":
            specs += [
                (p + "attn_norm", (C,), "ones"),
                (p + "qkvw", (qkv_rows, C), "normal"),
                (p + "w_o", (C, cfg.H * d), "normal_out"),
                (p + "mlp_norm", (C,), "ones"),
                (p + "w1", (F, C), "normal"),
                (p + "w3", (F, C), "normal"),
                (p + "w2", (C, F), "normal_out"),
            ]
        else:
            specs += [
                (p + "ln_g", (C,), "ones"),
                (p + "ln_b", (C,), "zeros"),
                (p + "qkvw", (qkv_rows, C), "normal"),
                (p + "fc_in", (F, C), "normal"),
                (p + "w_out", (C, cfg.H * d + F), "normal_out"),
            ]
    if cfg.block == "llama":
        specs += [("norm_f", (C,), "ones")]
    else:
        specs += [("lnf_g", (C,), "ones"), ("lnf_b", (C,), "zeros")]
    specs += [("lm_head", (cfg.V, C), "normal")]
    return specs


def n_params(cfg: Config) -> int:
    return int(sum(int(np.prod(s)) for _, s, _ in param_specs(cfg)))


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(stream)])))


def uniform_tokens(seed: int, B: int, T1: int, V: int) -> np.ndarray:
    """int32 [B, T1] ids uniform on [0, V)."""
    return _rng(seed, 1).integers(0, V, size=(B, T1), dtype=np.int64).astype(np.int32)


def zipf_tokens(seed: int, B: int, T1: int, V: int, s: float = 1.1) -> np.ndarray:
    """int32 [B, T1] ids with P(k) proportional to (k+1)^-s on [0, V), drawn by
    inverse CDF from seeded uniforms (a stand-in for natural-text rank/frequency)."""
    w = np.arange(1, V + 1, dtype=np.float64) ** (-s)
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    u = _rng(seed, 1).random(size=(B, T1))
    ids = np.searchsorted(cdf, u, side="right")
    return np.minimum(ids, V - 1).astype(np.int32)


def make_tokens(cfg: Config, seed: int, B: int | None = None) -> np.ndarray:
    """int32 [B, T+1]: inputs are [:, :T], next-token targets are [:, 1:]."""
    B = cfg.B if B is None else B
    if cfg.tokens == "zipf":
        return zipf_tokens(seed, B, cfg.T + 1, cfg.V)
    return uniform_tokens(seed, B, cfg.T + 1, cfg.V)


def make_params(cfg: Config, seed: int) -> dict:
    """Named fp32 master weights: matrices N(0, std^2) (output projections times
    1/sqrt(2L) when cfg.scale_out), gains 1, LayerNorm shifts 0."""
    out = {}
    for i, (name, shape, init) in enumerate(param_specs(cfg)):
        if init == "ones":
            out[name] = np.ones(shape, np.float32)
        elif init == "zeros":
            out[name] = np.zeros(shape, np.float32)
        else:
            std = cfg.init_std
            if init == "normal_out" and cfg.scale_out:
                std = std / np.sqrt(2.0 * cfg.L)
            out[name] = (_rng(seed, 100 + i).standard_normal(size=shape) * std).astype(np.float32)
    return out
