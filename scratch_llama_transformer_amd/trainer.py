"""Device buffers for one model and the three step calls.

Holds the fp32 master weights, their bf16 copy (bf16 configurations), the
AdamW moments, the gradient buffer, the activation arena and the scratch area,
all allocated with torch on the current GPU, and calls the library's
slt_forward_loss / slt_backward / slt_adamw_step on the current stream.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as B


class TrainStep:
    def __init__(self, wcfg, params: dict | None = None, seed: int = 0, device: str = "cuda", clip=None):
        """clip: None, or (kind, max_norm) with kind "l2" or "linf": the
        gradient is scaled by the global-norm clipping factor before AdamW."""
        self.w = wcfg
        self.clip = clip
        self.cfg = B.make_config(wcfg)
        B.slt_validate(self.cfg)
        self.layout, self.n = B.slt_param_layout(self.cfg)
        self.device = torch.device(device)
        self.bf16 = wcfg.act == "bf16"
        f32 = dict(dtype=torch.float32, device=self.device)
        self.master = torch.zeros(self.n, **f32)
        if params is not None:
            self.load_params(params)
        else:
            out_scale = float(1.0 / np.sqrt(2.0 * wcfg.L)) if wcfg.scale_out else 1.0
            B.slt_model_init(self.cfg, seed, wcfg.init_std, out_scale, self.master)
        self.shadow = torch.empty(self.n, dtype=torch.int16, device=self.device) if self.bf16 else None
        self.m = torch.zeros(self.n, **f32)
        self.v = torch.zeros(self.n, **f32)
        self.grads = torch.empty(self.n, **f32)
        act, scr = B.slt_workspace_bytes(self.cfg)
        self.acts = torch.empty(act, dtype=torch.uint8, device=self.device)
        self.scratch = torch.empty(scr, dtype=torch.uint8, device=self.device)
        self.loss = torch.zeros(1, **f32)
        self.gnorm = torch.zeros(2, **f32)  # [norm, clipping factor]
        self.clip_ws = torch.empty(B.slt_clip_workspace_bytes(), dtype=torch.uint8, device=self.device)
        self.t = 0
        self.refresh_shadow()

    # -- parameters ---------------------------------------------------------
    def load_params(self, params: dict) -> None:
        host = np.zeros(self.n, np.float32)
        for t in self.layout:
            a = np.asarray(params[t["name"]], np.float32).reshape(-1)
            if a.size != t["numel"]:
                raise ValueError(f"{t['name']}: {a.size} elements, layout says {t['numel']}")
            host[t["offset"]:t["offset"] + t["numel"]] = a
        self.master.copy_(torch.from_numpy(host))

    def unpack(self, flat: torch.Tensor) -> dict:
        host = flat.detach().float().cpu().numpy()
        return {t["name"]: host[t["offset"]:t["offset"] + t["numel"]].reshape(
            (t["cols"],) if t["rows"] == 1 else (t["rows"], t["cols"])) for t in self.layout}

    def refresh_shadow(self) -> None:
        if self.bf16:
            B.slt_cast_bf16(self.master, self.shadow, self.n)

    @property
    def compute_params(self) -> torch.Tensor:
        return self.shadow if self.bf16 else self.master

    # -- the step -----------------------------------------------------------
    def forward(self, tokens: torch.Tensor) -> None:
        B.slt_forward_loss(self.cfg, self.compute_params, tokens, self.acts, self.scratch, self.loss)

    def backward(self, tokens: torch.Tensor) -> None:
        B.slt_backward(self.cfg, self.compute_params, tokens, self.acts, self.scratch, self.grads)

    def clip_grads(self) -> None:
        kind, max_norm = self.clip
        B.slt_clip_grad_norm(self.n, self.grads, B.NORM_L2 if kind == "l2" else B.NORM_LINF, float(max_norm),
                             self.gnorm, self.gnorm.data_ptr() + 4, self.clip_ws)

    def adamw(self, lr=None, wd=None) -> None:
        self.t += 1
        w = self.w
        scale = None
        if self.clip is not None:
            self.clip_grads()
            scale = self.gnorm.data_ptr() + 4
        B.slt_adamw_step(self.n, self.master, self.shadow, self.grads, self.m, self.v, self.t,
                         w.lr if lr is None else lr, w.beta1, w.beta2, w.adam_eps, w.wd if wd is None else wd,
                         grad_scale=scale)

    def next_masks(self) -> None:
        """Moves the dropout key to the next value, so that the following
        forward draws fresh masks (a forward and its backward must share one
        key: the backward regenerates the forward's masks from it)."""
        self.cfg.dropout_seed = (self.cfg.dropout_seed + 1) & 0xFFFFFFFFFFFFFFFF

    def backward_adamw(self, tokens: torch.Tensor, lr=None, wd=None) -> None:
        """The backward with AdamW folded in (slt_backward_adamw): each
        layer's update runs as soon as its gradients are final; the same
        result as backward() then adamw() without clipping."""
        self.t += 1
        w = self.w
        B.slt_backward_adamw(self.cfg, self.compute_params, tokens, self.acts, self.scratch, self.grads, self.master,
                             self.shadow, self.m, self.v, self.t, w.lr if lr is None else lr, w.beta1, w.beta2,
                             w.adam_eps, w.wd if wd is None else wd)

    fuse_adamw = True  # step() folds AdamW into the backward when there is no clipping

    def step(self, tokens: torch.Tensor) -> None:
        self.forward(tokens)
        if self.clip is None and self.fuse_adamw:
            self.backward_adamw(tokens)
        else:
            self.backward(tokens)
            self.adamw()
        if self.cfg.dropout > 0:
            self.next_masks()

    def accumulate(self, micro_tokens) -> float:
        """Gradient of the mean loss over several equal micro-batches, each run
        through the arena in turn (this object's batch size is the
        micro-batch size): grads = sum_s (1/S) grad_s, and the mean loss
        sum_s (1/S) loss_s kept on the device by the library.  Returns the
        mean loss (one host synchronisation)."""
        S = len(micro_tokens)
        self.grads.zero_()
        mean_loss = torch.zeros(1, dtype=torch.float32, device=self.device)
        for tok in micro_tokens:
            self.forward(tok)
            B.slt_backward_accumulate(self.cfg, self.compute_params, tok, self.acts, self.scratch, self.grads,
                                      1.0 / S, self.loss, mean_loss)
            if self.cfg.dropout > 0:
                self.next_masks()
        return float(mean_loss.item())


class CachedForward:
    """Key/value cache and workspace for incremental forwards of one model:
    ``run(tokens)`` feeds the next Tq tokens of each of the B sequences
    (prefill when the cache is empty, then single tokens) through
    slt_forward_cached and returns their logits.  ``params`` is the compute
    copy of the flat parameters (a TrainStep's ``compute_params``)."""

    def __init__(self, wcfg, params: torch.Tensor, batch: int, Tmax: int, Tq_max: int, device: str = "cuda"):
        self.w = wcfg
        self.cfg = B.make_config(wcfg)
        B.slt_validate(self.cfg)
        self.params = params
        self.B, self.Tmax, self.Tq_max = batch, Tmax, Tq_max
        cache_bytes, ws_bytes = B.slt_kv_cache_bytes(self.cfg, batch, Tq_max, Tmax)
        self.cache = torch.empty(cache_bytes, dtype=torch.uint8, device=device)
        self.ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=device)
        self.dtype = torch.bfloat16 if wcfg.act == "bf16" else torch.float32
        self.pos = 0

    def run(self, tokens: torch.Tensor, last_only: bool = False) -> torch.Tensor:
        """tokens: int32 [B, Tq] on the device.  Returns logits [B, Tq, V]
        (or [B, V] with last_only) in the activation dtype."""
        Bn, Tq = tokens.shape
        if Bn != self.B or Tq > self.Tq_max:
            raise ValueError("batch or chunk length does not fit this cache")
        rows = Bn if last_only else Bn * Tq
        z = torch.empty(rows, self.w.V, dtype=self.dtype, device=self.cache.device)
        B.slt_forward_cached(self.cfg, self.params, tokens, Bn, Tq, tokens.stride(0), self.pos, self.cache,
                             self.Tmax, self.ws, last_only, z, self.w.V)
        self.pos += Tq
        return z if last_only else z.view(Bn, Tq, self.w.V)
