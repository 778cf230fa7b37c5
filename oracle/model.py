"""Plain float64 CPU oracle for one training step: forward, hand-written
backward and AdamW.

TEST INFRASTRUCTURE: imported only by tests, the smoke check and the
benchmark's CPU-baseline leg.  It shares no code with the GPU library.

Sources (page title, section):
  * Hephaistos, "Architecture at a glance": pre-norm block x + Attn(RMSNorm(x)),
    then x + SwiGLU(RMSNorm(x)); RMSNorm without centring or bias; RoPE on q and
    k inside attention; causal multi-head attention with a stable softmax;
    SwiGLU (silu(x W1) * x W3) W2; untied lm_head; AdamW with decoupled decay
    and bias correction.
  * Hephaistos, "Design notes": flat parameter buffers, an activation arena
    that caches what the backward needs (rstd, pre-SiLU gate, ...), backward as
    a straight reverse walk.
  * MicroGPT in Rust, "RMSNorm": scale = (mean square + 1e-5)^(-1/2).
  * strata, capability tables: backward rules for matmul, LayerNorm, RMSNorm,
    GELU, SiLU, embedding, cross-entropy and causal attention with independent
    n_head / n_kv_head and optional RoPE; AdamW decoupled and bias-corrected.
  * Transformer in Rust, "CodeGen: Parallel Sub-Block Design": one LayerNorm
    feeds attention and the FFN, both outputs join the residual in one add;
    "Key Features": RoPE with even-odd pair rotation; "Model Configurations":
    rotary_dim 32 of head dim 64.
  * randyGPT, "Training (Metal GPU path)": cross-entropy over all positions.

Readings taken where the pages are silent are stated next to the code.

Precision model.  For fp32 configurations the oracle runs in float64 without
rounding.  For bf16 configurations it applies ``bf16_round`` at every point
where the GPU path stores a bf16 tensor in memory (weights' compute copy,
residual stream, norm outputs, projections -- q and k after RoPE --, attention
output, MLP activations, logits, and every activation gradient); statistics,
weight gradients, optimizer state and the loss stay float64.  Values a GPU
kernel rounds only inside registers (probabilities, score gradients) are not
rounded here.
"""
from __future__ import annotations

import math
import numpy as np

from .dropout import dropout_multiplier

__all__ = [
    "bf16_round", "store_fn",
    "embedding_fwd", "embedding_bwd",
    "rmsnorm_fwd", "rmsnorm_bwd", "layernorm_fwd", "layernorm_bwd",
    "rope_tables", "rope_apply",
    "attention_fwd", "attention_bwd",
    "swiglu_fwd", "swiglu_bwd", "gelu_fwd", "gelu_bwd",
    "cross_entropy", "adamw", "grad_norm", "clip_scale",
    "forward", "backward", "train_step", "decay_mask_like", "accumulated_grads",
]


# ----------------------------------------------------------------------------
# bf16 storage rounding (IEEE-754 binary16-brain: 8 significant bits, the
# exponent range of binary32), round to nearest, ties to even.
# ----------------------------------------------------------------------------
_BF16_MIN_NORMAL = 2.0 ** -126
_BF16_SUBNORMAL_STEP = 2.0 ** -133
_BF16_OVERFLOW = 2.0 ** 128


def bf16_round(x):
    """Round float64 values to the nearest bfloat16 value (ties to even).

    Normal range: keep 8 significant bits.  Below 2^-126 the grid is the
    fixed subnormal spacing 2^-133.  Results of magnitude 2^128 or more are
    infinite.  NaN propagates."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                       # x = m * 2^e, 0.5 <= |m| < 1
    out = np.ldexp(np.rint(m * 256.0), e - 8)   # rint: ties to even
    small = np.abs(x) < _BF16_MIN_NORMAL
    if np.any(small):
        out = np.where(small, np.rint(x / _BF16_SUBNORMAL_STEP) * _BF16_SUBNORMAL_STEP, out)
    big = np.abs(out) >= _BF16_OVERFLOW
    if np.any(big):
        out = np.where(big, np.copysign(np.inf, x), out)
    return out


def _identity(x):
    return x


def store_fn(act: str, jitter: float = 0.0, seed: int = 0):
    """The storage rounding for an activation type ("bf16" or "f32").

    jitter > 0 multiplies every value by (1 + jitter * N(0, 1)) before it is
    rounded: with jitter = 2^-24 this mimics another fp32 summation order in
    front of each bf16 store, so the spread between a plain and a jittered run
    measures how far two valid bf16 computations of the same step may differ."""
    if act != "bf16":
        return _identity
    if jitter == 0.0:
        return bf16_round
    rng = np.random.default_rng(seed)

    def jittered(x):
        x = np.asarray(x, np.float64)
        return bf16_round(x * (1.0 + jitter * rng.standard_normal(x.shape)))
    return jittered


# ----------------------------------------------------------------------------
# Embedding (Hephaistos, "Architecture at a glance": token embedding, no
# position table; strata: embedding backward rule)
# ----------------------------------------------------------------------------
def embedding_fwd(wte, ids):
    """x[i] = wte[ids[i]].  ids: int array [N]."""
    return np.asarray(wte, np.float64)[np.asarray(ids)]


def embedding_bwd(dx, ids, V):
    """dwte[v] = sum of dx[i] over the positions i with ids[i] == v; rows of
    ids that never occur are exactly zero."""
    dx = np.asarray(dx, np.float64)
    out = np.zeros((V, dx.shape[1]), np.float64)
    np.add.at(out, np.asarray(ids), dx)
    return out


# ----------------------------------------------------------------------------
# Norms
# ----------------------------------------------------------------------------
def rmsnorm_fwd(x, g, eps):
    """RMSNorm (Hephaistos, "Architecture at a glance"; MicroGPT in Rust,
    "RMSNorm"): r = (mean_c x_c^2 + eps)^(-1/2), y = x * r * g.
    Reading: the mean runs over the C channels.  Returns (y, r)."""
    x = np.asarray(x, np.float64)
    ms = np.mean(x * x, axis=-1)
    r = 1.0 / np.sqrt(ms + eps)
    return x * r[..., None] * np.asarray(g, np.float64), r


def rmsnorm_bwd(x, g, r, dy):
    """Backward of rmsnorm_fwd, derived from y_c = g_c x_c r(x):
    with xh = x r and dxh = dy * g,  dx = r (dxh - xh * mean_c(dxh * xh)),
    dg = sum over rows of dy * xh.  Returns (dx, dg)."""
    x = np.asarray(x, np.float64)
    g = np.asarray(g, np.float64)
    dy = np.asarray(dy, np.float64)
    xh = x * r[..., None]
    dxh = dy * g
    dx = r[..., None] * (dxh - xh * np.mean(dxh * xh, axis=-1, keepdims=True))
    dg = np.sum((dy * xh).reshape(-1, x.shape[-1]), axis=0)
    return dx, dg


def layernorm_fwd(x, gamma, beta, eps):
    """LayerNorm (strata, GPT-2 reference; Transformer in Rust, "CodeGen:
    Parallel Sub-Block Design"): mu = mean x, var = mean (x - mu)^2 (biased),
    r = (var + eps)^(-1/2), y = (x - mu) r gamma + beta.  Reading: eps = 1e-5
    as for RMSNorm.  Returns (y, mu, r)."""
    x = np.asarray(x, np.float64)
    mu = np.mean(x, axis=-1)
    xc = x - mu[..., None]
    var = np.mean(xc * xc, axis=-1)
    r = 1.0 / np.sqrt(var + eps)
    return xc * r[..., None] * np.asarray(gamma, np.float64) + np.asarray(beta, np.float64), mu, r


def layernorm_bwd(x, gamma, mu, r, dy):
    """Backward of layernorm_fwd: with xh = (x - mu) r and dxh = dy * gamma,
    dx = r (dxh - mean(dxh) - xh mean(dxh * xh)); dgamma = sum dy * xh,
    dbeta = sum dy.  Returns (dx, dgamma, dbeta)."""
    x = np.asarray(x, np.float64)
    dy = np.asarray(dy, np.float64)
    xh = (x - mu[..., None]) * r[..., None]
    dxh = dy * np.asarray(gamma, np.float64)
    dx = r[..., None] * (dxh - np.mean(dxh, axis=-1, keepdims=True)
                         - xh * np.mean(dxh * xh, axis=-1, keepdims=True))
    C = x.shape[-1]
    dgamma = np.sum((dy * xh).reshape(-1, C), axis=0)
    dbeta = np.sum(dy.reshape(-1, C), axis=0)
    return dx, dgamma, dbeta


# ----------------------------------------------------------------------------
# RoPE (Hephaistos, "Architecture at a glance" and the GGUF export note:
# rotate-half layout in training; Transformer in Rust, "Key Features": even-odd
# pairs; "Model Configurations": rotary_dim 32; strata: relative-position law)
# ----------------------------------------------------------------------------
def rope_tables(T, R, base):
    """cos and sin of the angles pos * theta_j, theta_j = base^(-2j/R), for
    pos in [0, T) and j in [0, R/2).  Float64 [T, R/2]."""
    j = np.arange(R // 2, dtype=np.float64)
    theta = base ** (-2.0 * j / R)
    ang = np.arange(T, dtype=np.float64)[:, None] * theta[None, :]
    return np.cos(ang), np.sin(ang)


def _rope_pairs(R, mode):
    h = R // 2
    if mode == "half":      # pair (j, j + R/2)
        return np.arange(h), np.arange(h) + h
    if mode == "pairs":     # pair (2j, 2j + 1)
        return 2 * np.arange(h), 2 * np.arange(h) + 1
    raise ValueError(mode)


def rope_apply(u, cos, sin, R, mode, inverse=False):
    """Rotate each pair (a, b) of the first R dims of u[..., T, d] by the angle
    of its position: (a, b) -> (a cos - b sin, a sin + b cos).  Dims >= R are
    unchanged.  inverse=True applies the transpose (rotation by -angle), which
    is the backward of the rotation."""
    u = np.asarray(u, np.float64)
    out = u.copy()
    ia, ib = _rope_pairs(R, mode)
    s = -sin if inverse else sin
    a, b = u[..., ia], u[..., ib]
    out[..., ia] = a * cos - b * s
    out[..., ib] = a * s + b * cos
    return out


# ----------------------------------------------------------------------------
# Causal attention (Hephaistos, "Architecture at a glance"; strata: fused causal
# attention with independent n_head / n_kv_head)
# ----------------------------------------------------------------------------
def _expand_kv(k, H):
    """Query head h reads KV head floor(h * Hkv / H)."""
    Hkv = k.shape[1]
    return np.repeat(k, H // Hkv, axis=1)


def _causal_scores(q, k):
    d = q.shape[-1]
    T = q.shape[-2]
    s = np.matmul(q, np.swapaxes(_expand_kv(k, q.shape[1]), -1, -2)) / math.sqrt(d)
    mask = np.tril(np.ones((T, T), dtype=bool))
    return np.where(mask, s, -np.inf)


def attention_fwd(q, k, v, drop=None):
    """q [B,H,T,d], k and v [B,Hkv,T,d] (already rotated).
    s_ij = q_i . k_j / sqrt(d) for j <= i; p_i = softmax(s_i) computed after
    subtracting the row maximum; o_i = sum_j p_ij m_ij v_j, where m is the
    attention-weight dropout multiplier [B,H,T,T] (Hephaistos, "Architecture
    at a glance": dropout on the attention weights; m = 1 without dropout).
    Returns (o [B,H,T,d], lse [B,H,T] = log sum_j exp(s_ij))."""
    q = np.asarray(q, np.float64)
    s = _causal_scores(q, np.asarray(k, np.float64))
    mx = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - mx)
    den = np.sum(e, axis=-1, keepdims=True)
    p = e / den
    if drop is not None:
        p = p * drop
    o = np.matmul(p, _expand_kv(np.asarray(v, np.float64), q.shape[1]))
    return o, (mx + np.log(den))[..., 0]


def attention_bwd(q, k, v, do, drop=None):
    """Backward of attention_fwd, recomputing p.  With the dropout multiplier
    m (ones without dropout): dp_ij = m_ij (do_i . v_j);
    ds_ij = p_ij (dp_ij - sum_l p_il dp_il); dq_i = sum_j ds_ij k_j / sqrt(d);
    dk_j = sum_i ds_ij q_i / sqrt(d); dv_j = sum_i p_ij m_ij do_i.  dk and dv
    of a KV head sum over the query heads that read it.  Returns (dq, dk, dv)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    B, H, T, d = q.shape
    Hkv = k.shape[1]
    s = _causal_scores(q, k)
    mx = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - mx)
    p = e / np.sum(e, axis=-1, keepdims=True)
    ke, ve = _expand_kv(k, H), _expand_kv(v, H)
    dp = np.matmul(do, np.swapaxes(ve, -1, -2))
    pm = p
    if drop is not None:
        dp = dp * drop
        pm = p * drop
    ds = p * (dp - np.sum(p * dp, axis=-1, keepdims=True))
    scale = 1.0 / math.sqrt(d)
    dq = np.matmul(ds, ke) * scale
    dke = np.matmul(np.swapaxes(ds, -1, -2), q) * scale
    dve = np.matmul(np.swapaxes(pm, -1, -2), do)
    rep = H // Hkv
    dk = dke.reshape(B, Hkv, rep, T, d).sum(axis=2)
    dv = dve.reshape(B, Hkv, rep, T, d).sum(axis=2)
    return dq, dk, dv


# ----------------------------------------------------------------------------
# MLP activations
# ----------------------------------------------------------------------------
def _sigmoid(a):
    return 0.5 * (1.0 + np.tanh(0.5 * a))


def swiglu_fwd(a, b):
    """SwiGLU gate (Hephaistos, "Architecture at a glance"): h = silu(a) * b
    with silu(a) = a * sigmoid(a)."""
    a = np.asarray(a, np.float64)
    return a * _sigmoid(a) * np.asarray(b, np.float64)


def swiglu_bwd(a, b, dh):
    """db = dh * silu(a); da = dh * b * sigmoid(a) * (1 + a (1 - sigmoid(a)))."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    dh = np.asarray(dh, np.float64)
    sg = _sigmoid(a)
    return dh * b * sg * (1.0 + a * (1.0 - sg)), dh * a * sg


_GELU_K = math.sqrt(2.0 / math.pi)
_GELU_C = 0.044715


def gelu_fwd(a):
    """GELU, tanh form (reading: the pages name GELU without its formula; the
    GPT-2 / CodeGen family uses 0.5 a (1 + tanh(sqrt(2/pi)(a + 0.044715 a^3))))."""
    a = np.asarray(a, np.float64)
    return 0.5 * a * (1.0 + np.tanh(_GELU_K * (a + _GELU_C * a ** 3)))


def gelu_bwd(a, du):
    """d/da of gelu_fwd times du."""
    a = np.asarray(a, np.float64)
    t = np.tanh(_GELU_K * (a + _GELU_C * a ** 3))
    dt = (1.0 - t * t) * _GELU_K * (1.0 + 3.0 * _GELU_C * a * a)
    return np.asarray(du, np.float64) * (0.5 * (1.0 + t) + 0.5 * a * dt)


# ----------------------------------------------------------------------------
# Cross-entropy over all positions (randyGPT, "Training (Metal GPU path)";
# Hephaistos, "What you'll see": untrained loss close to ln V, a per-token mean)
# ----------------------------------------------------------------------------
def cross_entropy(z, y):
    """z [N, V] logits, y [N] targets.  loss = mean_i (logsumexp(z_i) - z_i[y_i]);
    dz = (softmax(z_i) - onehot(y_i)) / N.  Returns (loss, dz, lse)."""
    z = np.asarray(z, np.float64)
    y = np.asarray(y)
    N = z.shape[0]
    mx = np.max(z, axis=1, keepdims=True)
    lse = (mx + np.log(np.sum(np.exp(z - mx), axis=1, keepdims=True)))[:, 0]
    rows = np.arange(N)
    loss = float(np.mean(lse - z[rows, y]))
    dz = np.exp(z - lse[:, None])
    dz[rows, y] -= 1.0
    return loss, dz / N, lse


# ----------------------------------------------------------------------------
# AdamW (Hephaistos, "Architecture at a glance": decoupled weight decay and
# bias correction; strata: AdamW decoupled, bias-corrected)
# ----------------------------------------------------------------------------
def adamw(theta, g, m, v, t, lr, beta1, beta2, eps, wd, decay=None):
    """One AdamW update at step t >= 1:
    m <- b1 m + (1-b1) g;  v <- b2 v + (1-b2) g^2;
    mh = m / (1 - b1^t);   vh = v / (1 - b2^t);
    theta <- theta - lr (mh / (sqrt(vh) + eps) + wd * theta)   (decay on the
    pre-update theta; where decay is given, wd applies only where it is true).
    Returns (theta, m, v) as new float64 arrays."""
    theta = np.asarray(theta, np.float64)
    g = np.asarray(g, np.float64)
    m = beta1 * np.asarray(m, np.float64) + (1.0 - beta1) * g
    v = beta2 * np.asarray(v, np.float64) + (1.0 - beta2) * g * g
    mh = m / (1.0 - beta1 ** t)
    vh = v / (1.0 - beta2 ** t)
    w = wd if decay is None else wd * np.asarray(decay, np.float64)
    theta = theta - lr * (mh / (np.sqrt(vh) + eps) + w * theta)
    return theta, m, v


def grad_norm(grads, kind="l2"):
    """Global norm over every gradient element of every tensor: the L2 norm
    (MicroGPT in Rust, "Gradient Clipping"; Transformer in Rust, "Features":
    clipping by global norm) or the L-infinity norm max |g| (randyGPT,
    "Training (Metal GPU path)")."""
    flat = np.concatenate([np.asarray(g, np.float64).ravel() for g in grads.values()])
    if flat.size == 0:
        return 0.0
    if kind == "l2":
        return float(np.sqrt(np.sum(flat * flat)))
    if kind == "linf":
        return float(np.max(np.abs(flat)))
    raise ValueError(kind)


def clip_scale(norm, max_norm):
    """MicroGPT in Rust, "Gradient Clipping": max_norm / norm when the norm
    exceeds max_norm, else 1.  Reading: randyGPT's "L-infinity norm clipped
    at 1.0" is the same rule with the L-infinity norm (a scale, not an
    element-wise clamp)."""
    return max_norm / norm if norm > max_norm else 1.0


def decay_mask_like(params):
    """Reading: the pages exclude no tensor from weight decay, so every
    element decays."""
    return {k: np.ones_like(np.asarray(v, np.float64)) for k, v in params.items()}


# ----------------------------------------------------------------------------
# The model (Hephaistos, "Architecture at a glance" and "Design notes";
# Transformer in Rust, "CodeGen: Parallel Sub-Block Design")
# ----------------------------------------------------------------------------
def _heads(x2d, B, T, nh, d):
    """[N, nh*d] -> [B, nh, T, d]."""
    return x2d.reshape(B, T, nh, d).transpose(0, 2, 1, 3)


def _unheads(x4d):
    """[B, nh, T, d] -> [N, nh*d]."""
    B, nh, T, d = x4d.shape
    return x4d.transpose(0, 2, 1, 3).reshape(B * T, nh * d)


def forward(cfg, params, tokens, jitter=0.0, seed=0):
    """Forward pass and loss.

    cfg: a workload config (V, C, H, Hkv, L, T, F, R, rope_mode, block, act,
    eps, base); params: dict name -> master weights (matrices [out, in]);
    tokens: int [B, T+1], inputs tokens[:, :T], targets tokens[:, 1:].

    Llama block: x += W_o attn(rope(q), rope(k), v) with qkv = RMSNorm(x) W_qkv^T;
                 x += W_2 (silu(a) * b) with a, b = RMSNorm(x) W_1^T, RMSNorm(x) W_3^T.
    Parallel block: n = LayerNorm(x); x += [attn(n) | gelu(n W_in^T)] W_out^T.
    Final norm, then z = n_f W_head^T and the mean cross-entropy.
    jitter/seed: see store_fn (0 for the reference computation).  Jitter
    applies to stored activations and activation gradients only: the bf16
    compute copy of the weights is one rounding of the fp32 master with no
    summation in front of it, so every valid computation holds the same copy.
    Returns (loss, cache) where cache holds what the backward reads."""
    S = store_fn(cfg.act, jitter, seed)
    W = {k: store_fn(cfg.act)(np.asarray(v, np.float64)) for k, v in params.items()}
    tokens = np.asarray(tokens)
    B, T = tokens.shape[0], tokens.shape[1] - 1
    X, Y = tokens[:, :T].reshape(-1), tokens[:, 1:].reshape(-1)
    C, H, Hkv, d, R = cfg.C, cfg.H, cfg.Hkv, cfg.C // cfg.H, cfg.R
    cos, sin = rope_tables(T, R, cfg.base)
    qd, kd = H * d, Hkv * d

    # inverted dropout (training forward; Hephaistos, "Architecture at a
    # glance"; randyGPT, "Architecture Details"): multipliers of sites 0
    # (embedding output), 1 (attention projection / parallel block output),
    # 2 (MLP output) and 3 (attention weights, [B, H, T, T] with element
    # ((b H + h) T + i) T + j), cached for the backward
    p_drop = getattr(cfg, "dropout", 0.0)
    seed_drop = getattr(cfg, "dropout_seed", 0)

    def dmask(site, layer):
        return dropout_multiplier(p_drop, seed_drop, site, layer, B * T, C) if p_drop > 0 else None

    x = embedding_fwd(W["wte"], X)
    m_emb = dmask(0, 0)
    if m_emb is not None:
        x = S(x * m_emb)
    layers = []
    for l in range(cfg.L):
        p = f"h{l}."
        c = {"x_in": x}
        if cfg.block == "llama":
            n1, r1 = rmsnorm_fwd(x, W[p + "attn_norm"], cfg.eps)
            n1 = S(n1)
            qkv = n1 @ W[p + "qkvw"].T
        else:
            n1, mu1, r1 = layernorm_fwd(x, W[p + "ln_g"], W[p + "ln_b"], cfg.eps)
            n1 = S(n1)
            qkv = n1 @ W[p + "qkvw"].T
            a = S(n1 @ W[p + "fc_in"].T)
            c.update(mu1=mu1, a=a)
        # RoPE belongs to the q/k projection's output (Hephaistos, "Architecture
        # at a glance": RoPE applied to q and k inside attention): the stored
        # activation is the rotated q and k, rounded once, and v
        q = S(rope_apply(_heads(qkv[:, :qd], B, T, H, d), cos, sin, R, cfg.rope_mode))
        k = S(rope_apply(_heads(qkv[:, qd:qd + kd], B, T, Hkv, d), cos, sin, R, cfg.rope_mode))
        v = S(_heads(qkv[:, qd + kd:], B, T, Hkv, d))
        ma = None if p_drop <= 0 else dropout_multiplier(p_drop, seed_drop, 3, l, B * H * T, T).reshape(B, H, T, T)
        o4, lse = attention_fwd(q, k, v, ma)
        o = S(_unheads(o4))
        c.update(n1=n1, r1=r1, q=q, k=k, v=v, o=o, ma=ma)
        m1 = dmask(1, l)
        c["m1"] = m1
        drop1 = (lambda y: y) if m1 is None else (lambda y: y * m1)
        if cfg.block == "llama":
            x = S(x + drop1(o @ W[p + "w_o"].T))
            c["x_mid"] = x
            n2, r2 = rmsnorm_fwd(x, W[p + "mlp_norm"], cfg.eps)
            n2 = S(n2)
            a = S(n2 @ W[p + "w1"].T)
            b = S(n2 @ W[p + "w3"].T)
            h = S(swiglu_fwd(a, b))
            m2 = dmask(2, l)
            y2 = h @ W[p + "w2"].T
            x = S(x + (y2 if m2 is None else y2 * m2))
            c.update(n2=n2, r2=r2, a=a, b=b, h=h, m2=m2)
        else:
            u = S(gelu_fwd(c["a"]))
            x = S(x + drop1(np.concatenate([o, u], axis=1) @ W[p + "w_out"].T))
            c["u"] = u
        layers.append(c)
    x_f = x
    if cfg.block == "llama":
        nf, rf = rmsnorm_fwd(x_f, W["norm_f"], cfg.eps)
        muf = None
    else:
        nf, muf, rf = layernorm_fwd(x_f, W["lnf_g"], W["lnf_b"], cfg.eps)
    nf = S(nf)
    z = S(nf @ W["lm_head"].T)
    loss, dz, lse_z = cross_entropy(z, Y)
    cache = dict(store=S, W=W, X=X, Y=Y, B=B, T=T, cos=cos, sin=sin, layers=layers,
                 x_f=x_f, nf=nf, rf=rf, muf=muf, z=z, dz=dz, lse_z=lse_z, m_emb=m_emb)
    return loss, cache


def backward(cfg, cache):
    """Hand-written backward: a reverse walk over the cached forward.
    Matrix rules dX = dY W and dW = dY^T X; every weight gradient is written
    (not accumulated).  Returns dict name -> float64 gradient."""
    S = cache["store"]
    W = cache["W"]
    B, T = cache["B"], cache["T"]
    C, H, Hkv, d, R = cfg.C, cfg.H, cfg.Hkv, cfg.C // cfg.H, cfg.R
    cos, sin = cache["cos"], cache["sin"]
    qd, kd = H * d, Hkv * d
    grads = {}

    dz = S(cache["dz"])
    grads["lm_head"] = dz.T @ cache["nf"]
    dnf = S(dz @ W["lm_head"])
    if cfg.block == "llama":
        dx, grads["norm_f"] = rmsnorm_bwd(cache["x_f"], W["norm_f"], cache["rf"], dnf)
    else:
        dx, grads["lnf_g"], grads["lnf_b"] = layernorm_bwd(
            cache["x_f"], W["lnf_g"], cache["muf"], cache["rf"], dnf)
    dx = S(dx)

    for l in reversed(range(cfg.L)):
        p = f"h{l}."
        c = cache["layers"][l]
        # through dropout: the projection's output gradient is the incoming
        # one times the mask (stored like any activation gradient)
        if cfg.block == "llama":
            dy2 = dx if c.get("m2") is None else S(dx * c["m2"])
            grads[p + "w2"] = dy2.T @ c["h"]
            dh = S(dy2 @ W[p + "w2"])
            da, db = swiglu_bwd(c["a"], c["b"], dh)
            da, db = S(da), S(db)
            grads[p + "w1"] = da.T @ c["n2"]
            grads[p + "w3"] = db.T @ c["n2"]
            dn2 = S(da @ W[p + "w1"] + db @ W[p + "w3"])
            dxn, grads[p + "mlp_norm"] = rmsnorm_bwd(c["x_mid"], W[p + "mlp_norm"], c["r2"], dn2)
            dx = S(dx + dxn)
            dy1 = dx if c.get("m1") is None else S(dx * c["m1"])
            grads[p + "w_o"] = dy1.T @ c["o"]
            do = S(dy1 @ W[p + "w_o"])
        else:
            ou = np.concatenate([c["o"], c["u"]], axis=1)
            dy1 = dx if c.get("m1") is None else S(dx * c["m1"])
            grads[p + "w_out"] = dy1.T @ ou
            dou = S(dy1 @ W[p + "w_out"])
            do, du = dou[:, :C], dou[:, C:]
            da = S(gelu_bwd(c["a"], du))
        dq, dk, dv = attention_bwd(c["q"], c["k"], c["v"], _heads(do, B, T, H, d), c.get("ma"))
        dq = rope_apply(dq, cos, sin, R, cfg.rope_mode, inverse=True)
        dk = rope_apply(dk, cos, sin, R, cfg.rope_mode, inverse=True)
        dqkv = S(np.concatenate([_unheads(dq), _unheads(dk), _unheads(dv)], axis=1))
        grads[p + "qkvw"] = dqkv.T @ c["n1"]
        if cfg.block == "llama":
            dn1 = S(dqkv @ W[p + "qkvw"])
            dxn, grads[p + "attn_norm"] = rmsnorm_bwd(c["x_in"], W[p + "attn_norm"], c["r1"], dn1)
        else:
            grads[p + "fc_in"] = da.T @ c["n1"]
            dn1 = S(dqkv @ W[p + "qkvw"] + da @ W[p + "fc_in"])
            dxn, grads[p + "ln_g"], grads[p + "ln_b"] = layernorm_bwd(
                c["x_in"], W[p + "ln_g"], c["mu1"], c["r1"], dn1)
        dx = S(dx + dxn)
    m_emb = cache.get("m_emb")
    grads["wte"] = embedding_bwd(dx if m_emb is None else dx * m_emb, cache["X"], cfg.V)
    return grads


def accumulated_grads(cfg, params, micro_tokens):
    """Gradient accumulation (Transformer in Rust, "Configuration": several
    forward passes per optimizer step; "Features": gradient accumulation):
    the mean over S equal micro-batches of each micro-batch's gradient (of its
    own mean loss) -- the gradient of the mean loss over all of them.
    Returns (mean loss, grads)."""
    S = len(micro_tokens)
    total, acc = 0.0, None
    for tok in micro_tokens:
        loss, cache = forward(cfg, params, tok)
        g = backward(cfg, cache)
        total += loss
        acc = {k: v / S for k, v in g.items()} if acc is None else {k: acc[k] + g[k] / S for k in acc}
    return total / S, acc


def train_step(cfg, params, tokens, t=1, m=None, v=None, decay=None,
               lr=None, beta1=None, beta2=None, adam_eps=None, wd=None, jitter=0.0, seed=0, clip=None):
    """forward -> backward -> (optional clipping) -> AdamW on every tensor.
    m and v default to zero (first step).  clip: None or (kind, max_norm):
    every gradient is multiplied by clip_scale(grad_norm(grads, kind),
    max_norm) before AdamW sees it.  Returns dict(loss, grads, params, m, v,
    grad_norm, clip_scale); grads are the unclipped gradients."""
    loss, cache = forward(cfg, params, tokens, jitter, seed)
    grads = backward(cfg, cache)
    gn, cscale = None, 1.0
    if clip is not None:
        gn = grad_norm(grads, clip[0])
        cscale = clip_scale(gn, clip[1])
    lr = cfg.lr if lr is None else lr
    beta1 = cfg.beta1 if beta1 is None else beta1
    beta2 = cfg.beta2 if beta2 is None else beta2
    adam_eps = cfg.adam_eps if adam_eps is None else adam_eps
    wd = cfg.wd if wd is None else wd
    new_p, new_m, new_v = {}, {}, {}
    for name, th in params.items():
        m0 = np.zeros_like(np.asarray(th, np.float64)) if m is None else m[name]
        v0 = np.zeros_like(np.asarray(th, np.float64)) if v is None else v[name]
        dm = None if decay is None else decay[name]
        new_p[name], new_m[name], new_v[name] = adamw(
            th, cscale * np.asarray(grads[name], np.float64), m0, v0, t, lr, beta1, beta2, adam_eps, wd, dm)
    return dict(loss=loss, grads=grads, params=new_p, m=new_m, v=new_v, grad_norm=gn, clip_scale=cscale)
