"""Pins for the CPU oracle: closed forms, invariants, worked numbers from the
pages, library routines and finite differences.  None of these retypes the
oracle's formulas; each is chosen so that a plausible slip (a dropped term, a
wrong sign or index, a transposed operand) fails at least one of them."""
import math

import numpy as np
import pytest

import oracle as O
import slt_workloads as W


def tiny(block="llama", H=4, Hkv=4, act="f32", **kw):
    base = dict(name="tiny", V=23, C=16, H=H, Hkv=Hkv, L=2, T=7, B=2, F=24,
                R=16 // H, rope_mode="half", block=block, act=act,
                tokens="uniform", scale_out=False)
    if block == "parallel":
        base.update(rope_mode="pairs", R=2)   # partial: 2 of head dim 4
    base.update(kw)
    return W.Config(**base)


def rand_params(cfg, seed=0, std=0.3):
    """Weights large enough that every term of the step matters; gains and
    shifts randomised too so their gradients are exercised."""
    rng = np.random.default_rng(seed)
    out = {}
    for name, shape, init in W.param_specs(cfg):
        if init == "ones":
            out[name] = 1.0 + 0.2 * rng.standard_normal(shape)
        elif init == "zeros":
            out[name] = 0.2 * rng.standard_normal(shape)
        else:
            out[name] = std * rng.standard_normal(shape)
    return out


# --------------------------------------------------------------------------
# bf16 rounding against a library conversion (torch, fp32 -> bfloat16 RNE)
# --------------------------------------------------------------------------
def test_bf16_round_matches_torch_conversion():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    # ties: low 16 bits exactly 0x8000, both parities of bit 16
    ties = (rng.integers(0, 2 ** 16, size=20000, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    special = np.array([0, 0x80000000, 0x00000001, 0x007FFFFF, 0x00800000, 0x7F7FFFFF,
                        0x7F7F8000, 0x7F7F7FFF, 0xFF7FFFFF, 0x3F808000, 0x3F818000], np.uint32)
    bits = np.concatenate([bits, ties, special])
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).to(torch.float32).numpy().astype(np.float64)
    got = O.bf16_round(f.astype(np.float64))
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all(), (f[~same][:5], got[~same][:5], ref[~same][:5])


def test_bf16_round_ties_to_even_worked_values():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: ties go to the even one (1).
    assert O.bf16_round(1.0 + 2.0 ** -8) == 1.0
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even).
    assert O.bf16_round(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    assert O.bf16_round(1.0 + 2.0 ** -8 + 2.0 ** -30) == 1.0 + 2.0 ** -7


# --------------------------------------------------------------------------
# Parameter counts printed on the Hephaistos page ("What you'll see": 1,049,216
# for 4L/4H/C128/V1024; "The bigger run": 15.74M for 8L/8H/C384/V2048).
# --------------------------------------------------------------------------
def test_param_counts_match_hephaistos_page():
    small = W.Config("h", V=1024, C=128, H=4, Hkv=4, L=4, T=64, B=1, F=(8 * 128) // 3, R=32,
                     rope_mode="half", block="llama", act="f32", tokens="uniform", scale_out=False)
    assert W.n_params(small) == 1049216
    big = small.with_(V=2048, C=384, H=8, Hkv=8, L=8, T=256, F=(8 * 384) // 3, R=48)
    assert round(W.n_params(big) / 1e6, 2) == 15.74


def test_config_param_counts():
    assert [W.n_params(c) for c in W.CONFIGS] == [3952, 4974848, 17308032, 245924864, 356558848]


# --------------------------------------------------------------------------
# Finite-difference gradient checks at float64 (Hephaistos, "Why it's
# interesting" / "Tests": every parameter tensor against central differences;
# strata: f64 gradcheck of every backward rule)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("family", ["llama_mha", "llama_gqa", "parallel_partial_rope"])
def test_full_model_gradcheck_every_tensor(family):
    cfg = {"llama_mha": tiny(), "llama_gqa": tiny(H=4, Hkv=2),
           "parallel_partial_rope": tiny(block="parallel")}[family]
    params = rand_params(cfg, seed=3)
    tokens = np.random.default_rng(4).integers(0, cfg.V, size=(cfg.B, cfg.T + 1))
    loss, cache = O.forward(cfg, params, tokens)
    grads = O.backward(cfg, cache)
    assert set(grads) == set(params)
    rng = np.random.default_rng(5)
    h = 1e-6
    worst = 0.0
    for name, p in params.items():
        flat = p.reshape(-1)
        idx = rng.choice(flat.size, size=min(6, flat.size), replace=False)
        if name == "wte":   # include rows that occur in the batch
            idx = np.concatenate([idx, tokens[0, :3] * cfg.C])
        for i in idx:
            old = flat[i]
            flat[i] = old + h
            lp, _ = O.forward(cfg, params, tokens)
            flat[i] = old - h
            lm, _ = O.forward(cfg, params, tokens)
            flat[i] = old
            num = (lp - lm) / (2 * h)
            ana = grads[name].reshape(-1)[i]
            # central differences carry ~eps*|loss|/h = 3e-10 of rounding noise
            err = abs(ana - num) / max(abs(ana), abs(num), 1e-4)
            worst = max(worst, err)
            assert err < 1e-5, (name, i, ana, num)
    assert worst < 1e-5


def test_cross_entropy_gradcheck():
    rng = np.random.default_rng(0)
    z = rng.standard_normal((5, 7)) * 2
    y = rng.integers(0, 7, 5)
    _, dz, _ = O.cross_entropy(z, y)
    h = 1e-6
    for i in range(5):
        for j in range(7):
            zp, zm = z.copy(), z.copy()
            zp[i, j] += h
            zm[i, j] -= h
            num = (O.cross_entropy(zp, y)[0] - O.cross_entropy(zm, y)[0]) / (2 * h)
            assert abs(num - dz[i, j]) < 1e-8


# --------------------------------------------------------------------------
# Cross-check against an independent torch float64 autograd model (strata,
# rules: PyTorch allowed as a test oracle).  Library softmax, silu, gelu(tanh)
# and cross_entropy; autograd instead of hand-written backward.
# --------------------------------------------------------------------------
def torch_reference(cfg, params, tokens):
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    P = {k: torch.tensor(np.asarray(v, np.float64), requires_grad=True) for k, v in params.items()}
    tok = torch.tensor(np.asarray(tokens, np.int64))
    B, T = tok.shape[0], tok.shape[1] - 1
    C, H, Hkv = cfg.C, cfg.H, cfg.Hkv
    d = C // H
    R = cfg.R
    pos = torch.arange(T, dtype=torch.float64)
    inv = cfg.base ** (-torch.arange(0, R, 2, dtype=torch.float64) / R)
    ang = pos[:, None] * inv[None, :]
    cs, sn = torch.cos(ang), torch.sin(ang)

    def rope(u):  # u [B, nh, T, d]; rotate as complex numbers
        if cfg.rope_mode == "half":
            re, im = u[..., :R // 2], u[..., R // 2:R]
        else:
            re, im = u[..., 0:R:2], u[..., 1:R:2]
        zc = torch.complex(re, im) * torch.polar(torch.ones_like(ang), ang)
        if cfg.rope_mode == "half":
            rot = torch.cat([zc.real, zc.imag], dim=-1)
        else:
            rot = torch.stack([zc.real, zc.imag], dim=-1).flatten(-2)
        return torch.cat([rot, u[..., R:]], dim=-1)

    def rms(x, g):
        return x * torch.rsqrt(x.pow(2).mean(-1, keepdim=True) + cfg.eps) * g

    def ln(x, g, b):
        return F.layer_norm(x, (C,), g, b, cfg.eps)

    def attn(n, w):
        qkv = n @ w.T
        q = qkv[..., :H * d].reshape(B, T, H, d).transpose(1, 2)
        k = qkv[..., H * d:(H + Hkv) * d].reshape(B, T, Hkv, d).transpose(1, 2)
        v = qkv[..., (H + Hkv) * d:].reshape(B, T, Hkv, d).transpose(1, 2)
        q, k = rope(q), rope(k)
        k = k.repeat_interleave(H // Hkv, dim=1)
        v = v.repeat_interleave(H // Hkv, dim=1)
        s = (q @ k.transpose(-1, -2)) / math.sqrt(d)
        s = s.masked_fill(~torch.ones(T, T, dtype=torch.bool).tril(), float("-inf"))
        o = torch.softmax(s, dim=-1) @ v
        return o.transpose(1, 2).reshape(B, T, H * d)

    x = P["wte"][tok[:, :T]]
    for l in range(cfg.L):
        p = f"h{l}."
        if cfg.block == "llama":
            x = x + attn(rms(x, P[p + "attn_norm"]), P[p + "qkvw"]) @ P[p + "w_o"].T
            n = rms(x, P[p + "mlp_norm"])
            x = x + (F.silu(n @ P[p + "w1"].T) * (n @ P[p + "w3"].T)) @ P[p + "w2"].T
        else:
            n = ln(x, P[p + "ln_g"], P[p + "ln_b"])
            a = F.gelu(n @ P[p + "fc_in"].T, approximate="tanh")
            x = x + torch.cat([attn(n, P[p + "qkvw"]), a], dim=-1) @ P[p + "w_out"].T
    nf = rms(x, P["norm_f"]) if cfg.block == "llama" else ln(x, P["lnf_g"], P["lnf_b"])
    z = nf @ P["lm_head"].T
    loss = F.cross_entropy(z.reshape(-1, cfg.V), tok[:, 1:].reshape(-1))
    loss.backward()
    return float(loss.detach()), {k: v.grad.numpy() for k, v in P.items()}


@pytest.mark.parametrize("family", ["cfg1", "llama_gqa", "parallel_partial_rope", "cfg2_small_batch"])
def test_oracle_matches_torch_autograd(family):
    if family == "cfg1":
        cfg = W.get_config(1)
    elif family == "llama_gqa":
        cfg = tiny(H=8, Hkv=2, C=32, T=12, L=2)
    elif family == "parallel_partial_rope":
        cfg = tiny(block="parallel", C=32, H=4, R=4, T=12)
    else:
        cfg = W.get_config(2).with_(B=2, T=64, L=2)
    params = rand_params(cfg, seed=11, std=0.1)
    tokens = np.random.default_rng(12).integers(0, cfg.V, size=(cfg.B, cfg.T + 1))
    loss, cache = O.forward(cfg, params, tokens)
    grads = O.backward(cfg, cache)
    tloss, tgrads = torch_reference(cfg, params, tokens)
    assert abs(loss - tloss) <= 1e-12 * abs(tloss)
    for k in params:
        err = np.linalg.norm(grads[k] - tgrads[k]) / max(np.linalg.norm(tgrads[k]), 1e-300)
        assert err < 1e-10, (k, err)


# --------------------------------------------------------------------------
# Closed forms of the whole step
# --------------------------------------------------------------------------
@pytest.mark.parametrize("block", ["llama", "parallel"])
def test_zero_head_gives_ln_v_and_zero_lower_gradients(block):
    cfg = tiny(block=block)
    params = rand_params(cfg, seed=7)
    params["lm_head"][:] = 0.0
    tokens = np.random.default_rng(8).integers(0, cfg.V, size=(cfg.B, cfg.T + 1))
    loss, cache = O.forward(cfg, params, tokens)
    assert loss == pytest.approx(math.log(cfg.V), rel=1e-15, abs=0)
    N = cfg.B * cfg.T
    expect = np.full((N, cfg.V), 1.0 / cfg.V)
    expect[np.arange(N), tokens[:, 1:].reshape(-1)] -= 1.0
    np.testing.assert_allclose(cache["dz"], expect / N, rtol=1e-14, atol=1e-17)
    grads = O.backward(cfg, cache)
    for k, g in grads.items():
        if k != "lm_head":
            assert np.all(g == 0.0), k
    assert np.linalg.norm(grads["lm_head"]) > 0


def test_identity_blocks_reduce_to_closed_form_bigram():
    """With zero output projections each block is the identity; with one-hot
    embeddings of size alpha and lm_head = beta * I the logits are
    s * e_x with s = alpha * beta / sqrt(alpha^2 / C + eps), so the loss of a
    position is log(e^s + V - 1) - s [y == x]."""
    V = C = 16
    cfg = tiny(V=V, C=C)
    params = rand_params(cfg, seed=2)
    for l in range(cfg.L):
        params[f"h{l}.w_o"][:] = 0.0
        params[f"h{l}.w2"][:] = 0.0
    params["norm_f"][:] = 1.0
    alpha, beta = 1.7, 0.9
    params["wte"] = alpha * np.eye(V)
    params["lm_head"] = beta * np.eye(V)
    tokens = np.random.default_rng(3).integers(0, V, size=(cfg.B, cfg.T + 1))
    tokens[0, 1] = tokens[0, 0]     # make sure some targets equal their inputs
    loss, _ = O.forward(cfg, params, tokens)
    s = alpha * beta / math.sqrt(alpha ** 2 / C + cfg.eps)
    x, y = tokens[:, :-1].reshape(-1), tokens[:, 1:].reshape(-1)
    per = np.log(np.exp(s) + V - 1) - s * (x == y)
    assert loss == pytest.approx(per.mean(), rel=1e-14)


@pytest.mark.parametrize("block,H,Hkv", [("llama", 4, 4), ("llama", 4, 2), ("parallel", 4, 4)])
def test_prefix_forward_gate(block, H, Hkv):
    """strata rule: a decoder fed a prefix must reproduce the full forward's
    rows for that prefix (the cache-free form of the KV-cache gate); this
    pins causality and absolute positions starting at 0."""
    cfg = tiny(block=block, H=H, Hkv=Hkv, T=9, B=1)
    params = rand_params(cfg, seed=21)
    tokens = np.random.default_rng(22).integers(0, cfg.V, size=(1, cfg.T + 1))
    _, full = O.forward(cfg, params, tokens)
    for i in range(cfg.T):
        _, pre = O.forward(cfg, params, tokens[:, :i + 2])
        np.testing.assert_allclose(pre["z"][-1], full["z"][i], rtol=1e-12, atol=1e-13)


def test_gqa_equals_mha_with_repeated_kv_heads():
    """strata, "GPT-2 to modern": one attention op with independent n_head and
    n_kv_head; GQA is MHA whose KV heads are shared.  Forward equal; the GQA
    gradient of a KV row is the sum over its copies."""
    g = tiny(H=4, Hkv=2, T=6)
    m = tiny(H=4, Hkv=4, T=6)
    d = g.C // g.H
    pg = rand_params(g, seed=31)
    pm = {k: v.copy() for k, v in pg.items() if not k.endswith("qkvw")}
    for l in range(g.L):
        w = pg[f"h{l}.qkvw"]
        q = w[:g.H * d]
        k = w[g.H * d:(g.H + g.Hkv) * d].reshape(g.Hkv, d, g.C)
        v = w[(g.H + g.Hkv) * d:].reshape(g.Hkv, d, g.C)
        rep = g.H // g.Hkv
        pm[f"h{l}.qkvw"] = np.concatenate([q, np.repeat(k, rep, 0).reshape(-1, g.C),
                                           np.repeat(v, rep, 0).reshape(-1, g.C)])
    tokens = np.random.default_rng(32).integers(0, g.V, size=(g.B, g.T + 1))
    lg, cg = O.forward(g, pg, tokens)
    lm, cm = O.forward(m, pm, tokens)
    assert lg == pytest.approx(lm, rel=1e-13)
    gg, gm = O.backward(g, cg), O.backward(m, cm)
    for l in range(g.L):
        a = gg[f"h{l}.qkvw"]
        b = gm[f"h{l}.qkvw"]
        rep = g.H // g.Hkv
        np.testing.assert_allclose(a[:g.H * d], b[:g.H * d], rtol=1e-10, atol=1e-14)
        for part in range(2):
            sa = a[(g.H + part * g.Hkv) * d:(g.H + (part + 1) * g.Hkv) * d].reshape(g.Hkv, d, g.C)
            sb = b[(g.H + part * g.H) * d:(g.H + (part + 1) * g.H) * d].reshape(g.Hkv, rep, d, g.C)
            np.testing.assert_allclose(sa, sb.sum(1), rtol=1e-10, atol=1e-14)


def test_initial_loss_close_to_ln_vocab():
    """Hephaistos, "What you'll see": untrained loss ~ ln V (6.9847 vs 6.9315);
    strata lab 01: 3.1126 vs 3.1355.  With N(0, 0.02) weights the excess is
    about 2e-4 * C."""
    cfg = W.get_config(1)
    params = W.make_params(cfg, 1001)
    tokens = W.make_tokens(cfg, 1001)
    loss, _ = O.forward(cfg, params, tokens)
    assert abs(loss - math.log(cfg.V)) < 0.05


# --------------------------------------------------------------------------
# Norms
# --------------------------------------------------------------------------
def test_rmsnorm_worked_value_and_invariants():
    x = np.array([[3.0, 4.0]])
    y, r = O.rmsnorm_fwd(x, np.ones(2), 1e-5)
    assert r[0] == pytest.approx(1.0 / math.sqrt(12.5 + 1e-5), rel=1e-15)
    rng = np.random.default_rng(0)
    x = rng.standard_normal((6, 32)) * 3
    y, r = O.rmsnorm_fwd(x, np.ones(32), 1e-5)
    ms = np.mean(x * x, 1)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, 1)), np.sqrt(ms / (ms + 1e-5)), rtol=1e-13)
    y0, _ = O.rmsnorm_fwd(x, np.ones(32), 0.0)
    y1, _ = O.rmsnorm_fwd(7.5 * x, np.ones(32), 0.0)
    np.testing.assert_allclose(y0, y1, rtol=1e-13)
    g = rng.standard_normal(32)
    _, r0 = O.rmsnorm_fwd(x, g, 0.0)
    dx, _ = O.rmsnorm_bwd(x, g, r0, rng.standard_normal((6, 32)))
    np.testing.assert_allclose(np.sum(x * dx, 1), 0.0, atol=1e-12)


def test_layernorm_invariants():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 24)) * 2 + 3
    gm, bt = np.ones(24), np.zeros(24)
    y, mu, r = O.layernorm_fwd(x, gm, bt, 1e-5)
    np.testing.assert_allclose(y.mean(1), 0.0, atol=1e-13)
    var = ((x - x.mean(1, keepdims=True)) ** 2).mean(1)
    np.testing.assert_allclose((y * y).mean(1), var / (var + 1e-5), rtol=1e-12)
    y2, _, _ = O.layernorm_fwd(x + 11.0, gm, bt, 1e-5)
    np.testing.assert_allclose(y, y2, rtol=1e-9, atol=1e-12)
    g = rng.standard_normal(24)
    _, mu0, r0 = O.layernorm_fwd(x, g, bt, 0.0)
    dx, _, dbeta = O.layernorm_bwd(x, g, mu0, r0, rng.standard_normal((5, 24)))
    np.testing.assert_allclose(dx.sum(1), 0.0, atol=1e-12)
    np.testing.assert_allclose(np.sum(x * dx, 1), 0.0, atol=1e-11)


# --------------------------------------------------------------------------
# RoPE
# --------------------------------------------------------------------------
def test_rope_worked_angles():
    # R = 2: theta_0 = 1, so position 1 turns (1, 0) into (cos 1, sin 1).
    cos, sin = O.rope_tables(3, 2, 10000.0)
    u = np.zeros((3, 2))
    u[:, 0] = 1.0
    out = O.rope_apply(u, cos, sin, 2, "half")
    np.testing.assert_allclose(out[1], [math.cos(1.0), math.sin(1.0)], rtol=1e-15)
    np.testing.assert_allclose(out[2], [math.cos(2.0), math.sin(2.0)], rtol=1e-15)
    # R = 4: theta_1 = 10000^(-1/2) = 0.01; position 100 turns pair 1 by 1 rad.
    cos, sin = O.rope_tables(101, 4, 10000.0)
    u = np.zeros((101, 4))
    u[:, 1] = 1.0      # rotate-half: pair 1 is dims (1, 3)
    out = O.rope_apply(u, cos, sin, 4, "half")
    np.testing.assert_allclose(out[100, [1, 3]], [math.cos(1.0), math.sin(1.0)], rtol=1e-12)
    np.testing.assert_allclose(out[100, [0, 2]], 0.0, atol=0)
    v = np.zeros((101, 4))
    v[:, 2] = 1.0      # even-odd: pair 1 is dims (2, 3)
    out = O.rope_apply(v, cos, sin, 4, "pairs")
    np.testing.assert_allclose(out[100, [2, 3]], [math.cos(1.0), math.sin(1.0)], rtol=1e-12)


@pytest.mark.parametrize("mode", ["half", "pairs"])
def test_rope_invariants(mode):
    T, d = 12, 8
    cos, sin = O.rope_tables(T, d, 10000.0)
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal((T, d)), rng.standard_normal((T, d))
    rq = O.rope_apply(q, cos, sin, d, mode)
    np.testing.assert_allclose(rq[0], q[0], rtol=0, atol=0)                 # R_0 = I
    np.testing.assert_allclose(np.linalg.norm(rq, axis=1), np.linalg.norm(q, axis=1), rtol=1e-14)
    # strata: <R_i q, R_j k> depends only on i - j
    qq = np.repeat(q[:1], T, 0)
    kk = np.repeat(k[:1], T, 0)
    a = O.rope_apply(qq, cos, sin, d, mode)
    b = O.rope_apply(kk, cos, sin, d, mode)
    for i, j, s in [(5, 2, 4), (7, 7, 3), (3, 9, 2)]:
        assert a[i] @ b[j] == pytest.approx(a[i + s] @ b[j + s], rel=1e-12)
    back = O.rope_apply(rq, cos, sin, d, mode, inverse=True)
    np.testing.assert_allclose(back, q, rtol=1e-13, atol=1e-14)


def test_rope_rotate_half_equals_interleaved_after_permutation():
    """Hephaistos, GGUF export: rotate-half and interleaved layouts differ by a
    fixed permutation of each head's q/k rows."""
    T, d = 10, 8
    cos, sin = O.rope_tables(T, d, 10000.0)
    u = np.random.default_rng(3).standard_normal((T, d))
    perm = np.empty(d, int)
    perm[0::2] = np.arange(d // 2)
    perm[1::2] = np.arange(d // 2) + d // 2
    np.testing.assert_allclose(O.rope_apply(u, cos, sin, d, "half")[:, perm],
                               O.rope_apply(u[:, perm], cos, sin, d, "pairs"), rtol=1e-15)


def test_partial_rope_leaves_tail_and_full_case():
    T, d = 6, 8
    u = np.random.default_rng(4).standard_normal((T, d))
    cos, sin = O.rope_tables(T, 4, 10000.0)
    out = O.rope_apply(u, cos, sin, 4, "pairs")
    np.testing.assert_array_equal(out[:, 4:], u[:, 4:])
    np.testing.assert_allclose(out[:, :4], O.rope_apply(u[:, :4], cos, sin, 4, "pairs"), rtol=0)


# --------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------
def test_attention_two_position_closed_form():
    """Row 1 of a causal 2-position attention mixes v0 and v1 with weights
    sigmoid(s10 - s11), sigmoid(s11 - s10), s = q.k / sqrt(d); row 0 is v0."""
    rng = np.random.default_rng(5)
    d = 4
    q = rng.standard_normal((1, 1, 2, d))
    k = rng.standard_normal((1, 1, 2, d))
    v = rng.standard_normal((1, 1, 2, d))
    o, lse = O.attention_fwd(q, k, v)
    s10 = q[0, 0, 1] @ k[0, 0, 0] / 2.0
    s11 = q[0, 0, 1] @ k[0, 0, 1] / 2.0
    w0 = 1.0 / (1.0 + math.exp(s11 - s10))
    np.testing.assert_allclose(o[0, 0, 0], v[0, 0, 0], rtol=1e-15)
    np.testing.assert_allclose(o[0, 0, 1], w0 * v[0, 0, 0] + (1 - w0) * v[0, 0, 1], rtol=1e-13)
    assert lse[0, 0, 1] == pytest.approx(math.log(math.exp(s10) + math.exp(s11)), rel=1e-14)


def test_attention_zero_query_is_prefix_mean():
    rng = np.random.default_rng(6)
    B, H, T, d = 2, 3, 9, 4
    v = rng.standard_normal((B, H, T, d))
    o, _ = O.attention_fwd(np.zeros((B, H, T, d)), rng.standard_normal((B, H, T, d)), v)
    expect = np.cumsum(v, axis=2) / np.arange(1, T + 1)[None, None, :, None]
    np.testing.assert_allclose(o, expect, rtol=1e-13)


def test_attention_backward_finite_differences():
    rng = np.random.default_rng(7)
    B, H, Hkv, T, d = 1, 4, 2, 5, 4
    q = rng.standard_normal((B, H, T, d))
    k = rng.standard_normal((B, Hkv, T, d))
    v = rng.standard_normal((B, Hkv, T, d))
    w = rng.standard_normal((B, H, T, d))
    dq, dk, dv = O.attention_bwd(q, k, v, w)
    h = 1e-6
    for arr, grad in [(q, dq), (k, dk), (v, dv)]:
        for _ in range(6):
            idx = tuple(rng.integers(0, s) for s in arr.shape)
            old = arr[idx]
            arr[idx] = old + h
            fp = np.sum(O.attention_fwd(q, k, v)[0] * w)
            arr[idx] = old - h
            fm = np.sum(O.attention_fwd(q, k, v)[0] * w)
            arr[idx] = old
            assert (fp - fm) / (2 * h) == pytest.approx(grad[idx], rel=1e-6, abs=1e-9)


def test_online_softmax_tiled_attention_equals_materialized():
    """strata: flash-style attention (online softmax over key blocks) matches
    the materialized softmax.  The tiled loop is written here, independent of
    the oracle's one-shot softmax."""
    rng = np.random.default_rng(8)
    T, d, blk = 37, 8, 5
    q, k, v = (rng.standard_normal((T, d)) * 2 for _ in range(3))
    out = np.zeros((T, d))
    for i in range(T):
        m, l, acc = -np.inf, 0.0, np.zeros(d)
        for j0 in range(0, i + 1, blk):
            js = np.arange(j0, min(j0 + blk, i + 1))
            s = k[js] @ q[i] / math.sqrt(d)
            m_new = max(m, s.max())
            corr = math.exp(m - m_new) if np.isfinite(m) else 0.0
            e = np.exp(s - m_new)
            l = l * corr + e.sum()
            acc = acc * corr + e @ v[js]
            m = m_new
        out[i] = acc / l
    o, _ = O.attention_fwd(q[None, None], k[None, None], v[None, None])
    np.testing.assert_allclose(o[0, 0], out, rtol=1e-12)


# --------------------------------------------------------------------------
# MLP activations
# --------------------------------------------------------------------------
def test_swiglu_values():
    assert O.swiglu_fwd(1.0, 1.0) == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-15)
    assert O.swiglu_fwd(0.0, 5.0) == 0.0
    da, db = O.swiglu_bwd(np.array([0.0]), np.array([1.0]), np.array([1.0]))
    assert da[0] == pytest.approx(0.5) and db[0] == 0.0
    a = np.random.default_rng(9).standard_normal(50)
    da, db = O.swiglu_bwd(a, np.zeros(50), np.ones(50))
    assert np.all(da == 0.0) and np.all(O.swiglu_fwd(a, np.zeros(50)) == 0.0)
    b = np.random.default_rng(10).standard_normal(50)
    h = 1e-6
    num_a = (O.swiglu_fwd(a + h, b) - O.swiglu_fwd(a - h, b)) / (2 * h)
    num_b = (O.swiglu_fwd(a, b + h) - O.swiglu_fwd(a, b - h)) / (2 * h)
    da, db = O.swiglu_bwd(a, b, np.ones(50))
    np.testing.assert_allclose(da, num_a, rtol=1e-7, atol=1e-9)
    np.testing.assert_allclose(db, num_b, rtol=1e-7, atol=1e-9)


def test_gelu_against_library_and_erf_form():
    torch = pytest.importorskip("torch")
    a = np.linspace(-6, 6, 1001)
    ref = torch.nn.functional.gelu(torch.tensor(a), approximate="tanh").numpy()
    np.testing.assert_allclose(O.gelu_fwd(a), ref, rtol=1e-13, atol=1e-15)
    phi = np.array([0.5 * (1 + math.erf(x / math.sqrt(2))) for x in a])
    assert np.max(np.abs(O.gelu_fwd(a) - a * phi)) < 1e-3
    h = 1e-6
    np.testing.assert_allclose(O.gelu_bwd(a, np.ones_like(a)),
                               (O.gelu_fwd(a + h) - O.gelu_fwd(a - h)) / (2 * h), rtol=1e-7, atol=1e-9)
    assert O.gelu_bwd(np.array([0.0]), np.array([1.0]))[0] == pytest.approx(0.5)


# --------------------------------------------------------------------------
# Cross-entropy
# --------------------------------------------------------------------------
def test_cross_entropy_worked_values():
    loss, dz, lse = O.cross_entropy(np.array([[0.0, math.log(3.0)]]), np.array([0]))
    assert loss == pytest.approx(math.log(4.0), rel=1e-15)
    np.testing.assert_allclose(dz, [[0.25 - 1.0, 0.75]], rtol=1e-15)
    z = np.random.default_rng(11).standard_normal((7, 13)) * 4
    loss, dz, _ = O.cross_entropy(z, np.arange(7))
    np.testing.assert_allclose(dz.sum(1), 0.0, atol=1e-16)
    loss2, _, _ = O.cross_entropy(z + 100.0, np.arange(7))
    assert loss2 == pytest.approx(loss, rel=1e-13)
    assert O.cross_entropy(np.zeros((3, 27)), np.array([1, 2, 3]))[0] == pytest.approx(math.log(27), rel=1e-15)


# --------------------------------------------------------------------------
# AdamW
# --------------------------------------------------------------------------
def test_adamw_first_steps_closed_forms():
    lr, b1, b2, eps, wd = 1e-3, 0.9, 0.999, 1e-8, 0.1
    th0 = np.array([0.5, -0.25, 0.0, 1.0])
    g1 = np.array([0.3, -2.0, 1e-3, 0.0])
    th1, m1, v1 = O.adamw(th0, g1, 0, 0, 1, lr, b1, b2, eps, wd)
    # at t = 1 bias correction makes m_hat = g and v_hat = g^2
    np.testing.assert_allclose(th1, th0 - lr * (g1 / (np.abs(g1) + eps) + wd * th0), rtol=1e-14)
    np.testing.assert_allclose(m1, 0.1 * g1, rtol=1e-15)
    np.testing.assert_allclose(v1, 0.001 * g1 ** 2, rtol=1e-14)
    assert th1[3] == th0[3] * (1 - lr * wd)        # g = 0: pure decay
    g2 = np.array([-0.1, 1.0, 2e-3, 0.5])
    th2, _, _ = O.adamw(th1, g2, m1, v1, 2, lr, b1, b2, eps, wd)
    mh = (0.09 * g1 + 0.1 * g2) / 0.19
    vh = (0.000999 * g1 ** 2 + 0.001 * g2 ** 2) / 0.001999
    np.testing.assert_allclose(th2, th1 - lr * (mh / (np.sqrt(vh) + eps) + wd * th1), rtol=1e-12)
    thm, _, _ = O.adamw(th0, g1, 0, 0, 1, lr, b1, b2, eps, wd, decay=np.array([0, 1, 0, 1]))
    np.testing.assert_allclose(thm[0], th0[0] - lr * g1[0] / (abs(g1[0]) + eps), rtol=1e-14)


def test_adamw_converges_on_quadratic():
    """strata: AdamW converges on a quadratic."""
    c = np.array([1.0, -2.0, 0.5, 3.0])
    th = np.zeros(4)
    m = v = np.zeros(4)
    for t in range(1, 3001):
        th, m, v = O.adamw(th, th - c, m, v, t, 1e-2, 0.9, 0.999, 1e-8, 0.0)
    np.testing.assert_allclose(th, c, atol=1e-3)


# --------------------------------------------------------------------------
# Embedding
# --------------------------------------------------------------------------
def test_embedding_backward_unseen_rows_and_repeats():
    rng = np.random.default_rng(12)
    ids = np.array([3, 3, 3, 5, 3])
    dx = rng.standard_normal((5, 6))
    g = O.embedding_bwd(dx, ids, 8)
    np.testing.assert_allclose(g[3], dx[[0, 1, 2, 4]].sum(0), rtol=1e-15)
    np.testing.assert_array_equal(g[5], dx[3])
    assert np.all(g[[0, 1, 2, 4, 6, 7]] == 0.0)


# --------------------------------------------------------------------------
# bf16 storage emulation: the rounded forward stays close to the exact one
# --------------------------------------------------------------------------
def test_bf16_forward_close_to_exact():
    cfg = tiny(act="bf16", C=32, H=4, R=8)
    params = rand_params(cfg, seed=41, std=0.1)
    tokens = np.random.default_rng(42).integers(0, cfg.V, size=(cfg.B, cfg.T + 1))
    lb, cb = O.forward(cfg, params, tokens)
    lf, cf = O.forward(cfg.with_(act="f32"), params, tokens)
    assert abs(lb - lf) < 1e-2 * lf
    assert lb != lf
    gb, gf = O.backward(cfg, cb), O.backward(cfg.with_(act="f32"), cf)
    for k in gf:
        assert np.linalg.norm(gb[k] - gf[k]) <= 0.05 * np.linalg.norm(gf[k]) + 1e-12, k


# ---------------------------------------------------------------------------
# Global-norm gradient clipping (MicroGPT in Rust, "Gradient Clipping";
# Transformer in Rust, "Features"; randyGPT, "Training (Metal GPU path)")
# ---------------------------------------------------------------------------
def test_grad_norm_closed_forms():
    g = {"a": np.array([[3.0, 0.0]]), "b": np.array([-4.0]), "c": np.zeros((2, 2))}
    assert O.grad_norm(g, "l2") == 5.0            # 3-4-5 across tensors: the norm is global
    assert O.grad_norm(g, "linf") == 4.0          # largest magnitude, sign ignored
    assert O.grad_norm({"z": np.zeros(3)}, "l2") == 0.0
    assert O.clip_scale(5.0, 1.0) == 0.2
    assert O.clip_scale(0.5, 1.0) == 1.0          # below the threshold: untouched
    assert O.clip_scale(1.0, 1.0) == 1.0          # at the threshold: untouched
    rng = np.random.default_rng(40)
    g = {k: rng.standard_normal(s) * 3 for k, s in [("x", (7, 5)), ("y", (11,))]}
    for kind in ("l2", "linf"):
        s_ = O.clip_scale(O.grad_norm(g, kind), 0.75)
        clipped = {k: s_ * v for k, v in g.items()}
        assert abs(O.grad_norm(clipped, kind) - 0.75) < 1e-15   # clipped to exactly max_norm


def test_train_step_clipping_scales_first_moments():
    w = W.get_config(1)
    params = W.make_params(w, 41)
    tokens = W.make_tokens(w, 41)
    base = O.train_step(w, params, tokens)
    n2 = O.grad_norm(base["grads"], "l2")
    # a threshold above the norm changes nothing
    same = O.train_step(w, params, tokens, clip=("l2", 2.0 * n2))
    assert same["clip_scale"] == 1.0
    for k in params:
        assert np.array_equal(same["params"][k], base["params"][k])
    # below it, AdamW sees s g: m1 = 0.1 s g, v1 = 0.001 s^2 g^2 (t = 1)
    for kind in ("l2", "linf"):
        nrm = O.grad_norm(base["grads"], kind)
        out = O.train_step(w, params, tokens, clip=(kind, 0.25 * nrm))
        s_ = out["clip_scale"]
        assert abs(s_ - 0.25) < 1e-15 and out["grad_norm"] == nrm
        for k in params:
            g = base["grads"][k]
            np.testing.assert_allclose(out["m"][k], 0.1 * s_ * g, rtol=1e-14, atol=1e-300)
            np.testing.assert_allclose(out["v"][k], 0.001 * s_ * s_ * g * g, rtol=1e-14, atol=1e-300)


# ---------------------------------------------------------------------------
# Gradient accumulation (Transformer in Rust, "Configuration", "Features")
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("ci,S", [(1, 2), (1, 4), (3, 2)])
def test_accumulation_over_micro_batches_equals_full_batch(ci, S):
    # sequences are independent, so the mean of the micro-batch gradients is
    # the full batch's gradient; for bf16 storage the micro-batch dz is S times
    # the full batch's, an exact power-of-two scaling, so even the rounding
    # points agree
    w = W.get_config(ci)
    w = w.with_(B=4, L=1, T=16) if ci == 3 else w.with_(B=4)
    params = W.make_params(w, 42)
    tokens = W.make_tokens(w, 42)
    loss_full, cache = O.forward(w, params, tokens)
    full = O.backward(w, cache)
    micro = np.split(tokens, S, axis=0)
    wm = w.with_(B=w.B // S)
    loss_acc, acc = O.accumulated_grads(wm, params, micro)
    assert abs(loss_acc - loss_full) <= 1e-13 * abs(loss_full)
    for k in full:
        den = np.linalg.norm(full[k])
        assert np.linalg.norm(acc[k] - full[k]) <= 1e-12 * max(den, 1e-300), k


# --------------------------------------------------------------------------
# Key/value-cache forward (randyGPT, "Features": prefill once, then one
# single-token forward per new token; strata, "rules": the cached decoder
# equals the full forward to about 1e-9 at float64, with pre-rotated keys)
# --------------------------------------------------------------------------
KV_CASES = [("llama", 4, 4, {}), ("llama", 4, 2, {}), ("llama", 4, 1, {}), ("llama", 4, 4, {"R": 0}),
            ("parallel", 4, 4, {}), ("llama", 2, 2, {"rope_mode": "pairs", "R": 8})]


@pytest.mark.parametrize("block,H,Hkv,kw", KV_CASES)
def test_cached_decode_equals_full_forward(block, H, Hkv, kw):
    """Prefill a 3-token prompt, then decode one token at a time: the logits
    of every position equal that row of the full causal forward, and no
    sequence sees another's keys."""
    cfg = tiny(block=block, H=H, Hkv=Hkv, T=9, B=2, **kw)
    params = rand_params(cfg, seed=41)
    tokens = np.random.default_rng(42).integers(0, cfg.V, size=(2, cfg.T + 1))
    _, full = O.forward(cfg, params, tokens)
    zfull = full["z"].reshape(2, cfg.T, cfg.V)
    cache = O.kv_cache_new(cfg, 2, cfg.T + 3)
    got = [O.forward_cached(cfg, params, cache, tokens[:, :3])]
    for t in range(3, cfg.T):
        got.append(O.forward_cached(cfg, params, cache, tokens[:, t:t + 1]))
    got = np.concatenate(got, axis=1)
    assert cache["len"] == cfg.T
    assert np.max(np.abs(got - zfull)) <= 1e-9 * max(1.0, np.max(np.abs(zfull)))
    np.testing.assert_allclose(got, zfull, rtol=1e-11, atol=1e-12)


def test_chunked_prefill_equals_full_forward():
    """Chunks of 2, 4, 1 and 2 tokens: each query attends to every earlier
    cached position and to the earlier queries of its own chunk only."""
    cfg = tiny(H=4, Hkv=2, T=9, B=2)
    params = rand_params(cfg, seed=43)
    tokens = np.random.default_rng(44).integers(0, cfg.V, size=(2, cfg.T + 1))
    _, full = O.forward(cfg, params, tokens)
    cache = O.kv_cache_new(cfg, 2, cfg.T)
    got, t = [], 0
    for n in (2, 4, 1, 2):
        got.append(O.forward_cached(cfg, params, cache, tokens[:, t:t + n]))
        t += n
    np.testing.assert_allclose(np.concatenate(got, axis=1), full["z"].reshape(2, cfg.T, cfg.V),
                               rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("block,H,Hkv,kw", KV_CASES[:2] + KV_CASES[4:5])
def test_cache_holds_rotated_keys_and_values(block, H, Hkv, kw):
    """The cache rows of positions 0..T-1 are the full forward's rotated keys
    and its values, layer by layer; rows past the written length stay 0."""
    cfg = tiny(block=block, H=H, Hkv=Hkv, T=8, B=2, **kw)
    params = rand_params(cfg, seed=45)
    tokens = np.random.default_rng(46).integers(0, cfg.V, size=(2, cfg.T + 1))
    _, full = O.forward(cfg, params, tokens)
    cache = O.kv_cache_new(cfg, 2, cfg.T + 2)
    O.forward_cached(cfg, params, cache, tokens[:, :5])
    O.forward_cached(cfg, params, cache, tokens[:, 5:cfg.T])
    for l in range(cfg.L):
        np.testing.assert_allclose(cache["k"][l][:, :, :cfg.T], full["layers"][l]["k"], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(cache["v"][l][:, :, :cfg.T], full["layers"][l]["v"], rtol=1e-12, atol=1e-13)
        assert not np.any(cache["k"][l][:, :, cfg.T:]) and not np.any(cache["v"][l][:, :, cfg.T:])
    # the first head's keys at position 0 are the unrotated projection (angle 0)
    n1 = full["layers"][0]["n1"]
    qd = cfg.H * (cfg.C // cfg.H)
    d = cfg.C // cfg.H
    k0 = (n1 @ np.asarray(params["h0.qkvw"]).T)[0, qd:qd + d]
    np.testing.assert_allclose(cache["k"][0][0, 0, 0], k0, rtol=1e-12, atol=1e-13)


def test_cached_forward_rejects_overflowing_cache():
    cfg = tiny(T=4, B=1)
    params = rand_params(cfg, seed=47)
    cache = O.kv_cache_new(cfg, 1, 4)
    O.forward_cached(cfg, params, cache, np.zeros((1, 3), int))
    with pytest.raises(ValueError):
        O.forward_cached(cfg, params, cache, np.zeros((1, 2), int))


# --------------------------------------------------------------------------
# Inverted dropout (Hephaistos, "Architecture at a glance", "Design notes";
# randyGPT, "Architecture Details" and its default rate 0.1)
# --------------------------------------------------------------------------
def test_oracle_philox_published_vectors():
    """The oracle's own Philox-4x32-10 against the known-answer vectors its
    authors distribute with the generator."""
    from oracle.dropout import philox4x32_10
    cases = [
        ((0, 0, 0, 0), (0, 0), (0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8)),
        ((0xffffffff,) * 4, (0xffffffff,) * 2, (0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd)),
        ((0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344), (0xa4093822, 0x299f31d0),
         (0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1)),
    ]
    for ctr, key, want in cases:
        assert tuple(int(x) for x in philox4x32_10(ctr, key)) == want


def test_dropout_masks_rate_scale_and_independence():
    from oracle.dropout import dropout_multiplier
    p, rows, C = 0.1, 512, 384
    m = dropout_multiplier(p, 77, 1, 3, rows, C)
    kept = m > 0
    n = m.size
    # keep rate within 5 sigma of 1 - p; kept elements carry float32(1/(1-p))
    assert abs(kept.mean() - (1 - p)) < 5 * math.sqrt(p * (1 - p) / n)
    assert np.all(m[kept] == float(np.float32(1 / 0.9)))
    # inverted dropout preserves the mean: E[m] = (1-p) / (1-p)
    assert abs(m.mean() - 1.0) < 5 * math.sqrt(p * (1 - p) / n) / (1 - p) + 1e-7
    # other sites, layers and seeds draw other masks (agreement ~ p^2 + (1-p)^2)
    for other in (dropout_multiplier(p, 77, 2, 3, rows, C), dropout_multiplier(p, 77, 1, 4, rows, C),
                  dropout_multiplier(p, 78, 1, 3, rows, C)):
        agree = ((other > 0) == kept).mean()
        assert abs(agree - (p * p + (1 - p) ** 2)) < 0.01
    # no rate: every element kept with factor 1
    assert np.all(dropout_multiplier(0.0, 77, 1, 3, rows, C) == 1.0)


def test_dropout_rate_zero_is_the_plain_step():
    cfg = tiny()
    params = rand_params(cfg, seed=3)
    tokens = np.random.default_rng(4).integers(0, cfg.V, size=(cfg.B, cfg.T + 1))
    l0, c0 = O.forward(cfg, params, tokens)
    l1, c1 = O.forward(cfg.with_(dropout=0.0, dropout_seed=9), params, tokens)
    assert l0 == l1
    g0, g1 = O.backward(cfg, c0), O.backward(cfg, c1)
    assert all(np.array_equal(g0[k], g1[k]) for k in g0)


@pytest.mark.parametrize("block", ["llama", "parallel"])
def test_dropout_gradcheck_every_tensor(block):
    """With the masks fixed by the seed the loss is a smooth function of the
    weights: the backward through every dropout site against f64 central
    differences; a heavy rate so that every site drops elements."""
    cfg = tiny(block=block).with_(dropout=0.3, dropout_seed=12345)
    params = rand_params(cfg, seed=3)
    tokens = np.random.default_rng(4).integers(0, cfg.V, size=(cfg.B, cfg.T + 1))
    loss, cache = O.forward(cfg, params, tokens)
    assert loss != O.forward(cfg.with_(dropout=0.0), params, tokens)[0]
    grads = O.backward(cfg, cache)
    rng = np.random.default_rng(5)
    h = 1e-6
    for name, p in params.items():
        flat = p.reshape(-1)
        idx = rng.choice(flat.size, size=min(5, flat.size), replace=False)
        if name == "wte":
            idx = np.concatenate([idx, tokens[0, :3] * cfg.C])
        for i in idx:
            old = flat[i]
            flat[i] = old + h
            lp, _ = O.forward(cfg, params, tokens)
            flat[i] = old - h
            lm, _ = O.forward(cfg, params, tokens)
            flat[i] = old
            num = (lp - lm) / (2 * h)
            ana = grads[name].reshape(-1)[i]
            assert abs(ana - num) / max(abs(ana), abs(num), 1e-4) < 1e-5, (name, i, ana, num)


def test_attention_weight_dropout_gradcheck():
    """Attention with a dropout mask on its weights (site 3): the backward's
    dq, dk, dv (GQA: two query heads per KV head) against f64 central
    differences of L = sum(o * g), and D_i = sum_j p_ij dp_ij equal to
    do_i . o_i with the mask applied (the identity the kernels use)."""
    from oracle.dropout import dropout_multiplier
    rng = np.random.default_rng(21)
    B, H, Hkv, T, d = 2, 4, 2, 7, 4
    q = rng.standard_normal((B, H, T, d))
    k = rng.standard_normal((B, Hkv, T, d))
    v = rng.standard_normal((B, Hkv, T, d))
    g = rng.standard_normal((B, H, T, d))
    m = dropout_multiplier(0.4, 99, 3, 1, B * H * T, T).reshape(B, H, T, T)
    assert (m == 0).any() and (m > 0).any()
    o, _ = O.attention_fwd(q, k, v, m)
    assert not np.allclose(o, O.attention_fwd(q, k, v)[0])
    dq, dk, dv = O.attention_bwd(q, k, v, g, m)
    h = 1e-6
    for x, dx in ((q, dq), (k, dk), (v, dv)):
        for idx in [tuple(rng.integers(0, s) for s in x.shape) for _ in range(12)]:
            old = x[idx]
            x[idx] = old + h
            lp = np.sum(O.attention_fwd(q, k, v, m)[0] * g)
            x[idx] = old - h
            lm = np.sum(O.attention_fwd(q, k, v, m)[0] * g)
            x[idx] = old
            num = (lp - lm) / (2 * h)
            assert abs(dx[idx] - num) <= 1e-6 * max(1.0, abs(num)), (idx, dx[idx], num)
    # D from the probabilities equals do . o (o already holds the mask)
    s = np.einsum("bhid,bhjd->bhij", q, np.repeat(k, H // Hkv, axis=1)) / math.sqrt(d)
    s = np.where(np.tril(np.ones((T, T), bool)), s, -np.inf)
    p = np.exp(s - s.max(-1, keepdims=True))
    p /= p.sum(-1, keepdims=True)
    dp = np.einsum("bhid,bhjd->bhij", g, np.repeat(v, H // Hkv, axis=1)) * m
    assert np.allclose(np.sum(p * dp, -1), np.sum(g * o, -1), rtol=1e-12, atol=1e-12)
