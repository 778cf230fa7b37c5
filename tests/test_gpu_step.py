"""Whole-step parity (forward loss, every gradient, every post-AdamW weight)
of the HIP path against the oracle on the same seeded inputs, plus
properties that hold at the full benchmark sizes."""
import math
import os

import numpy as np
import pytest

import oracle as O
import slt_workloads as W
from parity import (COMPANION_JITTER, LOSS_TOL, check, check_bf16_step_tensor, check_bf16_step_weights,
                    check_weights)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def TS():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from scratch_llama_transformer_amd.trainer import TrainStep
    return TrainStep


def say(*a):
    print("[case]", *a, flush=True)


def run_step(TS, w, seed):
    params = W.make_params(w, seed)
    tokens = W.make_tokens(w, seed)
    ts = TS(w, params=params)
    tok = torch.from_numpy(tokens).cuda()
    ts.forward(tok)
    torch.cuda.synchronize()
    loss = float(ts.loss.item())
    ts.backward(tok)
    ts.adamw()
    torch.cuda.synchronize()
    return params, tokens, ts, loss


# (config index, batch, layers): every width, vocabulary and sequence length of
# the five configurations; batch and depth cut so the oracle stays in seconds.
STEP_CASES = [(1, None, None), (2, 8, None), (3, 8, None), (4, 1, 2), (5, 1, 2)]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("ci,Bn,L", STEP_CASES)
def test_full_step_parity(TS, ci, Bn, L):
    w = W.get_config(ci)
    w = w.with_(B=Bn or w.B, L=L or w.L)
    say("step", w)
    params, tokens, ts, loss = run_step(TS, w, 1000 + ci)
    ref = O.train_step(w, params, tokens)
    assert abs(loss - ref["loss"]) <= LOSS_TOL[w.act] * abs(ref["loss"]), (loss, ref["loss"])
    grads = ts.unpack(ts.grads)
    new = ts.unpack(ts.master)
    ties = 0
    if w.act == "f32":
        for name in params:
            check(grads[name], ref["grads"][name], w.act, f"grad {name}")
            ties += check_weights(new[name], ref["params"][name], ref["grads"][name], w.act, f"weight {name}")
    else:
        ties = check_bf16_step(w, params, tokens, grads, new, ref, f"step {w.name} B={w.B} L={w.L}")
    print(f"[result] {w.name} loss gpu {loss:.7f} oracle {ref['loss']:.7f}; tie-exempt weights {ties}")


def check_bf16_step(w, params, tokens, grads, new, ref, case, companion=True, grad_scale=1.0):
    """Every gradient and post-AdamW weight of a bf16 step under the fixed
    whole-step rule (tests/parity.py); the oracle's companion (2^-20 jitter
    in front of each activation store) is computed for the record only.
    Returns the number of sign-tie exempt weights."""
    comp = None
    if companion:
        _, ccache = O.forward(w, params, tokens, jitter=COMPANION_JITTER, seed=1)
        comp = O.backward(w, ccache)
    worst, ties, n = (0.0, 0.0, 0.0, 0.0), 0, 0
    for name in params:
        st = check_bf16_step_tensor(grads[name], ref["grads"][name], f"grad {name}",
                                    comp[name] if comp else None, case)
        worst = tuple(max(a, b) for a, b in zip(worst, st))
        ties += check_bf16_step_weights(new[name], ref["params"][name], grads[name], ref["grads"][name],
                                        params[name], w, f"weight {name}", case, grad_scale)
        n += np.asarray(params[name]).size
    print(f"[result] {case}: worst over gradients: normwise {worst[0]:.2e}, 99.9% quantile {worst[1]:.2f} bands, "
          f"worst element {worst[2]:.2f} bands, beyond band {worst[3]:.2e}; exempt weights {ties} of {n}")
    return ties


# The widest model the library accepts (C = 4096, 64 heads of 64): every norm,
# GEMM and attention kernel at its largest row width, one layer, 64 tokens.
MAX_WIDTH_CASES = [
    dict(V=384, C=4096, H=64, Hkv=8, L=1, T=64, B=1, F=11008, R=64),
    dict(V=384, C=4096, H=64, Hkv=64, L=1, T=64, B=1, F=4096, R=32),
]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("ci,over", [(4, MAX_WIDTH_CASES[0]), (5, MAX_WIDTH_CASES[1])])
def test_full_step_at_maximum_width(TS, ci, over):
    w = W.get_config(ci).with_(**over)
    say("maximum-width step", w)
    params, tokens, ts, loss = run_step(TS, w, 1700 + ci)
    ref = O.train_step(w, params, tokens)
    assert abs(loss - ref["loss"]) <= LOSS_TOL[w.act] * abs(ref["loss"]), (loss, ref["loss"])
    grads = ts.unpack(ts.grads)
    new = ts.unpack(ts.master)
    check_bf16_step(w, params, tokens, grads, new, ref, f"maximum width {w.name} C={w.C}")
    print(f"[result] {w.name} C={w.C}: loss gpu {loss:.7f} oracle {ref['loss']:.7f}")


# The whole batch of each bf16 workload (16384 tokens) through one layer:
# every product at its full token count (the fused SwiGLU launches, the
# grouped weight gradients, the 256 x 256 tiles, the attention kernels at the
# full sequence length).  Loss, every gradient and every post-AdamW weight
# against the oracle under the fixed whole-step rule (no companion: the
# oracle alone takes a minute or two at these sizes).
@pytest.mark.timeout(1200)
@pytest.mark.parametrize("ci", [3, 4, 5])
def test_full_batch_step_one_layer(TS, ci):
    w = W.get_config(ci).with_(L=1)
    say("full-batch step", w)
    params, tokens, ts, loss = run_step(TS, w, 1000 + ci)
    ref = O.train_step(w, params, tokens)
    assert abs(loss - ref["loss"]) <= LOSS_TOL[w.act] * abs(ref["loss"]), (loss, ref["loss"])
    grads = ts.unpack(ts.grads)
    new = ts.unpack(ts.master)
    check_bf16_step(w, params, tokens, grads, new, ref, f"full batch {w.name} B={w.B} L=1", companion=False)


# (config index, overrides, dropout p): p exactly representable in binary32,
# the library's type for it, so both sides draw the same threshold and scale.
# The attention kernels covered: the generic fp32 ones (tiny, d=256), the
# bf16 chunked ones (d=384; parallel block at T=2048) and the bf16 64-key
# dK/dV kernel (T not a multiple of 4).
DROPOUT_CASES = [(1, {}, 0.25), (2, dict(B=8), 0.125), (3, dict(B=8), 0.125), (3, dict(B=2, L=2, T=254), 0.25),
                 (5, dict(B=1, L=2), 0.25)]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("ci,over,pdrop", DROPOUT_CASES)
def test_full_step_with_dropout(TS, ci, over, pdrop):
    """Inverted dropout at the embedding output, the attention weights, the
    attention projection (the parallel block's combined projection) and the
    MLP output: the GPU's masks are regenerated from the same Philox counters
    as the oracle's, so loss, gradients and post-AdamW weights meet the same
    bars as without dropout."""
    w = W.get_config(ci)
    w = w.with_(**over, dropout=pdrop, dropout_seed=0x1234_5678_9ABC + ci)
    say("dropout step", w)
    params, tokens, ts, loss = run_step(TS, w, 1500 + ci)
    ref = O.train_step(w, params, tokens)
    plain = O.train_step(w.with_(dropout=0.0), params, tokens)
    gd = math.sqrt(sum(float(np.sum((ref["grads"][k] - plain["grads"][k]) ** 2)) for k in params))
    gn = math.sqrt(sum(float(np.sum(plain["grads"][k] ** 2)) for k in params))
    assert gd > 0.1 * gn, (gd, gn)      # the masks change the gradient
    assert abs(loss - ref["loss"]) <= LOSS_TOL[w.act] * abs(ref["loss"]), (loss, ref["loss"])
    grads = ts.unpack(ts.grads)
    new = ts.unpack(ts.master)
    if w.act == "f32":
        for name in params:
            check(grads[name], ref["grads"][name], w.act, f"grad {name}")
            check_weights(new[name], ref["params"][name], ref["grads"][name], w.act, f"weight {name}")
    else:
        check_bf16_step(w, params, tokens, grads, new, ref, f"dropout {w.name} p={pdrop} T={w.T}")
    print(f"[result] {w.name} p={pdrop} loss gpu {loss:.7f} oracle {ref['loss']:.7f} (no dropout "
          f"{plain['loss']:.7f}); gradient change {gd / gn:.2f} of its norm")


def test_dropout_key_advances_per_step(TS):
    """step() moves to the next key after its backward: a second forward on
    the same weights and tokens draws other masks (another loss), and going
    back to the first key reproduces the first loss bit for bit."""
    w = W.get_config(1).with_(dropout=0.25, dropout_seed=77)
    params = W.make_params(w, 1600)
    tok = torch.from_numpy(W.make_tokens(w, 1600)).cuda()
    ts = TS(w, params=params)
    ts.forward(tok)
    first = float(ts.loss.item())
    ts.next_masks()
    assert ts.cfg.dropout_seed == 78
    ts.forward(tok)
    second = float(ts.loss.item())
    ts.cfg.dropout_seed = 77
    ts.forward(tok)
    again = float(ts.loss.item())
    assert second != first and again == first, (first, second, again)
    ts.step(tok)
    assert ts.cfg.dropout_seed == 78


@pytest.mark.timeout(900)
@pytest.mark.parametrize("ci,Bn,kind", [(1, None, "l2"), (2, 8, "linf"), (3, 8, "l2")])
def test_full_step_with_gradient_clipping(TS, ci, Bn, kind):
    """Global-norm clipping between the backward and AdamW: the GPU's norm and
    factor against the oracle's, and the clipped step's weights."""
    w = W.get_config(ci)
    w = w.with_(B=Bn or w.B)
    say("clipped step", w, kind)
    params = W.make_params(w, 2000 + ci)
    tokens = W.make_tokens(w, 2000 + ci)
    plain = O.train_step(w, params, tokens)
    max_norm = 0.3 * O.grad_norm(plain["grads"], kind)        # clipping active
    ref = O.train_step(w, params, tokens, clip=(kind, max_norm))
    ts = TS(w, params=params, clip=(kind, max_norm))
    tok = torch.from_numpy(tokens).cuda()
    ts.forward(tok)
    ts.backward(tok)
    ts.adamw()
    torch.cuda.synchronize()
    nrm, sc = (float(x) for x in ts.gnorm.cpu().numpy())
    tol = 1e-5 if w.act == "f32" else 2e-2
    assert abs(nrm - ref["grad_norm"]) <= tol * ref["grad_norm"], (nrm, ref["grad_norm"])
    assert abs(sc - ref["clip_scale"]) <= tol * ref["clip_scale"], (sc, ref["clip_scale"])
    grads = ts.unpack(ts.grads)
    new = ts.unpack(ts.master)
    for name in params:
        if w.act == "f32":
            check_weights(new[name], ref["params"][name], ref["grads"][name], w.act, f"weight {name}")
            # every element: the oracle's AdamW on the GPU's gradient times the GPU's factor
            own, _, _ = O.adamw(params[name], sc * grads[name], 0.0, 0.0, 1, w.lr, w.beta1, w.beta2, w.adam_eps,
                                w.wd)
            check(new[name], own, "f32", f"weight {name} from the GPU gradient")
        else:
            check_bf16_step_tensor(grads[name], ref["grads"][name], f"grad {name}", None, f"clipped {w.name}")
            check_bf16_step_weights(new[name], ref["params"][name], grads[name], ref["grads"][name], params[name],
                                    w, f"weight {name}", f"clipped {w.name}", sc)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("ci,Bn,S", [(1, 4, 2), (2, 8, 2), (3, 8, 4)])
def test_gradient_accumulation(TS, ci, Bn, S):
    """S micro-batches through slt_backward_accumulate (scale 1/S) give the
    full batch's gradient: against the GPU's own full-batch step (same
    rounding points for power-of-two S, so only summation order differs) and
    against the oracle's accumulation."""
    w = W.get_config(ci).with_(B=Bn)
    say("accumulation", w, S)
    params = W.make_params(w, 3000 + ci)
    tokens = W.make_tokens(w, 3000 + ci)
    full = TS(w, params=params)
    tok = torch.from_numpy(tokens).cuda()
    full.forward(tok)
    full.backward(tok)
    torch.cuda.synchronize()
    full_loss = float(full.loss.item())
    gfull = full.unpack(full.grads)
    wm = w.with_(B=Bn // S)
    ts = TS(wm, params=params)
    micro = [torch.from_numpy(np.ascontiguousarray(t)).cuda() for t in np.split(tokens, S, axis=0)]
    loss = ts.accumulate(micro)
    gacc = ts.unpack(ts.grads)
    assert abs(loss - full_loss) <= 1e-5 * abs(full_loss), (loss, full_loss)
    for name in gfull:
        check(gacc[name], gfull[name], "f32", f"accumulated vs full-batch {name}")
    ref_loss, ref = O.accumulated_grads(wm, params, np.split(tokens, S, axis=0))
    assert abs(loss - ref_loss) <= LOSS_TOL[w.act] * abs(ref_loss)
    for name in ref:
        if w.act == "f32":
            check(gacc[name], ref[name], "f32", f"accumulated vs oracle {name}")
        else:
            check_bf16_step_tensor(gacc[name], ref[name], f"accumulated {name}", None, f"accumulation {w.name} S={S}")


def test_step_is_deterministic(TS):
    w = W.get_config(3).with_(B=4, L=2)
    say("determinism", w)
    params = W.make_params(w, 7)
    tok = torch.from_numpy(W.make_tokens(w, 7)).cuda()
    outs = []
    for _ in range(2):
        ts = TS(w, params=params)
        ts.forward(tok)
        ts.backward(tok)
        torch.cuda.synchronize()
        outs.append((ts.loss.clone(), ts.grads.clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


@pytest.mark.timeout(300)
@pytest.mark.parametrize("ci,over", [(1, {}), (3, dict(B=4, L=2)), (5, dict(B=1, L=1, T=256)),
                                     (2, dict(B=2, L=2, dropout=0.125, dropout_seed=5))])
def test_backward_adamw_equals_separate_calls(TS, ci, over):
    """slt_backward_adamw (each layer's update enqueued as its gradients
    become final) against slt_backward then slt_adamw_step: gradients,
    master weights, moments and the bf16 copy bitwise equal over two steps."""
    w = W.get_config(ci).with_(**over)
    say("fused AdamW", w)
    params = W.make_params(w, 41 + ci)
    tok = torch.from_numpy(W.make_tokens(w, 41 + ci)).cuda()
    a, b = TS(w, params=params), TS(w, params=params)
    for _ in range(2):
        a.forward(tok)
        a.backward(tok)
        a.adamw()
        b.forward(tok)
        b.backward_adamw(tok)
    torch.cuda.synchronize()
    for name in ("grads", "master", "m", "v", "shadow"):
        x, y = getattr(a, name), getattr(b, name)
        assert (x is None) == (y is None), name
        if x is not None:
            assert torch.equal(x, y), name


@pytest.mark.timeout(300)
def test_backward_from_two_host_threads(TS):
    """Two models stepped from two host threads at once, each on its own
    torch stream: the backward's second stream and events are shared per
    device (enqueues take turns), and every gradient equals the one a single
    thread computes."""
    import threading
    cases = [W.get_config(3).with_(B=2, L=2, T=128), W.get_config(5).with_(B=1, L=1, T=256)]
    toks = [torch.from_numpy(W.make_tokens(w, 31 + i)).cuda() for i, w in enumerate(cases)]
    params = [W.make_params(w, 31 + i) for i, w in enumerate(cases)]
    ref = []
    for w, p, tok in zip(cases, params, toks):
        ts = TS(w, params=p)
        ts.forward(tok)
        ts.backward(tok)
        torch.cuda.synchronize()
        ref.append(ts.grads.clone())
    steppers = [TS(w, params=p) for w, p in zip(cases, params)]
    torch.cuda.synchronize()  # their set-up ran on the default stream
    got, errors = [None, None], []

    def run(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                from scratch_llama_transformer_amd import binding as B
                ts = steppers[i]
                for _ in range(3):
                    B.slt_forward_loss(ts.cfg, ts.compute_params, toks[i], ts.acts, ts.scratch, ts.loss, s)
                    B.slt_backward(ts.cfg, ts.compute_params, toks[i], ts.acts, ts.scratch, ts.grads, s)
                s.synchronize()
                got[i] = ts.grads.clone()
        except Exception as e:  # reported below
            errors.append(e)

    th = [threading.Thread(target=run, args=(i,)) for i in range(2)]
    for t in th:
        t.start()
    for t in th:
        t.join()
    assert not errors, errors
    for i in range(2):
        assert torch.equal(got[i], ref[i]), i


@pytest.mark.parametrize("ci", [3, 5])
def test_full_size_forward_rows_match_oracle_on_sampled_sequences(TS, ci):
    """At the full benchmark shape, the per-position losses of a few sampled
    sequences equal an oracle forward over those sequences alone (attention
    never crosses sequences)."""
    w = W.get_config(ci)
    if ci == 5:
        w = w.with_(L=2)
    say("full-size rows", w)
    params = W.make_params(w, 2000 + ci)
    tokens = W.make_tokens(w, 2000 + ci)
    ts = TS(w, params=params)
    ts.forward(torch.from_numpy(tokens).cuda())
    torch.cuda.synchronize()
    rowloss = ts.scratch[: 4 * w.N].view(torch.float32).cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(ci)
    for b in rng.choice(w.B, size=2, replace=False):
        _, cache = O.forward(w.with_(B=1), params, tokens[b:b + 1])
        z = cache["z"]
        y = tokens[b, 1:]
        mx = z.max(1)
        ref = mx + np.log(np.exp(z - mx[:, None]).sum(1)) - z[np.arange(w.T), y]
        got = rowloss[b * w.T:(b + 1) * w.T]
        err = np.abs(got - ref) / np.abs(ref)
        tol = 2e-3 if w.act == "bf16" else 1e-5
        assert err.max() < tol, err.max()


@pytest.mark.parametrize("ci", [3, 4])
def test_full_size_zero_head_properties(TS, ci):
    """Full benchmark shape with lm_head = 0: the loss is ln V, every gradient
    below the head is exactly zero, and every weight except lm_head only
    decays: theta (1 - lr wd)."""
    w = W.get_config(ci)
    say("zero head", w)
    ts = TS(w, seed=ci)
    by = {t["name"]: t for t in ts.layout}
    h = by["lm_head"]
    ts.master[h["offset"]:h["offset"] + h["numel"]].zero_()
    ts.refresh_shadow()
    theta0 = ts.master.clone()
    tok = torch.from_numpy(W.make_tokens(w, 3000 + ci)).cuda()
    ts.forward(tok)
    torch.cuda.synchronize()
    assert abs(ts.loss.item() - math.log(w.V)) < 2e-6 * math.log(w.V)
    ts.backward(tok)
    ts.adamw()
    torch.cuda.synchronize()
    g = ts.grads.clone()
    g[h["offset"]:h["offset"] + h["numel"]] = 0
    assert int(torch.count_nonzero(g)) == 0
    body = torch.ones(ts.n, dtype=torch.bool, device="cuda")
    body[h["offset"]:h["offset"] + h["numel"]] = False
    expect = theta0 - w.lr * (w.wd * theta0)
    diff = (ts.master - expect)[body].abs()
    assert float(diff.max()) <= 2 * 2 ** -23 * float(theta0[body].abs().max())


@pytest.mark.timeout(300)
@pytest.mark.parametrize("ci,over", [(3, dict(B=4, L=2)), (5, dict(B=1, L=2, T=256)), (2, dict(B=2, L=2))])
def test_launch_timing_counts_and_leaves_results_unchanged(TS, ci, over):
    """slt_timing brackets every launch of the five classes in a step (the
    counts the step's structure fixes: one weight-gradient bracket per layer,
    around the layer's grouped launch or its separate fp32 products; every
    class's time positive), and a step with it on gives bitwise the
    gradients and weights of one with it off."""
    from scratch_llama_transformer_amd import binding as B
    w = W.get_config(ci).with_(**over)
    say("launch timing", w)
    params = W.make_params(w, 11)
    tok = torch.from_numpy(W.make_tokens(w, 11)).cuda()
    outs = []
    B.slt_timing_read()  # forget earlier records
    for on in (False, True):
        ts = TS(w, params=params)
        B.slt_timing(on)
        try:
            ts.step(tok)
            torch.cuda.synchronize()
        finally:
            B.slt_timing(False)
        outs.append((ts.grads.clone(), ts.master.clone()))
        rec = B.slt_timing_read()
        if not on:
            assert all(n == 0 for _, n in rec.values()), rec
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    per = 4 if w.block == "llama" else 2  # projections per layer
    want = {"gemm_fwd": per * w.L + 1, "gemm_dx": per * w.L + 1, "gemm_dw": w.L, "attention_fwd": w.L,
            "attention_bwd": w.L}
    for k, n in want.items():
        ms, got = rec[k]
        assert got == n, (k, got, n)
        assert ms > 0, (k, ms)
