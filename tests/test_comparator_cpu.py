"""The bf16 whole-step comparator (fixed limits, tests/parity.py) accepts
other valid bf16 computations of the step (the oracle with relative jitter in
front of each activation store stands for another fp32 summation order) and
rejects plausible mistakes, planted here in the oracle on the CPU."""
import numpy as np
import pytest

import oracle as O
import oracle.model as M
import slt_workloads as W
from parity import COMPANION_JITTER, check_bf16_step_tensor


def cfg():
    return W.get_config(3).with_(B=2, T=64, L=2, V=512, C=128, H=4, Hkv=4, F=256, R=32)


def run(w, params, tokens, jitter=0.0, seed=0):
    loss, cache = O.forward(w, params, tokens, jitter=jitter, seed=seed)
    return loss, O.backward(w, cache)


@pytest.fixture(scope="module")
def base():
    w = cfg()
    params = W.make_params(w, 5)
    tokens = W.make_tokens(w, 5)
    loss, ref = run(w, params, tokens)
    return w, params, tokens, loss, ref


def passes(got, ref):
    try:
        for k in ref:
            check_bf16_step_tensor(got[k], ref[k], k)
        return True
    except AssertionError:
        return False


@pytest.mark.parametrize("jitter,seed", [(2.0 ** -24, 7), (COMPANION_JITTER, 1), (COMPANION_JITTER, 9)])
def test_another_valid_rounding_order_passes(base, jitter, seed):
    w, params, tokens, loss, ref = base
    _, other = run(w, params, tokens, jitter=jitter, seed=seed)
    assert passes(other, ref)


@pytest.mark.parametrize("bug", ["rope_direction", "rmsnorm_no_eps_mean", "attention_dv_dropped_group",
                                 "swiglu_missing_term"])
def test_planted_mistakes_fail(base, monkeypatch, bug):
    w, params, tokens, loss, ref = base
    if bug == "rope_direction":
        orig = M.rope_apply
        monkeypatch.setattr(M, "rope_apply", lambda u, c, s, R, mode, inverse=False: orig(u, c, s, R, mode,
                                                                                           not inverse))
    elif bug == "rmsnorm_no_eps_mean":
        monkeypatch.setattr(M, "rmsnorm_fwd", lambda x, g, eps: (
            x / np.sqrt(np.sum(x * x, -1, keepdims=True)) * g, 1.0 / np.sqrt(np.sum(x * x, -1))))
    elif bug == "attention_dv_dropped_group":
        orig = M.attention_bwd
        monkeypatch.setattr(M, "attention_bwd", lambda q, k, v, do, drop=None: (lambda r: (r[0], r[1], 0.9 * r[2]))(
            orig(q, k, v, do, drop)))
    elif bug == "swiglu_missing_term":
        monkeypatch.setattr(M, "swiglu_bwd", lambda a, b, dh: (
            np.asarray(dh) * np.asarray(b) * M._sigmoid(np.asarray(a)), np.asarray(dh) * np.asarray(a) *
            M._sigmoid(np.asarray(a))))
    _, got = run(w, params, tokens)
    assert not passes(got, ref)
