"""Key/value-cache forward (prefill, chunked continuation, single-token
decode) of the HIP path against the oracle's cached forward on the same
seeded weights and tokens.  The oracle's cached forward is itself pinned to
the full causal forward (tests/test_oracle_pins.py), so these cases also tie
the GPU's decode to the full forward.

Comparators: fp32 logits normwise 1e-5.  bf16 logits come out of several
layers of stored bf16 activations, where a value within an fp32 summation-
order difference of a rounding boundary may round either way and later
layers amplify the flip; as for the whole training step, the GPU logits are
held to the fixed whole-step rule of tests/parity.py (normwise 2e-2, at most
0.5 % of the elements beyond their band, none beyond 8 bands); the spread
between the oracle and its companion (the same cached forward with 2^-20
relative jitter before each activation store) is reported beside it."""
import numpy as np
import pytest

import oracle as O
import slt_workloads as W
from parity import COMPANION_JITTER, check, check_bf16_step_tensor

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from scratch_llama_transformer_amd import binding, trainer
    return binding, trainer


def say(*a):
    print("[case]", *a, flush=True)


def compute_params(trainer, w, params):
    ts = trainer.TrainStep(w.with_(B=1), params=params)
    return ts.compute_params, ts


def logits_np(z):
    return z.float().cpu().numpy().astype(np.float64)


class OracleRun:
    """The oracle's cached forward, and for bf16 its jittered companion."""

    def __init__(self, w, params, Bn, Tmax):
        self.w, self.params = w, params
        self.cache = O.kv_cache_new(w, Bn, Tmax)
        self.comp = O.kv_cache_new(w, Bn, Tmax) if w.act == "bf16" else None
        self.calls = 0

    def __call__(self, ids):
        ref = O.forward_cached(self.w, self.params, self.cache, ids)
        comp = None
        if self.comp is not None:
            self.calls += 1
            comp = O.forward_cached(self.w, self.params, self.comp, ids, jitter=COMPANION_JITTER, seed=self.calls)
        return ref, comp


def check_logits(got, ref, comp, act, name):
    """Rows are (sequence, position) pairs; the band floor is each row's rms."""
    V = ref.shape[-1]
    got, ref = got.reshape(-1, V), ref.reshape(-1, V)
    if act == "f32":
        check(got, ref, act, name)
    else:
        nw, q, worst, frac = check_bf16_step_tensor(got, ref, name, comp.reshape(-1, V), "kv-cache forward")
        print(f"[result] {name}: normwise {nw:.2e}, 99.9% {q:.2f} bands, worst {worst:.2f} bands, "
              f"beyond band {frac:.2e}")


# (config, batch, layers, prompt, chunk after the prompt, single-token steps, Tmax)
#  - tiny fp32: a 5-token prompt goes through the cache kernel (below 16 rows)
#  - d=256 fp32 and d=384 bf16: the prompt through the training attention,
#    then a 3-token chunk over the cache, then single tokens
#  - GQA and the parallel block (partial even-odd RoPE): prompts past 256
#    positions, so the cache attention splits keys into chunks and merges
DECODE_CASES = [
    (1, 2, None, 5, None, 10, 16),
    (2, 2, 2, 40, 3, 4, 64),
    (3, 3, 2, 64, 3, 4, 80),
    (4, 1, 2, 270, None, 3, 300),
    (5, 1, 2, 300, 2, 3, 320),
]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("ci,Bn,L,P,chunk,steps,Tmax", DECODE_CASES)
def test_cached_forward_matches_oracle(lib, ci, Bn, L, P, chunk, steps, Tmax):
    binding, trainer = lib
    w = W.get_config(ci)
    w = w.with_(L=L or w.L, T=Tmax)
    say("cached forward", w.name, dict(B=Bn, L=w.L, prompt=P, chunk=chunk, steps=steps, Tmax=Tmax))
    params = W.make_params(w, 3000 + ci)
    ids = W.make_tokens(w, 3000 + ci, B=Bn)[:, :Tmax]
    cp, _keep = compute_params(trainer, w, params)
    run = trainer.CachedForward(w, cp, Bn, Tmax, max(P, chunk or 1))
    orc = OracleRun(w, params, Bn, Tmax)
    calls = [P] + ([chunk] if chunk else []) + [1] * steps
    pos = 0
    for Tq in calls:
        part = np.ascontiguousarray(ids[:, pos:pos + Tq])
        z = run.run(torch.from_numpy(part).cuda())
        ref, comp = orc(part)
        torch.cuda.synchronize()
        check_logits(logits_np(z), ref, comp, w.act, f"logits at positions {pos}..{pos + Tq - 1}")
        pos += Tq
    print(f"[result] {w.name}: {len(calls)} calls, {pos} positions")


@pytest.mark.timeout(300)
def test_last_only_logits_and_reuse(lib):
    """last_only returns the last row of each sequence; a second sequence
    started in the same cache (pos0 = 0 again) overwrites the first."""
    binding, trainer = lib
    w = W.get_config(3).with_(L=2, T=48)
    params = W.make_params(w, 3100)
    ids = W.make_tokens(w, 3100, B=2)[:, :48]
    cp, _keep = compute_params(trainer, w, params)
    for first in (ids[::-1].copy(), ids):
        run = trainer.CachedForward(w, cp, 2, 48, 40)
        orc = OracleRun(w, params, 2, 48)
        if first is not ids:
            run.run(torch.from_numpy(np.ascontiguousarray(first[:, :40])).cuda())
            run.pos = 0
        z = run.run(torch.from_numpy(np.ascontiguousarray(ids[:, :40])).cuda(), last_only=True)
        ref, comp = orc(ids[:, :40])
        torch.cuda.synchronize()
        check_logits(logits_np(z), ref[:, -1], comp[:, -1], w.act, "last-row logits")
        z = run.run(torch.from_numpy(np.ascontiguousarray(ids[:, 40:41])).cuda(), last_only=True)
        ref, comp = orc(ids[:, 40:41])
        check_logits(logits_np(z), ref[:, -1], comp[:, -1], w.act, "decode logits")


@pytest.mark.timeout(600)
def test_full_size_decode_sampled_sequences(lib):
    """The d=384 workload at its full batch of 64 sequences: a 192-token
    prefill and four single-token steps; sequences are independent, so the
    oracle runs only sequences 0, 17 and 63 and those rows are compared."""
    binding, trainer = lib
    w = W.get_config(3)
    Tmax = w.T
    params = W.make_params(w, 3200)
    ids = W.make_tokens(w, 3200)[:, :Tmax]
    cp, _keep = compute_params(trainer, w, params)
    run = trainer.CachedForward(w, cp, w.B, Tmax, 192)
    pick = [0, 17, 63]
    orc = OracleRun(w, params, len(pick), Tmax)
    pos = 0
    for Tq in [192, 1, 1, 1, 1]:
        say("full-size decode", w.name, "positions", pos, pos + Tq - 1)
        z = run.run(torch.from_numpy(np.ascontiguousarray(ids[:, pos:pos + Tq])).cuda())
        ref, comp = orc(np.ascontiguousarray(ids[pick, pos:pos + Tq]))
        torch.cuda.synchronize()
        check_logits(logits_np(z)[pick], ref, comp, w.act, f"logits at {pos}")
        pos += Tq


def test_rejects_overflow_and_bad_sizes(lib):
    binding, trainer = lib
    w = W.get_config(1)
    cfg = binding.make_config(w)
    with pytest.raises(binding.SltError):
        binding.slt_kv_cache_bytes(cfg, 1, 20, 16)
    cb, wb = binding.slt_kv_cache_bytes(cfg, 1, 4, 16)
    cache = torch.empty(cb, dtype=torch.uint8, device="cuda")
    ws = torch.empty(max(wb, 256), dtype=torch.uint8, device="cuda")
    tok = torch.zeros(1, 4, dtype=torch.int32, device="cuda")
    z = torch.empty(4, w.V, device="cuda")
    ts = trainer.TrainStep(w)
    with pytest.raises(binding.SltError):  # 14 + 4 > 16
        binding.slt_forward_cached(cfg, ts.compute_params, tok, 1, 4, 4, 14, cache, 16, ws, 0, z, w.V)
