"""slt_softmax_xent_noalloc (the entry point for callers that cannot
allocate: its per-row loss scratch is a static device array) against
slt_softmax_xent with a caller workspace: loss, lse and the logit gradient
written in place, bit for bit, on two calls in a row, the second with a
smaller input; and the host-side rejection of inputs beyond the static
scratch."""
import numpy as np
import pytest

import slt_workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

F32, BF16 = 0, 1


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from scratch_llama_transformer_amd import binding
    binding.load()
    return binding


def run_both(B, Bn, T, V, dtype, seed):
    rng = np.random.default_rng(seed)
    tdt = torch.bfloat16 if dtype == BF16 else torch.float32
    z0 = torch.from_numpy(rng.standard_normal((Bn * T, V)).astype(np.float32)).to(tdt).cuda()
    tok = torch.from_numpy(W.uniform_tokens(seed, Bn, T + 1, V)).cuda()
    out = []
    for noalloc in (False, True):
        z = z0.clone()
        loss = torch.full((1,), float("nan"), device="cuda")
        lse = torch.full((Bn * T,), float("nan"), device="cuda")
        if noalloc:
            B.slt_softmax_xent_noalloc(z, V, tok, Bn, T, T + 1, V, loss, lse, dtype)
        else:
            ws = torch.empty(4 * Bn * T, dtype=torch.uint8, device="cuda")
            B.slt_softmax_xent(z, V, tok, Bn, T, T + 1, V, loss, lse, dtype, ws)
        torch.cuda.synchronize()
        out.append((loss.cpu(), lse.cpu(), z.cpu()))
    return out


@pytest.mark.parametrize("dtype", [BF16, F32])
def test_noalloc_equals_workspace_call_twice(B, dtype):
    for Bn, T, V, seed in [(16, 256, 4096, 1), (3, 37, 500, 2)]:  # the second call smaller
        print("[case] softmax_xent_noalloc", Bn, T, V, dtype, flush=True)
        (l0, s0, z0), (l1, s1, z1) = run_both(B, Bn, T, V, dtype, seed)
        assert torch.isfinite(l0).all() and torch.equal(l0, l1), (l0, l1)
        assert torch.equal(s0, s1)
        assert torch.equal(z0, z1)


def test_noalloc_rejects_more_rows_than_its_scratch(B):
    z = torch.zeros((4, 8), dtype=torch.bfloat16, device="cuda")
    tok = torch.zeros((1, 5), dtype=torch.int32, device="cuda")
    loss = torch.zeros(1, device="cuda")
    with pytest.raises(B.SltError, match="static scratch"):
        B.slt_softmax_xent_noalloc(z, 8, tok, 1 << 11, 1 << 10, (1 << 10) + 1, 8, loss, None, BF16)
