"""Host-side checks of the C ABI (no kernel runs): the library loads, exports
every function include/slt.h declares, reports the parameter layout of the
workloads, validates configurations and sizes the arena."""
import ctypes as ct
import os
import re

import numpy as np
import pytest

import slt_workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "scratch_llama_transformer_amd", "libslt.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libslt.so not built")


def header_functions():
    src = open(os.path.join(ROOT, "include", "slt.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(slt_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    from scratch_llama_transformer_amd import binding as B
    lib = B.load()
    names = header_functions()
    assert len(names) >= 25
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) - {"slt_philox4x32_10"} == set(B.SIGNATURES)


def test_version_string():
    from scratch_llama_transformer_amd import binding as B
    assert "gfx950" in B.slt_version()


@pytest.mark.parametrize("i", [1, 2, 3, 4, 5])
def test_layout_matches_workload_tensors(i):
    from scratch_llama_transformer_amd import binding as B
    w = W.get_config(i)
    layout, n = B.slt_param_layout(B.make_config(w))
    specs = W.param_specs(w)
    assert n == W.n_params(w)
    assert [t["name"] for t in layout] == [s[0] for s in specs]
    off = 0
    for t, (name, shape, _) in zip(layout, specs):
        assert t["offset"] == off
        assert t["numel"] == int(np.prod(shape))
        assert (t["rows"], t["cols"]) == ((1, shape[0]) if len(shape) == 1 else shape)
        assert t["decay"] == 1
        off += t["numel"]
    # fused matrices: [w1; w3] and [qkvw; fc_in] are adjacent in the flat buffer
    by = {t["name"]: t for t in layout}
    if w.block == "llama":
        assert by["h0.w3"]["offset"] == by["h0.w1"]["offset"] + by["h0.w1"]["numel"]
    else:
        assert by["h0.fc_in"]["offset"] == by["h0.qkvw"]["offset"] + by["h0.qkvw"]["numel"]


@pytest.mark.parametrize("bad,code", [
    (dict(H=3), 1), (dict(Hkv=3), 1), (dict(R=5), 1), (dict(R=64), 1), (dict(V=0), 1),
    (dict(rope_mode=7), 1), (dict(block=2), 1), (dict(act=5), 1), (dict(C=2048, H=16), 2),
    (dict(dropout=1.0), 1), (dict(dropout=-0.25), 1), (dict(dropout=float("nan")), 1),
])
def test_validation_rejects(bad, code):
    from scratch_llama_transformer_amd import binding as B
    c = B.make_config(W.get_config(3))
    for k, v in bad.items():
        setattr(c, k, v)
    with pytest.raises(B.SltError) as e:
        B.slt_validate(c)
    assert e.value.code == code
    assert B.load().slt_last_error()


def test_workspace_sizes_grow_with_batch():
    from scratch_llama_transformer_amd import binding as B
    w = W.get_config(3)
    a1, s1 = B.slt_workspace_bytes(B.make_config(w.with_(B=8)))
    a2, s2 = B.slt_workspace_bytes(B.make_config(w))
    assert 0 < a1 < a2 and 0 < s1 <= s2
    # the arena holds at least the bf16 logits of the step
    assert a2 >= w.N * w.V * 2


def test_philox_known_answers():
    """Known-answer vectors of Philox-4x32-10 from its authors' distribution."""
    from scratch_llama_transformer_amd import binding as B
    lib = B.load()
    fn = lib.slt_philox4x32_10
    fn.restype = None
    U4, U2 = ct.c_uint32 * 4, ct.c_uint32 * 2
    cases = [
        ((0, 0, 0, 0), (0, 0), (0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8)),
        ((0xffffffff,) * 4, (0xffffffff,) * 2, (0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd)),
        ((0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344), (0xa4093822, 0x299f31d0),
         (0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1)),
    ]
    for ctr, key, want in cases:
        out = U4()
        fn(U4(*ctr), U2(*key), out)
        assert tuple(out) == want, [hex(x) for x in out]


def test_host_calls_reject_bad_arguments_before_launch():
    from scratch_llama_transformer_amd import binding as B
    lib = B.load()
    # negative sizes and NULL operands are caught on the host; stream NULL is fine
    assert lib.slt_gemm(-1, 4, 4, None, 4, 1, None, 4, 1, None, 4, None, 0, 1, 1, None, 0, None) == 1
    assert lib.slt_gemm(4, 4, 4, None, 4, 1, None, 4, 1, None, 4, None, 0, 1, 1, None, 0, None) == 1
    assert lib.slt_adamw_step(10, None, None, None, None, None, 1, 1e-3, 0.9, 0.999, 1e-8, 0.1, None, None, None) == 1
    assert lib.slt_clip_grad_norm(-1, None, 0, 1.0, None, None, None, None) == 1
    assert lib.slt_clip_grad_norm(8, None, 2, 1.0, None, None, None, None) == 1      # bad kind
    assert lib.slt_clip_grad_norm(8, None, 0, 0.0, None, None, None, None) == 1      # max_norm <= 0
    assert B.slt_clip_workspace_bytes() > 0
    assert lib.slt_attention_fwd(None, None, None, None, None, None, 8, 8, 8, 8, 1, 4, 2, 1, 128, 0, 0, None, 1,
                                 None, None) == 2
    # a bf16 head dim the tiled kernels take needs room for one rotated bf16 copy of q and k
    assert B.slt_attention_fwd_workspace(2, 64, 4, 2, 48, 1) == 2 * 6 * 64 * 48 * 2
    assert B.slt_attention_fwd_workspace(2, 64, 4, 2, 48, 0) == 0
    assert B.slt_attention_fwd_workspace(2, 64, 4, 2, 24, 1) == 0
    assert B.slt_attention_bwd_workspace(2, 64, 4, 2, 24, 1) == 2 * 4 * 64 * 4
    assert lib.slt_softmax_xent(None, 10, None, 1, 4, 5, 10, None, None, 1, None, None) == 1
    # RoPE: odd R, R > d, bad mode, narrow strides, NULL pointers
    assert lib.slt_rope_fwd(None, 16, None, 16, 1, 4, 2, 8, 7, 0, None, 1, None) == 1
    assert lib.slt_rope_bwd(None, 16, None, 16, 1, 4, 2, 8, 10, 0, None, 1, None) == 1
    assert lib.slt_rope_fwd(None, 16, None, 16, 1, 4, 2, 8, 8, 5, None, 1, None) == 1
    assert lib.slt_rope_fwd(None, 12, None, 16, 1, 4, 2, 8, 8, 0, None, 1, None) == 1
    assert lib.slt_rope_fwd(None, 16, None, 16, 1, 4, 2, 8, 8, 0, None, 1, None) == 1
    assert lib.slt_rope_fwd(None, 16, None, 16, 0, 4, 2, 8, 8, 0, None, 1, None) == 0   # nothing to do
    # QKV with RoPE: heads wider than N, odd R
    assert lib.slt_qkv_rope_fwd(4, 16, 8, None, None, None, 16, 4, 2, 2, 8, 8, 0, None, 1, None) == 1
    assert lib.slt_qkv_rope_fwd(4, 64, 8, None, None, None, 64, 4, 2, 2, 8, 7, 0, None, 1, None) == 1
    # machine-bound kernels: bad variant, size not a multiple of 16, NULL
    assert lib.slt_stream_copy(None, None, 32, 5, None) == 1
    assert lib.slt_stream_copy(None, None, 24, 0, None) == 1
    assert lib.slt_stream_copy(None, None, 32, 0, None) == 1
    assert lib.slt_stream_copy(None, None, 0, 0, None) == 0
    assert lib.slt_mfma_loop(8, 4, 3, None, None) == 1
    assert lib.slt_mfma_loop(0, 4, 0, None, None) == 1
    assert B.slt_mfma_loop_flops(8, 4, 0) == 8 * 4 * 4 * 8 * 16384
    assert B.slt_mfma_loop_flops(8, 4, 1) == 8 * 4 * 4 * 8 * 32768
    assert B.slt_mfma_loop_flops(8, 4, 2) == 8 * 4 * 4 * 16 * 16384
    # launch timing: NULL outputs or a negative class count are rejected; with
    # nothing recorded every class reads zero
    assert lib.slt_timing_read(None, None, 5) == 1
    ms, cnt = (ct.c_double * 5)(), (ct.c_int64 * 5)()
    assert lib.slt_timing_read(ms, cnt, -1) == 1
    assert lib.slt_timing(0) == 0
    assert B.slt_timing_read() == {c: (0.0, 0) for c in B.TIMING_CLASSES}


def test_kv_cache_sizes():
    """Cache = per layer K and V [B, Hkv, Tmax, d] (256-byte aligned each),
    then the RoPE table [Tmax, R] fp32; bad sizes are rejected on the host."""
    from scratch_llama_transformer_amd import binding as B
    a256 = lambda n: (n + 255) // 256 * 256
    for i in (1, 3, 4, 5):
        w = W.get_config(i)
        cfg = B.make_config(w)
        d, es = w.C // w.H, (2 if w.act == "bf16" else 4)
        for Bn, Tq, Tmax in ((1, 1, 16), (3, 5, 300)):
            cb, wb = B.slt_kv_cache_bytes(cfg, Bn, Tq, Tmax)
            assert cb == 2 * w.L * a256(Bn * w.Hkv * Tmax * d * es) + a256(Tmax * max(w.R, 2) * 4)
            assert wb > 0
        for bad in ((0, 1, 16), (1, 0, 16), (1, 17, 16), (1, 1, 0)):
            with pytest.raises(B.SltError):
                B.slt_kv_cache_bytes(cfg, *bad)
