"""ctypes binding of libslt.so.

Every ``slt_*`` function here has the name and argument order of the C entry
point in include/slt.h; it only turns torch tensors into device pointers,
passes the current HIP stream, and raises ``SltError`` on a non-zero status.
All arithmetic runs in the library's HIP kernels.  There is no fallback: if
the library is missing or no GPU is visible, calls raise.
"""
from __future__ import annotations

import ctypes as ct
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libslt.so")

F32, BF16 = 0, 1
ROPE_HALF, ROPE_PAIRS = 0, 1
BLOCK_LLAMA, BLOCK_PARALLEL = 0, 1
NORM_L2, NORM_LINF = 0, 1
STATUS = {0: "SLT_OK", 1: "SLT_EINVAL", 2: "SLT_EUNSUPPORTED", 3: "SLT_EHIP"}


class SltError(RuntimeError):
    def __init__(self, fn, code, msg):
        super().__init__(f"{fn}: {STATUS.get(code, code)}: {msg}")
        self.code = code


class slt_config(ct.Structure):
    _fields_ = [("V", ct.c_int32), ("C", ct.c_int32), ("H", ct.c_int32), ("Hkv", ct.c_int32),
                ("L", ct.c_int32), ("T", ct.c_int32), ("B", ct.c_int32), ("F", ct.c_int32),
                ("R", ct.c_int32), ("rope_mode", ct.c_int32), ("block", ct.c_int32), ("act", ct.c_int32),
                ("eps", ct.c_float), ("rope_base", ct.c_float), ("dropout", ct.c_float),
                ("dropout_seed", ct.c_uint64)]


class slt_tensor(ct.Structure):
    _fields_ = [("name", ct.c_char * 40), ("offset", ct.c_int64), ("numel", ct.c_int64),
                ("rows", ct.c_int64), ("cols", ct.c_int64), ("decay", ct.c_int32)]


_P = ct.c_void_p
_I32, _I64, _F = ct.c_int32, ct.c_int64, ct.c_float


class slt_gemm_group_item(ct.Structure):
    _fields_ = [("M", _I32), ("N", _I32), ("A", _P), ("lda", _I64), ("B", _P), ("ldb", _I64), ("C", _P),
                ("ldc", _I64), ("alpha", _F), ("accumulate", _I32)]

# name -> (restype, argtypes)
SIGNATURES = {
    "slt_last_error": (ct.c_char_p, []),
    "slt_version": (ct.c_char_p, []),
    "slt_validate": (_I32, [ct.POINTER(slt_config)]),
    "slt_param_layout": (_I32, [ct.POINTER(slt_config), ct.POINTER(slt_tensor), _I32,
                                ct.POINTER(_I32), ct.POINTER(_I64)]),
    "slt_workspace_bytes": (_I32, [ct.POINTER(slt_config), ct.POINTER(_I64), ct.POINTER(_I64)]),
    "slt_model_init": (_I32, [ct.POINTER(slt_config), ct.c_uint64, _F, _F, _P, _P]),
    "slt_cast_bf16": (_I32, [_P, _P, _I64, _P]),
    "slt_forward_loss": (_I32, [ct.POINTER(slt_config), _P, _P, _P, _P, _P, _P]),
    "slt_backward": (_I32, [ct.POINTER(slt_config), _P, _P, _P, _P, _P, _P]),
    "slt_backward_accumulate": (_I32, [ct.POINTER(slt_config), _P, _P, _P, _P, _P, _F, _P, _P, _P]),
    "slt_kv_cache_bytes": (_I32, [ct.POINTER(slt_config), _I32, _I32, _I32, ct.POINTER(_I64), ct.POINTER(_I64)]),
    "slt_forward_cached": (_I32, [ct.POINTER(slt_config), _P, _P, _I32, _I32, _I64, _I32, _P, _I32, _P, _I32,
                                  _P, _I64, _P]),
    "slt_adamw_step": (_I32, [_I64, _P, _P, _P, _P, _P, _I64, _F, _F, _F, _F, _F, _P, _P, _P]),
    "slt_clip_workspace_bytes": (_I64, []),
    "slt_clip_grad_norm": (_I32, [_I64, _P, _I32, _F, _P, _P, _P, _P]),
    "slt_backward_adamw": (_I32, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _F, _F, _F, _F, _F, _P, _P]),
    "slt_gemm": (_I32, [_I32, _I32, _I32, _P, _I64, _I32, _P, _I64, _I32, _P, _I64, _P, _I64,
                        _I32, _I32, _P, _I64, _P]),
    "slt_mlp_swiglu_fwd": (_I32, [_I32, _I32, _I32, _P, _P, _P, _P, _I32, _P]),
    "slt_proj_gelu_fwd": (_I32, [_I32, _I32, _I32, _P, _P, _P, _I64, _I32, _P, _I64, _I32, _P]),
    "slt_mlp_swiglu_bwd": (_I32, [_I32, _I32, _I32, _P, _P, _P, _P, _P, _I32, _P]),
    "slt_qkv_rope_fwd": (_I32, [_I32, _I32, _I32, _P, _P, _P, _I64, _I32, _I32, _I32, _I32, _I32, _I32, _P, _I32,
                                _P]),
    "slt_gemm_dw_group": (_I32, [ct.POINTER(slt_gemm_group_item), _I32, _I32, _P, _I64, _P]),
    "slt_embedding_fwd": (_I32, [_P, _I32, _I32, _I64, _P, _P, _I32, _I32, _I32, _P]),
    "slt_embedding_bwd_workspace": (_I64, [_I64, _I32]),
    "slt_embedding_bwd": (_I32, [_P, _I32, _I32, _I64, _P, _P, _I32, _I32, _I32, _P, _P]),
    "slt_rmsnorm_fwd": (_I32, [_P, _P, _P, _P, _I32, _I32, _F, _I32, _P]),
    "slt_norm_bwd_workspace": (_I64, [_I32, _I32]),
    "slt_rmsnorm_bwd": (_I32, [_P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _P, _P]),
    "slt_layernorm_fwd": (_I32, [_P, _P, _P, _P, _P, _P, _I32, _I32, _F, _I32, _P]),
    "slt_layernorm_bwd": (_I32, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _P, _P]),
    "slt_rope_table": (_I32, [_I32, _I32, _F, _P, _P]),
    "slt_rope_fwd": (_I32, [_P, _I64, _P, _I64, _I32, _I32, _I32, _I32, _I32, _I32, _P, _I32, _P]),
    "slt_rope_bwd": (_I32, [_P, _I64, _P, _I64, _I32, _I32, _I32, _I32, _I32, _I32, _P, _I32, _P]),
    "slt_attention_fwd_workspace": (_I64, [_I32, _I32, _I32, _I32, _I32, _I32]),
    "slt_attention_fwd": (_I32, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I32, _I32, _I32, _I32,
                                 _I32, _I32, _I32, _P, _I32, _P, _P]),
    "slt_attention_bwd_workspace": (_I64, [_I32, _I32, _I32, _I32, _I32, _I32]),
    "slt_attention_bwd": (_I32, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64,
                                 _I64, _I64, _I64, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _P, _I32,
                                 _P, _P]),
    "slt_swiglu_fwd": (_I32, [_P, _P, _P, _I32, _I32, _I64, _I64, _I64, _I32, _P]),
    "slt_swiglu_bwd": (_I32, [_P, _P, _P, _P, _P, _I32, _I32, _I64, _I64, _I64, _I64, _I64, _I32, _P]),
    "slt_gelu_fwd": (_I32, [_P, _P, _I32, _I32, _I64, _I64, _I32, _P]),
    "slt_gelu_bwd": (_I32, [_P, _P, _P, _I32, _I32, _I64, _I64, _I64, _I32, _P]),
    "slt_softmax_xent": (_I32, [_P, _I64, _P, _I32, _I32, _I64, _I32, _P, _P, _I32, _P, _P]),
    "slt_softmax_xent_noalloc": (_I32, [_P, _I64, _P, _I32, _I32, _I64, _I32, _P, _P, _I32, _P]),
    "slt_timing": (_I32, [_I32]),
    "slt_timing_read": (_I32, [_P, _P, _I32]),
    "slt_stream_copy": (_I32, [_P, _P, _I64, _I32, _P]),
    "slt_mfma_loop_flops": (_I64, [_I32, _I32, _I32]),
    "slt_mfma_loop": (_I32, [_I32, _I32, _I32, _P, _P]),
}

_lib = None


def load(path: str = LIB_PATH):
    """Load libslt.so and declare every signature.  Raises if it is absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run scratch_llama_transformer_amd.build first")
    lib = ct.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(x):
    """Device pointer of a tensor, None, or an int address."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not x.is_cuda:
        raise ValueError("expected a GPU tensor")
    return x.data_ptr()


def _stream(stream):
    import torch
    if stream is None:
        if not torch.cuda.is_available():
            raise RuntimeError("no GPU visible: libslt runs only on an MI355X (gfx950)")
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _check(name, code):
    if code != 0:
        raise SltError(name, code, (_lib.slt_last_error() or b"").decode())


def make_config(w) -> slt_config:
    """slt_config from a workload config (the fields of slt_workloads.Config)."""
    return slt_config(V=w.V, C=w.C, H=w.H, Hkv=w.Hkv, L=w.L, T=w.T, B=w.B, F=w.F, R=w.R,
                      rope_mode=ROPE_HALF if w.rope_mode == "half" else ROPE_PAIRS,
                      block=BLOCK_LLAMA if w.block == "llama" else BLOCK_PARALLEL,
                      act=BF16 if w.act == "bf16" else F32, eps=w.eps, rope_base=w.base,
                dropout=getattr(w, "dropout", 0.0), dropout_seed=getattr(w, "dropout_seed", 0))


# ---------------------------------------------------------------------------
# Host-only entry points
# ---------------------------------------------------------------------------
def slt_version() -> str:
    return load().slt_version().decode()


def slt_validate(cfg: slt_config) -> None:
    _check("slt_validate", load().slt_validate(ct.byref(cfg)))


def slt_param_layout(cfg: slt_config):
    lib = load()
    n, p = _I32(), _I64()
    _check("slt_param_layout", lib.slt_param_layout(ct.byref(cfg), None, 0, ct.byref(n), ct.byref(p)))
    arr = (slt_tensor * n.value)()
    _check("slt_param_layout", lib.slt_param_layout(ct.byref(cfg), arr, n.value, ct.byref(n), ct.byref(p)))
    return [dict(name=t.name.decode(), offset=t.offset, numel=t.numel, rows=t.rows, cols=t.cols,
                 decay=t.decay) for t in arr], p.value


def slt_workspace_bytes(cfg: slt_config):
    a, s = _I64(), _I64()
    _check("slt_workspace_bytes", load().slt_workspace_bytes(ct.byref(cfg), ct.byref(a), ct.byref(s)))
    return a.value, s.value


def slt_embedding_bwd_workspace(N, V) -> int:
    return int(load().slt_embedding_bwd_workspace(N, V))


def slt_norm_bwd_workspace(rows, C) -> int:
    return int(load().slt_norm_bwd_workspace(rows, C))


def slt_attention_fwd_workspace(B, T, H, Hkv, d, dtype) -> int:
    return int(load().slt_attention_fwd_workspace(B, T, H, Hkv, d, dtype))


def slt_attention_bwd_workspace(B, T, H, Hkv, d, dtype) -> int:
    return int(load().slt_attention_bwd_workspace(B, T, H, Hkv, d, dtype))


# ---------------------------------------------------------------------------
# Device entry points
# ---------------------------------------------------------------------------
def slt_model_init(cfg, seed, std, out_scale, master, stream=None):
    _check("slt_model_init", load().slt_model_init(ct.byref(cfg), seed, std, out_scale, _ptr(master),
                                                   _stream(stream)))


def slt_cast_bf16(src, dst, n, stream=None):
    _check("slt_cast_bf16", load().slt_cast_bf16(_ptr(src), _ptr(dst), n, _stream(stream)))


def slt_forward_loss(cfg, params, tokens, acts, scratch, loss, stream=None):
    _check("slt_forward_loss", load().slt_forward_loss(ct.byref(cfg), _ptr(params), _ptr(tokens), _ptr(acts),
                                                       _ptr(scratch), _ptr(loss), _stream(stream)))


def slt_backward_adamw(cfg, params, tokens, acts, scratch, grads, master, shadow, m, v, t, lr, beta1, beta2, eps,
                       wd, decay_mask=None, stream=None):
    _check("slt_backward_adamw", load().slt_backward_adamw(
        ct.byref(cfg), _ptr(params), _ptr(tokens), _ptr(acts), _ptr(scratch), _ptr(grads), _ptr(master),
        _ptr(shadow), _ptr(m), _ptr(v), t, lr, beta1, beta2, eps, wd, _ptr(decay_mask), _stream(stream)))


def slt_backward(cfg, params, tokens, acts, scratch, grads, stream=None):
    _check("slt_backward", load().slt_backward(ct.byref(cfg), _ptr(params), _ptr(tokens), _ptr(acts),
                                               _ptr(scratch), _ptr(grads), _stream(stream)))


def slt_backward_accumulate(cfg, params, tokens, acts, scratch, grads, scale, loss=None, loss_sum=None, stream=None):
    _check("slt_backward_accumulate", load().slt_backward_accumulate(
        ct.byref(cfg), _ptr(params), _ptr(tokens), _ptr(acts), _ptr(scratch), _ptr(grads), scale, _ptr(loss),
        _ptr(loss_sum), _stream(stream)))


def slt_kv_cache_bytes(cfg, B, Tq, Tmax):
    """(cache bytes, workspace bytes) of the key/value-cache forward."""
    cb, wb = ct.c_int64(0), ct.c_int64(0)
    _check("slt_kv_cache_bytes", load().slt_kv_cache_bytes(ct.byref(cfg), B, Tq, Tmax, ct.byref(cb), ct.byref(wb)))
    return cb.value, wb.value


def slt_forward_cached(cfg, params, tokens, B, Tq, ld_tokens, pos0, cache, Tmax, workspace, last_only, logits,
                       ld_logits, stream=None):
    _check("slt_forward_cached", load().slt_forward_cached(
        ct.byref(cfg), _ptr(params), _ptr(tokens), B, Tq, ld_tokens, pos0, _ptr(cache), Tmax, _ptr(workspace),
        int(last_only), _ptr(logits), ld_logits, _stream(stream)))


def slt_adamw_step(n, master, shadow, grads, m, v, t, lr, beta1, beta2, eps, wd, decay_mask=None, grad_scale=None,
                   stream=None):
    _check("slt_adamw_step", load().slt_adamw_step(n, _ptr(master), _ptr(shadow), _ptr(grads), _ptr(m), _ptr(v),
                                                   t, lr, beta1, beta2, eps, wd, _ptr(decay_mask), _ptr(grad_scale),
                                                   _stream(stream)))


def slt_clip_workspace_bytes() -> int:
    return int(load().slt_clip_workspace_bytes())


def slt_clip_grad_norm(n, grads, kind, max_norm, norm, scale, workspace, stream=None):
    _check("slt_clip_grad_norm", load().slt_clip_grad_norm(n, _ptr(grads), kind, max_norm, _ptr(norm), _ptr(scale),
                                                           _ptr(workspace), _stream(stream)))


def slt_gemm(M, N, K, A, lda, a_kmajor, B, ldb, b_kmajor, C, ldc, R, ldr, in_dtype, out_dtype,
             workspace=None, workspace_bytes=0, stream=None):
    _check("slt_gemm", load().slt_gemm(M, N, K, _ptr(A), lda, int(a_kmajor), _ptr(B), ldb, int(b_kmajor), _ptr(C),
                                       ldc, _ptr(R), ldr, in_dtype, out_dtype, _ptr(workspace), workspace_bytes,
                                       _stream(stream)))


def slt_mlp_swiglu_fwd(M, F, C, x, w13, ab, h, dtype, stream=None):
    _check("slt_mlp_swiglu_fwd", load().slt_mlp_swiglu_fwd(M, F, C, _ptr(x), _ptr(w13), _ptr(ab), _ptr(h), dtype,
                                                           _stream(stream)))


def slt_proj_gelu_fwd(M, N, K, x, w, y, ldy, col0, u, ldu, dtype, stream=None):
    _check("slt_proj_gelu_fwd", load().slt_proj_gelu_fwd(M, N, K, _ptr(x), _ptr(w), _ptr(y), ldy, col0, _ptr(u), ldu,
                                                         dtype, _stream(stream)))


def slt_qkv_rope_fwd(M, N, K, x, w, y, ldy, T, H, Hkv, d, R, rope_mode, cs, dtype, stream=None):
    _check("slt_qkv_rope_fwd", load().slt_qkv_rope_fwd(M, N, K, _ptr(x), _ptr(w), _ptr(y), ldy, T, H, Hkv, d, R,
                                                       rope_mode, _ptr(cs), dtype, _stream(stream)))


def slt_mlp_swiglu_bwd(M, F, C, dy, w2, ab, dab, dh_workspace, dtype, stream=None):
    _check("slt_mlp_swiglu_bwd", load().slt_mlp_swiglu_bwd(M, F, C, _ptr(dy), _ptr(w2), _ptr(ab), _ptr(dab),
                                                           _ptr(dh_workspace), dtype, _stream(stream)))


def slt_gemm_dw_group(items, K, workspace=None, workspace_bytes=0, stream=None):
    """items: sequence of (M, N, A, lda, B, ldb, C, ldc, alpha, accumulate)."""
    arr = (slt_gemm_group_item * len(items))()
    for i, (M, N, A, lda, Bm, ldb, C, ldc, alpha, acc) in enumerate(items):
        arr[i] = slt_gemm_group_item(M, N, _ptr(A), lda, _ptr(Bm), ldb, _ptr(C), ldc, alpha, int(acc))
    _check("slt_gemm_dw_group", load().slt_gemm_dw_group(arr, len(items), K, _ptr(workspace), workspace_bytes,
                                                         _stream(stream)))


def slt_embedding_fwd(tokens, B, T, ld_tokens, wte, x, V, C, dtype, stream=None):
    _check("slt_embedding_fwd", load().slt_embedding_fwd(_ptr(tokens), B, T, ld_tokens, _ptr(wte), _ptr(x), V, C,
                                                         dtype, _stream(stream)))


def slt_embedding_bwd(tokens, B, T, ld_tokens, dx, dwte, V, C, dtype, workspace, stream=None):
    _check("slt_embedding_bwd", load().slt_embedding_bwd(_ptr(tokens), B, T, ld_tokens, _ptr(dx), _ptr(dwte), V,
                                                         C, dtype, _ptr(workspace), _stream(stream)))


def slt_rmsnorm_fwd(x, g, y, rstd, rows, C, eps, dtype, stream=None):
    _check("slt_rmsnorm_fwd", load().slt_rmsnorm_fwd(_ptr(x), _ptr(g), _ptr(y), _ptr(rstd), rows, C, eps, dtype,
                                                     _stream(stream)))


def slt_rmsnorm_bwd(x, g, rstd, dy, dres, dx, dg, rows, C, dtype, workspace, stream=None):
    _check("slt_rmsnorm_bwd", load().slt_rmsnorm_bwd(_ptr(x), _ptr(g), _ptr(rstd), _ptr(dy), _ptr(dres), _ptr(dx),
                                                     _ptr(dg), rows, C, dtype, _ptr(workspace), _stream(stream)))


def slt_layernorm_fwd(x, gamma, beta, y, mean, rstd, rows, C, eps, dtype, stream=None):
    _check("slt_layernorm_fwd", load().slt_layernorm_fwd(_ptr(x), _ptr(gamma), _ptr(beta), _ptr(y), _ptr(mean),
                                                         _ptr(rstd), rows, C, eps, dtype, _stream(stream)))


def slt_layernorm_bwd(x, gamma, mean, rstd, dy, dres, dx, dgamma, dbeta, rows, C, dtype, workspace, stream=None):
    _check("slt_layernorm_bwd", load().slt_layernorm_bwd(_ptr(x), _ptr(gamma), _ptr(mean), _ptr(rstd), _ptr(dy),
                                                         _ptr(dres), _ptr(dx), _ptr(dgamma), _ptr(dbeta), rows, C,
                                                         dtype, _ptr(workspace), _stream(stream)))


def slt_rope_table(T, R, base, cs, stream=None):
    _check("slt_rope_table", load().slt_rope_table(T, R, base, _ptr(cs), _stream(stream)))


def slt_rope_fwd(x, ldx, y, ldy, B, T, nheads, d, R, rope_mode, cs, dtype, stream=None):
    _check("slt_rope_fwd", load().slt_rope_fwd(_ptr(x), ldx, _ptr(y), ldy, B, T, nheads, d, R, rope_mode, _ptr(cs),
                                               dtype, _stream(stream)))


def slt_rope_bwd(dy, lddy, dx, lddx, B, T, nheads, d, R, rope_mode, cs, dtype, stream=None):
    _check("slt_rope_bwd", load().slt_rope_bwd(_ptr(dy), lddy, _ptr(dx), lddx, B, T, nheads, d, R, rope_mode,
                                               _ptr(cs), dtype, _stream(stream)))


def slt_attention_fwd(q, k, v, o, lse, o_res, ldq, ldk, ldv, ldo, B, T, H, Hkv, d, R, rope_mode, cs, dtype,
                      workspace=None, stream=None):
    _check("slt_attention_fwd", load().slt_attention_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(o_res),
                                                         ldq, ldk,
                                                         ldv, ldo, B, T, H, Hkv, d, R, rope_mode, _ptr(cs), dtype,
                                                         _ptr(workspace), _stream(stream)))


def slt_attention_bwd(q, k, v, o, o_res, dout, lse, dq, dk, dv, ldq, ldk, ldv, ldo, lddo, lddq, lddk, lddv,
                      B, T, H, Hkv, d, R, rope_mode, cs, dtype, workspace, stream=None):
    _check("slt_attention_bwd", load().slt_attention_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(o_res), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), ldq, ldk, ldv,
        ldo, lddo, lddq, lddk, lddv, B, T, H, Hkv, d, R, rope_mode, _ptr(cs), dtype, _ptr(workspace),
        _stream(stream)))


def slt_swiglu_fwd(a, b, h, rows, F, lda, ldb, ldh, dtype, stream=None):
    _check("slt_swiglu_fwd", load().slt_swiglu_fwd(_ptr(a), _ptr(b), _ptr(h), rows, F, lda, ldb, ldh, dtype,
                                                   _stream(stream)))


def slt_swiglu_bwd(a, b, dh, da, db, rows, F, lda, ldb, lddh, ldda, lddb, dtype, stream=None):
    _check("slt_swiglu_bwd", load().slt_swiglu_bwd(_ptr(a), _ptr(b), _ptr(dh), _ptr(da), _ptr(db), rows, F, lda,
                                                   ldb, lddh, ldda, lddb, dtype, _stream(stream)))


def slt_gelu_fwd(a, u, rows, F, lda, ldu, dtype, stream=None):
    _check("slt_gelu_fwd", load().slt_gelu_fwd(_ptr(a), _ptr(u), rows, F, lda, ldu, dtype, _stream(stream)))


def slt_gelu_bwd(a, du, da, rows, F, lda, lddu, ldda, dtype, stream=None):
    _check("slt_gelu_bwd", load().slt_gelu_bwd(_ptr(a), _ptr(du), _ptr(da), rows, F, lda, lddu, ldda, dtype,
                                               _stream(stream)))


def slt_softmax_xent(z, ldz, tokens, B, T, ld_tokens, V, loss, lse, dtype, workspace, stream=None):
    _check("slt_softmax_xent", load().slt_softmax_xent(_ptr(z), ldz, _ptr(tokens), B, T, ld_tokens, V, _ptr(loss),
                                                       _ptr(lse), dtype, _ptr(workspace), _stream(stream)))


def slt_softmax_xent_noalloc(z, ldz, tokens, B, T, ld_tokens, V, loss, lse, dtype, stream=None):
    _check("slt_softmax_xent_noalloc", load().slt_softmax_xent_noalloc(_ptr(z), ldz, _ptr(tokens), B, T, ld_tokens, V,
                                                                       _ptr(loss), _ptr(lse), dtype, _stream(stream)))


TIMING_CLASSES = ("gemm_fwd", "gemm_dx", "gemm_dw", "attention_fwd", "attention_bwd")


def slt_timing(on: bool):
    _check("slt_timing", load().slt_timing(1 if on else 0))


def slt_timing_read():
    """{class: (milliseconds, launches)} recorded since the previous read."""
    n = len(TIMING_CLASSES)
    ms = (ct.c_double * n)()
    cnt = (ct.c_int64 * n)()
    _check("slt_timing_read", load().slt_timing_read(ms, cnt, n))
    return {c: (ms[i], int(cnt[i])) for i, c in enumerate(TIMING_CLASSES)}


def slt_stream_copy(src, dst, nbytes, variant=0, stream=None):
    _check("slt_stream_copy", load().slt_stream_copy(_ptr(src), _ptr(dst), nbytes, variant, _stream(stream)))


def slt_mfma_loop_flops(blocks, iters, variant=0) -> int:
    return int(load().slt_mfma_loop_flops(blocks, iters, variant))


def slt_mfma_loop(blocks, iters, out, variant=0, stream=None):
    _check("slt_mfma_loop", load().slt_mfma_loop(blocks, iters, variant, _ptr(out), _stream(stream)))
