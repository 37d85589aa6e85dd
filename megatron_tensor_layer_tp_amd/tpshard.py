"""Thin ctypes binding of libtpshard (include/tpshard.h).

Each function has the C entry point's name and argument order and only
marshals arguments: a torch tensor (or any object with ``data_ptr()``) becomes
its device address, ``None`` becomes NULL, and ``stream=None`` means torch's
current stream on the current device.  Every computation happens in the
library's HIP kernels; there is no fallback.  A non-zero status raises
``TpError`` carrying ``tp_last_error()``.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtpshard.so")

TP_OK, TP_EINVAL, TP_ESHAPE, TP_EDTYPE, TP_EALIGN, TP_EWORKSPACE, TP_EHIP, TP_EUNSUPPORTED = range(8)
TP_DT_F32, TP_DT_BF16 = 0, 1
TP_ACT_RELU, TP_ACT_GELU = 0, 1

_i64 = ctypes.c_int64
_int = ctypes.c_int
_vp = ctypes.c_void_p
_sz = ctypes.c_size_t

_SIGS = {
    "tp_mlp_fwd": (_int, [_int, _int, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "tp_mlp_bwd_workspace": (_sz, [_int, _i64, _i64, _i64]),
    "tp_mlp_bwd": (_int, [_int, _int, _i64, _i64, _i64] + [_vp] * 9 + [_vp, _sz, _vp]),
    "tp_swiglu_fwd": (_int, [_int, _i64, _i64, _i64] + [_vp] * 8 + [_vp]),
    "tp_swiglu_bwd_workspace": (_sz, [_int, _i64, _i64, _i64]),
    "tp_swiglu_bwd": (_int, [_int, _i64, _i64, _i64] + [_vp] * 12 + [_vp, _sz, _vp]),
    "tp_attn_proj_fwd": (_int, [_int, _i64, _i64, _i64, _i64] + [_vp] * 10 + [_vp]),
    "tp_attn_proj_bwd_workspace": (_sz, [_int, _i64, _i64, _i64, _i64]),
    "tp_attn_proj_bwd": (_int, [_int, _i64, _i64, _i64, _i64] + [_vp] * 16 + [_vp, _sz, _vp]),
    "tp_lm_head_fwd": (_int, [_int, _i64, _i64, _i64, _vp, _vp, _vp, _vp]),
    "tp_vocab_ce": (_int, [_i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp]),
    "tp_vocab_ce_bwd": (_int, [_int, _i64, _i64, _i64] + [_vp] * 6 + [_vp]),
    "tp_attn_core_fwd": (_int, [_int, _i64, _i64, _i64, _i64] + [_vp] * 5 + [_vp]),
    "tp_attn_core_bwd_workspace": (_sz, [_int, _i64, _i64, _i64, _i64]),
    "tp_attn_core_bwd": (_int, [_int, _i64, _i64, _i64, _i64] + [_vp] * 9 + [_vp, _sz, _vp]),
    "tp_attn_out_bwd_workspace": (_sz, [_int, _i64, _i64, _i64]),
    "tp_attn_out_bwd": (_int, [_int, _i64, _i64, _i64] + [_vp] * 5 + [_vp, _sz, _vp]),
    "tp_attn_qkv_bwd_workspace": (_sz, [_int, _i64, _i64, _i64, _i64]),
    "tp_attn_qkv_bwd": (_int, [_int, _i64, _i64, _i64, _i64] + [_vp] * 11 + [_vp, _sz, _vp]),
    "tp_sp_ln_fwd": (_int, [_int, _i64, _i64, ctypes.c_float, ctypes.c_float] + [_vp] * 9 + [_vp]),
    "tp_sp_ln_bwd_workspace": (_sz, [_int, _i64, _i64]),
    "tp_sp_ln_bwd": (_int, [_int, _i64, _i64, ctypes.c_float] + [_vp] * 11 + [_vp, _sz, _vp]),
    "tp_lm_head_ce_workspace": (_sz, [_int, _i64, _i64, _i64]),
    "tp_lm_head_ce_fwd": (_int, [_int, _i64, _i64, _i64, _i64] + [_vp] * 6 + [_vp, _sz, _vp]),
    "tp_lm_head_ce_noalloc_max_bytes": (_sz, []),
    "tp_lm_head_ce_fwd_noalloc": (_int, [_int, _i64, _i64, _i64, _i64] + [_vp] * 6 + [_vp]),
    "tp_vocab_embed": (_int, [_int, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _vp]),
    "tp_status_string": (ctypes.c_char_p, [_int]),
    "tp_last_error": (ctypes.c_char_p, []),
    "tp_abi_version": (_int, []),
}

EXPORTS = tuple(_SIGS)


class TpError(RuntimeError):
    def __init__(self, call: str, status: int, detail: str):
        super().__init__(f"{call} failed with status {status}: {detail}")
        self.status = status
        self.call = call


_lib = None


def lib() -> ctypes.CDLL:
    """Load libtpshard.so (built in-tree by build.py); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m megatron_tensor_layer_tp_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _call(name, *args):
    st = getattr(lib(), name)(*args)
    if st != TP_OK:
        detail = lib().tp_last_error().decode(errors="replace")
        raise TpError(name, st, detail)
    return st


def tp_status_string(status: int) -> str:
    return lib().tp_status_string(status).decode()


def tp_last_error() -> str:
    return lib().tp_last_error().decode(errors="replace")


def tp_abi_version() -> int:
    return lib().tp_abi_version()


# ---------------------------------------------------------------- MLP
def tp_mlp_fwd(act, dt, s, h, ft, X, W1, W2, Z, H, Y, stream=None):
    return _call("tp_mlp_fwd", act, dt, s, h, ft, _ptr(X), _ptr(W1), _ptr(W2), _ptr(Z), _ptr(H),
                 _ptr(Y), _stream(stream))


def tp_mlp_bwd_workspace(dt, s, h, ft) -> int:
    return lib().tp_mlp_bwd_workspace(dt, s, h, ft)


def tp_mlp_bwd(act, dt, s, h, ft, X, W1, W2, Z, H, dY, dX, dW1, dW2, ws, ws_bytes, stream=None):
    return _call("tp_mlp_bwd", act, dt, s, h, ft, _ptr(X), _ptr(W1), _ptr(W2), _ptr(Z), _ptr(H),
                 _ptr(dY), _ptr(dX), _ptr(dW1), _ptr(dW2), _ptr(ws), ws_bytes, _stream(stream))


# ---------------------------------------------------------------- SwiGLU
def tp_swiglu_fwd(dt, s, h, ft, X, Wg, Wu, Wd, G, U, A, Y, stream=None):
    return _call("tp_swiglu_fwd", dt, s, h, ft, _ptr(X), _ptr(Wg), _ptr(Wu), _ptr(Wd), _ptr(G),
                 _ptr(U), _ptr(A), _ptr(Y), _stream(stream))


def tp_swiglu_bwd_workspace(dt, s, h, ft) -> int:
    return lib().tp_swiglu_bwd_workspace(dt, s, h, ft)


def tp_swiglu_bwd(dt, s, h, ft, X, Wg, Wu, Wd, G, U, A, dY, dX, dWg, dWu, dWd, ws, ws_bytes,
                  stream=None):
    return _call("tp_swiglu_bwd", dt, s, h, ft, _ptr(X), _ptr(Wg), _ptr(Wu), _ptr(Wd), _ptr(G),
                 _ptr(U), _ptr(A), _ptr(dY), _ptr(dX), _ptr(dWg), _ptr(dWu), _ptr(dWd), _ptr(ws),
                 ws_bytes, _stream(stream))


# ---------------------------------------------------------------- attention projections
def tp_attn_proj_fwd(dt, s, h, dq, dkv, X, Wq, Wk, Wv, O, Wo, Q, K, V, Y, stream=None):
    return _call("tp_attn_proj_fwd", dt, s, h, dq, dkv, _ptr(X), _ptr(Wq), _ptr(Wk), _ptr(Wv),
                 _ptr(O), _ptr(Wo), _ptr(Q), _ptr(K), _ptr(V), _ptr(Y), _stream(stream))


def tp_attn_proj_bwd_workspace(dt, s, h, dq, dkv) -> int:
    return lib().tp_attn_proj_bwd_workspace(dt, s, h, dq, dkv)


def tp_attn_proj_bwd(dt, s, h, dq, dkv, X, Wq, Wk, Wv, O, Wo, dQ, dK, dV, dY, dX, dWq, dWk, dWv,
                     dO, dWo, ws, ws_bytes, stream=None):
    return _call("tp_attn_proj_bwd", dt, s, h, dq, dkv, _ptr(X), _ptr(Wq), _ptr(Wk), _ptr(Wv),
                 _ptr(O), _ptr(Wo), _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(dY), _ptr(dX), _ptr(dWq),
                 _ptr(dWk), _ptr(dWv), _ptr(dO), _ptr(dWo), _ptr(ws), ws_bytes, _stream(stream))


def tp_attn_out_bwd_workspace(dt, s, h, dq) -> int:
    return lib().tp_attn_out_bwd_workspace(dt, s, h, dq)


def tp_attn_out_bwd(dt, s, h, dq, O, Wo, dY, dO, dWo, ws, ws_bytes, stream=None):
    return _call("tp_attn_out_bwd", dt, s, h, dq, _ptr(O), _ptr(Wo), _ptr(dY), _ptr(dO), _ptr(dWo), _ptr(ws),
                 ws_bytes, _stream(stream))


def tp_attn_qkv_bwd_workspace(dt, s, h, dq, dkv) -> int:
    return lib().tp_attn_qkv_bwd_workspace(dt, s, h, dq, dkv)


def tp_attn_qkv_bwd(dt, s, h, dq, dkv, X, Wq, Wk, Wv, dQ, dK, dV, dX, dWq, dWk, dWv, ws, ws_bytes, stream=None):
    return _call("tp_attn_qkv_bwd", dt, s, h, dq, dkv, _ptr(X), _ptr(Wq), _ptr(Wk), _ptr(Wv), _ptr(dQ), _ptr(dK),
                 _ptr(dV), _ptr(dX), _ptr(dWq), _ptr(dWk), _ptr(dWv), _ptr(ws), ws_bytes, _stream(stream))


# ---------------------------------------------------------------- vocab
def tp_lm_head_fwd(dt, s, h, Vs, Hf, Wlm, logits, stream=None):
    return _call("tp_lm_head_fwd", dt, s, h, Vs, _ptr(Hf), _ptr(Wlm), _ptr(logits), _stream(stream))


def tp_attn_core_fwd(dt, s, nq, nkv, d, Q, K, V, O, lse, stream=None):
    return _call("tp_attn_core_fwd", dt, s, nq, nkv, d, _ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(lse),
                 _stream(stream))


def tp_attn_core_bwd_workspace(dt, s, nq, nkv, d) -> int:
    return lib().tp_attn_core_bwd_workspace(dt, s, nq, nkv, d)


def tp_attn_core_bwd(dt, s, nq, nkv, d, Q, K, V, O, dO, lse, dQ, dK, dV, ws, ws_bytes, stream=None):
    return _call("tp_attn_core_bwd", dt, s, nq, nkv, d, _ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(dO), _ptr(lse),
                 _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(ws), ws_bytes, _stream(stream))


def tp_sp_ln_fwd(dt, n, h, p, eps, y, x, mask, gamma, beta, u, z, mean, rstd, stream=None):
    return _call("tp_sp_ln_fwd", dt, n, h, p, eps, _ptr(y), _ptr(x), _ptr(mask), _ptr(gamma), _ptr(beta),
                 _ptr(u), _ptr(z), _ptr(mean), _ptr(rstd), _stream(stream))


def tp_sp_ln_bwd_workspace(dt, n, h):
    return lib().tp_sp_ln_bwd_workspace(dt, n, h)


def tp_sp_ln_bwd(dt, n, h, p, dz, dun, u, mean, rstd, gamma, mask, dx, dy, dgamma, dbeta, ws, ws_bytes,
                 stream=None):
    return _call("tp_sp_ln_bwd", dt, n, h, p, _ptr(dz), _ptr(dun), _ptr(u), _ptr(mean), _ptr(rstd), _ptr(gamma),
                 _ptr(mask), _ptr(dx), _ptr(dy), _ptr(dgamma), _ptr(dbeta), _ptr(ws), ws_bytes, _stream(stream))


def tp_vocab_ce_bwd(dt, s, Vs, vocab_start, logits, target, gmax, gsum, dloss, dlogits, stream=None):
    return _call("tp_vocab_ce_bwd", dt, s, Vs, vocab_start, _ptr(logits), _ptr(target), _ptr(gmax), _ptr(gsum),
                 _ptr(dloss), _ptr(dlogits), _stream(stream))


def tp_lm_head_ce_workspace(dt, s, h, Vs):
    return lib().tp_lm_head_ce_workspace(dt, s, h, Vs)


def tp_lm_head_ce_fwd(dt, s, h, Vs, vocab_start, Hf, Wlm, target, lmax, lsumexp, tlogit, ws, ws_bytes,
                      stream=None):
    return _call("tp_lm_head_ce_fwd", dt, s, h, Vs, vocab_start, _ptr(Hf), _ptr(Wlm), _ptr(target), _ptr(lmax),
                 _ptr(lsumexp), _ptr(tlogit), _ptr(ws), ws_bytes, _stream(stream))


def tp_lm_head_ce_noalloc_max_bytes() -> int:
    return lib().tp_lm_head_ce_noalloc_max_bytes()


def tp_lm_head_ce_fwd_noalloc(dt, s, h, Vs, vocab_start, Hf, Wlm, target, lmax, lsumexp, tlogit, stream=None):
    return _call("tp_lm_head_ce_fwd_noalloc", dt, s, h, Vs, vocab_start, _ptr(Hf), _ptr(Wlm), _ptr(target),
                 _ptr(lmax), _ptr(lsumexp), _ptr(tlogit), _stream(stream))


def tp_vocab_ce(s, Vs, vocab_start, logits, target, lmax, lsumexp, tlogit, stream=None):
    return _call("tp_vocab_ce", s, Vs, vocab_start, _ptr(logits), _ptr(target), _ptr(lmax),
                 _ptr(lsumexp), _ptr(tlogit), _stream(stream))


def tp_vocab_embed(dt, n, Vs, h, vocab_start, ids, table, out, stream=None):
    return _call("tp_vocab_embed", dt, n, Vs, h, vocab_start, _ptr(ids), _ptr(table), _ptr(out),
                 _stream(stream))
