"""CPU checks of the C ABI: the library loads, exports every entry point the
header declares, and rejects bad arguments before anything reaches the GPU.

No call here launches a kernel: every call either fails validation or has
nothing to compute (an empty batch), so these run without a GPU.
"""
import ctypes
import os
import re

import pytest

from megatron_tensor_layer_tp_amd import tpshard as T

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tpshard.h")

A16 = 1 << 20  # a fake, 16-byte aligned "device address" that validation never dereferences


def header_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(tp_\w+)\s*\(", txt, flags=re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(T.LIB_PATH):
        from megatron_tensor_layer_tp_amd import build
        build.build(verbose=False)
    return T.lib()


def test_exports_every_declared_symbol(L):
    names = header_functions()
    assert len(names) == 30, names
    raw = ctypes.CDLL(T.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n
    assert set(names) == set(T.EXPORTS)
    assert T.tp_abi_version() == 1
    assert T.tp_status_string(T.TP_ESHAPE) == "TP_ESHAPE"
    assert T.tp_status_string(99) == "TP_UNKNOWN_STATUS"


def _st(L, name, *args):
    return getattr(L, name)(*args)


def mlp_args(**kw):
    a = dict(act=T.TP_ACT_GELU, dt=T.TP_DT_BF16, s=8, h=16, ft=32, X=A16, W1=A16, W2=A16, Z=A16,
             H=A16, Y=A16, stream=None)
    a.update(kw)
    return list(a.values())


def test_mlp_fwd_validation(L):
    assert _st(L, "tp_mlp_fwd", *mlp_args(act=7)) == T.TP_EINVAL
    assert "act 7" in T.tp_last_error()
    assert _st(L, "tp_mlp_fwd", *mlp_args(dt=5)) == T.TP_EINVAL
    assert _st(L, "tp_mlp_fwd", *mlp_args(s=-1)) == T.TP_ESHAPE
    assert "s = -1" in T.tp_last_error()
    assert _st(L, "tp_mlp_fwd", *mlp_args(h=1 << 31)) == T.TP_ESHAPE
    assert _st(L, "tp_mlp_fwd", *mlp_args(X=None)) == T.TP_EINVAL
    assert "X is NULL" in T.tp_last_error()
    assert _st(L, "tp_mlp_fwd", *mlp_args(W2=A16 + 2)) == T.TP_EALIGN
    # GeLU needs the pre-activation Z; ReLU may drop it
    assert _st(L, "tp_mlp_fwd", *mlp_args(Z=None)) == T.TP_EINVAL
    # an empty batch is legal and has nothing to do (no launch, no GPU needed)
    assert _st(L, "tp_mlp_fwd", *mlp_args(s=0, X=None, Z=None, H=None, Y=None, act=T.TP_ACT_RELU)) == T.TP_OK
    assert T.tp_last_error() == ""


def test_bwd_workspace_rules(L):
    need = T.tp_mlp_bwd_workspace(T.TP_DT_BF16, 8192, 768, 1536)
    assert need >= 8192 * 1536 * 2          # dZ is staged in the workspace
    assert T.tp_mlp_bwd_workspace(T.TP_DT_F32, 8, 16, 32) >= 8 * 32 * 4
    assert T.tp_mlp_bwd_workspace(T.TP_DT_BF16, -1, 16, 32) == 0
    args = [T.TP_ACT_RELU, T.TP_DT_BF16, 8192, 768, 1536] + [A16] * 9
    assert _st(L, "tp_mlp_bwd", *args, None, 0, None) == T.TP_EWORKSPACE
    assert _st(L, "tp_mlp_bwd", *args, A16, need - 1, None) == T.TP_EWORKSPACE
    assert _st(L, "tp_mlp_bwd", *args, A16 + 16, need, None) == T.TP_EALIGN
    assert T.tp_swiglu_bwd_workspace(T.TP_DT_BF16, 8192, 8192, 3584) >= 2 * 8192 * 3584 * 2
    assert T.tp_attn_proj_bwd_workspace(T.TP_DT_BF16, 8192, 8192, 1024, 128) >= 0
    # the query is a pure function of the sizes
    assert need == T.tp_mlp_bwd_workspace(T.TP_DT_BF16, 8192, 768, 1536)


def test_vocab_validation(L):
    ce = [16, 32, 0, A16, A16, A16, A16, A16, None]
    bad = list(ce)
    bad[2] = -5
    assert _st(L, "tp_vocab_ce", *bad) == T.TP_ESHAPE
    bad = list(ce)
    bad[4] = None
    assert _st(L, "tp_vocab_ce", *bad) == T.TP_EINVAL
    assert _st(L, "tp_vocab_ce", 0, 32, 0, None, None, None, None, None, None) == T.TP_OK
    em = [T.TP_DT_BF16, 16, 32, 64, 0, A16, A16, A16, None]
    bad = list(em)
    bad[0] = 9
    assert _st(L, "tp_vocab_embed", *bad) == T.TP_EINVAL
    bad = list(em)
    bad[7] = A16 + 8
    assert _st(L, "tp_vocab_embed", *bad) == T.TP_EALIGN
    assert _st(L, "tp_lm_head_fwd", T.TP_DT_BF16, 8, -2, 16, A16, A16, A16, None) == T.TP_ESHAPE


def test_layer_calls_validation(L):
    sw = [T.TP_DT_BF16, 8, 16, 32] + [A16] * 8 + [None]
    bad = list(sw)
    bad[6] = None  # Wu
    assert _st(L, "tp_swiglu_fwd", *bad) == T.TP_EINVAL
    assert "Wu" in T.tp_last_error()
    at = [T.TP_DT_BF16, 8, 16, 16, 8] + [A16] * 10 + [None]
    bad = list(at)
    bad[4] = -8
    assert _st(L, "tp_attn_proj_fwd", *bad) == T.TP_ESHAPE
    # zero-width K/V heads are legal sizes (nothing to write for them)
    ok = [T.TP_DT_BF16, 0, 16, 16, 0] + [A16, A16, None, None, None, A16, A16, None, None, None] + [None]
    assert _st(L, "tp_attn_proj_fwd", *ok) == T.TP_OK


def test_lm_head_ce_validation(L):
    need = T.tp_lm_head_ce_workspace(T.TP_DT_BF16, 8192, 8192, 16032)
    # two fp32 partials per position for every tile column (at most 256 wide), plus the target logit
    assert need >= 8192 * 4 * (2 * (16032 // 256) + 1)
    assert need == T.tp_lm_head_ce_workspace(T.TP_DT_BF16, 8192, 8192, 16032)
    assert T.tp_lm_head_ce_workspace(T.TP_DT_F32, 8, 8, 8) == 0
    args = [T.TP_DT_BF16, 8192, 8192, 16032, 0] + [A16] * 6
    bad = list(args)
    bad[0] = T.TP_DT_F32
    assert _st(L, "tp_lm_head_ce_fwd", *bad, A16, need, None) == T.TP_EUNSUPPORTED
    bad = list(args)
    bad[4] = -1
    assert _st(L, "tp_lm_head_ce_fwd", *bad, A16, need, None) == T.TP_ESHAPE
    bad = list(args)
    bad[7] = None  # target
    assert _st(L, "tp_lm_head_ce_fwd", *bad, A16, need, None) == T.TP_EINVAL
    assert _st(L, "tp_lm_head_ce_fwd", *args, A16, need - 1, None) == T.TP_EWORKSPACE
    assert _st(L, "tp_lm_head_ce_fwd", *args, A16 + 16, need, None) == T.TP_EALIGN
    # nothing to compute: no positions
    assert _st(L, "tp_lm_head_ce_fwd", T.TP_DT_BF16, 0, 64, 100, 0, None, A16, None, None, None, None,
               None, 0, None) == T.TP_OK


def test_vocab_ce_bwd_validation(L):
    args = [T.TP_DT_F32, 16, 32, 0] + [A16] * 6 + [None]
    bad = list(args)
    bad[0] = 3
    assert _st(L, "tp_vocab_ce_bwd", *bad) == T.TP_EINVAL
    bad = list(args)
    bad[3] = -1
    assert _st(L, "tp_vocab_ce_bwd", *bad) == T.TP_ESHAPE
    bad = list(args)
    bad[8] = None  # dloss
    assert _st(L, "tp_vocab_ce_bwd", *bad) == T.TP_EINVAL
    assert "dloss" in T.tp_last_error()
    bad = list(args)
    bad[9] = A16 + 4
    assert _st(L, "tp_vocab_ce_bwd", *bad) == T.TP_EALIGN
    # nothing to compute: an empty shard
    assert _st(L, "tp_vocab_ce_bwd", T.TP_DT_BF16, 16, 0, 0, None, A16, A16, A16, A16, None, None) == T.TP_OK


def test_attn_core_validation(L):
    args = [T.TP_DT_BF16, 64, 8, 1, 128] + [A16] * 5 + [None]
    bad = list(args)
    bad[4] = 64
    assert _st(L, "tp_attn_core_fwd", *bad) == T.TP_EUNSUPPORTED
    bad = list(args)
    bad[0] = T.TP_DT_F32
    assert _st(L, "tp_attn_core_fwd", *bad) == T.TP_EUNSUPPORTED
    bad = list(args)
    bad[3] = 3
    assert _st(L, "tp_attn_core_fwd", *bad) == T.TP_ESHAPE
    bad = list(args)
    bad[9] = None  # lse
    assert _st(L, "tp_attn_core_fwd", *bad) == T.TP_EINVAL
    bad = list(args)
    bad[8] = A16 + 2
    assert _st(L, "tp_attn_core_fwd", *bad) == T.TP_EALIGN
    # nothing to compute: no positions
    assert _st(L, "tp_attn_core_fwd", T.TP_DT_BF16, 0, 8, 1, 128, None, None, None, None, None, None) == T.TP_OK


def test_sp_validation(L):
    import ctypes as C
    f = [T.TP_DT_BF16, 16, 64, C.c_float(0.1), C.c_float(1e-5)] + [A16] * 9 + [None]
    bad = list(f)
    bad[3] = C.c_float(1.0)
    assert _st(L, "tp_sp_ln_fwd", *bad) == T.TP_EINVAL
    bad = list(f)
    bad[4] = C.c_float(0.0)
    assert _st(L, "tp_sp_ln_fwd", *bad) == T.TP_EINVAL
    bad = list(f)
    bad[2] = 20000
    assert _st(L, "tp_sp_ln_fwd", *bad) == T.TP_EUNSUPPORTED
    bad = list(f)
    bad[7] = None  # mask
    assert _st(L, "tp_sp_ln_fwd", *bad) == T.TP_EINVAL
    need = T.tp_sp_ln_bwd_workspace(T.TP_DT_BF16, 1024, 8192)
    assert need >= (1024 // 16) * 2 * 8192 * 4
    b = [T.TP_DT_BF16, 1024, 8192, C.c_float(0.1)] + [A16] * 11
    assert _st(L, "tp_sp_ln_bwd", *b, A16, need - 1, None) == T.TP_EWORKSPACE
    assert _st(L, "tp_sp_ln_bwd", *b, A16 + 64, need, None) == T.TP_EALIGN
    assert _st(L, "tp_sp_ln_fwd", T.TP_DT_BF16, 0, 64, C.c_float(0.1), C.c_float(1e-5), None, None, None, A16, A16,
               None, None, None, None, None) == T.TP_OK


def test_attn_core_bwd_validation(L):
    need = T.tp_attn_core_bwd_workspace(T.TP_DT_BF16, 8192, 8, 1, 128)
    # per-query-head fp32 partials of dK and dV, plus the per-query statistics
    assert need >= 2 * 8 * 8192 * 128 * 4 + 8 * 8192 * 2 * 4
    assert need == T.tp_attn_core_bwd_workspace(T.TP_DT_BF16, 8192, 8, 1, 128)
    assert T.tp_attn_core_bwd_workspace(T.TP_DT_BF16, 8192, 8, 1, 64) == 0
    args = [T.TP_DT_BF16, 8192, 8, 1, 128] + [A16] * 9
    assert _st(L, "tp_attn_core_bwd", *args, A16, need - 1, None) == T.TP_EWORKSPACE
    assert _st(L, "tp_attn_core_bwd", *args, A16 + 32, need, None) == T.TP_EALIGN
    bad = list(args)
    bad[4] = 64
    assert _st(L, "tp_attn_core_bwd", *bad, A16, need, None) == T.TP_EUNSUPPORTED
    bad = list(args)
    bad[0] = T.TP_DT_F32
    assert _st(L, "tp_attn_core_bwd", *bad, A16, need, None) == T.TP_EUNSUPPORTED
    bad = list(args)
    bad[3] = 3
    assert _st(L, "tp_attn_core_bwd", *bad, A16, need, None) == T.TP_ESHAPE
    bad = list(args)
    bad[2], bad[3] = 0, 1  # no query heads for a KV head
    assert _st(L, "tp_attn_core_bwd", *bad, A16, need, None) == T.TP_ESHAPE
    bad = list(args)
    bad[10] = None  # lse
    assert _st(L, "tp_attn_core_bwd", *bad, A16, need, None) == T.TP_EINVAL
    assert "lse" in T.tp_last_error()
    bad = list(args)
    bad[13] = A16 + 2  # dV
    assert _st(L, "tp_attn_core_bwd", *bad, A16, need, None) == T.TP_EALIGN
    # nothing to compute: no positions
    assert _st(L, "tp_attn_core_bwd", T.TP_DT_BF16, 0, 8, 1, 128, *([None] * 9), None, 0, None) == T.TP_OK


def test_attn_proj_bwd_halves_validation(L):
    no = T.tp_attn_out_bwd_workspace(T.TP_DT_BF16, 8192, 8192, 1024)
    nq = T.tp_attn_qkv_bwd_workspace(T.TP_DT_BF16, 8192, 8192, 1024, 128)
    # the halves' workspaces are the whole call's two regions
    assert no + nq == T.tp_attn_proj_bwd_workspace(T.TP_DT_BF16, 8192, 8192, 1024, 128)
    o = [T.TP_DT_BF16, 8192, 8192, 1024] + [A16] * 5
    if no:
        assert _st(L, "tp_attn_out_bwd", *o, A16, no - 1, None) == T.TP_EWORKSPACE
    bad = list(o)
    bad[6] = None  # dY
    assert _st(L, "tp_attn_out_bwd", *bad, A16, no, None) == T.TP_EINVAL
    q = [T.TP_DT_BF16, 8192, 8192, 1024, 128] + [A16] * 11
    if nq:
        assert _st(L, "tp_attn_qkv_bwd", *q, A16, nq - 1, None) == T.TP_EWORKSPACE
    bad = list(q)
    bad[4] = -1
    assert _st(L, "tp_attn_qkv_bwd", *bad, A16, nq, None) == T.TP_ESHAPE
    bad = list(q)
    bad[11] = A16 + 8  # dX
    assert _st(L, "tp_attn_qkv_bwd", *bad, A16, nq, None) == T.TP_EALIGN


def test_lm_head_ce_noalloc_validation(L):
    cap = T.tp_lm_head_ce_noalloc_max_bytes()
    assert cap == 32 << 20
    args = [T.TP_DT_BF16, 8192, 8192, 16032, 0] + [A16] * 6 + [None]
    bad = list(args)
    bad[0] = T.TP_DT_F32
    assert _st(L, "tp_lm_head_ce_fwd_noalloc", *bad) == T.TP_EUNSUPPORTED
    bad = list(args)
    bad[7] = None  # target
    assert _st(L, "tp_lm_head_ce_fwd_noalloc", *bad) == T.TP_EINVAL
    # beyond the scratch: refused before anything is enqueued
    bad = list(args)
    bad[1], bad[3] = 65536, 32064
    assert T.tp_lm_head_ce_workspace(T.TP_DT_BF16, 65536, 8192, 32064) > cap
    assert _st(L, "tp_lm_head_ce_fwd_noalloc", *bad) == T.TP_EWORKSPACE
    assert "scratch" in T.tp_last_error()
    # nothing to compute: no positions (no device touched)
    assert _st(L, "tp_lm_head_ce_fwd_noalloc", T.TP_DT_BF16, 0, 64, 100, 0, None, A16, None, None, None, None,
               None) == T.TP_OK
