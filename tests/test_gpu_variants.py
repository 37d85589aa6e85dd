"""Every built bf16 GEMM variant (tile shape x residency: LDS stages and
workgroups per CU) on the same products, each checked against the fp64 oracle.

The planner normally picks one variant per product from its cost model, so most
variants would only run at the sizes where they win; TP_GEMM_VARIANT restricts
every product that has the variant built to it (split-K and pairing still
planned), which puts each variant through the MLP, the attention projections
and SwiGLU's gate/up pass with integer inputs (bit-exact), the SwiGLU and
attention-projection paths with float inputs, and the fused LM-head + CE path,
at ragged sizes."""
import numpy as np
import pytest

from gpu_util import need_gpu
from megatron_tensor_layer_tp_amd import inputs as I
from megatron_tensor_layer_tp_amd import tpshard as T
from test_gpu_layer import attn_integer_case, bf, close, run_attn, run_swiglu, swiglu_integer_case
from test_gpu_lm_ce import check_vs_oracle, run_fused
from test_gpu_mlp import integer_exact_case

pytestmark = pytest.mark.gpu

VARIANTS = ["256x256:two", "256x256:waves8", "256x192:two", "256x128:three", "128x256:three", "128x192:three",
            "128x128:three", "128x192:shared", "128x128:shared"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    T.lib()


@pytest.fixture(params=VARIANTS)
def variant(request, monkeypatch):
    monkeypatch.setenv("TP_GEMM_VARIANT", request.param)
    return request.param


@pytest.mark.parametrize("s,h,ft", [(520, 200, 1000), (2056, 136, 392)])
def test_mlp_integer_exact(oracle_mod, variant, s, h, ft):
    integer_exact_case(oracle_mod, s, h, ft)


@pytest.mark.parametrize("s,h,dq,dkv", [(520, 264, 256, 32), (2056, 136, 392, 136)])
def test_attn_proj_integer_exact(oracle_mod, variant, s, h, dq, dkv):
    attn_integer_case(oracle_mod, s, h, dq, dkv)


def test_swiglu_gate_up_integer_exact(oracle_mod, variant):
    swiglu_integer_case(oracle_mod, 520, 264, 392)


def test_swiglu(oracle_mod, variant):
    s, h, ft = 520, 264, 392
    g = np.random.default_rng(11)
    X = bf(g.standard_normal((s, h)))
    Wg, Wu = bf(g.standard_normal((h, ft)) * 0.1), bf(g.standard_normal((h, ft)) * 0.1)
    Wd = bf(g.standard_normal((ft, h)) * 0.1)
    dY = bf(g.standard_normal((s, h)))
    o = run_swiglu(True, X, Wg, Wu, Wd, dY)
    f = [I.bf16_bits_to_f64(v) for v in (X, Wg, Wu, Wd, dY)]
    G, U, A, Y = oracle_mod.swiglu_fwd(*f[:4])
    dX, dWg, dWu, dWd = oracle_mod.swiglu_bwd(*f)
    for k, w in dict(G=G, U=U, A=A, Y=Y, dX=dX, dWg=dWg, dWu=dWu, dWd=dWd).items():
        close(o[k], w, k)


def test_attn_proj(oracle_mod, variant):
    s, h, dq, dkv = 520, 264, 256, 32
    g = np.random.default_rng(12)
    X = bf(g.standard_normal((s, h)))
    Wq, Wk, Wv = (bf(g.standard_normal(sh) * 0.05) for sh in ((h, dq), (h, dkv), (h, dkv)))
    O, Wo = bf(g.standard_normal((s, dq))), bf(g.standard_normal((dq, h)) * 0.05)
    dQ, dK, dV, dY = (bf(g.standard_normal(sh)) for sh in ((s, dq), (s, dkv), (s, dkv), (s, h)))
    o = run_attn(True, X, Wq, Wk, Wv, O, Wo, dQ, dK, dV, dY)
    f = [I.bf16_bits_to_f64(v) for v in (X, Wq, Wk, Wv, O, Wo, dQ, dK, dV, dY)]
    Q, K, V, Y = oracle_mod.attn_fwd(*f[:6])
    dX, dWq, dWk, dWv, dO, dWo = oracle_mod.attn_bwd(*f)
    for k, w in dict(Q=Q, K=K, V=V, Y=Y, dX=dX, dWq=dWq, dWk=dWk, dWv=dWv, dO=dO, dWo=dWo).items():
        close(o[k], w, k)


def test_lm_head_ce(oracle_mod, variant):
    s, h, Vs, start = 520, 136, 2056, 77
    g = np.random.default_rng(13)
    Hf, W = bf(g.standard_normal((s, h))), bf(g.standard_normal((h, Vs)) * 0.05)
    tgt = g.integers(-3, start + Vs + 4, s).astype(np.int64)
    tgt[0], tgt[1] = start, start + Vs - 1
    got = run_fused(Hf, W, tgt, start)
    z = oracle_mod.lm_head(I.bf16_bits_to_f64(Hf), I.bf16_bits_to_f64(W))
    check_vs_oracle(got, oracle_mod.ce_stats(z, tgt, start))
