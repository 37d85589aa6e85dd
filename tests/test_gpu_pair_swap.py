"""Paired launches in the swapped order: the activation gradient's blocks (NT,
a store or the activation-backward epilogue) dispatched first and the weight
gradient's (TN) after them, as the planner picks for shards with few tokens,
where the weight gradients' K (the token count) is the short one.  Every output
element is still one fp32 sum over K in increasing order, whatever the pairing
and the tile shape, so:

  * bit-exact integer cases ({-1,0,1} inputs: every accumulation exact) of the
    MLP backward with the swapped order forced (TP_GEMM_PAIR=swap) for each
    residency the swapped pairs are built for, at ragged sizes that span
    several tiles;
  * at the GPT-3-175B t=8 MLP shard, where the planner itself takes the swapped
    order, the results equal those with pairing switched off, bit for bit.
"""
import pytest

from gpu_util import need_gpu, torch
from megatron_tensor_layer_tp_amd import inputs as I
from megatron_tensor_layer_tp_amd import tpshard as T
from test_gpu_mlp import integer_exact_case, run_mlp

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    T.lib()


@pytest.mark.parametrize("variant", ["", "256x256:waves8", "128x192:shared", "128x128:shared"])
@pytest.mark.parametrize("s,h,ft", [(264, 1032, 520), (136, 784, 1296)])
def test_mlp_bwd_swapped_integer_exact(oracle_mod, monkeypatch, variant, s, h, ft):
    monkeypatch.setenv("TP_GEMM_PAIR", "swap")
    if variant:
        monkeypatch.setenv("TP_GEMM_VARIANT", variant)
    integer_exact_case(oracle_mod, s, h, ft)


def test_gpt3_mlp_swapped_pairs_equal_unpaired(monkeypatch):
    d = I.mlp_inputs(3, shards=[0])
    args = (T.TP_ACT_GELU, True, d["X"], d["W1"][0], d["W2"][0], d["dY"])
    a = run_mlp(*args)
    monkeypatch.setenv("TP_GEMM_PAIR", "off")
    b = run_mlp(*args)
    for k in a:
        assert torch.equal(a[k], b[k]), k
