"""The last-round re-tiling of a launch (a launch whose last round would fill at
most half of the workgroup slots runs its whole rounds first, then the
remaining tiles -- a rectangle of the output -- as a product of their own with
smaller tiles).  Every output element is still one fp32 sum over K in
increasing order, so the results must not change:

  * bit-exact integer cases ({-1,0,1} inputs: every accumulation exact) through
    the re-tiled path of every layout it serves -- the column GEMM with its
    ReLU epilogue (NN), dZ with the ReLU-mask epilogue (NT), the weight
    gradients dW1 and dW2 (TN), and SwiGLU's dual gate/up pass -- forced at
    small sizes with TP_GEMM_TAIL=force on 256x256 tiles, pairing off;
  * at the GPT-3-175B t=8 MLP shard (its dW1 and dW2 launches take the path)
    and the Llama-3-70B SwiGLU shard (its gate/up launch does), the default
    results equal those with the re-tiling switched off, bit for bit.
"""
import pytest

from gpu_util import need_gpu, torch
from megatron_tensor_layer_tp_amd import inputs as I
from megatron_tensor_layer_tp_amd import tpshard as T
from test_gpu_layer import run_swiglu, swiglu_integer_case
from test_gpu_mlp import integer_exact_case, run_mlp

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    T.lib()


@pytest.fixture
def forced_tail(monkeypatch):
    monkeypatch.setenv("TP_GEMM_VARIANT", "256x256:waves8")
    monkeypatch.setenv("TP_GEMM_TAIL", "force")
    monkeypatch.setenv("TP_GEMM_PAIR", "off")


# (s, h, ft): 17 x 16 tiles of the column GEMM and of dZ; 16 x 17 and 17 x 16 tiles of dW2 and dW1
@pytest.mark.parametrize("s,h,ft", [(4352, 128, 4096), (128, 4352, 4096)])
def test_mlp_tail_integer_exact(oracle_mod, forced_tail, s, h, ft):
    integer_exact_case(oracle_mod, s, h, ft)


def test_swiglu_gate_up_tail_integer_exact(oracle_mod, forced_tail):
    swiglu_integer_case(oracle_mod, 4352, 128, 2048)


def test_gpt3_mlp_tail_equals_untiled(monkeypatch):
    d = I.mlp_inputs(3, shards=[0])
    args = (T.TP_ACT_GELU, True, d["X"], d["W1"][0], d["W2"][0], d["dY"])
    a = run_mlp(*args)
    monkeypatch.setenv("TP_GEMM_TAIL", "off")
    b = run_mlp(*args)
    for k in a:
        assert torch.equal(a[k], b[k]), k


def test_llama3_swiglu_tail_equals_untiled(monkeypatch):
    d = I.swiglu_inputs(4)
    args = (True, d["X"], d["Wg"][0], d["Wu"][0], d["Wd"][0], d["dY"])
    a = run_swiglu(*args)
    monkeypatch.setenv("TP_GEMM_TAIL", "off")
    b = run_swiglu(*args)
    for k in a:
        assert torch.equal(a[k], b[k]), k
