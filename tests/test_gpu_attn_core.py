"""GPU parity of the attention core on a shard's heads (tp_attn_core_fwd;
"7.3 模型并行与张量并行" §7.3.4: the card's query heads share its key/value
head) against the fp64 oracle.

  * O (bf16) within 5e-3 relative Frobenius of the oracle per head and within
    the element-wise bound of gpu_util.elem_bound, at small, ragged (s not a
    multiple of the 128-row query block or the 64-key tile) and grouped
    (nq / nkv = 1, 2, 4, 8) sizes, and on stratified sampled rows (one in every
    64-row half of each query block) of the Llama-3-70B t=8 shard (s = 8192,
    8 query heads, 1 KV head);
  * the log-sum-exp of each row's scores within 1e-4 absolute;
  * run twice, bit-identical.
"""
import numpy as np
import pytest

from gpu_util import check_bf16, dev, fill_garbage, host, host_f64, need_gpu, torch
from megatron_tensor_layer_tp_amd import inputs as I
from megatron_tensor_layer_tp_amd import tpshard as T

pytestmark = pytest.mark.gpu
D = 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    T.lib()


def run_core(Q, K, V, nq, nkv):
    s = Q.shape[0]
    O = fill_garbage(torch.empty((s, nq * D), dtype=torch.int16, device="cuda:0"))
    lse = fill_garbage(torch.empty((nq, s), dtype=torch.float32, device="cuda:0"))
    T.tp_attn_core_fwd(T.TP_DT_BF16, s, nq, nkv, D, dev(Q), dev(K), dev(V), O, lse)
    torch.cuda.synchronize()
    return O, lse


def check(got_O, got_lse, want_O, want_lse, nq, rows=None):
    O = host_f64(got_O)
    lse = host(got_lse).astype(np.float64)
    if rows is not None:
        O, lse = O[rows], lse[:, rows]
    for j in range(nq):
        check_bf16(O[:, j * D:(j + 1) * D], want_O[:, j * D:(j + 1) * D], f"O head {j}")
    assert np.abs(lse - want_lse).max() <= 1e-4


@pytest.mark.parametrize("s,nq,nkv", [(128, 8, 1), (200, 4, 2), (64, 2, 1), (1, 8, 1), (513, 8, 1),
                                      (300, 2, 2), (1000, 8, 4)])
def test_core_small(oracle_mod, s, nq, nkv):
    g = np.random.default_rng(s + 10 * nq + nkv)
    bf = lambda a: I.f32_to_bf16_bits(a.astype(np.float32))  # noqa: E731
    Q, K, V = bf(g.standard_normal((s, nq * D))), bf(g.standard_normal((s, nkv * D))), \
        bf(g.standard_normal((s, nkv * D)))
    O, lse = run_core(Q, K, V, nq, nkv)
    wO, wl = oracle_mod.attn_core_fwd(*(I.bf16_bits_to_f64(a) for a in (Q, K, V)), nq, nkv)
    check(O, lse, wO, wl, nq)


def test_core_llama3_shard_sampled(oracle_mod):
    d = I.attn_core_inputs(4)
    Q, K, V = d["Q"][0], d["K"][0], d["V"][0]
    nq, nkv, s = d["nq"], d["nkv"], d["s"]
    O, lse = run_core(Q, K, V, nq, nkv)
    rows = I.sample_rows(s, 64, 4, 31)
    wO, wl = oracle_mod.attn_core_fwd(*(I.bf16_bits_to_f64(a) for a in (Q, K, V)), nq, nkv, rows=rows)
    check(O, lse, wO, wl, nq, rows)
    O2, lse2 = run_core(Q, K, V, nq, nkv)
    assert torch.equal(O, O2) and torch.equal(lse, lse2)
