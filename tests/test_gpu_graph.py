"""The library's calls under HIP graph capture.  No call allocates, frees,
synchronizes or clears memory with hipMemsetAsync (workspaces come from the
caller; the allocation-free CE call uses its own device array), so a sequence
of calls can be captured once and replayed: a layer's MLP forward and backward
(paired launches, split-K with its deferred reduction), the attention core
forward and backward, the fused LM head + CE statistics without a workspace
and the embedding gather, captured into one graph on torch's capture stream.
Every replay, with eager work and synchronizations between replays, must give
the eager results bit for bit (every kernel sums in a fixed order)."""
import numpy as np
import pytest

from gpu_util import dev, fill_garbage, need_gpu, torch, workspace
from megatron_tensor_layer_tp_amd import inputs as I
from megatron_tensor_layer_tp_amd import tpshard as T

pytestmark = pytest.mark.gpu
BF = T.TP_DT_BF16


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    T.lib()


def bf(g, shape, scale=1.0):
    return dev(I.f32_to_bf16_bits((g.standard_normal(shape) * scale).astype(np.float32)))


def i16(*shape):
    return fill_garbage(torch.empty(shape, dtype=torch.int16, device="cuda:0"))


def f32(*shape):
    return fill_garbage(torch.empty(shape, dtype=torch.float32, device="cuda:0"))


def test_graph_replays_equal_eager():
    g = np.random.default_rng(17)
    # MLP shard (GeLU): s long beside h and f/t, so the weight gradients split along K
    s, h, ft = 2048, 128, 256
    X, W1, W2, dY = bf(g, (s, h)), bf(g, (h, ft), h ** -0.5), bf(g, (ft, h), ft ** -0.5), bf(g, (s, h))
    Z, H, Y, dX, dW1, dW2 = i16(s, ft), i16(s, ft), i16(s, h), i16(s, h), i16(h, ft), i16(ft, h)
    ws_m, nb_m = workspace(T.tp_mlp_bwd_workspace(BF, s, h, ft))
    # attention core, grouped (4 query heads on 2 KV heads), ragged length
    sa, nq, nkv, d = 300, 4, 2, 128
    Q, K, V, dO = bf(g, (sa, nq * d)), bf(g, (sa, nkv * d)), bf(g, (sa, nkv * d)), bf(g, (sa, nq * d))
    O, lse = i16(sa, nq * d), f32(nq, sa)
    dQ, dK, dV = i16(sa, nq * d), i16(sa, nkv * d), i16(sa, nkv * d)
    ws_a, nb_a = workspace(T.tp_attn_core_bwd_workspace(BF, sa, nq, nkv, d))
    # fused LM head + CE statistics (no workspace) and the embedding gather of a vocab shard
    sv, hv, Vs, start = 200, 128, 2056, 1000
    Hf, Wlm = bf(g, (sv, hv)), bf(g, (hv, Vs), 0.05)
    tgt = torch.from_numpy(g.integers(0, 4 * Vs, sv).astype(np.int64)).to("cuda:0")
    m, se, tl = f32(sv), f32(sv), f32(sv)
    table, emb = bf(g, (Vs, hv)), i16(sv, hv)
    outs = [Z, H, Y, dX, dW1, dW2, O, lse, dQ, dK, dV, m, se, tl, emb]

    def step():
        T.tp_mlp_fwd(T.TP_ACT_GELU, BF, s, h, ft, X, W1, W2, Z, H, Y)
        T.tp_mlp_bwd(T.TP_ACT_GELU, BF, s, h, ft, X, W1, W2, Z, H, dY, dX, dW1, dW2, ws_m, nb_m)
        T.tp_attn_core_fwd(BF, sa, nq, nkv, d, Q, K, V, O, lse)
        T.tp_attn_core_bwd(BF, sa, nq, nkv, d, Q, K, V, O, dO, lse, dQ, dK, dV, ws_a, nb_a)
        T.tp_lm_head_ce_fwd_noalloc(BF, sv, hv, Vs, start, Hf, Wlm, tgt, m, se, tl)
        T.tp_vocab_embed(BF, sv, Vs, hv, start, tgt, table, emb)

    step()  # eager (also sets up the allocation-free call's device array)
    torch.cuda.synchronize()
    want = [t.clone() for t in outs]
    for t in outs:
        fill_garbage(t)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outs:
            fill_garbage(t)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, want)):
            assert torch.equal(a, b), (rep, i)
