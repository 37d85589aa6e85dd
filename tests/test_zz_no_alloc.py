"""The allocation-free fused LM head + CE call (tp_lm_head_ce_fwd_noalloc)
against the same call with a caller's workspace (tp_lm_head_ce_fwd), through
the C ABI: the same kernels on the same inputs, so the three statistics must be
equal bit for bit -- on two calls in a row, the second on a smaller input
(the library's scratch keeps the first call's contents, none of which the
second may read), then a request beyond the scratch is refused before
anything is enqueued.  Inputs follow the vocab shard (bf16 activations and an
N(0, 0.01) weight slice, targets uniform over the whole vocabulary)."""
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


def stats_t(s):
    return [fill_garbage(torch.empty(s, dtype=torch.float32, device="cuda:0")) for _ in range(3)]


def run_both(Hf, W, tgt, start):
    s, h = Hf.shape
    Vs = W.shape[1]
    Hd, Wd, td = dev(Hf), dev(W), dev(tgt)
    with_ws = stats_t(s)
    ws, nb = workspace(T.tp_lm_head_ce_workspace(BF, s, h, Vs))
    T.tp_lm_head_ce_fwd(BF, s, h, Vs, start, Hd, Wd, td, *with_ws, ws, nb)
    no_ws = stats_t(s)
    T.tp_lm_head_ce_fwd_noalloc(BF, s, h, Vs, start, Hd, Wd, td, *no_ws)
    torch.cuda.synchronize()
    return with_ws, no_ws


def inputs(seed, s, h, Vs, start):
    g = np.random.default_rng(seed)
    Hf = I.f32_to_bf16_bits(g.standard_normal((s, h)).astype(np.float32))
    W = I.f32_to_bf16_bits((g.standard_normal((h, Vs)) * 0.01).astype(np.float32))
    tgt = g.integers(0, 128256, s).astype(np.int64)
    tgt[: s // 4] = start + g.integers(0, Vs, s // 4)   # a quarter of the targets inside the shard
    return Hf, W, tgt


def test_noalloc_matches_workspace_call_twice():
    # first call: the vocab shard's full width and 4096 positions (about 12 MiB of scratch)
    a = run_both(*inputs(1, 4096, 1024, 16032, 16032), 16032)
    # second call, smaller: every slot it reads must be its own
    b = run_both(*inputs(2, 520, 136, 2056, 77), 77)
    for (w, n) in (a, b):
        for x, y in zip(w, n):
            assert torch.equal(x, y)
        assert torch.isfinite(n[0]).all() and (n[1] > 0).all()


def test_noalloc_refuses_more_than_its_scratch():
    cap = T.tp_lm_head_ce_noalloc_max_bytes()
    assert cap == 32 << 20
    s, h, Vs = 65536, 64, 32064     # at least 65536 * (2 * 126 + 1) * 4 bytes > 32 MiB
    assert T.tp_lm_head_ce_workspace(BF, s, h, Vs) > cap
    A = torch.empty(16, dtype=torch.int16, device="cuda:0")
    with pytest.raises(T.TpError) as e:
        T.tp_lm_head_ce_fwd_noalloc(BF, s, h, Vs, 0, A, A, A, A, A, A)
    assert e.value.status == T.TP_EWORKSPACE and "scratch" in str(e.value)
