"""GPU parity of the fused LM head + cross-entropy statistics
(tp_lm_head_ce_fwd; lecture 16 notes §5.5, the fused vocab-parallel cross
entropy that never writes the logits out).

  * Against the fp64 oracle (its own fp64 logits, then the CE statistics):
    max and target logit within 2e-5 absolute (fp32 accumulation of the same
    bf16 products), sum of exponentials within 1e-4 relative, loss within
    1e-4 absolute -- at small and ragged sizes, over all 8 shards of a
    V=128256 vocabulary, and on sampled rows of the [8192,8192] x [8192,16032]
    shard.
  * Against the unfused GPU path (tp_lm_head_fwd then tp_vocab_ce) on the same
    inputs: max and target logit are the same fp32 values (bit-exact), the sum
    of exponentials agrees within 1e-5 relative.
"""
import numpy as np
import pytest

from gpu_util import dev, fill_garbage, host, need_gpu, torch
from megatron_tensor_layer_tp_amd import inputs as I
from megatron_tensor_layer_tp_amd import tpshard as T

pytestmark = pytest.mark.gpu
BF = T.TP_DT_BF16


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    T.lib()


def bf(a):
    return I.f32_to_bf16_bits(np.asarray(a, np.float32))


def f32_out(n):
    return fill_garbage(torch.empty(n, dtype=torch.float32, device="cuda:0"))


def run_fused(Hf, W, tgt, start):
    s, h = Hf.shape
    Vs = W.shape[1]
    nb = T.tp_lm_head_ce_workspace(BF, s, h, Vs)
    ws = torch.full((max(nb, 256),), 0xff, dtype=torch.uint8, device="cuda:0")  # NaN garbage
    m, se, tl = f32_out(s), f32_out(s), f32_out(s)
    T.tp_lm_head_ce_fwd(BF, s, h, Vs, start, dev(Hf), dev(W), dev(np.asarray(tgt, np.int64)), m, se, tl, ws, nb)
    torch.cuda.synchronize()
    return host(m), host(se), host(tl)


def run_unfused(Hf, W, tgt, start):
    s, h = Hf.shape
    Vs = W.shape[1]
    z = torch.empty((s, Vs), dtype=torch.float32, device="cuda:0")
    T.tp_lm_head_fwd(BF, s, h, Vs, dev(Hf), dev(W), z)
    m, se, tl = f32_out(s), f32_out(s), f32_out(s)
    T.tp_vocab_ce(s, Vs, start, z, dev(np.asarray(tgt, np.int64)), m, se, tl)
    torch.cuda.synchronize()
    return host(m), host(se), host(tl)


def check_vs_oracle(got, want):
    m, se, tl = (np.asarray(a, np.float64) for a in got)
    om, ose, otl = want
    fin = np.isfinite(om)
    assert np.array_equal(np.isfinite(m), fin)
    assert np.all(m[~fin] == om[~fin])
    assert np.abs(m[fin] - om[fin]).max(initial=0) <= 2e-5
    assert np.abs(tl - otl).max(initial=0) <= 2e-5
    ok = ose > 0
    assert np.all(se[~ok] == 0)
    assert (np.abs(se[ok] - ose[ok]) / ose[ok]).max(initial=0) <= 1e-4


def check_vs_unfused(got, ref):
    m, se, tl = got
    um, use, utl = ref
    assert np.array_equal(m, um)
    assert np.array_equal(tl, utl)
    ok = use > 0
    assert np.all(se[~ok] == 0)
    assert (np.abs(se[ok] - use[ok]) / use[ok]).max(initial=0) <= 1e-5


@pytest.mark.parametrize("s,h,Vs,start", [(136, 128, 200, 0), (300, 72, 1001, 2002), (64, 256, 1000, 5),
                                          (257, 64, 16032 // 4, 0), (5, 8, 1, 3), (9, 16, 0, 4),
                                          (10, 0, 50, 0), (520, 136, 2056, 77),
                                          (40, 64, 40000, 1000),  # 313 tile columns: the merge's general loop
                                          (70, 64, 8192, 3),       # 64 tile columns: every load in registers
                                          (70, 64, 8200, 5)])      # 65: the general loop
def test_fused_small(oracle_mod, s, h, Vs, start):
    g = np.random.default_rng(s * 7 + Vs)
    Hf, W = bf(g.standard_normal((s, h))), bf(g.standard_normal((h, Vs)) * 0.05)
    tgt = g.integers(-3, start + Vs + 4, s).astype(np.int64)
    if s > 2 and Vs > 0:
        tgt[0] = start
        tgt[1] = start + Vs - 1
    got = run_fused(Hf, W, tgt, start)
    z = oracle_mod.lm_head(I.bf16_bits_to_f64(Hf), I.bf16_bits_to_f64(W))
    check_vs_oracle(got, oracle_mod.ce_stats(z, tgt, start))
    check_vs_unfused(got, run_unfused(Hf, W, tgt, start))


def test_fused_loss_over_all_shards(oracle_mod):
    """8 vocab shards of V=128256 for 192 positions, h=128: the fused per-shard
    statistics, combined, give the oracle's direct loss within 1e-4."""
    s, h, V, t = 192, 128, 128256, 8
    Vs = V // t
    g = np.random.default_rng(11)
    Hf = bf(g.standard_normal((s, h)))
    W = bf(g.standard_normal((h, V)) * (0.905 / np.sqrt(h)))
    tgt = I.ids_uniform(s, V, 5, I.T_TGT)
    ms, ses, tls = [], [], []
    for i in range(t):
        m, se, tl = run_fused(Hf, np.ascontiguousarray(W[:, i * Vs:(i + 1) * Vs]), tgt, i * Vs)
        ms.append(m)
        ses.append(se)
        tls.append(tl)
    loss = oracle_mod.ce_combine(ms, ses, tls)
    z = oracle_mod.lm_head(I.bf16_bits_to_f64(Hf), I.bf16_bits_to_f64(W))
    direct = oracle_mod.ce_direct(z, tgt)
    assert np.abs(loss - direct).max() <= 1e-4
    assert abs(loss.mean() - direct.mean()) <= 1e-4


def test_fused_vocab_shard(oracle_mod):
    """The [8192,8192] x [8192,16032] shard 0: every position against the
    unfused GPU path, sampled positions against the oracle."""
    d = I.vocab_inputs(5, with_table=False, with_logits=False)
    Hf, W, tgt = d["Hf"], d["Wlm"][0], d["targets"]
    got = run_fused(Hf, W, tgt, 0)
    check_vs_unfused(got, run_unfused(Hf, W, tgt, 0))
    rows = I.sample_rows(d["s"], 64, 5, 22)
    # make sure some sampled targets fall inside the shard
    z = oracle_mod.lm_head_rows(I.bf16_bits_to_f64(Hf), I.bf16_bits_to_f64(W), rows)
    want = oracle_mod.ce_stats(z, tgt[rows], 0)
    check_vs_oracle(tuple(a[rows] for a in got), want)
    tgt_in = tgt.copy()
    tgt_in[rows] = (np.arange(len(rows)) * 997) % d["Vs"]
    got_in = run_fused(Hf, W, tgt_in, 0)
    check_vs_oracle(tuple(a[rows] for a in got_in), oracle_mod.ce_stats(z, tgt_in[rows], 0))
    assert np.all(got_in[2][rows] != 0)
