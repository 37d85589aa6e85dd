"""GPU parity of the MLP shard (tp_mlp_fwd / tp_mlp_bwd) against the fp64 oracle.

Exact cases (bit for bit):
  * the book's two-card worked example ("7.3 模型并行与张量并行" §7.3.2/§7.3.3),
    fp32 and bf16 storage, each shard and the sum of the shards;
  * configuration 1 (X[8,16], W1[16,64] split in two, integers in [-3,3]), fp32;
  * integer inputs in {-1,0,1} with bf16 storage at multi-tile, ragged and
    split-K sizes: every fp32 accumulation is then exact, so the only rounding
    is the bf16 store of each output and of the saved Z / H / dZ, and the GPU
    must reproduce the oracle's values rounded at exactly those points.
Floating-point cases: relative Frobenius error <= 5e-3 per output against the
fp64 oracle (no intermediate rounding on the oracle side) plus the element-wise
bound of gpu_util.elem_bound, on full outputs for small sizes and on
stratified sampled rows / columns (one in every 64-row or 64-column strip, at
least 64) at the GPT-2-small and GPT-3-175B shard sizes.
"""
import json
import os

import numpy as np
import pytest

from gpu_util import (DEV, check_bf16, dev, empty_like_dt, fill_garbage, host, host_f64, need_gpu,
                      torch, workspace)
from megatron_tensor_layer_tp_amd import inputs as I
from megatron_tensor_layer_tp_amd import tpshard as T

pytestmark = pytest.mark.gpu
TOL = 5e-3
GOLD = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    T.lib()


def run_mlp(act, bf16, X, W1, W2, dY, with_z=True):
    """One shard's forward and backward on the GPU.  X, W1, W2, dY are host
    arrays in the storage type (uint16 bf16 bits or float32)."""
    s, h = X.shape
    ft = W1.shape[1]
    dt = T.TP_DT_BF16 if bf16 else T.TP_DT_F32
    Xd, W1d, W2d, dYd = dev(X), dev(W1), dev(W2), dev(dY)
    Z = fill_garbage(empty_like_dt((s, ft), bf16)) if with_z else None
    H = fill_garbage(empty_like_dt((s, ft), bf16))
    Y = fill_garbage(empty_like_dt((s, h), bf16))
    T.tp_mlp_fwd(act, dt, s, h, ft, Xd, W1d, W2d, Z, H, Y)
    dX = fill_garbage(empty_like_dt((s, h), bf16))
    dW1 = fill_garbage(empty_like_dt((h, ft), bf16))
    dW2 = fill_garbage(empty_like_dt((ft, h), bf16))
    ws, nb = workspace(T.tp_mlp_bwd_workspace(dt, s, h, ft))
    T.tp_mlp_bwd(act, dt, s, h, ft, Xd, W1d, W2d, Z, H, dYd, dX, dW1, dW2, ws, nb)
    torch.cuda.synchronize()
    out = dict(H=H, Y=Y, dX=dX, dW1=dW1, dW2=dW2)
    if with_z:
        out["Z"] = Z
    return out


def rne(x):
    """Round fp64 values (exact integers below 2^24 here) to bf16, back to fp64."""
    return I.bf16_bits_to_f64(I.f32_to_bf16_bits(np.asarray(x, dtype=np.float32)))


# ---------------------------------------------------------------- exact cases
@pytest.mark.parametrize("bf16", [False, True])
def test_worked_example_each_shard_and_sum(bf16):
    g = json.load(open(GOLD))
    X = np.array(g["X"], np.float32)
    W1 = np.array(g["W1"], np.float32)
    W2 = np.array(g["W2"], np.float32)
    dY = np.array(g["dY"], np.float32)
    conv = I.f32_to_bf16_bits if bf16 else (lambda a: a)
    Ys, dXs = 0, 0
    for i in range(g["t"]):
        sl = slice(2 * i, 2 * i + 2)
        o = run_mlp(T.TP_ACT_RELU, bf16, conv(X), conv(np.ascontiguousarray(W1[:, sl])),
                    conv(np.ascontiguousarray(W2[sl])), conv(dY))
        assert np.array_equal(host_f64(o["H"]), np.array(g["H_partial"][i], float))
        assert np.array_equal(host_f64(o["Y"]), np.array(g["Y_partial"][i], float))
        assert np.array_equal(host_f64(o["dX"]), np.array(g["dX_partial"][i], float))
        Ys = Ys + host_f64(o["Y"])
        dXs = dXs + host_f64(o["dX"])
    assert np.array_equal(Ys, np.array(g["Y"], float))
    assert np.array_equal(dXs, np.array(g["dX"], float))


@pytest.mark.parametrize("with_z", [True, False])
def test_config1_fp32_bit_exact(oracle_mod, with_z):
    d = I.mlp_inputs(1)
    X, dY = d["X"], d["dY"]
    Yt, dXt = 0, 0
    for i in range(d["t"]):
        o = run_mlp(T.TP_ACT_RELU, False, X, d["W1"][i], d["W2"][i], dY, with_z=with_z)
        Z, H, Y = oracle_mod.mlp_fwd("relu", X, d["W1"][i], d["W2"][i])
        dX, dW1, dW2 = oracle_mod.mlp_bwd("relu", X, d["W1"][i], d["W2"][i], dY)
        want = dict(Z=Z, H=H, Y=Y, dX=dX, dW1=dW1, dW2=dW2)
        for k, t in o.items():
            assert np.array_equal(host_f64(t), want[k]), k
        Yt = Yt + host_f64(o["Y"])
        dXt = dXt + host_f64(o["dX"])
    W1 = np.concatenate([d["W1"][i] for i in range(d["t"])], axis=1)
    W2 = np.concatenate([d["W2"][i] for i in range(d["t"])], axis=0)
    assert np.array_equal(Yt, oracle_mod.mlp_fwd("relu", X, W1, W2)[2])
    assert np.array_equal(dXt, oracle_mod.mlp_bwd("relu", X, W1, W2, dY)[0])


EXACT_SHAPES = [
    (300, 200, 136),   # s not a multiple of 8: element-wise loads, ragged tiles
    (512, 384, 640),   # 16-byte loads, several tiles
    (264, 136, 264),   # 16-byte loads, tails of 8 past the tile edge
    (2048, 128, 256),  # long K for the weight gradients: split-K
    (4104, 8, 8),      # one output tile, K long enough for more than 8 splits
    (520, 200, 1000),  # 128x192 tiles with ragged M, N (1000 = 5*192 + 40) and K edges
    (1032, 392, 776),  # 192-column tiles in the paired backward, ragged everywhere
    (1, 8, 8),
]


def integer_exact_case(oracle_mod, s, h, ft):
    """Integer inputs in {-1,0,1}, bf16 storage: the GPU must match the oracle
    rounded to bf16 exactly where the kernels store."""
    g = np.random.default_rng(s * 7 + h)
    X, W1, W2, dY = (g.integers(-1, 2, size=sh).astype(np.float32)
                     for sh in ((s, h), (h, ft), (ft, h), (s, h)))
    o = run_mlp(T.TP_ACT_RELU, True, *(I.f32_to_bf16_bits(a) for a in (X, W1, W2, dY)))
    mm = oracle_mod.matmul
    Z = mm(X, W1)
    Zb = rne(Z)
    Hb = oracle_mod.act("relu", Zb)
    Y = rne(mm(Hb, W2))
    dZb = rne(mm(dY, W2, tb=True) * oracle_mod.act_grad("relu", Zb))
    want = dict(Z=Zb, H=Hb, Y=Y, dX=rne(mm(dZb, W1, tb=True)), dW1=rne(mm(X, dZb, ta=True)),
                dW2=rne(mm(Hb, dY, ta=True)))
    for k, t in o.items():
        got = host_f64(t)
        bad = np.argwhere(got != want[k])
        assert bad.size == 0, (k, bad[:5], got[tuple(bad[0])], want[k][tuple(bad[0])])


@pytest.mark.parametrize("s,h,ft", EXACT_SHAPES)
def test_integer_bf16_exact(oracle_mod, s, h, ft):
    integer_exact_case(oracle_mod, s, h, ft)


# ---------------------------------------------------------------- floating point
def check_close(got_t, want, name, tol=TOL, rows=None, cols=None):
    got = host_f64(got_t)
    if rows is not None:
        got = got[rows]
    if cols is not None:
        got = got[:, cols]
    return check_bf16(got, want, name, tol=tol)


@pytest.mark.parametrize("s,h,ft", [(300, 200, 136), (520, 264, 392), (256, 256, 512)])
@pytest.mark.parametrize("act", ["gelu", "relu"])
def test_float_small_full(oracle_mod, s, h, ft, act):
    g = np.random.default_rng(3)
    X = I.f32_to_bf16_bits(g.standard_normal((s, h)).astype(np.float32))
    W1 = I.f32_to_bf16_bits((g.standard_normal((h, ft)) * 0.05).astype(np.float32))
    W2 = I.f32_to_bf16_bits((g.standard_normal((ft, h)) * 0.05).astype(np.float32))
    dY = I.f32_to_bf16_bits(g.standard_normal((s, h)).astype(np.float32))
    a = T.TP_ACT_GELU if act == "gelu" else T.TP_ACT_RELU
    o = run_mlp(a, True, X, W1, W2, dY)
    f = [I.bf16_bits_to_f64(v) for v in (X, W1, W2, dY)]
    Z, H, Y = oracle_mod.mlp_fwd(act, *f[:3])
    dX, dW1, dW2 = oracle_mod.mlp_bwd(act, *f)
    for k, w in dict(Z=Z, H=H, Y=Y, dX=dX, dW1=dW1, dW2=dW2).items():
        check_close(o[k], w, k)


def _sampled_config(oracle_mod, cfg, n_rows, n_cols):
    d = I.mlp_inputs(cfg, shards=[0])
    s, h, ft = d["s"], d["h"], d["ft"]
    o = run_mlp(T.TP_ACT_GELU, True, d["X"], d["W1"][0], d["W2"][0], d["dY"])
    X, W1, W2, dY = (I.bf16_bits_to_f64(v) for v in (d["X"], d["W1"][0], d["W2"][0], d["dY"]))
    rows = I.sample_rows(s, n_rows, cfg, 1)
    c1 = I.sample_rows(ft, n_cols, cfg, 2)
    r2 = I.sample_rows(ft, n_cols, cfg, 3)
    Z, H, Y = oracle_mod.mlp_fwd_rows("gelu", X, W1, W2, rows)
    check_close(o["Z"], Z, "Z", rows=rows)
    check_close(o["H"], H, "H", rows=rows)
    check_close(o["Y"], Y, "Y", rows=rows)
    dX, dW1, dW2 = oracle_mod.mlp_bwd_sampled("gelu", X, W1, W2, dY, rows, c1, r2)
    check_close(o["dX"], dX, "dX", rows=rows)
    check_close(o["dW1"], dW1, "dW1", cols=c1)
    check_close(o["dW2"], dW2, "dW2", rows=r2)
    return o


def test_gpt2_small_shard_sampled(oracle_mod):
    o = _sampled_config(oracle_mod, 2, 64, 64)
    # run-twice determinism: no atomics, split-K summed in a fixed order
    d = I.mlp_inputs(2, shards=[0])
    o2 = run_mlp(T.TP_ACT_GELU, True, d["X"], d["W1"][0], d["W2"][0], d["dY"])
    for k in o:
        assert torch.equal(o[k], o2[k]), k


def test_gpt3_shard_sampled(oracle_mod):
    _sampled_config(oracle_mod, 3, 64, 64)
