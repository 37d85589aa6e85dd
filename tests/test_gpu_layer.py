"""GPU parity of the SwiGLU and attention-projection shards against the fp64
oracle ("7.3 模型并行与张量并行" §7.3.4): full outputs at small sizes (ragged
tiles, several segments), stratified sampled rows / columns at the
Llama-3-70B t=8 shard size (at least one in every 64-row or 64-column strip,
so every tile of every launch is compared).  Bar: relative Frobenius error
<= 5e-3 per output tensor and the element-wise bound of gpu_util.elem_bound.

Exact cases: integer inputs in {-1,0,1} make every fp32 accumulation exact,
so all ten attention-projection outputs (N-segments Q|K|V, K-segments
dQ.Wq^T + dK.Wk^T + dV.Wv^T, the paired launches, split-K weight gradients)
and SwiGLU's G and U must equal the oracle's values rounded to bf16, bit for
bit."""
import numpy as np
import pytest

from gpu_util import (check_bf16, dev, empty_like_dt, fill_garbage, host_f64, need_gpu, torch,
                      workspace)
from megatron_tensor_layer_tp_amd import inputs as I
from megatron_tensor_layer_tp_amd import tpshard as T

pytestmark = pytest.mark.gpu
TOL = 5e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    T.lib()


def close(got_t, want, name, rows=None, cols=None, tol=TOL):
    got = host_f64(got_t)
    if rows is not None:
        got = got[rows]
    if cols is not None:
        got = got[:, cols]
    if tol == TOL:
        check_bf16(got, want, name)
    else:  # fp32 storage: the same two bars, scaled to fp32 accumulation
        check_bf16(got, want, name, tol=tol, rel=tol, rms_frac=10 * tol)


def bf(a):
    return I.f32_to_bf16_bits(np.asarray(a, np.float32))


# ---------------------------------------------------------------- SwiGLU
def run_swiglu(bf16, X, Wg, Wu, Wd, dY):
    s, h = X.shape
    ft = Wg.shape[1]
    dt = T.TP_DT_BF16 if bf16 else T.TP_DT_F32
    Xd, Wgd, Wud, Wdd, dYd = map(dev, (X, Wg, Wu, Wd, dY))
    G, U, A = (fill_garbage(empty_like_dt((s, ft), bf16)) for _ in range(3))
    Y = fill_garbage(empty_like_dt((s, h), bf16))
    T.tp_swiglu_fwd(dt, s, h, ft, Xd, Wgd, Wud, Wdd, G, U, A, Y)
    dX = fill_garbage(empty_like_dt((s, h), bf16))
    dWg, dWu = (fill_garbage(empty_like_dt((h, ft), bf16)) for _ in range(2))
    dWd = fill_garbage(empty_like_dt((ft, h), bf16))
    ws, nb = workspace(T.tp_swiglu_bwd_workspace(dt, s, h, ft))
    T.tp_swiglu_bwd(dt, s, h, ft, Xd, Wgd, Wud, Wdd, G, U, A, dYd, dX, dWg, dWu, dWd, ws, nb)
    torch.cuda.synchronize()
    return dict(G=G, U=U, A=A, Y=Y, dX=dX, dWg=dWg, dWu=dWu, dWd=dWd)


@pytest.mark.parametrize("s,h,ft", [(136, 96, 72), (520, 264, 392), (300, 200, 100), (256, 512, 256)])
def test_swiglu_small_full(oracle_mod, s, h, ft):
    g = np.random.default_rng(s + ft)
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


def test_swiglu_fp32_small(oracle_mod):
    g = np.random.default_rng(1)
    s, h, ft = 70, 40, 24
    X, dY = g.standard_normal((s, h)).astype(np.float32), g.standard_normal((s, h)).astype(np.float32)
    Wg, Wu = (g.standard_normal((h, ft)) * 0.2).astype(np.float32), (g.standard_normal((h, ft)) * 0.2).astype(np.float32)
    Wd = (g.standard_normal((ft, h)) * 0.2).astype(np.float32)
    o = run_swiglu(False, X, Wg, Wu, Wd, dY)
    G, U, A, Y = oracle_mod.swiglu_fwd(X, Wg, Wu, Wd)
    dX, dWg, dWu, dWd = oracle_mod.swiglu_bwd(X, Wg, Wu, Wd, dY)
    for k, w in dict(G=G, U=U, A=A, Y=Y, dX=dX, dWg=dWg, dWu=dWu, dWd=dWd).items():
        close(o[k], w, k, tol=1e-5)


def test_swiglu_llama3_shard_sampled(oracle_mod):
    d = I.swiglu_inputs(4)
    s, h, ft = d["s"], d["h"], d["ft"]
    o = run_swiglu(True, d["X"], d["Wg"][0], d["Wu"][0], d["Wd"][0], d["dY"])
    X, Wg, Wu, Wd, dY = (I.bf16_bits_to_f64(v) for v in (d["X"], d["Wg"][0], d["Wu"][0], d["Wd"][0], d["dY"]))
    rows = I.sample_rows(s, 64, 4, 1)
    cols = I.sample_rows(ft, 64, 4, 2)
    rd = I.sample_rows(ft, 64, 4, 3)
    G, U, A, Y = oracle_mod.swiglu_fwd_rows(X, Wg, Wu, Wd, rows)
    for k, w in dict(G=G, U=U, A=A, Y=Y).items():
        close(o[k], w, k, rows=rows)
    dX, dWg, dWu, dWd = oracle_mod.swiglu_bwd_sampled(X, Wg, Wu, Wd, dY, rows, cols, rd)
    close(o["dX"], dX, "dX", rows=rows)
    close(o["dWg"], dWg, "dWg", cols=cols)
    close(o["dWu"], dWu, "dWu", cols=cols)
    close(o["dWd"], dWd, "dWd", rows=rd)


# ---------------------------------------------------------------- attention projections
def run_attn(bf16, X, Wq, Wk, Wv, O, Wo, dQ, dK, dV, dY):
    s, h = X.shape
    dq, dkv = Wq.shape[1], Wk.shape[1]
    dt = T.TP_DT_BF16 if bf16 else T.TP_DT_F32
    dv = list(map(dev, (X, Wq, Wk, Wv, O, Wo, dQ, dK, dV, dY)))
    Q = fill_garbage(empty_like_dt((s, dq), bf16))
    K, V = (fill_garbage(empty_like_dt((s, dkv), bf16)) for _ in range(2))
    Y = fill_garbage(empty_like_dt((s, h), bf16))
    T.tp_attn_proj_fwd(dt, s, h, dq, dkv, *dv[:6], Q, K, V, Y)
    dX = fill_garbage(empty_like_dt((s, h), bf16))
    dWq = fill_garbage(empty_like_dt((h, dq), bf16))
    dWk, dWv = (fill_garbage(empty_like_dt((h, dkv), bf16)) for _ in range(2))
    dO = fill_garbage(empty_like_dt((s, dq), bf16))
    dWo = fill_garbage(empty_like_dt((dq, h), bf16))
    ws, nb = workspace(T.tp_attn_proj_bwd_workspace(dt, s, h, dq, dkv))
    T.tp_attn_proj_bwd(dt, s, h, dq, dkv, *dv, dX, dWq, dWk, dWv, dO, dWo, ws, nb)
    torch.cuda.synchronize()
    return dict(Q=Q, K=K, V=V, Y=Y, dX=dX, dWq=dWq, dWk=dWk, dWv=dWv, dO=dO, dWo=dWo)


@pytest.mark.parametrize("s,h,dq,dkv", [(136, 128, 64, 8), (520, 264, 256, 32), (300, 200, 48, 16),
                                        (256, 512, 1024, 128)])
def test_attn_small_full(oracle_mod, s, h, dq, dkv):
    g = np.random.default_rng(s + dq)
    X = bf(g.standard_normal((s, h)))
    Wq, Wk, Wv = bf(g.standard_normal((h, dq)) * 0.05), bf(g.standard_normal((h, dkv)) * 0.05), \
        bf(g.standard_normal((h, dkv)) * 0.05)
    O, Wo = bf(g.standard_normal((s, dq))), bf(g.standard_normal((dq, h)) * 0.05)
    dQ, dK, dV, dY = (bf(g.standard_normal(sh)) for sh in ((s, dq), (s, dkv), (s, dkv), (s, h)))
    o = run_attn(True, X, Wq, Wk, Wv, O, Wo, dQ, dK, dV, dY)
    f = [I.bf16_bits_to_f64(v) for v in (X, Wq, Wk, Wv, O, Wo, dQ, dK, dV, dY)]
    Q, K, V, Y = oracle_mod.attn_fwd(*f[:6])
    dX, dWq, dWk, dWv, dO, dWo = oracle_mod.attn_bwd(*f)
    for k, w in dict(Q=Q, K=K, V=V, Y=Y, dX=dX, dWq=dWq, dWk=dWk, dWv=dWv, dO=dO, dWo=dWo).items():
        close(o[k], w, k)


def test_attn_llama3_shard_sampled(oracle_mod):
    d = I.attn_inputs(4)
    s = d["s"]
    names = ("X", "Wq", "Wk", "Wv", "O", "Wo", "dQ", "dK", "dV", "dY")
    raw = [d[n] if n in ("X", "dY") else d[n][0] for n in names]
    o = run_attn(True, *raw)
    f = [I.bf16_bits_to_f64(v) for v in raw]
    rows = I.sample_rows(s, 64, 4, 11)
    cq = I.sample_rows(d["dq"], 64, 4, 12)
    ckv = I.sample_rows(d["dkv"], 64, 4, 13)
    ro = I.sample_rows(d["dq"], 64, 4, 14)
    Q, K, V, Y = oracle_mod.attn_fwd_rows(*f[:6], rows)
    for k, w in dict(Q=Q, K=K, V=V, Y=Y).items():
        close(o[k], w, k, rows=rows)
    dX, dWq, dWk, dWv, dO, dWo = oracle_mod.attn_bwd_sampled(*f, rows, cq, ckv, ro)
    close(o["dX"], dX, "dX", rows=rows)
    close(o["dO"], dO, "dO", rows=rows)
    close(o["dWq"], dWq, "dWq", cols=cq)
    close(o["dWk"], dWk, "dWk", cols=ckv)
    close(o["dWv"], dWv, "dWv", cols=ckv)
    close(o["dWo"], dWo, "dWo", rows=ro)


# ---------------------------------------------------------------- exact integer cases
def rne(x):
    """Round fp64 values (exact integers below 2^24 here) to bf16, back to fp64."""
    return I.bf16_bits_to_f64(I.f32_to_bf16_bits(np.asarray(x, dtype=np.float32)))


def assert_bits(got_t, want, name):
    got = host_f64(got_t)
    bad = np.argwhere(got != want)
    assert bad.size == 0, (name, bad.shape[0], bad[:5], got[tuple(bad[0])], want[tuple(bad[0])])


def ints(g, shape):
    return g.integers(-1, 2, size=shape).astype(np.float32)


ATTN_EXACT = [
    (300, 200, 48, 16),     # s, h not multiples of 8: element-wise loads
    (520, 264, 256, 32),    # 16-byte loads, ragged tiles, several segments
    (2048, 136, 256, 128),  # long K for the weight gradients: split-K
    (1032, 392, 392, 136),  # 192-column tiles, K-segments not multiples of 64
    (4104, 128, 128, 8),    # few output tiles, K long enough for many splits
    (1, 8, 8, 8),
]


def attn_integer_case(oracle_mod, s, h, dq, dkv):
    g = np.random.default_rng(s * 13 + dq)
    X, O, dY = ints(g, (s, h)), ints(g, (s, dq)), ints(g, (s, h))
    Wq, Wk, Wv, Wo = ints(g, (h, dq)), ints(g, (h, dkv)), ints(g, (h, dkv)), ints(g, (dq, h))
    dQ, dK, dV = ints(g, (s, dq)), ints(g, (s, dkv)), ints(g, (s, dkv))
    args = (X, Wq, Wk, Wv, O, Wo, dQ, dK, dV, dY)
    o = run_attn(True, *(I.f32_to_bf16_bits(a) for a in args))
    Q, K, V, Y = oracle_mod.attn_fwd(*args[:6])
    dX, dWq, dWk, dWv, dO, dWo = oracle_mod.attn_bwd(*args)
    for k, w in dict(Q=Q, K=K, V=V, Y=Y, dX=dX, dWq=dWq, dWk=dWk, dWv=dWv, dO=dO, dWo=dWo).items():
        assert_bits(o[k], rne(w), k)


@pytest.mark.parametrize("s,h,dq,dkv", ATTN_EXACT)
def test_attn_proj_integer_exact(oracle_mod, s, h, dq, dkv):
    attn_integer_case(oracle_mod, s, h, dq, dkv)


SWIGLU_EXACT = [(300, 200, 136), (520, 264, 392), (2048, 136, 256), (1032, 392, 776), (1, 8, 8)]


def swiglu_integer_case(oracle_mod, s, h, ft):
    """G and U are plain products: bit-exact.  A = SiLU(G) U and everything
    after it go through the fp32 SiLU, so they keep the tolerance bar."""
    g = np.random.default_rng(s * 17 + ft)
    X, dY = ints(g, (s, h)), ints(g, (s, h))
    Wg, Wu, Wd = ints(g, (h, ft)), ints(g, (h, ft)), ints(g, (ft, h))
    o = run_swiglu(True, *(I.f32_to_bf16_bits(a) for a in (X, Wg, Wu, Wd, dY)))
    assert_bits(o["G"], rne(oracle_mod.matmul(X, Wg)), "G")
    assert_bits(o["U"], rne(oracle_mod.matmul(X, Wu)), "U")


@pytest.mark.parametrize("s,h,ft", SWIGLU_EXACT)
def test_swiglu_gate_up_integer_exact(oracle_mod, s, h, ft):
    swiglu_integer_case(oracle_mod, s, h, ft)
