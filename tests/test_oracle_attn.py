"""Pins of the oracle's attention core on a shard's heads ("7.3 模型并行与张量
并行" §7.3.4: each card runs attention on its own query heads, which share the
card's key/value head, and concatenates them).

- against torch's fp64 scaled_dot_product_attention (causal and not), with the
  key/value heads repeated for the grouped query heads, and the log-sum-exp
  against torch.logsumexp of the masked scaled scores;
- closed forms: V = 1 gives O = 1; the first position sees only key 0; equal
  keys give the running mean of V;
- causality: keys and values after position r do not change row r;
- the grouping (query head j reads KV head j // (nq / nkv)) against plain
  multi-head attention on repeated heads;
- sampled rows equal the same rows of the full computation, bit for bit;
- brute force in pure Python on a tiny case.
"""
import math

import numpy as np
import pytest
import torch


def _rand(seed, s, nq, nkv, d, scale=1.0):
    g = np.random.default_rng(seed)
    return (g.standard_normal((s, nq * d)) * scale, g.standard_normal((s, nkv * d)) * scale,
            g.standard_normal((s, nkv * d)))


def _torch_ref(Q, K, V, nq, nkv, causal):
    s = Q.shape[0]
    d = Q.shape[1] // nq
    q = torch.tensor(Q).reshape(s, nq, d).transpose(0, 1)            # [nq, s, d]
    k = torch.tensor(K).reshape(s, nkv, d).transpose(0, 1).repeat_interleave(nq // nkv, dim=0).contiguous()
    v = torch.tensor(V).reshape(s, nkv, d).transpose(0, 1).repeat_interleave(nq // nkv, dim=0).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal)
    sc = q @ k.transpose(1, 2) / math.sqrt(d)
    if causal:
        sc = sc.masked_fill(torch.ones(s, s, dtype=torch.bool).triu(1), float("-inf"))
    lse = torch.logsumexp(sc, dim=-1)
    return o.transpose(0, 1).reshape(s, nq * d).numpy(), lse.numpy()


@pytest.mark.parametrize("s,nq,nkv,d,causal", [(33, 8, 1, 16, True), (20, 4, 2, 8, True), (17, 2, 2, 32, False),
                                               (64, 8, 1, 128, True)])
def test_matches_torch_sdpa(oracle_mod, s, nq, nkv, d, causal):
    Q, K, V = _rand(s + d, s, nq, nkv, d)
    O, lse = oracle_mod.attn_core_fwd(Q, K, V, nq, nkv, causal)
    wo, wl = _torch_ref(Q, K, V, nq, nkv, causal)
    np.testing.assert_allclose(O, wo, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, wl, rtol=1e-12, atol=1e-12)


def test_closed_forms(oracle_mod):
    s, nq, nkv, d = 24, 4, 1, 8
    Q, K, V = _rand(5, s, nq, nkv, d, scale=2.0)
    O, _ = oracle_mod.attn_core_fwd(Q, K, np.ones_like(V), nq, nkv)
    np.testing.assert_allclose(O, 1.0, rtol=1e-14)
    O, lse = oracle_mod.attn_core_fwd(Q, K, V, nq, nkv)
    for j in range(nq):                      # position 0 sees key 0 only
        assert np.array_equal(O[0, j * d:(j + 1) * d], V[0])
    np.testing.assert_allclose(lse[:, 0], (Q[0].reshape(nq, d) @ K[0]) / math.sqrt(d), rtol=1e-14)
    # equal (zero) keys: uniform weights over the visible positions, the running mean of V
    O, lse = oracle_mod.attn_core_fwd(Q, np.zeros_like(K), V, nq, nkv)
    mean = np.cumsum(V, axis=0) / np.arange(1, s + 1)[:, None]
    for j in range(nq):
        np.testing.assert_allclose(O[:, j * d:(j + 1) * d], mean, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, np.log(np.arange(1, s + 1))[None, :].repeat(nq, 0), rtol=1e-14)


def test_causality(oracle_mod):
    s, nq, nkv, d, r = 30, 2, 1, 8, 11
    Q, K, V = _rand(6, s, nq, nkv, d)
    O, lse = oracle_mod.attn_core_fwd(Q, K, V, nq, nkv)
    K2, V2 = K.copy(), V.copy()
    K2[r + 1:] += 5.0
    V2[r + 1:] -= 3.0
    O2, lse2 = oracle_mod.attn_core_fwd(Q, K2, V2, nq, nkv)
    assert np.array_equal(O[:r + 1], O2[:r + 1]) and np.array_equal(lse[:, :r + 1], lse2[:, :r + 1])
    assert not np.allclose(O[r + 1:], O2[r + 1:])


def test_grouping_equals_repeated_heads(oracle_mod):
    s, nq, nkv, d = 19, 8, 2, 8
    Q, K, V = _rand(7, s, nq, nkv, d)
    O, lse = oracle_mod.attn_core_fwd(Q, K, V, nq, nkv)
    rep = lambda X: np.concatenate([X[:, (j // 4) * d:(j // 4 + 1) * d] for j in range(nq)], axis=1)  # noqa: E731
    O2, lse2 = oracle_mod.attn_core_fwd(Q, rep(K), rep(V), nq, nq)
    np.testing.assert_allclose(O, O2, rtol=1e-15, atol=0)
    np.testing.assert_allclose(lse, lse2, rtol=1e-15, atol=0)


def test_sampled_rows_equal_full(oracle_mod):
    s, nq, nkv, d = 40, 4, 1, 16
    Q, K, V = _rand(8, s, nq, nkv, d)
    O, lse = oracle_mod.attn_core_fwd(Q, K, V, nq, nkv)
    rows = np.array([0, 7, 39, 13])
    Or, lr = oracle_mod.attn_core_fwd(Q, K, V, nq, nkv, rows=rows)
    assert np.array_equal(Or, O[rows]) and np.array_equal(lr, lse[:, rows])


def test_brute_force_tiny(oracle_mod):
    s, nq, nkv, d = 4, 2, 1, 2
    Q, K, V = _rand(9, s, nq, nkv, d)
    O, lse = oracle_mod.attn_core_fwd(Q, K, V, nq, nkv)
    for j in range(nq):
        for r in range(s):
            sc = [sum(Q[r, j * d + k] * K[c, k] for k in range(d)) / math.sqrt(d) for c in range(r + 1)]
            z = sum(math.exp(x) for x in sc)
            assert abs(lse[j, r] - math.log(z)) <= 1e-13
            for k in range(d):
                want = sum(math.exp(sc[c]) / z * V[c, k] for c in range(r + 1))
                assert abs(O[r, j * d + k] - want) <= 1e-13


# ---------------------------------------------------------------- backward
# Pins of attn_core_bwd (dO -> dQ, dK, dV of the same attention):
# - torch fp64 autograd through scaled_dot_product_attention, the key/value
#   heads repeated for the grouped query heads (autograd then sums a shared
#   head's gradient over its group);
# - central differences of L = sum(dO * O) with the oracle's own forward;
# - grouping: the grouped dK, dV equal the per-head gradients of plain
#   multi-head attention on repeated heads, summed over each group;
# - closed form of uniform attention (all keys zero): dQ = 0,
#   dV[c] = sum_j sum_{r>=c} dO_j[r] / (r+1), and
#   dK[c] = sum_j sum_{r>=c} (dO_j[r].V[c] - dO_j[r].mean_{c'<=r} V[c']) Q_j[r] / ((r+1) sqrt d);
# - shifting every key by one vector leaves all three unchanged (the softmax
#   is shift invariant per row and each dS row sums to zero);
# - sampled positions equal the full computation, bit for bit.
def _torch_bwd(Q, K, V, dO, nq, nkv, causal):
    s = Q.shape[0]
    d = Q.shape[1] // nq
    q = torch.tensor(Q).reshape(s, nq, d).transpose(0, 1).requires_grad_(True)
    k = torch.tensor(K).reshape(s, nkv, d).transpose(0, 1).requires_grad_(True)
    v = torch.tensor(V).reshape(s, nkv, d).transpose(0, 1).requires_grad_(True)
    kr = k.repeat_interleave(nq // nkv, dim=0)
    vr = v.repeat_interleave(nq // nkv, dim=0)
    o = torch.nn.functional.scaled_dot_product_attention(q, kr, vr, is_causal=causal)
    o.backward(torch.tensor(dO).reshape(s, nq, d).transpose(0, 1))
    f = lambda t, n: t.grad.transpose(0, 1).reshape(s, n * d).numpy()  # noqa: E731
    return f(q, nq), f(k, nkv), f(v, nkv)


@pytest.mark.parametrize("s,nq,nkv,d,causal", [(33, 8, 1, 16, True), (20, 4, 2, 8, True), (17, 2, 2, 32, False),
                                               (64, 8, 1, 128, True), (9, 4, 4, 8, False)])
def test_bwd_matches_torch_autograd(oracle_mod, s, nq, nkv, d, causal):
    Q, K, V = _rand(s + 3 * d, s, nq, nkv, d)
    dO = np.random.default_rng(s + 7).standard_normal((s, nq * d))
    dQ, dK, dV = oracle_mod.attn_core_bwd(Q, K, V, dO, nq, nkv, causal)
    wq, wk, wv = _torch_bwd(Q, K, V, dO, nq, nkv, causal)
    for got, want in ((dQ, wq), (dK, wk), (dV, wv)):
        np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-11)


def test_bwd_central_differences(oracle_mod):
    s, nq, nkv, d = 12, 4, 2, 8
    Q, K, V = _rand(21, s, nq, nkv, d)
    dO = np.random.default_rng(22).standard_normal((s, nq * d))
    dQ, dK, dV = oracle_mod.attn_core_bwd(Q, K, V, dO, nq, nkv)
    loss = lambda q, k, v: float(np.sum(dO * oracle_mod.attn_core_fwd(q, k, v, nq, nkv)[0]))  # noqa: E731
    h = 1e-5
    g = np.random.default_rng(23)
    for which, grad in ((0, dQ), (1, dK), (2, dV)):
        for _ in range(6):
            r, c = int(g.integers(s)), int(g.integers(grad.shape[1]))
            args_p = [Q.copy(), K.copy(), V.copy()]
            args_m = [Q.copy(), K.copy(), V.copy()]
            args_p[which][r, c] += h
            args_m[which][r, c] -= h
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(fd - grad[r, c]) <= 1e-7 * max(1.0, abs(fd)), (which, r, c, fd, grad[r, c])


def test_bwd_grouping_sums_repeated_heads(oracle_mod):
    s, nq, nkv, d = 19, 8, 2, 8
    Q, K, V = _rand(24, s, nq, nkv, d)
    dO = np.random.default_rng(25).standard_normal((s, nq * d))
    dQ, dK, dV = oracle_mod.attn_core_bwd(Q, K, V, dO, nq, nkv)
    grp = nq // nkv
    rep = lambda X: np.concatenate([X[:, (j // grp) * d:(j // grp + 1) * d] for j in range(nq)], axis=1)  # noqa: E731
    dQ2, dK2, dV2 = oracle_mod.attn_core_bwd(Q, rep(K), rep(V), dO, nq, nq)
    np.testing.assert_allclose(dQ, dQ2, rtol=1e-13, atol=1e-14)
    for g in range(nkv):
        heads = range(g * grp, (g + 1) * grp)
        np.testing.assert_allclose(dK[:, g * d:(g + 1) * d], sum(dK2[:, j * d:(j + 1) * d] for j in heads),
                                   rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(dV[:, g * d:(g + 1) * d], sum(dV2[:, j * d:(j + 1) * d] for j in heads),
                                   rtol=1e-12, atol=1e-13)


def test_bwd_uniform_attention_closed_form(oracle_mod):
    s, nq, nkv, d = 14, 2, 1, 8
    Q, _, V = _rand(26, s, nq, nkv, d)
    K = np.zeros((s, nkv * d))
    dO = np.random.default_rng(27).standard_normal((s, nq * d))
    dQ, dK, dV = oracle_mod.attn_core_bwd(Q, K, V, dO, nq, nkv)
    assert np.array_equal(dQ, np.zeros_like(dQ))
    mean = np.cumsum(V, axis=0) / np.arange(1, s + 1)[:, None]
    wv = np.zeros((s, d))
    wk = np.zeros((s, d))
    for j in range(nq):
        dOj, Qj = dO[:, j * d:(j + 1) * d], Q[:, j * d:(j + 1) * d]
        for c in range(s):
            for r in range(c, s):
                wv[c] += dOj[r] / (r + 1)
                wk[c] += (dOj[r] @ V[c] - dOj[r] @ mean[r]) * Qj[r] / ((r + 1) * math.sqrt(d))
    np.testing.assert_allclose(dV, wv, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dK, wk, rtol=1e-10, atol=1e-12)


def test_bwd_key_shift_invariance(oracle_mod):
    s, nq, nkv, d = 21, 4, 1, 16
    Q, K, V = _rand(28, s, nq, nkv, d)
    dO = np.random.default_rng(29).standard_normal((s, nq * d))
    a = np.random.default_rng(30).standard_normal(d)
    base = oracle_mod.attn_core_bwd(Q, K, V, dO, nq, nkv)
    shifted = oracle_mod.attn_core_bwd(Q, K + a[None, :], V, dO, nq, nkv)
    for x, y in zip(base, shifted):
        np.testing.assert_allclose(x, y, rtol=1e-9, atol=1e-11)


def test_bwd_sampled_equals_full(oracle_mod):
    s, nq, nkv, d = 40, 4, 2, 16
    Q, K, V = _rand(31, s, nq, nkv, d)
    dO = np.random.default_rng(32).standard_normal((s, nq * d))
    dQ, dK, dV = oracle_mod.attn_core_bwd(Q, K, V, dO, nq, nkv)
    rows, cols = np.array([0, 7, 39, 13]), np.array([39, 0, 5])
    sq, sk, sv = oracle_mod.attn_core_bwd(Q, K, V, dO, nq, nkv, rows=rows, cols=cols)
    assert np.array_equal(sq, dQ[rows]) and np.array_equal(sk, dK[cols]) and np.array_equal(sv, dV[cols])
