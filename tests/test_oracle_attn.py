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
