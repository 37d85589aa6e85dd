"""Pins of the oracle's vocab-parallel LM head, cross-entropy statistics and
embedding lookup ("7.3 模型并行与张量并行" §7.3.4; lecture 16 notes §5.5).

- the direct loss against torch's fp64 cross_entropy (the library comparison the
  lecture notes themselves make);
- the shard statistics combined over t shards against the direct loss;
- closed forms: uniform logits give ln V, shift invariance, loss >= 0;
- brute force over every target on tiny vocabularies;
- the embedding against numpy indexing of the full table and the one-owner rule.
"""
import math

import numpy as np
import pytest
import torch

from megatron_tensor_layer_tp_amd import inputs as I


def _split_stats(oracle_mod, z, y, t):
    V = z.shape[1]
    Vs = V // t
    st = [oracle_mod.ce_stats(np.ascontiguousarray(z[:, i * Vs:(i + 1) * Vs]), y, i * Vs) for i in range(t)]
    return [a[0] for a in st], [a[1] for a in st], [a[2] for a in st]


def test_direct_loss_matches_torch_cross_entropy(oracle_mod):
    g = np.random.default_rng(1)
    s, V = 16, 96
    z = g.standard_normal((s, V)) * 3
    y = g.integers(0, V, s)
    want = torch.nn.functional.cross_entropy(torch.tensor(z), torch.tensor(y), reduction="none").numpy()
    np.testing.assert_allclose(oracle_mod.ce_direct(z, y), want, rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("t", [1, 2, 3, 4, 8])
def test_shard_statistics_combine_to_full_loss(oracle_mod, t):
    g = np.random.default_rng(2 + t)
    s, V = 10, 48
    z = g.standard_normal((s, V)) * 4
    y = g.integers(0, V, s)
    ms, ses, tls = _split_stats(oracle_mod, z, y, t)
    loss = oracle_mod.ce_combine(ms, ses, tls)
    want = torch.nn.functional.cross_entropy(torch.tensor(z), torch.tensor(y), reduction="none").numpy()
    np.testing.assert_allclose(loss, want, rtol=1e-13, atol=1e-13)
    # exactly one shard holds each target; the others report 0
    owner = y // (V // t)
    for i in range(t):
        assert np.all((tls[i] != 0) | (owner != i) | (z[np.arange(s), y] == 0))
        assert np.all(tls[i][owner != i] == 0.0)
    # the shard maxima are the row maxima of the slices, and their max is the row max
    assert np.array_equal(np.max(np.stack(ms), axis=0), z.max(axis=1))


def test_closed_forms(oracle_mod):
    s, V = 4, 64
    z = np.full((s, V), 0.37)
    y = np.array([0, 5, 63, 17])
    np.testing.assert_allclose(oracle_mod.ce_direct(z, y), np.full(s, math.log(V)), rtol=1e-15)
    ms, ses, tls = _split_stats(oracle_mod, z, y, 4)
    np.testing.assert_allclose(oracle_mod.ce_combine(ms, ses, tls), np.full(s, math.log(V)), rtol=1e-14)
    # shift invariance and non-negativity
    g = np.random.default_rng(4)
    z = g.standard_normal((s, V)) * 5
    a = oracle_mod.ce_direct(z, y)
    np.testing.assert_allclose(oracle_mod.ce_direct(z + 123.25, y), a, rtol=1e-12, atol=1e-12)
    assert np.all(a >= 0)
    # se of one shard is in [1, Vs]: the maximal term contributes exp(0) = 1
    m, se, tl = oracle_mod.ce_stats(np.ascontiguousarray(z[:, :16]), y, 0)
    assert np.all(se >= 1.0) and np.all(se <= 16)


def test_brute_force_tiny_vocab(oracle_mod):
    """All targets, V <= 16, every t dividing V; each loss computed by a plain
    Python loop with math.exp / math.log."""
    g = np.random.default_rng(8)
    for V in (1, 2, 6, 12, 16):
        z = g.standard_normal((V, V)) * 2  # one row per target id
        y = np.arange(V)
        brute = np.array([math.log(sum(math.exp(v) for v in z[r])) - z[r, y[r]] for r in range(V)])
        for t in [d for d in range(1, V + 1) if V % d == 0]:
            ms, ses, tls = _split_stats(oracle_mod, z, y, t)
            np.testing.assert_allclose(oracle_mod.ce_combine(ms, ses, tls), brute, rtol=1e-13, atol=1e-13)


def test_out_of_shard_and_empty_shard(oracle_mod):
    z = np.arange(12, dtype=np.float64).reshape(3, 4)
    y = np.array([-1, 4, 999])  # below, in (global id 4 = local 0 of shard [4,8)), beyond
    m, se, tl = oracle_mod.ce_stats(z, y, 4)
    assert list(tl) == [0.0, z[1, 0], 0.0]
    assert list(m) == [3.0, 7.0, 11.0]
    m0, se0, tl0 = oracle_mod.ce_stats(np.zeros((3, 0)), y, 0)
    assert np.all(m0 == -np.inf) and np.all(se0 == 0.0) and np.all(tl0 == 0.0)


def test_lm_head_matches_numpy(oracle_mod):
    g = np.random.default_rng(6)
    Hf, W = g.standard_normal((5, 9)), g.standard_normal((9, 7))
    np.testing.assert_allclose(oracle_mod.lm_head(Hf, W), Hf @ W, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(oracle_mod.lm_head_rows(Hf, W, np.array([1, 4])), (Hf @ W)[[1, 4]],
                               rtol=1e-14, atol=1e-14)


def test_embedding_matches_full_lookup_and_single_owner(oracle_mod):
    g = np.random.default_rng(10)
    V, h, t, n = 40, 12, 4, 64
    full = I.f32_to_bf16_bits(g.standard_normal((V, h)).astype(np.float32))
    full[full == 0] = 1  # no zero rows: a missed copy must show
    ids = g.integers(0, V, n)
    ids[:3] = [0, V - 1, V // t]  # shard edges
    Vs = V // t
    outs = [oracle_mod.embed(ids, full[i * Vs:(i + 1) * Vs], i * Vs) for i in range(t)]
    # numpy indexing of the whole table is the unsharded lookup
    want = full[ids]
    for r in range(n):
        owner = ids[r] // Vs
        for i in range(t):
            if i == owner:
                assert np.array_equal(outs[i][r], want[r])
            else:
                assert np.all(outs[i][r] == 0)
    # summing the shards (as numbers) reproduces the lookup, as the all-reduce would
    tot = sum(I.bf16_bits_to_f64(o) for o in outs)
    assert np.array_equal(tot, I.bf16_bits_to_f64(want))


def test_embedding_out_of_range_ids_give_zero_rows(oracle_mod):
    table = np.arange(1, 1 + 4 * 3, dtype=np.uint16).reshape(4, 3)
    ids = np.array([-5, 3, 4, 7, 8, 1 << 40])
    out = oracle_mod.embed(ids, table, 4)
    assert np.array_equal(out, np.array([[0, 0, 0], [0, 0, 0], table[0], table[3], [0, 0, 0], [0, 0, 0]],
                                        dtype=np.uint16))
    f32 = np.arange(6, dtype=np.float32).reshape(2, 3) + 1
    out32 = oracle_mod.embed(np.array([1, 2]), f32, 0)
    assert np.array_equal(out32, np.array([f32[1], [0, 0, 0]], dtype=np.float32))


# ---------------------------------------------------------------- CE backward
def _shard_grads(oracle_mod, z, y, t, g):
    """Each shard's gradient slice from the combined (M, S), concatenated."""
    V = z.shape[1]
    Vs = V // t
    ms, ses, _ = _split_stats(oracle_mod, z, y, t)
    M, S = oracle_mod.ce_global(ms, ses)
    parts = [oracle_mod.ce_bwd(np.ascontiguousarray(z[:, i * Vs:(i + 1) * Vs]), y, i * Vs, M, S, g)
             for i in range(t)]
    return np.concatenate(parts, axis=1)


@pytest.mark.parametrize("t", [1, 2, 4, 8])
def test_ce_bwd_matches_torch_autograd(oracle_mod, t):
    """Sharded gradients, concatenated, equal torch's fp64 autograd of
    cross_entropy with per-position upstream gradients."""
    rng = np.random.default_rng(30 + t)
    s, V = 12, 64
    z = rng.standard_normal((s, V)) * 3
    y = rng.integers(0, V, s)
    g = rng.standard_normal(s)
    zt = torch.tensor(z, requires_grad=True)
    loss = torch.nn.functional.cross_entropy(zt, torch.tensor(y), reduction="none")
    loss.backward(torch.tensor(g))
    got = _shard_grads(oracle_mod, z, y, t, g)
    np.testing.assert_allclose(got, zt.grad.numpy(), rtol=1e-12, atol=1e-14)


def test_ce_bwd_finite_differences(oracle_mod):
    """Central differences of the direct loss, entry by entry, on a tiny case."""
    rng = np.random.default_rng(7)
    s, V, t = 3, 12, 3
    z = rng.standard_normal((s, V)) * 2
    y = np.array([0, 7, 11])
    g = np.ones(s)
    got = _shard_grads(oracle_mod, z, y, t, g)
    eps = 1e-6
    for r in range(s):
        for j in range(V):
            zp, zm = z.copy(), z.copy()
            zp[r, j] += eps
            zm[r, j] -= eps
            fd = (oracle_mod.ce_direct(zp, y)[r] - oracle_mod.ce_direct(zm, y)[r]) / (2 * eps)
            assert abs(got[r, j] - fd) <= 1e-8, (r, j, got[r, j], fd)


def test_ce_bwd_invariants(oracle_mod):
    """Every full row sums to 0 (softmax sums to 1, minus the one-hot); the
    entries are p - 1 at the target and p >= 0 elsewhere; a target outside the
    shard adds nothing to it; uniform logits give 1/V - onehot."""
    rng = np.random.default_rng(8)
    s, V, t = 6, 40, 4
    z = rng.standard_normal((s, V)) * 5
    y = rng.integers(0, V, s)
    g = np.full(s, 0.5)
    dz = _shard_grads(oracle_mod, z, y, t, g)
    np.testing.assert_allclose(dz.sum(axis=1), 0.0, atol=1e-15)
    mask = np.zeros_like(dz, dtype=bool)
    mask[np.arange(s), y] = True
    assert np.all(dz[~mask] >= 0) and np.all(dz[mask] < 0)
    zu = np.full((2, V), -1.25)
    yu = np.array([3, 39])
    du = _shard_grads(oracle_mod, zu, yu, t, np.ones(2))
    want = np.full((2, V), 1.0 / V)
    want[[0, 1], yu] -= 1.0
    np.testing.assert_allclose(du, want, rtol=1e-14, atol=1e-16)
    # a shard that holds no target: its slice is the softmax slice only
    M, S = oracle_mod.ce_global(*_split_stats(oracle_mod, z, y, 1)[:2])
    sl = oracle_mod.ce_bwd(z[:, :10], np.full(s, 10_000), 0, M, S, np.ones(s))
    np.testing.assert_allclose(sl, np.exp(z[:, :10] - M[:, None]) / S[:, None], rtol=1e-14)
