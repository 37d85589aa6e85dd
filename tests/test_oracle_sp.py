"""Pins of the oracle's sequence-parallel region ("7.3 模型并行与张量并行" §7.3.6:
LayerNorm and dropout act on each position independently, so each card keeps
s/t positions between a sublayer's reduce-scatter and the next all-gather):
residual add with an explicit dropout mask, LayerNorm, and their backward.

- forward and backward against torch fp64 layer_norm and autograd;
- closed forms: a constant row gives beta, unit gamma / zero beta give zero
  mean and variance var / (var + eps), p = 0 with an all-ones mask is x + y;
- the t shards' slices equal the same rows of the unsharded region, and the
  shards' dgamma / dbeta sum to the unsharded ones (what the all-reduce of the
  LayerNorm parameters' gradients adds up);
- central differences on a tiny case.
"""
import numpy as np
import pytest
import torch


def _case(seed, n, h, p):
    g = np.random.default_rng(seed)
    y, x = g.standard_normal((n, h)), g.standard_normal((n, h)) * 2
    mask = (g.random((n, h)) >= p).astype(np.uint8)
    gamma, beta = 1 + 0.1 * g.standard_normal(h), 0.1 * g.standard_normal(h)
    dz, dun = g.standard_normal((n, h)), g.standard_normal((n, h))
    return y, x, mask, gamma, beta, dz, dun


@pytest.mark.parametrize("n,h,p", [(8, 64, 0.1), (5, 33, 0.0), (16, 128, 0.5)])
def test_matches_torch(oracle_mod, n, h, p):
    y, x, mask, gamma, beta, dz, dun = _case(n + h, n, h, p)
    u, z, mean, rstd = oracle_mod.sp_ln_fwd(y, x, mask, gamma, beta, p)
    ty, tx, tg, tb = (torch.tensor(a, requires_grad=True) for a in (y, x, gamma, beta))
    tu = tx + ty * torch.tensor(mask, dtype=torch.float64) / (1 - p)
    tz = torch.nn.functional.layer_norm(tu, (h,), tg, tb, eps=oracle_mod.LN_EPS)
    np.testing.assert_allclose(u, tu.detach().numpy(), rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(z, tz.detach().numpy(), rtol=1e-12, atol=1e-12)
    ((tz * torch.tensor(dz)).sum() + (tu * torch.tensor(dun)).sum()).backward()
    dx, dy, dg, db = oracle_mod.sp_ln_bwd(dz, dun, u, mean, rstd, gamma, mask, p)
    np.testing.assert_allclose(dx, tx.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dy, ty.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dg, tg.grad.numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(db, tb.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_closed_forms(oracle_mod):
    n, h = 4, 32
    y, x, mask, gamma, beta, _, _ = _case(1, n, h, 0.2)
    u, z, _, _ = oracle_mod.sp_ln_fwd(np.zeros((n, h)), np.full((n, h), 3.25), mask, gamma, beta, 0.2)
    np.testing.assert_allclose(z, np.broadcast_to(beta, (n, h)), rtol=0, atol=1e-12)
    u, z, mean, rstd = oracle_mod.sp_ln_fwd(y, x, mask, np.ones(h), np.zeros(h), 0.2)
    np.testing.assert_allclose(z.mean(axis=1), 0.0, atol=1e-14)
    var = ((u - u.mean(axis=1, keepdims=True)) ** 2).mean(axis=1)
    np.testing.assert_allclose(z.var(axis=1), var / (var + oracle_mod.LN_EPS), rtol=1e-12)
    np.testing.assert_allclose(rstd, 1 / np.sqrt(var + oracle_mod.LN_EPS), rtol=1e-13)
    u0, _, _, _ = oracle_mod.sp_ln_fwd(y, x, np.ones((n, h), np.uint8), gamma, beta, 0.0)
    assert np.array_equal(u0, x + y)


@pytest.mark.parametrize("t", [2, 4])
def test_slices_equal_unsharded(oracle_mod, t):
    n, h, p = 16, 48, 0.25
    y, x, mask, gamma, beta, dz, dun = _case(3, n, h, p)
    u, z, mean, rstd = oracle_mod.sp_ln_fwd(y, x, mask, gamma, beta, p)
    dx, dy, dg, db = oracle_mod.sp_ln_bwd(dz, dun, u, mean, rstd, gamma, mask, p)
    k = n // t
    sdg, sdb = np.zeros(h), np.zeros(h)
    for i in range(t):
        r = slice(i * k, (i + 1) * k)
        ui, zi, mi, ri = oracle_mod.sp_ln_fwd(y[r], x[r], mask[r], gamma, beta, p)
        assert np.array_equal(ui, u[r]) and np.array_equal(zi, z[r])
        dxi, dyi, dgi, dbi = oracle_mod.sp_ln_bwd(dz[r], dun[r], ui, mi, ri, gamma, mask[r], p)
        assert np.array_equal(dxi, dx[r]) and np.array_equal(dyi, dy[r])
        sdg += dgi
        sdb += dbi
    np.testing.assert_allclose(sdg, dg, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(sdb, db, rtol=1e-13, atol=1e-13)


def test_finite_differences(oracle_mod):
    n, h, p = 2, 6, 0.5
    y, x, mask, gamma, beta, dz, dun = _case(4, n, h, p)

    def loss(y_, x_, g_, b_):
        u, z, _, _ = oracle_mod.sp_ln_fwd(y_, x_, mask, g_, b_, p)
        return float((z * dz).sum() + (u * dun).sum())

    u, z, mean, rstd = oracle_mod.sp_ln_fwd(y, x, mask, gamma, beta, p)
    dx, dy, dg, db = oracle_mod.sp_ln_bwd(dz, dun, u, mean, rstd, gamma, mask, p)
    eps = 1e-6
    for arr, grad, idx in ((x, dx, 0), (y, dy, 1), (gamma, dg, 2), (beta, db, 3)):
        flat = arr.reshape(-1)
        for i in range(flat.size):
            args = [y.copy(), x.copy(), gamma.copy(), beta.copy()]
            a_p, a_m = [a.copy() for a in args], [a.copy() for a in args]
            pos = {0: 1, 1: 0, 2: 2, 3: 3}[idx]
            a_p[pos].reshape(-1)[i] += eps
            a_m[pos].reshape(-1)[i] -= eps
            fd = (loss(*a_p) - loss(*a_m)) / (2 * eps)
            assert abs(grad.reshape(-1)[i] - fd) <= 1e-6 * max(1.0, abs(fd)), (idx, i, grad.reshape(-1)[i], fd)
