"""The seeded input generator: bf16 rounding, determinism and shard keys."""
import numpy as np
import pytest
import torch

from megatron_tensor_layer_tp_amd import inputs as I


def test_bf16_rounding_matches_torch_rne():
    g = np.random.default_rng(0)
    x = np.concatenate([g.standard_normal(100000).astype(np.float32) * 7,
                        np.array([0.0, -0.0, 1.0, np.inf, -np.inf, 3.4e38, 1e-40, -1e-45], np.float32),
                        # exact ties between two bf16 values: even mantissa wins
                        (np.array([0x3F808000, 0x3F818000, 0xBF808000], np.uint32)).view(np.float32)])
    want = torch.tensor(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(I.f32_to_bf16_bits(x), want)
    back = I.bf16_bits_to_f32(want)
    assert np.array_equal(back, torch.tensor(x).to(torch.bfloat16).float().numpy())


def test_draws_are_deterministic_and_keyed_by_shard():
    a = I.normal_bf16((4, 8), 0.02, 2, I.T_W1, 0)
    b = I.normal_bf16((4, 8), 0.02, 2, I.T_W1, 0)
    c = I.normal_bf16((4, 8), 0.02, 2, I.T_W1, 1)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    d = I.mlp_inputs(1)
    assert d["X"].shape == (8, 16) and d["W1"][1].shape == (16, 32) and d["W2"][0].shape == (32, 16)
    assert set(np.unique(d["X"])) <= set(range(-3, 4))


def test_sigma_is_standard_deviation():
    w = I.bf16_bits_to_f64(I.normal_bf16((512, 512), 0.02, 99, I.T_W1))
    assert abs(w.std() - 0.02) < 0.0005


def test_sample_rows_include_edges():
    r = I.sample_rows(1000, 64, 3)
    assert r[0] == 0 and r[-1] == 999 and len(set(r)) == len(r) and np.all(np.diff(r) > 0)
    assert np.array_equal(I.sample_rows(5, 64, 3), np.arange(5))


@pytest.mark.parametrize("n,k,stratum", [(8192, 64, 64), (8192, 64, 128), (6144, 64, 64), (16032, 64, 64),
                                         (1024, 64, 64), (128, 64, 64), (100, 64, 32), (8200, 64, 64)])
def test_sample_rows_stratified(n, k, stratum):
    """Every run of `stratum` consecutive indices (every tile strip) holds a
    sampled index, there are at least k of them, and the draw is seeded."""
    r = I.sample_rows(n, k, 4, 7, stratum=stratum)
    assert len(r) >= min(n, k) and r[0] == 0 and r[-1] == n - 1 and np.all(np.diff(r) > 0)
    assert r.min() >= 0 and r.max() < n
    for s0 in range(0, n, stratum):
        assert np.any((r >= s0) & (r < s0 + stratum)), s0
    assert np.array_equal(r, I.sample_rows(n, k, 4, 7, stratum=stratum))
