"""Pins of oracle.layernorm (CPU only)."""

import numpy as np
import torch

from oracle import layernorm


def test_matches_torch_layer_norm_float64():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((37, 96)) * 3 + 0.5
    g = rng.standard_normal(96)
    b = rng.standard_normal(96)
    y, mu, rs = layernorm(x, g, b, 1e-5)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (96,), torch.from_numpy(g), torch.from_numpy(b), 1e-5)
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-12)
    var, mean = torch.var_mean(torch.from_numpy(x), dim=1, unbiased=False)
    np.testing.assert_allclose(mu, mean.numpy(), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(rs, 1.0 / np.sqrt(var.numpy() + 1e-5), rtol=1e-13)


def test_constant_rows_give_beta():
    x = np.repeat(np.array([[2.5], [-7.0], [0.0]]), 16, axis=1)
    g = np.linspace(-2, 2, 16)
    b = np.arange(16, dtype=np.float64)
    y, mu, rs = layernorm(x, g, b, 1e-5)
    np.testing.assert_array_equal(y, np.broadcast_to(b, (3, 16)))
    np.testing.assert_array_equal(mu, [2.5, -7.0, 0.0])
    np.testing.assert_allclose(rs, 1.0 / np.sqrt(1e-5), rtol=1e-15)


def test_normalized_row_invariants():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((8, 64)) * 10
    eps = 0.25
    y, mu, rs = layernorm(x, np.ones(64), np.zeros(64), eps)
    var = x.var(axis=1)
    np.testing.assert_allclose(y.mean(axis=1), 0.0, atol=1e-12)
    np.testing.assert_allclose(y.var(axis=1), var / (var + eps), rtol=1e-12)


def test_python_loop_tiny():
    x = np.array([[1.0, 2.0, 4.0, 8.0], [-1.0, 0.5, 0.25, 3.0]])
    g = np.array([1.0, -2.0, 0.5, 3.0])
    b = np.array([0.0, 1.0, -1.0, 2.0])
    eps = 1e-3
    y, _, _ = layernorm(x, g, b, eps)
    for r in range(2):
        m = sum(x[r]) / 4
        v = sum((t - m) ** 2 for t in x[r]) / 4
        for c in range(4):
            assert abs(y[r, c] - ((x[r, c] - m) / (v + eps) ** 0.5 * g[c] + b[c])) < 1e-12
