"""Pins of the feed-forward oracle to facts outside itself (no GPU needed).

gelu against values of the normal CDF (Phi(1) = 0.8413447460685429..., Phi(-1) = 1 - Phi(1), and
the lower tail Phi(-5), Phi(-10) to relative precision), its
limits and odd-part identity gelu(z) - gelu(-z) = z; the whole feed-forward against torch's exact
gelu and float64 matmuls (library routines); closed forms (zero first weights give the same row for
every token; zero second weights give the bias; gelu and relu agree far from zero); and position-wise structure (permuting tokens
permutes the output, so any blocking of the tokens gives the same result).
"""
import numpy as np
import pytest
import torch

import oracle


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def test_gelu_values():
    phi1 = 0.8413447460685429  # standard normal CDF at 1
    assert abs(oracle.gelu(1.0) - phi1) < 1e-15
    assert abs(oracle.gelu(-1.0) - (-(1.0 - phi1))) < 1e-15
    assert oracle.gelu(0.0) == 0.0
    z = np.linspace(-6, 6, 101)
    assert np.abs(oracle.gelu(z) - oracle.gelu(-z) - z).max() < 1e-13  # z Phi(z) + z Phi(-z) = z
    assert abs(oracle.gelu(40.0) - 40.0) < 1e-12 and abs(oracle.gelu(-40.0)) < 1e-12
    # the lower tail keeps its relative precision: Phi(-10) = 7.619853024160527e-24, Phi(-5) = 2.866515718791939e-07
    assert abs(oracle.gelu(-10.0) / (-10.0 * 7.619853024160527e-24) - 1) < 1e-12
    assert abs(oracle.gelu(-5.0) / (-5.0 * 2.866515718791939e-07) - 1) < 1e-12


@pytest.mark.parametrize("activation", ["gelu", "relu"])
@pytest.mark.parametrize("N,dm,dff", [(5, 8, 16), (37, 32, 64)])
def test_ffn_matches_torch(N, dm, dff, activation):
    x, w1, b1, w2, b2 = _rand((N, dm), 1), _rand((dm, dff), 2, 0.2), _rand(dff, 3), _rand((dff, dm), 4, 0.2), _rand(dm, 5)
    y = oracle.ffn_reference(x, w1, b1, w2, b2, activation=activation)
    t = lambda a: torch.tensor(a, dtype=torch.float64)
    h = t(x) @ t(w1) + t(b1)
    h = torch.nn.functional.gelu(h, approximate="none") if activation == "gelu" else torch.relu(h)
    ref = h @ t(w2) + t(b2)
    assert np.abs(y - ref.numpy()).max() < 1e-12


def test_relu_and_gelu_agree_far_from_zero():
    # Phi(z) -> 1 for large z and z Phi(z) -> 0 for very negative z: both activations coincide there
    z = np.concatenate([np.linspace(-40, -12, 20), np.linspace(12, 40, 20)])
    assert np.abs(oracle.gelu(z) - oracle.relu(z)).max() < 1e-12
    assert np.all(oracle.relu(-np.abs(z)) == 0) and np.all(oracle.relu(np.abs(z)) == np.abs(z))


def test_ffn_closed_forms_and_position_wise():
    N, dm, dff = 12, 8, 24
    x, w1, b1, w2, b2 = _rand((N, dm), 11), _rand((dm, dff), 12), _rand(dff, 13), _rand((dff, dm), 14), _rand(dm, 15)
    # W1 = 0: every token gives gelu(b1) W2 + b2
    y0 = oracle.ffn_reference(x, np.zeros_like(w1), b1, w2, b2)
    want = oracle.gelu(b1) @ w2 + b2
    assert np.abs(y0 - want[None, :]).max() < 1e-12
    # W2 = 0: the bias
    assert np.abs(oracle.ffn_reference(x, w1, b1, np.zeros_like(w2), b2) - b2[None, :]).max() == 0
    # permuting tokens permutes the output; blocks of tokens give the same rows
    perm = np.random.default_rng(16).permutation(N)
    y = oracle.ffn_reference(x, w1, b1, w2, b2)
    assert np.abs(oracle.ffn_reference(x[perm], w1, b1, w2, b2) - y[perm]).max() < 1e-12
    blocks = np.concatenate([oracle.ffn_reference(x[i:i + 5], w1, b1, w2, b2) for i in range(0, N, 5)])
    assert np.abs(blocks - y).max() < 1e-12
