"""Pins of the oracle's future-attention target (CPU only).

y[g][j] = sum over the query heads h of group g and the queries i >= j + W
of the causal softmax weight of query i on key j.  Checked against a closed
form (uniform attention gives harmonic sums), the unit mass of every query,
the empty case, and PyTorch's attention routine in float64 (probabilities
read out through an identity value matrix).
"""
import math

import numpy as np
import pytest
import torch

from oracle import bf16_to_f64, future_attention_target
from fixed_budget_learned_amd.inputs import bf16_bits_rne


def _bits(rng, shape, scale=1.0):
    return bf16_bits_rne((scale * rng.standard_normal(shape)).astype(np.float32))


def _harmonic(n):
    return sum(1.0 / i for i in range(1, n + 1))


@pytest.mark.parametrize("W", [0, 1, 5, 17])
def test_uniform_attention_gives_harmonic_sums(W):
    """q = 0: every query spreads its mass evenly over keys 0..i, so
    y[j] = G * (H_T - H_{j+W}) with H the harmonic numbers."""
    T, D, Hq, Hkv = 40, 16, 4, 2
    rng = np.random.default_rng(1)
    q = np.zeros((Hq, T, D), np.uint16)
    k = _bits(rng, (Hkv, T, D))
    y = future_attention_target(q, k, W, 1.0 / math.sqrt(D))
    G = Hq // Hkv
    for g in range(Hkv):
        for j in range(T):
            want = G * (_harmonic(T) - _harmonic(min(T, j + W))) if j + W < T else 0.0
            assert abs(y[g][j] - want) < 1e-12, (g, j)


def test_every_query_spreads_unit_mass():
    """W = 0: summing y over keys counts each query's unit mass once."""
    T, D, Hq, Hkv = 33, 8, 8, 2
    rng = np.random.default_rng(2)
    y = future_attention_target(_bits(rng, (Hq, T, D)), _bits(rng, (Hkv, T, D)), 0,
                                1.0 / math.sqrt(D))
    assert abs(y.sum() - Hq * T) < 1e-9
    for g in range(Hkv):
        assert abs(y[g].sum() - (Hq // Hkv) * T) < 1e-9


def test_window_longer_than_sequence_gives_zero():
    rng = np.random.default_rng(3)
    y = future_attention_target(_bits(rng, (2, 10, 8)), _bits(rng, (1, 10, 8)), 10, 0.3)
    assert np.all(y == 0.0)


@pytest.mark.parametrize("W", [0, 3, 9])
def test_matches_torch_attention_probabilities(W):
    """PyTorch's scaled_dot_product_attention with V = identity returns the
    causal attention probabilities; their masked column sums are y."""
    T, D, Hq, Hkv = 24, 16, 4, 2
    rng = np.random.default_rng(4 + W)
    qb, kb = _bits(rng, (Hq, T, D), 2.0), _bits(rng, (Hkv, T, D), 2.0)
    scale = 1.0 / math.sqrt(D)
    y = future_attention_target(qb, kb, W, scale)
    Q = torch.from_numpy(bf16_to_f64(qb))
    K = torch.from_numpy(bf16_to_f64(kb))
    eye = torch.eye(T, dtype=torch.float64)
    want = np.zeros((Hkv, T))
    for h in range(Hq):
        g = h * Hkv // Hq
        P = torch.nn.functional.scaled_dot_product_attention(
            Q[h][None, None], K[g][None, None], eye[None, None], is_causal=True,
            scale=scale)[0, 0].numpy()   # [i][j]
        for j in range(T):
            want[g][j] += P[j + W:, j].sum()
    assert np.abs(y - want).max() < 1e-12


def test_planted_window_off_by_one_is_caught():
    """Counting queries i >= j + W - 1 instead of i >= j + W breaks the
    closed form."""
    T, D, W = 20, 8, 4
    rng = np.random.default_rng(5)
    k = _bits(rng, (1, T, D))
    q = np.zeros((1, T, D), np.uint16)
    y = future_attention_target(q, k, W - 1, 1.0)  # the mistake
    want = [(_harmonic(T) - _harmonic(j + W)) if j + W < T else 0.0 for j in range(T)]
    assert np.abs(y[0] - np.array(want)).max() > 1e-3
