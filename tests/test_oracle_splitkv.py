"""Pins for the cross-length oracle (queries against a longer key sequence,
used by the split-KV forward), CPU only: the self-attention oracle at equal
lengths, the last rows of a causal self-attention, per-element brute force,
and the single-query (decode) case against scipy's softmax.
"""
import math

import numpy as np
import pytest
from scipy.special import softmax

import oracle
from tests.test_oracle import _brute_forward


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("causal", [False, True])
def test_equal_lengths_is_self_attention(causal):
    q, k, v = (_rand((2, 300, 2, 8), s) for s in (1, 2, 3))
    o, lse = oracle.forward_cross(q, k, v, 0.3, causal)
    o2, lse2 = oracle.forward(q, k, v, 0.3, causal)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)


@pytest.mark.parametrize("nq", [1, 7, 300, 513])
def test_causal_queries_are_the_last_positions(nq):
    """Causal cross attention of the last nq queries equals the last nq rows
    of causal self-attention over the whole sequence."""
    N = 600
    q, k, v = (_rand((1, N, 2, 6), s) for s in (4, 5, 6))
    o, lse = oracle.forward_cross(q[:, N - nq:], k, v, 0.4, True)
    o2, lse2 = oracle.forward(q, k, v, 0.4, True)
    assert np.max(np.abs(o - o2[:, N - nq:])) <= 1e-12
    assert np.max(np.abs(lse - lse2[:, :, N - nq:])) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_cross(causal):
    Nq, Nk, d = 5, 9, 3
    q, k, v = _rand((1, Nq, 1, d), 7), _rand((1, Nk, 1, d), 8), _rand((1, Nk, 1, d), 9)
    o, lse = oracle.forward_cross(q, k, v, 0.7, causal)
    off = Nk - Nq
    for i in range(Nq):
        keys = [j for j in range(Nk) if not (causal and j > i + off)]
        x = [0.7 * sum(q[0, i, 0, c] * k[0, j, 0, c] for c in range(d)) for j in keys]
        mx = max(x)
        den = sum(math.exp(t - mx) for t in x)
        assert abs(lse[0, 0, i] - (mx + math.log(den))) <= 1e-12
        ref = sum(math.exp(t - mx) / den * v[0, j, 0] for t, j in zip(x, keys))
        assert np.max(np.abs(o[0, i, 0] - ref)) <= 1e-12
    # Nq = Nk reduces to the self-attention brute force of the fixed-length pins
    qs = _rand((4, 3), 10)
    ob, lb = _brute_forward(qs, qs, qs, 0.5, causal)
    o3, l3 = oracle.forward_cross(qs[None, :, None], qs[None, :, None], qs[None, :, None], 0.5, causal)
    assert np.max(np.abs(o3[0, :, 0] - ob)) <= 1e-12 and np.max(np.abs(l3[0, 0] - lb)) <= 1e-12


def test_decode_single_query_sees_every_key():
    Nk, d = 4000, 16
    q, k, v = _rand((1, 1, 3, d), 11), _rand((1, Nk, 3, d), 12), _rand((1, Nk, 3, d), 13)
    o, lse = oracle.forward_cross(q, k, v, 0.25, True)
    for h in range(3):
        logits = 0.25 * k[0, :, h] @ q[0, 0, h]
        p = softmax(logits)
        assert np.max(np.abs(o[0, 0, h] - p @ v[0, :, h])) <= 1e-12
        assert abs(lse[0, h, 0] - (np.log(np.sum(np.exp(logits - logits.max()))) + logits.max())) <= 1e-12
