"""Pins for the packed variable-length oracle (oracle/varlen.py), CPU only:
brute force, the padded -inf formulation of "FlashAttention for Efficient
Training" section 5.2, the fixed-length oracle at equal lengths, sequence
isolation, closed forms for length-1 sequences and finite differences.
"""
import math

import numpy as np
import pytest
from scipy.special import logsumexp

import oracle
from oracle import varlen as V
from tests.test_oracle import _brute_forward
from workloads import VarlenWorkload, make_varlen_inputs, varlen_lengths


def _packed(lengths, H, d, seed, amp=1.0):
    rng = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    t = int(cu[-1])
    q, k, v, do = (amp * rng.standard_normal((t, H, d)) for _ in range(4))
    return cu, q, k, v, do


# --------------------------------------------------------------------------
# Brute force per sequence with per-element loops; the dropout hash is keyed
# by the sequence index and positions within the sequence.
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("p_drop", [0.0, 0.3])
def test_brute_force_packed(causal, p_drop):
    lengths = [3, 1, 0, 5, 2]
    H, d, seed = 2, 3, 17
    cu, q, k, v, _ = _packed(lengths, H, d, 5)
    scale = 1.0 / math.sqrt(d)
    o, lse = V.forward_varlen(q, k, v, cu, scale, causal, p_drop, seed)
    assert o.shape == q.shape and lse.shape == (H, cu[-1])
    for s, n in enumerate(lengths):
        a = int(cu[s])
        for h in range(H):
            if n == 0:
                continue
            keep = None
            if p_drop > 0:
                keep = oracle.keep_mask(seed, s, h, H, p_drop, np.arange(n), np.arange(n)).astype(float)
            ob, lb = _brute_forward(q[a:a + n, h], k[a:a + n, h], v[a:a + n, h], scale, causal, keep,
                                    float(np.float32(p_drop)))
            assert np.max(np.abs(o[a:a + n, h] - ob)) <= 1e-12
            assert np.max(np.abs(lse[h, a:a + n] - lb)) <= 1e-12


# --------------------------------------------------------------------------
# Section 5.2's padded formulation: pad every sequence to the longest length
# with arbitrary values, score key j of a sequence of length L as -inf when
# j >= L (0-based), take the softmax over all padded keys (scipy's
# logsumexp), and compare the valid rows. Catches wrong slicing, offsets or
# a mask that leaks across sequences.
@pytest.mark.parametrize("causal", [False, True])
def test_matches_padded_minus_inf_formulation(causal):
    lengths = [7, 1, 12, 4]
    H, d = 3, 5
    cu, q, k, v, _ = _packed(lengths, H, d, 6)
    scale = 0.4
    S, Lmax = len(lengths), max(lengths)
    rng = np.random.default_rng(8)
    pad = {n: 50.0 * rng.standard_normal((S, Lmax, H, d)) for n in "qkv"}
    for s, n in enumerate(lengths):
        a = int(cu[s])
        pad["q"][s, :n], pad["k"][s, :n], pad["v"][s, :n] = q[a:a + n], k[a:a + n], v[a:a + n]
    o, lse = V.forward_varlen(q, k, v, cu, scale, causal)
    for s, n in enumerate(lengths):
        a = int(cu[s])
        for h in range(H):
            A = scale * pad["q"][s, :, h] @ pad["k"][s, :, h].T
            j = np.arange(Lmax)[None, :]
            i = np.arange(Lmax)[:, None]
            A = np.where(j >= n, -np.inf, A)
            if causal:
                A = np.where(j > i, -np.inf, A)
            l_ = logsumexp(A, axis=1)
            P = np.exp(A - l_[:, None])
            O = P @ pad["v"][s, :, h]
            assert np.max(np.abs(o[a:a + n, h] - O[:n])) <= 1e-12
            assert np.max(np.abs(lse[h, a:a + n] - l_[:n])) <= 1e-12


# --------------------------------------------------------------------------
# Equal lengths: the packed oracle is the fixed-length oracle with sequence s
# as batch item s (outputs, statistics and gradients, dropout included).
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("p_drop", [0.0, 0.2])
def test_equal_lengths_equal_fixed_batch(causal, p_drop):
    S, n, H, d = 3, 20, 2, 4
    cu, q, k, v, do = _packed([n] * S, H, d, 9)
    scale, seed = 0.5, 31
    o, lse = V.forward_varlen(q, k, v, cu, scale, causal, p_drop, seed)
    dq, dk, dv, dd = V.backward_varlen(q, k, v, do, cu, scale, causal, p_drop, seed)
    r = lambda x: x.reshape(S, n, H, d)
    o2, lse2 = oracle.forward(r(q), r(k), r(v), scale, causal, p_drop, seed)
    dq2, dk2, dv2, dd2 = oracle.backward(r(q), r(k), r(v), r(do), scale, causal, p_drop, seed)
    np.testing.assert_array_equal(r(o), o2)
    np.testing.assert_array_equal(lse.reshape(H, S, n).transpose(1, 0, 2), lse2)
    for got, ref in ((dq, dq2), (dk, dk2), (dv, dv2)):
        np.testing.assert_array_equal(r(got), ref)
    np.testing.assert_array_equal(dd.reshape(H, S, n).transpose(1, 0, 2), dd2)


# --------------------------------------------------------------------------
# Isolation: changing one sequence's inputs changes no other sequence's
# outputs or gradients.
def test_sequences_are_isolated():
    lengths = [6, 9, 4]
    H, d = 2, 3
    cu, q, k, v, do = _packed(lengths, H, d, 10)
    o, lse = V.forward_varlen(q, k, v, cu, 0.6, True, 0.1, 3)
    g = V.backward_varlen(q, k, v, do, cu, 0.6, True, 0.1, 3)
    q2, k2, v2, do2 = q.copy(), k.copy(), v.copy(), do.copy()
    a, e = int(cu[1]), int(cu[2])
    for x in (q2, k2, v2, do2):
        x[a:e] += 1.0
    o2, lse2 = V.forward_varlen(q2, k2, v2, cu, 0.6, True, 0.1, 3)
    g2 = V.backward_varlen(q2, k2, v2, do2, cu, 0.6, True, 0.1, 3)
    keep = np.r_[0:a, e:int(cu[-1])]
    np.testing.assert_array_equal(o[keep], o2[keep])
    np.testing.assert_array_equal(lse[:, keep], lse2[:, keep])
    for x, y in zip(g[:3], g2[:3]):
        np.testing.assert_array_equal(x[keep], y[keep])
    assert np.max(np.abs(o[a:e] - o2[a:e])) > 1e-3


# --------------------------------------------------------------------------
# A sequence of length 1 attends to itself only: O = V, LSE = scale q.k,
# dQ = dK = 0, dV = dO (without dropout).
def test_length_one_closed_form():
    lengths = [1, 5, 1]
    H, d = 2, 4
    cu, q, k, v, do = _packed(lengths, H, d, 12)
    o, lse = V.forward_varlen(q, k, v, cu, 0.8, False)
    dq, dk, dv, _ = V.backward_varlen(q, k, v, do, cu, 0.8, False)
    for t in (0, int(cu[-1]) - 1):
        np.testing.assert_allclose(o[t], v[t], rtol=0, atol=1e-15)
        np.testing.assert_allclose(lse[:, t], 0.8 * np.sum(q[t] * k[t], axis=1), rtol=0, atol=1e-14)
        assert np.max(np.abs(dq[t])) <= 1e-15 and np.max(np.abs(dk[t])) <= 1e-15
        np.testing.assert_allclose(dv[t], do[t], rtol=0, atol=1e-15)


# --------------------------------------------------------------------------
# Central finite differences of L = sum(dO * O) over a packed batch.
@pytest.mark.parametrize("causal,p_drop", [(False, 0.0), (True, 0.15)])
def test_finite_difference_gradients_packed(causal, p_drop):
    lengths = [4, 1, 6]
    H, d = 2, 2
    cu, q, k, v, do = _packed(lengths, H, d, 13)
    scale, seed, step = 0.9, 77, 1e-6
    dq, dk, dv, _ = V.backward_varlen(q, k, v, do, cu, scale, causal, p_drop, seed)

    def loss(**kw):
        args = {"q": q, "k": k, "v": v}
        args.update(kw)
        o, _ = V.forward_varlen(args["q"], args["k"], args["v"], cu, scale, causal, p_drop, seed)
        return float(np.sum(do * o))

    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += step
            xm[idx] -= step
            num[idx] = (loss(**{name: xp}) - loss(**{name: xm})) / (2 * step)
        err = np.max(np.abs(num - g)) / max(np.max(np.abs(g)), 1e-30)
        assert err <= 1e-6, (name, err)


# --------------------------------------------------------------------------
# The packed-batch input recipe.
@pytest.mark.parametrize("p_drop", [0.0, 0.2])
def test_given_output_per_sequence(p_drop):
    """backward_varlen(o=...) reads D from the given output: with the varlen
    oracle's own O it returns the default gradients, and with a perturbed O
    each sequence's gradients are the dense oracle's on that sequence alone
    (batch slot = sequence index) with the same O."""
    lengths = [5, 0, 13, 1, 8]
    H, d = 2, 4
    cu, q, k, v, do = _packed(lengths, H, d, 77)
    scale, seed = 0.6, 9
    o, _ = V.forward_varlen(q, k, v, cu, scale, True, p_drop, seed)
    ref = V.backward_varlen(q, k, v, do, cu, scale, True, p_drop, seed)
    same = V.backward_varlen(q, k, v, do, cu, scale, True, p_drop, seed, o=o)
    for x, y in zip(ref, same):
        assert np.max(np.abs(x - y)) <= 1e-12
    og = o + 0.05 * np.random.default_rng(5).standard_normal(o.shape)
    got = V.backward_varlen(q, k, v, do, cu, scale, True, p_drop, seed, o=og)
    B = len(lengths)
    for s, (a, e) in enumerate(zip(cu[:-1], cu[1:])):
        if e == a:
            continue
        n = e - a
        pad = lambda x: np.zeros((B, n) + x.shape[1:])  # noqa: E731
        qq, kk, vv, dd, oo = (pad(x) for x in (q, k, v, do, og))
        for x, src in ((qq, q), (kk, k), (vv, v), (dd, do), (oo, og)):
            x[s] = src[a:e]
        dq, dk, dv, _ = oracle.backward(qq, kk, vv, dd, scale, True, p_drop, seed, heads=[(s, h) for h in range(H)],
                                        o=oo)
        for name, full, part in (("dQ", got[0], dq), ("dK", got[1], dk), ("dV", got[2], dv)):
            assert np.max(np.abs(full[a:e] - part[s])) <= 1e-12, (name, s)


def test_varlen_inputs_recipe():
    w = VarlenWorkload("t", 5, 2, 64, "bf16", True, 0.0, min_len=1, max_len=40, seed=4)
    cu, inp = make_varlen_inputs(w)
    lengths = varlen_lengths(w)
    assert cu.dtype == np.int32 and cu[0] == 0
    np.testing.assert_array_equal(np.diff(cu), lengths)
    assert inp["q"][0].shape == (int(cu[-1]), 2, 64) and inp["q"][0].dtype == np.uint16
    w2 = w.with_(lengths=(3, 0, 2))
    cu2, _ = make_varlen_inputs(w2)
    np.testing.assert_array_equal(cu2, [0, 3, 3, 5])
