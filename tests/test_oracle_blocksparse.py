"""Pins for the block-sparse oracle (block mask over 128 x 128 blocks of the
score matrix), CPU only: brute force with the mask applied per element, the
dense oracle for an all-ones mask, the causal oracle for the block-lower
triangle, the packed variable-length oracle for a block-diagonal mask, fully
masked rows, and finite differences.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import varlen as V
from tests.test_oracle import _brute_forward
from workloads import block_mask_local_global, block_mask_random

BLK = 128


def _rand(B, N, H, d, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((B, N, H, d)) for _ in range(4)]


def _brute_masked(q, k, v, scale, causal, bm):
    """Per-element loops: key j of query i is used iff bm[i//128][j//128]
    (and j <= i under the causal mask); no key left: O = 0, LSE = -inf."""
    N, d = q.shape
    o = np.zeros((N, v.shape[1]))
    lse = np.full(N, -np.inf)
    for i in range(N):
        logits = [(j, scale * sum(q[i][c] * k[j][c] for c in range(d)))
                  for j in range(N) if bm[i // BLK][j // BLK] and not (causal and j > i)]
        if not logits:
            continue
        mx = max(x for _, x in logits)
        den = sum(math.exp(x - mx) for _, x in logits)
        lse[i] = mx + math.log(den)
        for j, x in logits:
            o[i] += math.exp(x - mx) / den * v[j]
    return o, lse


@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_masked(causal):
    B, N, H, d = 1, 300, 2, 2
    q, k, v, _ = _rand(B, N, H, d, 1)
    bm = np.array([[[1, 0, 1], [0, 1, 1], [0, 0, 0]],
                   [[0, 1, 0], [1, 0, 0], [1, 1, 1]]], np.uint8)[None]
    o, lse = oracle.forward(q, k, v, 0.7, causal, block_mask=bm)
    for h in range(H):
        ob, lb = _brute_masked(q[0, :, h], k[0, :, h], v[0, :, h], 0.7, causal, bm[0, h])
        assert np.max(np.abs(o[0, :, h] - ob)) <= 1e-12
        fin = np.isfinite(lb)
        np.testing.assert_array_equal(fin, np.isfinite(lse[0, h]))
        assert np.max(np.abs(lse[0, h][fin] - lb[fin])) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("p_drop", [0.0, 0.2])
def test_all_ones_mask_is_dense(causal, p_drop):
    B, N, H, d = 2, 300, 2, 4
    q, k, v, do = _rand(B, N, H, d, 2)
    bm = np.ones((B, H, 3, 3), np.uint8)
    o, lse = oracle.forward(q, k, v, 0.5, causal, p_drop, 9, block_mask=bm)
    o2, lse2 = oracle.forward(q, k, v, 0.5, causal, p_drop, 9)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)
    g = oracle.backward(q, k, v, do, 0.5, causal, p_drop, 9, block_mask=bm)
    g2 = oracle.backward(q, k, v, do, 0.5, causal, p_drop, 9)
    for a, b in zip(g, g2):
        np.testing.assert_array_equal(a, b)


def test_block_lower_triangle_with_causal_is_causal():
    B, N, H, d = 1, 333, 1, 3
    q, k, v, do = _rand(B, N, H, d, 3)
    bm = np.tril(np.ones((3, 3), np.uint8))[None, None]
    o, lse = oracle.forward(q, k, v, 0.4, True, block_mask=bm)
    o2, lse2 = oracle.forward(q, k, v, 0.4, True)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)


@pytest.mark.parametrize("p_drop", [0.0, 0.1])
def test_block_diagonal_mask_equals_packed_sequences(p_drop):
    """A block-diagonal mask splits the sequence into independent 128-token
    sequences: outputs and gradients equal the packed variable-length oracle
    on those pieces (without dropout; with dropout the hash keys differ, so
    only the dropout-free case is compared exactly and the dropout case checks
    that rows only mix within their block)."""
    B, N, H, d = 1, 300, 2, 3
    q, k, v, do = _rand(B, N, H, d, 4)
    nb = 3
    bm = np.eye(nb, dtype=np.uint8)[None, None].repeat(H, axis=1)
    o, lse = oracle.forward(q, k, v, 0.6, False, p_drop, 5, block_mask=bm)
    dq, dk, dv, _ = oracle.backward(q, k, v, do, 0.6, False, p_drop, 5, block_mask=bm)
    if p_drop == 0.0:
        cu = np.array([0, 128, 256, 300])
        o2, lse2 = V.forward_varlen(q[0], k[0], v[0], cu, 0.6, False)
        g2 = V.backward_varlen(q[0], k[0], v[0], do[0], cu, 0.6, False)
        assert np.max(np.abs(o[0] - o2)) <= 1e-12
        assert np.max(np.abs(lse[0] - lse2)) <= 1e-12
        for a, b in zip((dq, dk, dv), g2[:3]):
            assert np.max(np.abs(a[0] - b)) <= 1e-12
    else:
        # Perturbing block 1's keys and values leaves blocks 0 and 2 unchanged.
        k2, v2 = k.copy(), v.copy()
        k2[:, 128:256] += 1.0
        v2[:, 128:256] -= 1.0
        o3, _ = oracle.forward(q, k2, v2, 0.6, False, p_drop, 5, block_mask=bm)
        np.testing.assert_array_equal(o3[:, :128], o[:, :128])
        np.testing.assert_array_equal(o3[:, 256:], o[:, 256:])
        assert np.max(np.abs(o3[:, 128:256] - o[:, 128:256])) > 1e-3


def test_fully_masked_rows_and_unused_keys():
    B, N, H, d = 1, 300, 1, 4
    q, k, v, do = _rand(B, N, H, d, 6)
    bm = np.array([[1, 1, 0], [0, 0, 0], [1, 0, 0]], np.uint8)[None, None]
    o, lse = oracle.forward(q, k, v, 0.5, False, block_mask=bm)
    dq, dk, dv, dd = oracle.backward(q, k, v, do, 0.5, False, block_mask=bm)
    assert np.all(o[0, 128:256] == 0.0) and np.all(np.isneginf(lse[0, 0, 128:256]))
    assert np.all(np.isfinite(lse[0, 0, :128])) and np.all(np.isfinite(lse[0, 0, 256:]))
    assert np.all(dq[0, 128:256] == 0.0) and np.all(dd[0, 0, 128:256] == 0.0)
    # key block 2 is used by no query block
    assert np.all(dk[0, 256:] == 0.0) and np.all(dv[0, 256:] == 0.0)


@pytest.mark.parametrize("causal,p_drop", [(False, 0.0), (True, 0.15)])
def test_finite_difference_gradients_masked(causal, p_drop):
    B, N, H, d = 1, 140, 1, 2
    q, k, v, do = _rand(B, N, H, d, 7)
    bm = np.array([[1, 0], [1, 1]], np.uint8)[None, None] if causal else \
        np.array([[0, 1], [1, 0]], np.uint8)[None, None]
    scale, seed, step = 0.8, 21, 1e-6
    dq, dk, dv, _ = oracle.backward(q, k, v, do, scale, causal, p_drop, seed, block_mask=bm)

    def loss(**kw):
        a = {"q": q, "k": k, "v": v}
        a.update(kw)
        o, _ = oracle.forward(a["q"], a["k"], a["v"], scale, causal, p_drop, seed, block_mask=bm)
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


def test_sampled_head_with_mask_matches_full():
    B, N, H, d = 1, 400, 2, 4
    q, k, v, do = _rand(B, N, H, d, 8)
    bm = block_mask_random((B, H), N, 0.5, 3)
    bm[0, 1, 2, :] = 0  # a fully masked query block
    o, lse = oracle.forward(q, k, v, 0.5, True, 0.1, 4, block_mask=bm)
    dq, dk, dv, _ = oracle.backward(q, k, v, do, 0.5, True, 0.1, 4, block_mask=bm)
    rows = np.array([0, 5, 130, 257, 300, 399])
    cols = np.array([0, 127, 128, 256, 399])
    for h in range(H):
        r = oracle.sampled_head(q, k, v, do, 0.5, True, 0.1, 4, 0, h, rows, cols, bmask=bm[0, h])
        assert np.max(np.abs(r["o"] - o[0, rows, h])) <= 1e-12
        np.testing.assert_array_equal(np.isfinite(r["lse"]), np.isfinite(lse[0, h, rows]))
        assert np.max(np.abs(r["dq"] - dq[0, rows, h])) <= 1e-12
        assert np.max(np.abs(r["dk"] - dk[0, cols, h])) <= 1e-12
        assert np.max(np.abs(r["dv"] - dv[0, cols, h])) <= 1e-12


def test_mask_generators():
    m = block_mask_local_global(1000, 1, 1)
    assert m.shape == (8, 8) and m.dtype == np.uint8
    assert m[5, 4] and m[5, 6] and not m[5, 3] and m[5, 0] and m[0, 0]
    r = block_mask_random((2, 3), 300, 0.5, 1)
    assert r.shape == (2, 3, 3, 3) and set(np.unique(r)) <= {0, 1}
