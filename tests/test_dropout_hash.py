"""Pins for the dropout counter hash of the oracle (CPU only).

The mixers are pinned by published known-answer values; the combined mask by
its defining properties (keep rate, independence across rows and columns,
seed sensitivity, exact threshold)."""
import json
import os

import numpy as np
import pytest

from oracle import dropout_hash as DH

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hash_vectors.json")


def _vectors():
    with open(GOLDEN) as f:
        return json.load(f)


def test_splitmix64_published_outputs():
    g = _vectors()["splitmix64"]
    state = int(g["seed"])
    for want in g["outputs"]:
        state = (state + DH.GOLDEN_GAMMA) & DH.MASK64
        got = int(DH.mix64(np.array([state], np.uint64))[0])
        assert got == int(want, 16)


def _murmur3_x86_32(data: bytes, seed: int) -> int:
    """MurmurHash3_x86_32 body and tail written out here; the finalizer is the
    oracle's fmix32, which the published values therefore pin."""
    c1, c2 = 0xCC9E2D51, 0x1B873593
    m = 0xFFFFFFFF

    def rotl(x, r):
        return ((x << r) | (x >> (32 - r))) & m

    h = seed & m
    nblocks = len(data) // 4
    for i in range(nblocks):
        k = int.from_bytes(data[4 * i:4 * i + 4], "little")
        k = rotl((k * c1) & m, 15) * c2 & m
        h = (rotl(h ^ k, 13) * 5 + 0xE6546B64) & m
    tail = data[4 * nblocks:]
    k = 0
    for j in reversed(range(len(tail))):
        k ^= tail[j] << (8 * j)
    if tail:
        h ^= rotl((k * c1) & m, 15) * c2 & m
    h ^= len(data)
    return int(DH.fmix32(np.array([h], np.uint32))[0])


def test_murmur3_published_outputs():
    for case in _vectors()["murmurhash3_x86_32"]["cases"]:
        data = bytes.fromhex(case["hex_input"])
        assert _murmur3_x86_32(data, int(case["seed"], 16)) == int(case["hash"], 16), case


def test_threshold_for_p_0_1():
    # 0.1 in float32 is 13421773 * 2^-27, so floor(p * 2^32) = 13421773 * 32
    assert DH.keep_threshold(0.1) == 13421773 * 32 == 429496736
    assert DH.keep_threshold(0.0) == 0
    with pytest.raises(ValueError):
        DH.keep_threshold(1.0)


def test_keep_rate_and_independence():
    p = 0.1
    rows, cols = np.arange(0, 4096), np.arange(1000, 1000 + 4096)
    m = DH.keep_mask(2026, 0, 3, 8, p, rows, cols)  # 16.8M draws
    n = m.size
    q = 1.0 - DH.keep_threshold(p) / 2.0 ** 32
    sigma = np.sqrt(q * (1 - q) / n)
    assert abs(m.mean() - q) <= 5 * sigma
    # no drift of the keep rate across rows or columns
    rsd = np.sqrt(q * (1 - q) / m.shape[1])
    assert np.max(np.abs(m.mean(axis=1) - q)) <= 6 * rsd
    assert np.max(np.abs(m.mean(axis=0) - q)) <= 6 * rsd
    # adjacent rows / columns uncorrelated
    x = m.astype(np.float64) - q
    for a, b in ((x[1:], x[:-1]), (x[:, 1:], x[:, :-1])):
        corr = np.mean(a * b) / (q * (1 - q))
        assert abs(corr) <= 5.0 / np.sqrt(a.size)


def test_seed_and_head_sensitivity():
    r, c = np.arange(256), np.arange(256)
    base = DH.keep_mask(1, 0, 0, 4, 0.5, r, c)
    for other in (DH.keep_mask(2, 0, 0, 4, 0.5, r, c), DH.keep_mask(1, 0, 1, 4, 0.5, r, c),
                  DH.keep_mask(1, 1, 0, 4, 0.5, r, c)):
        agree = np.mean(base == other)
        assert 0.45 < agree < 0.55


def test_mask_is_layout_independent():
    # Any window of the mask equals the same window cut from a larger one.
    big = DH.keep_mask(7, 1, 2, 3, 0.3, np.arange(100), np.arange(100))
    win = DH.keep_mask(7, 1, 2, 3, 0.3, np.arange(40, 70), np.arange(13, 91))
    assert np.array_equal(big[40:70, 13:91], win)
