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
    # 0.1 in float32 is 13421773 * 2^-27, so p * 2^16 = 13421773 / 2048 = 6553.6...
    assert DH.keep_threshold(0.1) == 13421773 // 2048 == 6553
    assert DH.keep_threshold(0.0) == 0
    assert DH.keep_threshold(0.5) == 32768
    assert DH.keep_threshold(float(np.float32(1.0) - np.float32(2.0 ** -24))) == 65535
    assert DH.keep_threshold(2.0 ** -16) == 1
    with pytest.raises(ValueError):
        DH.keep_threshold(1.0)
    # below the draws' resolution a nonzero p would drop nothing: rejected
    for p in (1e-6, 2.0 ** -17, 2.0 ** -16 * 0.999):
        with pytest.raises(ValueError):
            DH.keep_threshold(p)


@pytest.mark.parametrize("p", [2.0 ** -16, 0.001, 0.1, 0.25, 0.5, 0.9])
def test_keep_rate_times_rescale(p):
    """Kept values are scaled by 1/(1 - p) (the float32 value the kernels
    use), the keep probability is 1 - T/2^16 with T = floor(p 2^16), so the
    expected dropped probability is (keep rate) * (rescale) times P. That
    factor is within 2^-16 / (1 - p) of 1 (the 16-bit draws' resolution; at
    p = 0.1 it is 1.0000102), and an empirical keep rate over 4M draws
    matches 1 - T/2^16."""
    pf = float(np.float32(p))
    t = DH.keep_threshold(p)
    keep = 1.0 - t / 65536.0
    rescale = float(np.float32(1.0 / (1.0 - pf)))
    # lower end: the float32 rounding of 1/(1 - p) (at most 2^-24 relative)
    assert -2.0 ** -23 <= keep * rescale - 1.0 <= 2.0 ** -16 / (1.0 - pf) + 1e-7
    m = DH.keep_mask(31, 0, 0, 1, p, np.arange(2048), np.arange(2048))
    sigma = np.sqrt(max(keep * (1 - keep), 1e-12) / m.size)
    assert abs(m.mean() - keep) <= 6 * sigma + 2.0 ** -22
    if p == 0.1:
        assert abs(keep * rescale - 1.0000102) < 1e-7


def test_row_and_pair_keys_do_not_coincide():
    """Row keys A_i and pair keys B_c come from disjoint counters (odd and
    even multiples of G past the head key). Over the N = 65536 dropout
    workload's index ranges (seed 2026, 8 heads, rows < 65536, pairs <
    32768) the two key sets share only the chance coincidences of 32-bit
    values (about 0.5 per head expected), and no row key equals the pair
    key of the same index or its neighbours. A derivation slip that aligned
    the counters (say A_i from 2i + 2) would make A_i = B_i for every i and
    zero the draws fmix32(0) = 0 of a whole diagonal."""
    rows, pairs = np.arange(65536), np.arange(32768)
    for h in range(8):
        key = DH.head_key(2026, 0, h, 8)
        a, bk = DH.row_keys(key, rows), DH.pair_keys(key, pairs)
        assert len(np.intersect1d(a, bk)) <= 8  # Poisson(0.5): P(> 8) < 1e-9
        for shift in (-1, 0, 1):
            i = np.arange(max(0, -shift), 32768 - max(0, shift))
            assert not np.any(a[i] == bk[i + shift])


@pytest.mark.parametrize("diag", ["c = i", "c = i // 2 (query's own pair)", "c = 2i"])
def test_keep_rate_on_diagonals(diag):
    """The keep rate along systematic diagonals of (row, key pair) equals the
    rate elsewhere: 65536 decisions per head and diagonal of the N = 65536
    dropout workload (seed 2026, heads 0 and 5)."""
    keep = 1.0 - DH.keep_threshold(0.1) / 65536.0
    for h in (0, 5):
        key = DH.head_key(2026, 0, h, 8)
        i = np.arange(32768) if diag != "c = 2i" else np.arange(16384)
        c = {"c = i": i, "c = i // 2 (query's own pair)": i // 2, "c = 2i": 2 * i}[diag]
        if diag == "c = i // 2 (query's own pair)":
            i = np.arange(65536)
            c = i // 2
        w = DH.fmix32(DH.row_keys(key, i) ^ DH.pair_keys(key, c))
        u = np.concatenate([w & np.uint32(0xFFFF), w >> np.uint32(16)])
        rate = float(np.mean(u >= DH.keep_threshold(0.1)))
        sigma = np.sqrt(keep * (1 - keep) / u.size)
        assert abs(rate - keep) <= 6 * sigma, (h, diag, rate)


def test_keep_rate_and_independence():
    p = 0.1
    rows, cols = np.arange(0, 4096), np.arange(1000, 1000 + 4096)
    m = DH.keep_mask(2026, 0, 3, 8, p, rows, cols)  # 16.8M draws
    n = m.size
    q = 1.0 - DH.keep_threshold(p) / 2.0 ** 16
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


def test_pair_convention():
    """Columns 2c and 2c + 1 of row i take the low and the high 16 bits of
    fmix32(A_i ^ B_c), built here from the separately pinned mixers."""
    seed, b, h, H = 99, 1, 2, 5
    key = int(DH.mix64(np.array([(seed + DH.GOLDEN_GAMMA * (1 + b * H + h)) & DH.MASK64], np.uint64))[0])
    assert key == DH.head_key(seed, b, h, H)
    rows, cols = np.array([0, 7, 1000]), np.array([0, 1, 2, 3, 4095, 4096])
    u = DH.uniforms16(seed, b, h, H, rows, cols)
    for ri, i in enumerate(rows):
        a = int(DH.mix64(np.array([(key + DH.GOLDEN_GAMMA * (2 * int(i) + 1)) & DH.MASK64], np.uint64))[0])
        for ci, j in enumerate(cols):
            c = int(j) // 2
            bc = int(DH.mix64(np.array([(key + DH.GOLDEN_GAMMA * (2 * c + 2)) & DH.MASK64], np.uint64))[0])
            w = int(DH.fmix32(np.array([(a ^ bc) & 0xFFFFFFFF], np.uint32))[0])
            assert int(u[ri, ci]) == ((w >> 16) if j % 2 else (w & 0xFFFF))


def test_draws_uniform_16_bit():
    """Both halves of the hash are uniform: chi-square over 256 bins of the
    high and the low byte of the draws of even and of odd columns."""
    u = DH.uniforms16(5, 0, 0, 1, np.arange(1024), np.arange(2048))  # 2M draws
    for sub in (u[:, 0::2], u[:, 1::2]):
        for byte in (sub >> 8, sub & 0xFF):
            cnt = np.bincount(byte.ravel().astype(np.int64), minlength=256)
            e = byte.size / 256
            chi2 = float(np.sum((cnt - e) ** 2 / e))
            assert chi2 < 255 + 6 * np.sqrt(2 * 255), chi2  # mean 255, sd 22.6


def test_pair_halves_and_rectangles_independent():
    """The two draws of one hash are uncorrelated, and so are the four keep
    decisions of rectangles (i, j), (i, j'), (i', j), (i', j'), whose hash
    inputs A ^ B XOR to zero (a structure the finalizer must break)."""
    p = 0.5
    rows, cols = np.arange(2048), np.arange(2048)
    u = DH.uniforms16(11, 0, 1, 2, rows, cols).astype(np.float64) / 65536.0 - 0.5
    n = u[:, 0::2].size
    corr = np.mean(u[:, 0::2] * u[:, 1::2]) / (1.0 / 12.0)
    assert abs(corr) <= 5.0 / np.sqrt(n)
    m = DH.keep_mask(11, 0, 1, 2, p, rows, cols).astype(np.float64) - 0.5
    rng = np.random.default_rng(0)
    i, i2 = rng.integers(0, 2048, 200000), rng.integers(0, 2048, 200000)
    j, j2 = rng.integers(0, 2048, 200000), rng.integers(0, 2048, 200000)
    ok = (i != i2) & (j != j2)
    prod = (m[i, j] * m[i, j2] * m[i2, j] * m[i2, j2])[ok] / 0.0625  # each factor +-0.5
    assert abs(prod.mean()) <= 5.0 / np.sqrt(ok.sum())
    # the same statistic does detect the structure when the finalizer is skipped
    key = DH.head_key(11, 0, 1, 2)
    raw = DH.row_keys(key, rows)[:, None] ^ DH.pair_keys(key, cols // 2)[None, :]
    mr = ((raw >> np.uint32(31)) & np.uint32(1)).astype(np.float64) - 0.5
    prod_raw = (mr[i, j] * mr[i, j2] * mr[i2, j] * mr[i2, j2])[ok] / 0.0625
    assert abs(prod_raw.mean()) > 0.9
