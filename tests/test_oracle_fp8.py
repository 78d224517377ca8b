"""Pins for the FP8 oracle (oracle/fp8.py), CPU only: the E4M3 rounding
against the format's own bit layout (every value, every midpoint, random
values by brute-force nearest), worked values, the per-block scale rule, and
attention on inputs the quantisation leaves unchanged."""
import numpy as np
import pytest

import oracle
from oracle import fp8


def _e4m3_table():
    """All finite E4M3 values decoded from the bit layout: sign, 4 exponent
    bits (bias 7), 3 mantissa bits; exponent field 0 is subnormal; S.1111.111
    is NaN."""
    vals = {}
    for code in range(256):
        s, e, m = code >> 7, (code >> 3) & 15, code & 7
        if e == 15 and m == 7:
            continue
        x = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
        vals[code] = -x if s else x
    return vals


def test_every_value_is_fixed_and_max_is_448():
    t = _e4m3_table()
    v = np.array(sorted(set(t.values())))
    np.testing.assert_array_equal(fp8.e4m3_round(v), v)
    assert v.max() == 448.0 and np.min(v[v > 0]) == 2.0 ** -9
    assert t[0x38] == 1.0


def test_midpoints_round_to_even():
    t = _e4m3_table()
    pos = sorted((c, x) for c, x in t.items() if x >= 0 and c < 0x80)
    for (c0, a), (c1, b) in zip(pos, pos[1:]):
        mid = (a + b) / 2
        even = a if (c0 & 1) == 0 else b
        assert fp8.e4m3_round(mid) == even, (a, b)
        assert fp8.e4m3_round(-mid) == -even


def test_random_values_round_to_nearest():
    grid = np.array(sorted(set(_e4m3_table().values())))
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(20000) * np.exp2(rng.integers(-12, 9, 20000))).astype(np.float32)
    x = np.clip(x, -448, 448)
    r = fp8.e4m3_round(x)
    d = np.abs(grid[None, :] - x.astype(np.float64)[:, None])
    best = np.min(d, axis=1)
    np.testing.assert_array_equal(np.abs(r - x), best)


def test_worked_values():
    cases = {1.0: 1.0, 1.0625: 1.0, 1.1875: 1.25, 448.0: 448.0, 2.0 ** -9: 2.0 ** -9,
             2.0 ** -10: 0.0, 3 * 2.0 ** -11: 2.0 ** -9, 1.97: 2.0, 0.3: 0.3125}
    for x, want in cases.items():
        assert fp8.e4m3_round(x) == want, x
    # relative error at most 2^-4 in the normal range
    x = np.linspace(2.0 ** -6, 448, 10001)
    assert np.max(np.abs(fp8.e4m3_round(x) - x) / x) <= 2.0 ** -4


def test_block_scales():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, 300, 3, 8)).astype(np.float32)
    x[1, 128:256, 2] = 0.0  # an all-zero block
    codes, sc = fp8.quantize(x, 128)
    assert sc.shape == (2, 3, 3)
    assert sc[1, 2, 1] == 1.0 and np.all(codes[1, 128:256, 2] == 0)
    for b in range(2):
        for h in range(3):
            for j in range(3):
                blk = codes[b, 128 * j:128 * (j + 1), h]
                if sc[b, h, j] != 1.0 or np.any(blk):
                    assert np.max(np.abs(blk)) == 448.0  # the largest element maps to 448
                    amax = np.max(np.abs(x[b, 128 * j:128 * (j + 1), h]))
                    assert sc[b, h, j] == np.float32(amax) / np.float32(448)
    deq = fp8.dequantize(codes, sc, 128)
    err = np.abs(deq - x)
    rep = np.repeat(sc, 128, axis=2)[:, :, :300].transpose(0, 2, 1)[:, :, :, None]
    assert np.all(err <= np.maximum(2.0 ** -4 * np.abs(x), rep * 2.0 ** -10) + 1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_grid_inputs_are_not_changed(causal):
    """Inputs already on the E4M3 grid whose every block reaches 448 quantise
    to themselves with scale 1, so the FP8 oracle equals the plain one."""
    grid = np.array(sorted(set(_e4m3_table().values())))
    rng = np.random.default_rng(2)
    B, N, H, d = 1, 200, 2, 8
    q = rng.choice(grid, size=(B, N, H, d))
    k = rng.choice(grid, size=(B, N, H, d))
    for x, r in ((q, 128), (k, 64)):
        for j in range(0, N, r):
            x[:, j, :, 0] = 448.0
    v = rng.standard_normal((B, N, H, d))
    o, lse = fp8.forward_fp8(q, k, v, 1e-4, causal)
    o2, lse2 = oracle.forward(q, k, v, 1e-4, causal)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)


def test_fp8_scores_stay_close_to_exact():
    rng = np.random.default_rng(3)
    q, k, v = (rng.standard_normal((1, 256, 2, 128)).astype(np.float32) for _ in range(3))
    o, lse = fp8.forward_fp8(q, k, v, 128 ** -0.5, True)
    o2, lse2 = oracle.forward(q, k, v, 128 ** -0.5, True)
    assert np.max(np.abs(o - o2)) < 0.1 and np.max(np.abs(lse - lse2)) < 0.1


def _bf16(x):
    """Round-to-nearest-even to bf16 (8 significant bits), in float64."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).double().numpy()


@pytest.mark.parametrize("amp,N,d,causal", [(1.0, 300, 128, False), (8.0, 127, 80, True)])
def test_bf16_probability_rounding_error_bound(amp, N, d, causal):
    """The tolerance of the random-shape FP8 test: an otherwise exact forward
    that rounds P to bf16 before P V (with the row sum on the rounded values)
    and stores O in bf16 is off by at most 2^-8 * sum_j P_ij |V_j| + 2^-7 |O_i|
    per element to first order (bf16 keeps 8 significant bits, relative
    rounding up to 2^-8: once on each P in P V, once through the row sum of
    the rounded P, once on the stored O), well within
    2e-2 * max(1, sum_j P_ij |V_j|). On the inputs of
    that test's amplitude-8 draw of N = 127, d = 80 it misses
    2e-2 * max(1, |O|): there |O| does not set the scale."""
    from workloads import Workload, make_inputs
    w = Workload(65, "f8r", 2, 1, N, d, "bf16", causal, 0.0, False, amp=amp)
    inp = make_inputs(w, with_grad=False)
    q, k, v = (inp[n][1].astype(np.float64) for n in ("q", "k", "v"))
    o, _ = fp8.forward_fp8(q, k, v, w.scale, causal)
    mag = fp8.forward_fp8(q, k, np.abs(v), w.scale, causal)[0]
    qd = fp8.dequantize(*fp8.quantize(q, fp8.Q_BLOCK), fp8.Q_BLOCK)
    kd = fp8.dequantize(*fp8.quantize(k, fp8.K_BLOCK), fp8.K_BLOCK)
    worst_o = 0.0
    for b in range(w.B):
        s = oracle.attention_scores(qd[b, :, 0], kd[b, :, 0], w.scale, causal)
        p = _bf16(np.exp(s - s.max(axis=1, keepdims=True)))
        emu = _bf16((p @ v[b, :, 0]) / p.sum(axis=1, keepdims=True))
        ob, mb = o[b, :, 0], mag[b, :, 0]
        err = np.abs(emu - ob)
        assert np.all(err <= 2.0 ** -8 * mb + 2.0 ** -7 * np.abs(ob) + 1e-12)
        assert np.max(err / (2e-2 * np.maximum(1.0, mb))) <= 0.5
        worst_o = max(worst_o, float(np.max(err / (2e-2 * np.maximum(1.0, np.abs(ob))))))
    if amp == 8.0:
        assert worst_o > 1.0
