"""Pins for the fp64 oracle, checked against facts that do not come from the
oracle itself: brute-force loops, finite differences, closed forms,
invariants and special cases. CPU only.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import attention as A
from workloads import Workload, make_inputs

RNG = np.random.default_rng(7)


def _rand(B, N, H, d, rng=RNG, amp=1.0):
    return amp * rng.standard_normal((B, N, H, d))


# --------------------------------------------------------------------------
# Pin 1: every row of P is a probability distribution.
@pytest.mark.parametrize("causal", [False, True])
def test_prob_rows_sum_to_one(causal):
    q = _rand(1, 64, 1, 16)[0, :, 0]
    k = _rand(1, 64, 1, 16)[0, :, 0]
    s = A.attention_scores(q, k, 0.25, causal)
    _, _, lse = A.softmax_stats(s)
    p = A.attention_probs(s, lse)
    assert np.all(p >= 0.0)
    assert np.max(np.abs(p.sum(axis=1) - 1.0)) <= 1e-12
    if causal:
        assert np.all(p[np.triu_indices(64, 1)] == 0.0)


# --------------------------------------------------------------------------
# Pin 2: brute force with per-element Python loops and math.exp.
def _brute_forward(q, k, v, scale, causal, keep=None, p_drop=0.0):
    N, d = q.shape
    o = [[0.0] * v.shape[1] for _ in range(N)]
    lse = [0.0] * N
    for i in range(N):
        logits = []
        for j in range(N):
            if causal and j > i:
                continue
            logits.append((j, scale * sum(q[i][c] * k[j][c] for c in range(d))))
        mx = max(x for _, x in logits)
        den = sum(math.exp(x - mx) for _, x in logits)
        lse[i] = mx + math.log(den)
        for j, x in logits:
            pij = math.exp(x - mx) / den
            if keep is not None:
                pij = pij * keep[i][j] / (1.0 - p_drop)
            for c in range(v.shape[1]):
                o[i][c] += pij * v[j][c]
    return np.array(o), np.array(lse)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("p_drop", [0.0, 0.3])
@pytest.mark.parametrize("N,d", [(1, 1), (5, 3), (8, 4)])
def test_brute_force_forward(causal, p_drop, N, d):
    B, H = 2, 2
    q, k, v = _rand(B, N, H, d), _rand(B, N, H, d), _rand(B, N, H, d)
    scale = 1.0 / math.sqrt(d)
    seed = 11
    o, lse = oracle.forward(q, k, v, scale, causal, p_drop, seed)
    for b in range(B):
        for h in range(H):
            keep = None
            if p_drop > 0:
                keep = oracle.keep_mask(seed, b, h, H, p_drop, np.arange(N), np.arange(N)).astype(float)
            ob, lb = _brute_forward(q[b, :, h], k[b, :, h], v[b, :, h], scale, causal, keep,
                                    float(np.float32(p_drop)))
            assert np.max(np.abs(o[b, :, h] - ob)) <= 1e-12
            assert np.max(np.abs(lse[b, h] - lb)) <= 1e-12


# --------------------------------------------------------------------------
# Pin 3: central finite differences of L = sum(dO * O).
def _loss(q, k, v, do, scale, causal, p, seed):
    o, _ = oracle.forward(q, k, v, scale, causal, p, seed)
    return float(np.sum(do * o))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("p_drop", [0.0, 0.1])
def test_finite_difference_gradients(causal, p_drop):
    rng = np.random.default_rng(123)
    B, N, H, d = 1, 12, 2, 3
    q, k, v, do = (rng.standard_normal((B, N, H, d)) for _ in range(4))
    scale, seed = 0.7, 99
    dq, dk, dv, _ = oracle.backward(q, k, v, do, scale, causal, p_drop, seed)
    step = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp = x.copy()
            xm = x.copy()
            xp[idx] += step
            xm[idx] -= step
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = _loss(args["q"], args["k"], args["v"], do, scale, causal, p_drop, seed)
            args[name] = xm
            lm = _loss(args["q"], args["k"], args["v"], do, scale, causal, p_drop, seed)
            num[idx] = (lp - lm) / (2 * step)
        err = np.max(np.abs(num - g)) / max(np.max(np.abs(g)), 1e-30)
        assert err <= 1e-6, (name, err)


# --------------------------------------------------------------------------
# Pin: D read from a given (stored) forward output. D moves by
# dD_i = rowsum(dO_i * (o_i - O_i)); since dLSE_i/dS_ij = P_ij, dQ and dK
# become the gradients of sum(dO * O) - sum_i dD_i LSE_i with dD held fixed,
# and dV is unchanged. Finite differences of the forward check all three.
def _num_grad(loss, args, name, step=1e-6):
    x = args[name]
    num = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        vals = []
        for sgn in (1, -1):
            xs = x.copy()
            xs[idx] += sgn * step
            vals.append(loss(**{**args, name: xs}))
        num[idx] = (vals[0] - vals[1]) / (2 * step)
    return num


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("p_drop", [0.0, 0.1])
def test_given_output_gradients_by_finite_differences(causal, p_drop):
    rng = np.random.default_rng(321)
    B, N, H, d = 1, 10, 2, 3
    q, k, v, do = (rng.standard_normal((B, N, H, d)) for _ in range(4))
    scale, seed = 0.7, 99
    o_exact, _ = oracle.forward(q, k, v, scale, causal, p_drop, seed)
    o_given = o_exact + 0.05 * rng.standard_normal(o_exact.shape)
    shift = np.einsum("bnhd,bnhd->bhn", do, o_given - o_exact)
    dq, dk, dv, _ = oracle.backward(q, k, v, do, scale, causal, p_drop, seed, o=o_given)

    def loss(q, k, v):
        o, lse = oracle.forward(q, k, v, scale, causal, p_drop, seed)
        return float(np.sum(do * o) - np.sum(shift * lse))

    args = {"q": q, "k": k, "v": v}
    for name, g in (("q", dq), ("k", dk), ("v", dv)):
        num = _num_grad(loss, args, name)
        err = np.max(np.abs(num - g)) / max(np.max(np.abs(g)), 1e-30)
        assert err <= 1e-6, (name, err)
    # and the move is not zero: the given output does change dQ and dK
    dq0, dk0, dv0, _ = oracle.backward(q, k, v, do, scale, causal, p_drop, seed)
    assert np.max(np.abs(dq - dq0)) > 1e-3 and np.max(np.abs(dk - dk0)) > 1e-3
    assert np.max(np.abs(dv - dv0)) == 0.0


def test_given_output_single_key_and_exact_output():
    # one key: P = 1 and dP = dO . V, so dS = -dO . (o - V)
    q, k, v, do = (_rand(2, 1, 3, 5) for _ in range(4))
    e = 0.1 * _rand(2, 1, 3, 5)
    scale = 0.4
    dq, dk, dv, _ = oracle.backward(q, k, v, do, scale, True, o=v + e)
    ds = -np.sum(do * e, axis=3, keepdims=True)
    assert np.max(np.abs(dq - scale * ds * k)) <= 1e-14
    assert np.max(np.abs(dk - scale * ds * q)) <= 1e-14
    assert np.array_equal(dv, do)
    # the exact output gives the default gradients
    q, k, v, do = (_rand(1, 40, 2, 6) for _ in range(4))
    o, _ = oracle.forward(q, k, v, 0.5, True, 0.2, 5)
    a = oracle.backward(q, k, v, do, 0.5, True, 0.2, 5)
    b = oracle.backward(q, k, v, do, 0.5, True, 0.2, 5, o=o)
    for x, y in zip(a, b):
        assert np.max(np.abs(x - y)) <= 1e-12


# --------------------------------------------------------------------------
# Closed forms and special cases.
@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_gives_uniform_attention(causal):
    B, N, H, d = 1, 40, 2, 8
    q = np.zeros((B, N, H, d))
    k, v = _rand(B, N, H, d), _rand(B, N, H, d)
    o, lse = oracle.forward(q, k, v, 0.3, causal)
    for h in range(H):
        if causal:
            cnt = np.arange(1, N + 1)
            expect = np.cumsum(v[0, :, h], axis=0) / cnt[:, None]
            assert np.max(np.abs(lse[0, h] - np.log(cnt))) <= 1e-13
        else:
            expect = np.broadcast_to(v[0, :, h].mean(axis=0), (N, d))
            assert np.max(np.abs(lse[0, h] - np.log(N))) <= 1e-13
        assert np.max(np.abs(o[0, :, h] - expect)) <= 1e-13


def test_zero_query_with_dropout_is_masked_mean():
    B, N, H, d = 1, 30, 1, 4
    q = np.zeros((B, N, H, d))
    k, v = _rand(B, N, H, d), _rand(B, N, H, d)
    p, seed = 0.25, 5
    o, _ = oracle.forward(q, k, v, 1.0, True, p, seed)
    z = oracle.keep_mask(seed, 0, 0, 1, p, np.arange(N), np.arange(N)).astype(float)
    z = np.tril(z)
    expect = (z @ v[0, :, 0]) / np.arange(1, N + 1)[:, None] / (1 - float(np.float32(p)))
    assert np.max(np.abs(o[0, :, 0] - expect)) <= 1e-13


def test_single_key():
    q, k, v, do = (_rand(2, 1, 3, 5) for _ in range(4))
    scale = 0.4
    o, lse = oracle.forward(q, k, v, scale, True)
    dq, dk, dv, _ = oracle.backward(q, k, v, do, scale, True)
    assert np.array_equal(o, v)
    assert np.max(np.abs(lse - scale * np.einsum("bnhd,bnhd->bhn", q, k))) <= 1e-14
    assert np.all(dq == 0) and np.all(dk == 0)
    assert np.array_equal(dv, do)


@pytest.mark.parametrize("causal", [False, True])
def test_gradient_invariants(causal):
    B, N, H, d = 2, 33, 2, 6
    q, k, v, do = (_rand(B, N, H, d) for _ in range(4))
    dq, dk, dv, _ = oracle.backward(q, k, v, do, 0.5, causal)
    # rows of dS sum to zero  =>  sum_j dK_j = scale * sum_i (sum_j dS_ij) Q_i = 0
    assert np.max(np.abs(dk.sum(axis=1))) <= 1e-12
    # rows of P sum to one    =>  sum_j dV_j = sum_i dO_i
    assert np.max(np.abs(dv.sum(axis=1) - do.sum(axis=1))) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_invariance(causal):
    B, N, H, d = 1, 20, 1, 5
    q, k, v, do = (_rand(B, N, H, d) for _ in range(4))
    c = RNG.standard_normal(d)
    scale = 0.6
    o1, l1 = oracle.forward(q, k, v, scale, causal)
    o2, l2 = oracle.forward(q, k + c, v, scale, causal)
    dq1, _, dv1, _ = oracle.backward(q, k, v, do, scale, causal)
    dq2, _, dv2, _ = oracle.backward(q, k + c, v, do, scale, causal)
    assert np.max(np.abs(o1 - o2)) <= 1e-12
    assert np.max(np.abs(l2 - l1 - scale * np.einsum("bnhd,d->bhn", q, c))) <= 1e-12
    assert np.max(np.abs(dq1 - dq2)) <= 1e-11
    assert np.max(np.abs(dv1 - dv2)) <= 1e-12


def test_key_value_permutation_invariance():
    B, N, H, d = 1, 25, 2, 4
    q, k, v, do = (_rand(B, N, H, d) for _ in range(4))
    perm = RNG.permutation(N)
    o1, l1 = oracle.forward(q, k, v, 0.5, False)
    o2, l2 = oracle.forward(q, k[:, perm], v[:, perm], 0.5, False)
    assert np.max(np.abs(o1 - o2)) <= 1e-13
    assert np.max(np.abs(l1 - l2)) <= 1e-13
    _, dk1, dv1, _ = oracle.backward(q, k, v, do, 0.5, False)
    _, dk2, dv2, _ = oracle.backward(q, k[:, perm], v[:, perm], do, 0.5, False)
    assert np.max(np.abs(dk1[:, perm] - dk2)) <= 1e-12
    assert np.max(np.abs(dv1[:, perm] - dv2)) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_lse_bounds(causal):
    B, N, H, d = 1, 50, 1, 8
    q, k = _rand(B, N, H, d, amp=3.0), _rand(B, N, H, d, amp=3.0)
    v = _rand(B, N, H, d)
    scale = 0.35
    _, lse = oracle.forward(q, k, v, scale, causal)
    s = A.attention_scores(q[0, :, 0], k[0, :, 0], scale, causal)
    mx = s.max(axis=1)
    nkeys = np.arange(1, N + 1) if causal else np.full(N, N)
    assert np.all(lse[0, 0] >= mx - 1e-12)
    assert np.all(lse[0, 0] <= mx + np.log(nkeys) + 1e-12)


def test_zero_dropout_equals_no_dropout():
    q, k, v, do = (_rand(1, 17, 2, 4) for _ in range(4))
    a = oracle.forward(q, k, v, 0.5, True, 0.0, 123)
    b = oracle.forward(q, k, v, 0.5, True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    # and the mask at p = 0 keeps everything
    assert oracle.keep_mask(3, 0, 0, 1, 0.0, np.arange(50), np.arange(50)).all()


def test_panels_do_not_change_results():
    q, k, v, do = (_rand(1, 70, 1, 4) for _ in range(4))
    for causal in (False, True):
        a = oracle.forward(q, k, v, 0.5, causal, 0.2, 9, panel=7)
        b = oracle.forward(q, k, v, 0.5, causal, 0.2, 9, panel=256)
        assert np.max(np.abs(a[0] - b[0])) <= 1e-13
        ga = oracle.backward(q, k, v, do, 0.5, causal, 0.2, 9, panel=9)
        gb = oracle.backward(q, k, v, do, 0.5, causal, 0.2, 9, panel=256)
        for x, y in zip(ga, gb):
            assert np.max(np.abs(x - y)) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_row_panel_with_offsets_matches_full(causal):
    """Rows r0..r1 computed alone (query i at row and key position r0 + i)
    equal those rows of the whole problem, dropout included: the offsets key
    the causal mask and the dropout hash by absolute row."""
    B, N, H, d = 1, 50, 2, 4
    q, k, v = (_rand(B, N, H, d) for _ in range(3))
    scale, p_drop, seed = 0.5, 0.3, 21
    o, lse = oracle.forward(q, k, v, scale, causal, p_drop, seed)
    for h in range(H):
        for r0, r1 in ((0, 7), (13, 29), (44, 50)):
            po, pl = oracle.head_forward(q[0, r0:r1, h].astype(np.float64), k[0, :, h].astype(np.float64),
                                         v[0, :, h].astype(np.float64), scale, causal, p_drop, seed, 0, h,
                                         H, row_offset=r0, hash_row_offset=r0)
            assert np.max(np.abs(po - o[0, r0:r1, h])) <= 1e-13
            assert np.max(np.abs(pl - lse[0, h, r0:r1])) <= 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_backward_row_panels_with_offsets_match_full(causal):
    """The backward over row panels computed alone: each panel's dQ and D are
    those rows of the whole problem, and the panels' shares of dK and dV add
    up to the whole dK and dV (dropout included)."""
    B, N, H, d = 1, 50, 2, 4
    q, k, v, do = (_rand(B, N, H, d) for _ in range(4))
    scale, p_drop, seed = 0.5, 0.3, 21
    dq, dk, dv, dd = oracle.backward(q, k, v, do, scale, causal, p_drop, seed)
    for h in range(H):
        sk = np.zeros((N, d))
        sv = np.zeros((N, d))
        for r0, r1 in ((0, 7), (7, 29), (29, 44), (44, 50)):
            pq, pk, pv, pd = oracle.head_backward(q[0, r0:r1, h], k[0, :, h], v[0, :, h], do[0, r0:r1, h],
                                                  scale, causal, p_drop, seed, 0, h, H,
                                                  row_offset=r0, hash_row_offset=r0)
            assert np.max(np.abs(pq - dq[0, r0:r1, h])) <= 1e-12
            assert np.max(np.abs(pd - dd[0, h, r0:r1])) <= 1e-12
            sk += pk
            sv += pv
        assert np.max(np.abs(sk - dk[0, :, h])) <= 1e-12
        assert np.max(np.abs(sv - dv[0, :, h])) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("p_drop", [0.0, 0.15])
def test_sampled_head_matches_full(causal, p_drop):
    B, N, H, d = 2, 45, 3, 5
    q, k, v, do = (_rand(B, N, H, d) for _ in range(4))
    scale, seed = 0.45, 77
    o, lse = oracle.forward(q, k, v, scale, causal, p_drop, seed)
    dq, dk, dv, dd = oracle.backward(q, k, v, do, scale, causal, p_drop, seed)
    rows = np.array([0, 3, 44, 20])
    cols = np.array([44, 0, 7])
    s = oracle.sampled_head(q, k, v, do, scale, causal, p_drop, seed, 1, 2, rows, cols, panel=8)
    assert np.max(np.abs(s["o"] - o[1, rows, 2])) <= 1e-13
    assert np.max(np.abs(s["lse"] - lse[1, 2, rows])) <= 1e-13
    assert np.max(np.abs(s["dq"] - dq[1, rows, 2])) <= 1e-12
    assert np.max(np.abs(s["D"] - dd[1, 2, rows])) <= 1e-12
    assert np.max(np.abs(s["dk"] - dk[1, cols, 2])) <= 1e-12
    assert np.max(np.abs(s["dv"] - dv[1, cols, 2])) <= 1e-12


# --------------------------------------------------------------------------
# Planted mistakes: a plausible error in the backward must fail a pin above.
def _planted_backward(kind):
    def bwd(q, k, v, do, scale, causal, p=0.0, seed=0):
        qh, kh, vh, doh = q[0, :, 0], k[0, :, 0], v[0, :, 0], do[0, :, 0]
        s = A.attention_scores(qh, kh, scale, causal)
        _, _, lse = A.softmax_stats(s)
        pm = A.attention_probs(s, lse)
        dp = doh @ vh.T
        dd = np.sum(pm * dp, axis=1)
        if kind == "drop_D":
            ds = pm * dp
        elif kind == "sign":
            ds = pm * (dd[:, None] - dp)
        else:
            ds = pm * (dp - dd[:, None])
        dq = scale * (ds @ kh)
        dk = scale * (ds @ qh) if kind == "transpose" else scale * (ds.T @ qh)
        return dq, dk
    return bwd


@pytest.mark.parametrize("kind", ["drop_D", "sign", "transpose"])
def test_finite_differences_catch_planted_mistakes(kind):
    rng = np.random.default_rng(5)
    q, k, v, do = (rng.standard_normal((1, 6, 1, 6)) for _ in range(4))
    dq, dk = _planted_backward(kind)(q, k, v, do, 0.5, True)
    step = 1e-6
    worst = 0.0
    for name, x, g in (("q", q, dq), ("k", k, dk)):
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += step
            xm[idx] -= step
            a = {"q": q, "k": k}
            a[name] = xp
            lp = _loss(a["q"], a["k"], v, do, 0.5, True, 0.0, 0)
            a[name] = xm
            lm = _loss(a["q"], a["k"], v, do, 0.5, True, 0.0, 0)
            worst = max(worst, abs((lp - lm) / (2 * step) - g[idx[1], idx[3]]))
    assert worst > 1e-3  # the finite-difference pin would reject this backward


# --------------------------------------------------------------------------
# Inputs: bf16 rounding of the generator against torch's conversion.
def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    from workloads import f32_to_bf16_bits, bf16_bits_to_f32
    x = np.concatenate([
        RNG.standard_normal(100000).astype(np.float32),
        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e38, -1e-40, np.inf, -np.inf], np.float32),
    ])
    # exact ties: 1 + 2^-8 rounds to 1 (even), 1 + 3*2^-8 rounds up
    bits = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, ref)
    assert np.array_equal(bf16_bits_to_f32(bits), torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_input_recipe_is_deterministic():
    w = Workload(99, "t", 1, 3, 10, 8, "bf16", True, 0.0, True, amp=0.5)
    a = make_inputs(w)
    b = make_inputs(w)
    for name in ("q", "k", "v", "do"):
        assert np.array_equal(a[name][0], b[name][0])
    # values are exactly representable bf16 numbers scaled from N(0,1) * 0.5
    rng = np.random.default_rng(1099)
    x = (rng.standard_normal((1, 10, 3, 8), dtype=np.float32) * np.float32(0.5)).astype(np.float32)
    assert np.max(np.abs(a["q"][1] - x)) <= np.max(np.abs(x)) * 2.0 ** -8


# --------------------------------------------------------------------------
# Tolerance reasoning of the large-norm GPU stress tests: a backward that is
# exact except for rounding dS to bf16 before dQ = scale dS K (as the kernels
# feed the matrix cores) is off by at most scale 2^-8 (|dS| |K|) per element
# (2^-8: the unit roundoff of 8 significant bits), the allowance those tests
# add; on keys of norm 40 that error exceeds 2e-2 max(1, |dQ|) while staying
# within half of the bar plus the allowance.
def test_bf16_ds_rounding_bound_on_shifted_logits():
    import torch
    w = Workload(71, "shift", 1, 2, 257, 64, "bf16", True, 0.0, True)
    inp = make_inputs(w, with_grad=True)
    bf = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).double().numpy()  # noqa: E731
    q, k = inp["q"][1].copy(), inp["k"][1].copy()
    q[..., 0], k[..., 0] = 16.0, 40.0
    q, k, v, do = bf(q), bf(k), inp["v"][1].astype(np.float64), inp["do"][1].astype(np.float64)
    o, lse = oracle.forward(q, k, v, w.scale, True)
    o_st = bf(o)
    ref = oracle.backward(q, k, v, do, w.scale, True, o=o_st)[0]
    worst_plain = worst_bound = 0.0
    for h in range(w.H):
        s = A.attention_scores(q[0, :, h], k[0, :, h], w.scale, True)
        p = A.attention_probs(s, lse[0, h])
        ds = p * (do[0, :, h] @ v[0, :, h].T - np.sum(do[0, :, h] * o_st[0, :, h], axis=1)[:, None])
        emu = w.scale * bf(ds) @ k[0, :, h]
        err = np.abs(emu - ref[0, :, h])
        assert np.all(err <= w.scale * 2.0 ** -8 * (np.abs(ds) @ np.abs(k[0, :, h])) + 1e-12)
        worst_plain = max(worst_plain, float(np.max(err / (2e-2 * np.maximum(1.0, np.abs(ref[0, :, h]))))))
        allow = 2e-2 * np.maximum(1.0, np.abs(ref[0, :, h])) + w.scale * 2.0 ** -8 * (np.abs(ds) @ np.abs(k[0, :, h]))
        worst_bound = max(worst_bound, float(np.max(err / allow)))
    assert worst_plain > 1.0
    assert worst_bound <= 0.5
