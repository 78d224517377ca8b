"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on
the same seeded inputs, element by element, at sizes the oracle finishes in
seconds that still span several tiles and a ragged tail; plus dropout masks
bit for bit, determinism, and the degenerate cases."""
import numpy as np
import pytest

import oracle
from helpers import assert_close, device_inputs, to_device, to_host
from workloads import WORKLOADS, Workload, make_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import exact_io_aware_72_amd as fa  # noqa: E402


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run_fwd(dev, w):
    o, lse = fa.forward(dev["q"], dev["k"], dev["v"], w.causal, w.dropout_p, w.dropout_seed, w.scale)
    torch.cuda.synchronize()
    return to_host(o), to_host(lse)


def _run_bwd(dev, w, o, lse):
    dq, dk, dv = fa.backward(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, w.causal, w.dropout_p,
                             w.dropout_seed, w.scale)
    torch.cuda.synchronize()
    return to_host(dq), to_host(dk), to_host(dv)


def _case(cfg, **kw):
    return WORKLOADS[cfg].with_(**kw)


# Small variants of every workload: same seed recipe, dtype, head dim, mask,
# dropout and amplitude; sequence lengths with ragged tails.
FWD_CASES = [
    _case(1),                                                    # fp32, N=256, d=64, full (exact workload)
    _case(1, N=300, causal=True),
    _case(1, N=77, d=128),
    _case(1, N=130, d=80, dropout_p=0.2),
    _case(2, B=2, H=3, N=300),                                   # bf16 causal d=64
    _case(2, B=1, H=2, N=1000, causal=False),
    _case(3, B=1, H=2, N=513),                                   # bf16 causal d=128
    _case(3, B=2, H=1, N=256, causal=False),
    _case(4, B=1, H=2, N=257),                                   # bf16 causal d=80, amp 0.5
    _case(4, B=1, H=3, N=200, causal=False),
    _case(5, B=1, H=2, N=300),                                   # bf16 causal d=128, dropout 0.1
    _case(5, B=1, H=1, N=191, causal=False, d=64),
    _case(3, B=1, H=1, N=1),
    _case(3, B=1, H=2, N=17),
    _case(4, B=1, H=1, N=100, causal=False),
    _case(2, B=1, H=1, N=129, dropout_p=0.5),
    # Head dims up to 80 from N = 8192 (and dropout from N = 32768) take the
    # eight-wave forward: 256-row work-groups with a ragged last one.
    _case(2, B=1, H=2, N=8200),
    _case(4, B=1, H=1, N=8300, causal=False),
    _case(2, B=1, H=1, N=8250, causal=False, dropout_p=0.1),
]


def _ids(cases):
    return [f"{w.dtype}-d{w.d}-N{w.N}-B{w.B}H{w.H}-{'causal' if w.causal else 'full'}-p{w.dropout_p}"
            for w in cases]


@pytest.mark.parametrize("w", FWD_CASES, ids=_ids(FWD_CASES))
def test_forward_matches_oracle(w):
    inp = make_inputs(w, with_grad=False)
    dev, val = device_inputs(inp, w.dtype)
    o, lse = _run_fwd(dev, w)
    o_ref, lse_ref = oracle.forward(val["q"], val["k"], val["v"], w.scale, w.causal, w.dropout_p,
                                    w.dropout_seed)
    assert_close("O", o, o_ref, w.dtype)
    assert_close("LSE", lse, lse_ref, w.dtype)


# Causal grids that the device holds at once as an even number of work-groups
# per CU (256 CUs): the launcher pairs the blocks (r, nblk - 1 - r) per CU.
# Two and four work-groups per CU at d = 64, two at d = 128.
PAIR_CASES = [
    _case(2, B=4, H=16, N=1024),
    _case(2, B=8, H=16, N=1024),
    _case(3, B=4, H=16, N=1024),
]


@pytest.mark.parametrize("w", PAIR_CASES, ids=_ids(PAIR_CASES))
def test_forward_resident_grid_pairs(w):
    inp = make_inputs(w, with_grad=False)
    dev, val = device_inputs(inp, w.dtype)
    o, lse = _run_fwd(dev, w)
    o_ref, lse_ref = oracle.forward(val["q"], val["k"], val["v"], w.scale, w.causal, w.dropout_p,
                                    w.dropout_seed)
    assert_close("O", o, o_ref, w.dtype)
    assert_close("LSE", lse, lse_ref, w.dtype)


# Causal grids several times larger than the device holds at once (one
# block per work-group, heaviest first, at these lengths; block pairs per
# work-group, taken from N = 32768 and by packed batches, are checked in
# test_gpu_fullsize.py and test_gpu_varlen.py). Four-wave groups at d = 128
# (two per CU), d = 64 (four per CU) and d = 80, with dropout, and with an
# odd block count, a ragged tail and a head count that is not a multiple of
# 8 (the non-XCD-aware mapping).
SWEEP_PAIR_CASES = [
    _case(3, B=2, H=64, N=1024),
    _case(2, B=4, H=64, N=1024),
    _case(4, B=2, H=64, N=1024),
    _case(5, B=1, H=128, N=1024),
    _case(3, B=1, H=105, N=1100),
]


@pytest.mark.parametrize("w", SWEEP_PAIR_CASES, ids=_ids(SWEEP_PAIR_CASES))
def test_forward_large_causal_grids(w):
    inp = make_inputs(w, with_grad=False)
    dev, val = device_inputs(inp, w.dtype)
    o, lse = _run_fwd(dev, w)
    o_ref, lse_ref = oracle.forward(val["q"], val["k"], val["v"], w.scale, w.causal, w.dropout_p,
                                    w.dropout_seed)
    assert_close("O", o, o_ref, w.dtype)
    assert_close("LSE", lse, lse_ref, w.dtype)


def test_eight_wave_large_grid_heads():
    """Eight-wave forward groups (d = 80, N = 8192) over a grid twice the
    device's. Three whole heads, on different XCDs, against the oracle."""
    w = _case(4, B=1, H=32, N=8192)
    inp = make_inputs(w, with_grad=False)
    dev, val = device_inputs(inp, w.dtype)
    o, lse = _run_fwd(dev, w)
    heads = [(0, 0), (0, 13), (0, 31)]
    o_ref, lse_ref = oracle.forward(val["q"], val["k"], val["v"], w.scale, w.causal, heads=heads)
    for b, h in heads:
        assert_close(f"O[{b},{h}]", o[b, :, h], o_ref[b, :, h], w.dtype)
        assert_close(f"LSE[{b},{h}]", lse[b, h], lse_ref[b, h], w.dtype)


def test_eight_wave_dropout_forward_rows():
    """Dropout runs from N = 32768 take the eight-wave forward; at N = 32800
    the last 256-row work-group holds 32 rows. Rows at the start, across a
    256-row group boundary and at the end are checked against the oracle,
    which computes those row panels alone (query i at row r0 + i for the
    causal mask and the dropout hash)."""
    w = _case(5, B=1, H=2, N=32800)
    inp = make_inputs(w, with_grad=False)
    dev, val = device_inputs(inp, w.dtype)
    o, lse = _run_fwd(dev, w)
    for h in range(w.H):
        for r0, r1 in ((0, 40), (16360, 16424), (32704, 32800)):
            po, pl = oracle.head_forward(val["q"][0, r0:r1, h], val["k"][0, :, h], val["v"][0, :, h],
                                         w.scale, w.causal, w.dropout_p, w.dropout_seed, 0, h, w.H,
                                         row_offset=r0, hash_row_offset=r0)
            assert_close(f"O[{h},{r0}:{r1}]", o[0, r0:r1, h], po, w.dtype)
            assert_close(f"LSE[{h},{r0}:{r1}]", lse[0, h, r0:r1], pl, w.dtype)


BWD_CASES = [
    _case(3, B=1, H=2, N=300),
    _case(3, B=1, H=1, N=260, causal=False),
    _case(4, B=1, H=2, N=257),
    _case(4, B=1, H=1, N=150, causal=False),
    _case(5, B=1, H=2, N=300),
    _case(5, B=1, H=1, N=200, causal=False),
    _case(2, B=1, H=2, N=333, backward=True),
    _case(1, N=256, backward=True),                              # fp32 backward
    _case(1, N=100, causal=True, d=80, dropout_p=0.1, backward=True),
    _case(3, B=1, H=1, N=1),
    _case(4, B=2, H=1, N=33),
]


@pytest.mark.parametrize("w", BWD_CASES, ids=_ids(BWD_CASES))
def test_backward_matches_oracle(w):
    inp = make_inputs(w, with_grad=True)
    dev, val = device_inputs(inp, w.dtype)
    o, lse = fa.forward(dev["q"], dev["k"], dev["v"], w.causal, w.dropout_p, w.dropout_seed, w.scale)
    dq, dk, dv = _run_bwd(dev, w, o, lse)
    dq_r, dk_r, dv_r, _ = oracle.backward(val["q"], val["k"], val["v"], val["do"], w.scale, w.causal,
                                          w.dropout_p, w.dropout_seed)
    assert_close("dQ", dq, dq_r, w.dtype)
    assert_close("dK", dk, dk_r, w.dtype)
    assert_close("dV", dv, dv_r, w.dtype)


def test_preprocess_matches_oracle():
    # The preprocess reads O as stored; it is handed the oracle's O in bf16,
    # and the oracle's backward reads D from that same O.
    w = _case(3, B=2, H=3, N=77)
    inp = make_inputs(w, with_grad=True)
    dev, val = device_inputs(inp, w.dtype)
    o_r, _ = oracle.forward(val["q"], val["k"], val["v"], w.scale, w.causal)
    o_st = torch.from_numpy(o_r).to(torch.bfloat16).cuda()
    dd = to_host(fa.backward_preprocess(o_st, dev["do"]))
    ref = oracle.backward(val["q"], val["k"], val["v"], val["do"], w.scale, w.causal, o=to_host(o_st))[3]
    assert np.max(np.abs(dd - ref)) <= 1e-4 * max(1.0, np.max(np.abs(ref)))


def test_backward_steps_equal_fused_call():
    w = _case(4, B=1, H=2, N=200)
    inp = make_inputs(w, with_grad=True)
    dev, _ = device_inputs(inp, w.dtype)
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    o, lse = fa.forward(q, k, v, True, 0.0, 0, w.scale)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, True, 0.0, 0, w.scale)
    ws = fa.backward_preprocess(o, do)
    dk2, dv2 = fa.backward_dkdv(q, k, v, do, lse, ws, True, 0.0, 0, w.scale)
    dq2 = fa.backward_dq(q, k, v, do, lse, ws, True, 0.0, 0, w.scale)
    torch.cuda.synchronize()
    for a, b in ((dq, dq2), (dk, dk2), (dv, dv2)):
        assert torch.equal(a, b)


# ---------------------------------------------------------------------------
# Dropout masks, bit for bit.
@pytest.mark.parametrize("b,h,H,p,row0,col0,rows,cols", [
    (0, 0, 8, 0.1, 0, 0, 257, 300),
    (0, 7, 8, 0.1, 65536 - 200, 65536 - 333, 200, 333),
    (1, 3, 16, 0.37, 12345, 40000, 64, 129),
    (0, 0, 1, 0.0, 0, 0, 31, 17),
])
def test_dropout_mask_bit_exact(b, h, H, p, row0, col0, rows, cols):
    got = fa.dropout_mask(2026, b, h, H, p, row0, col0, rows, cols).cpu().numpy().astype(bool)
    ref = oracle.keep_mask(2026, b, h, H, p, np.arange(row0, row0 + rows), np.arange(col0, col0 + cols))
    assert np.array_equal(got, ref)


def _onehot_window(N, d, j0):
    v = np.zeros((1, N, 1, d), np.float32)
    for c in range(d):
        if j0 + c < N:
            v[0, j0 + c, 0, c] = 1.0
    return v


@pytest.mark.parametrize("causal", [True, False])
def test_dropout_mask_read_out_of_forward(causal):
    """V rows j0..j0+d-1 set to unit vectors make O[i, c] = P~[i, j0+c], so the
    kernel's keep mask is (O != 0) wherever the probability is positive."""
    N, d, p, seed, j0 = 300, 64, 0.1, 2026, 40
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, N, 1, d), dtype=np.float32)
    k = rng.standard_normal((1, N, 1, d), dtype=np.float32)
    v = _onehot_window(N, d, j0)
    tq, tk, tv = (to_device(x, "f32") for x in (q, k, v))
    o, _ = fa.forward(tq, tk, tv, causal, p, seed, 0.125)
    for dt, (a, b_, c) in (("f32", (tq, tk, tv)),
                           ("bf16", (tq.bfloat16(), tk.bfloat16(), tv.bfloat16()))):
        o, _ = fa.forward(a, b_, c, causal, p, seed, 0.125)
        got = to_host(o)[0, :, 0, :] != 0.0
        ref = oracle.keep_mask(seed, 0, 0, 1, p, np.arange(N), np.arange(j0, j0 + d))
        valid = np.ones((N, d), bool)
        if causal:
            valid = (np.arange(j0, j0 + d)[None, :] <= np.arange(N)[:, None])
        assert np.array_equal(got[valid], ref[valid]), dt
        assert not got[~valid].any()


def test_dropout_mask_read_out_of_dkdv():
    """dO rows i0..i0+d-1 set to unit vectors make dV[j, c] = P~[i0+c, j]."""
    N, d, p, seed, i0 = 260, 64, 0.1, 77, 100
    rng = np.random.default_rng(4)
    q, k, v = (rng.standard_normal((1, N, 1, d), dtype=np.float32) for _ in range(3))
    do = _onehot_window(N, d, i0)
    tq, tk, tv, tdo = (to_device(x, "f32").bfloat16() for x in (q, k, v, do))
    o, lse = fa.forward(tq, tk, tv, True, p, seed, 0.125)
    _, _, dv = fa.backward(tq, tk, tv, o, tdo, lse, True, p, seed, 0.125)
    got = (to_host(dv)[0, :, 0, :] != 0.0)           # [key j, c]
    ref = oracle.keep_mask(seed, 0, 0, 1, p, np.arange(i0, i0 + d), np.arange(N)).T
    valid = np.arange(N)[:, None] <= np.arange(i0, i0 + d)[None, :]
    assert np.array_equal(got[valid], ref[valid])
    assert not got[~valid].any()


# ---------------------------------------------------------------------------
def test_deterministic_bitwise():
    w = _case(5, B=1, H=2, N=700)
    inp = make_inputs(w, with_grad=True)
    dev, _ = device_inputs(inp, w.dtype)
    outs = []
    for _ in range(2):
        o, lse = fa.forward(dev["q"], dev["k"], dev["v"], True, w.dropout_p, w.dropout_seed, w.scale)
        g = fa.backward(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, True, w.dropout_p,
                        w.dropout_seed, w.scale)
        torch.cuda.synchronize()
        outs.append([o.clone(), lse.clone()] + [x.clone() for x in g])
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.uint8) if a.dtype != torch.float32 else a, b.view(torch.uint8)
                           if b.dtype != torch.float32 else b)


def test_autograd_function_matches_backward():
    w = _case(3, B=1, H=2, N=130)
    inp = make_inputs(w, with_grad=True)
    dev, _ = device_inputs(inp, w.dtype)
    q, k, v = (dev[n].clone().requires_grad_(True) for n in ("q", "k", "v"))
    o = fa.flash_attention(q, k, v, causal=True)
    o.backward(dev["do"])
    o2, lse = fa.forward(dev["q"], dev["k"], dev["v"], True)
    dq, dk, dv = fa.backward(dev["q"], dev["k"], dev["v"], o2, dev["do"], lse, True)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
    assert torch.equal(q.grad, dq) and torch.equal(k.grad, dk) and torch.equal(v.grad, dv)


def test_autograd_dropout_draws_a_fresh_seed_per_call():
    """flash_attention with dropout and no seed: two calls draw different
    seeds (different keep masks, so different outputs), each seed is kept on
    the autograd node, and the gradients equal fa.backward run with that
    seed; under torch.manual_seed the draws repeat."""
    w = _case(5, B=1, H=2, N=200)
    inp = make_inputs(w, with_grad=True)
    dev, _ = device_inputs(inp, w.dtype)
    runs = []
    for _ in range(2):
        q, k, v = (dev[n].clone().requires_grad_(True) for n in ("q", "k", "v"))
        o = fa.flash_attention(q, k, v, causal=True, dropout_p=0.1)
        o.backward(dev["do"])
        runs.append((o.grad_fn.seed, o.detach(), q.grad, k.grad, v.grad))
    (s1, o1, *g1), (s2, o2, *_) = runs
    assert s1 != s2
    assert not torch.equal(o1, o2)
    m1 = fa.dropout_mask(s1, 0, 0, 2, 0.1, 0, 0, 200, 200)
    m2 = fa.dropout_mask(s2, 0, 0, 2, 0.1, 0, 0, 200, 200)
    assert not torch.equal(m1, m2)
    o_ref, lse = fa.forward(dev["q"], dev["k"], dev["v"], True, 0.1, s1)
    g_ref = fa.backward(dev["q"], dev["k"], dev["v"], o_ref, dev["do"], lse, True, 0.1, s1)
    torch.cuda.synchronize()
    assert torch.equal(o1, o_ref)
    for a, b in zip(g1, g_ref):
        assert torch.equal(a, b)
    torch.manual_seed(7)
    a = fa.draw_seed()
    torch.manual_seed(7)
    assert fa.draw_seed() == a


@pytest.mark.parametrize("causal", [True, False])
def test_zero_query_closed_form(causal):
    """Q = 0 gives uniform attention: O_i is the mean of the visible V rows and
    LSE_i = ln(number of visible keys), at a length spanning many tiles."""
    N, d = 3000, 80
    rng = np.random.default_rng(9)
    v = rng.standard_normal((1, N, 2, d), dtype=np.float32)
    k = rng.standard_normal((1, N, 2, d), dtype=np.float32)
    tq = torch.zeros((1, N, 2, d), dtype=torch.bfloat16, device="cuda")
    tk, tv = to_device(k, "f32").bfloat16(), to_device(v, "f32").bfloat16()
    o, lse = fa.forward(tq, tk, tv, causal, 0.0, 0, 1.0 / np.sqrt(d))
    vv = to_host(tv)
    cnt = np.arange(1, N + 1) if causal else np.full(N, N)
    exp_o = (np.cumsum(vv, axis=1) / cnt[None, :, None, None]) if causal else \
        np.broadcast_to(vv.mean(axis=1, keepdims=True), vv.shape)
    assert_close("O", to_host(o), exp_o, "bf16")
    assert_close("LSE", to_host(lse), np.broadcast_to(np.log(cnt), (1, 2, N)), "bf16")
