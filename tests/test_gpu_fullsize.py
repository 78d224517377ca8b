"""Full-size workloads on the GPU, in the launch configuration the benchmark
times: sampled outputs against stored oracle values (tests/golden, written by
make_golden.py from the oracle alone), properties that hold at any size, and
the absence of any N x N buffer."""
import hashlib
import os

import numpy as np
import pytest

import oracle
from helpers import assert_close, to_device, to_host
from workloads import WORKLOADS, make_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import exact_io_aware_72_amd as fa  # noqa: E402

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.empty_cache()


def _full(cfg):
    w = WORKLOADS[cfg]
    inp = make_inputs(w)
    dev = {k: to_device(v[0], w.dtype) for k, v in inp.items()}
    return w, inp, dev


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_full_size_sampled_parity(cfg):
    path = os.path.join(GOLDEN, f"sampled_cfg{cfg}.npz")
    if not os.path.exists(path):
        pytest.skip(f"{path} missing")
    g = np.load(path)
    w, inp, dev = _full(cfg)
    for name, v in inp.items():
        digest = hashlib.sha256(np.ascontiguousarray(v[0]).tobytes()).hexdigest()
        assert digest == str(g[f"sha256_{name}"]), f"input {name} differs from the stored recipe"
    print(f"config {cfg}: {w.name}", flush=True)
    o, lse = fa.forward(dev["q"], dev["k"], dev["v"], w.causal, w.dropout_p, w.dropout_seed, w.scale)
    grads = None
    if w.backward:
        grads = fa.backward(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, w.causal, w.dropout_p,
                            w.dropout_seed, w.scale)
    torch.cuda.synchronize()
    rows = torch.from_numpy(g["rows"]).cuda()
    cols = torch.from_numpy(g["cols"]).cuda()
    for hi, (b, h) in enumerate(g["heads"]):
        assert_close(f"O[{b},{h}]", to_host(o[b, rows, h]), g[f"h{hi}_o"], w.dtype)
        assert_close(f"LSE[{b},{h}]", to_host(lse[b, h, rows]), g[f"h{hi}_lse"], w.dtype)
        if grads is not None:
            dq, dk, dv = grads
            assert_close(f"dQ[{b},{h}]", to_host(dq[b, rows, h]), g[f"h{hi}_dq"], w.dtype)
            assert_close(f"dK[{b},{h}]", to_host(dk[b, cols, h]), g[f"h{hi}_dk"], w.dtype)
            assert_close(f"dV[{b},{h}]", to_host(dv[b, cols, h]), g[f"h{hi}_dv"], w.dtype)


def test_full_size_forward_whole_tensor_n2048():
    """The B = 4, H = 16, N = 2048, d = 64 causal forward, whole: every row of
    O and LSE of all 64 heads from the full-size launch against the oracle,
    element by element, the mean bar taken over the whole tensor."""
    w = WORKLOADS[2]
    inp = make_inputs(w)
    dev = {k: to_device(v[0], w.dtype) for k, v in inp.items()}
    print(f"config 2: {w.name}", flush=True)
    o, lse = fa.forward(dev["q"], dev["k"], dev["v"], w.causal, w.dropout_p, w.dropout_seed, w.scale)
    torch.cuda.synchronize()
    val = {k: v[1] for k, v in inp.items()}
    ro, rl = oracle.forward(val["q"], val["k"], val["v"], w.scale, w.causal, w.dropout_p, w.dropout_seed)
    assert_close("O", to_host(o), ro, w.dtype)
    assert_close("LSE", to_host(lse), rl, w.dtype)


@pytest.mark.parametrize("cfg,heads", [(3, [(0, 0), (1, 15)]), (4, [(0, 0), (0, 9)]), (5, [(0, 3)])])
def test_full_size_whole_heads(cfg, heads):
    """Whole heads of the N = 8192 (d = 128), N = 32768 (d = 80) and
    N = 65536 (dropout 0.1) workloads, element by element at the bar: every
    row of O, LSE and dQ and every key row of dK and dV, from the full-size
    launches, against the oracle run on those heads (a few seconds per head
    at N = 8192, about 10 s at N = 32768 and 50 s at N = 65536 on 16 host
    cores)."""
    w = WORKLOADS[cfg]
    inp = make_inputs(w, with_grad=True)
    dev = {k: to_device(v[0], w.dtype) for k, v in inp.items()}
    print(f"config {cfg}: {w.name}, heads {heads}", flush=True)
    args = (w.causal, w.dropout_p, w.dropout_seed, w.scale)
    o, lse = fa.forward(dev["q"], dev["k"], dev["v"], *args)
    dq, dk, dv = fa.backward(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, *args)
    torch.cuda.synchronize()
    got = {(b, h): {"O": to_host(o[b, :, h]), "LSE": to_host(lse[b, h]), "dQ": to_host(dq[b, :, h]),
                    "dK": to_host(dk[b, :, h]), "dV": to_host(dv[b, :, h])} for b, h in heads}
    del dev, o, lse, dq, dk, dv
    torch.cuda.empty_cache()
    val = {k: v[1] for k, v in inp.items()}
    for b, h in heads:
        ro, rl = oracle.forward(val["q"], val["k"], val["v"], w.scale, w.causal, w.dropout_p,
                                w.dropout_seed, heads=[(b, h)])
        rq, rk, rv, _ = oracle.backward(val["q"], val["k"], val["v"], val["do"], w.scale, w.causal,
                                        w.dropout_p, w.dropout_seed, heads=[(b, h)], check_d=False)
        ref = {"O": ro[b, :, h], "LSE": rl[b, h], "dQ": rq[b, :, h], "dK": rk[b, :, h], "dV": rv[b, :, h]}
        for name, r in ref.items():
            assert_close(f"{name}[{b},{h}]", got[(b, h)][name], r, w.dtype)
        print(f"  head ({b},{h}) ok", flush=True)


@pytest.mark.parametrize("d,causal,N", [(80, False, 32768), (64, True, 32768), (64, True, 32800)])
def test_long_sequence_wide_groups(d, causal, N):
    """N = 32768 runs the sixteen-wave forward groups (head dims up to 80, no
    dropout) and the eight-wave dQ groups; causal ones pair their blocks
    per work-group. Shapes the workloads do not cover (full mask at d = 80,
    causal at d = 64, and N = 32800: odd block counts, 65 forward and 129
    dQ blocks, with a ragged last block), at sampled rows and columns of one
    head against the oracle."""
    w = WORKLOADS[4].with_(H=2, d=d, causal=causal, N=N)
    inp = make_inputs(w, with_grad=True)
    dev = {k: to_device(v[0], w.dtype) for k, v in inp.items()}
    print(f"N={N} d={d} causal={causal}", flush=True)
    args = (w.causal, 0.0, 0, w.scale)
    o, lse = fa.forward(dev["q"], dev["k"], dev["v"], *args)
    dq, dk, dv = fa.backward(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, *args)
    torch.cuda.synchronize()
    N = w.N
    rng = np.random.default_rng(77)
    rows = np.unique(np.concatenate([[0, 255, 256, 511, 512, N // 2, N - 513, N - 512, N - 1],
                                     rng.choice(N, 7, replace=False)]))
    cols = np.unique(np.concatenate([[0, 1, 32767 - 300, N - 1], rng.choice(N, 6, replace=False)]))
    b, h = 0, 1
    val = {k: v[1] for k, v in inp.items()}
    ref = oracle.sampled_head(val["q"], val["k"], val["v"], val["do"], w.scale, w.causal, 0.0, 0,
                              b, h, rows, cols)
    r_t, c_t = torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()
    assert_close("O", to_host(o[b, r_t, h]), ref["o"], w.dtype)
    assert_close("LSE", to_host(lse[b, h, r_t]), ref["lse"], w.dtype)
    assert_close("dQ", to_host(dq[b, r_t, h]), ref["dq"], w.dtype)
    assert_close("dK", to_host(dk[b, c_t, h]), ref["dk"], w.dtype)
    assert_close("dV", to_host(dv[b, c_t, h]), ref["dv"], w.dtype)


@pytest.mark.parametrize("cfg", [3, 4])
def test_full_size_gradient_invariants(cfg):
    """Rows of dS sum to zero, so sum_j dK_j = 0; rows of P sum to one, so
    sum_j dV_j = sum_i dO_i (no dropout). Checked per (b, h) and column, with
    a bound from bf16 rounding of the stored gradients."""
    w, _, dev = _full(cfg)
    o, lse = fa.forward(dev["q"], dev["k"], dev["v"], w.causal, 0.0, 0, w.scale)
    dq, dk, dv = fa.backward(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, w.causal, 0.0, 0, w.scale)
    torch.cuda.synchronize()
    dk64, dv64, do64 = (x.to(torch.float64) for x in (dk, dv, dev["do"]))
    # each stored value is off by up to 2^-8 of itself (bf16's unit roundoff, far less on
    # average); errors add like a random walk, and 8 * 2^-9 * root-sum-square is several sigma
    for name, s, ref, mag in (
        ("sum dK", dk64.sum(dim=1), torch.zeros_like(dk64.sum(dim=1)), dk64.pow(2).sum(dim=1).sqrt()),
        ("sum dV", dv64.sum(dim=1), do64.sum(dim=1), dv64.pow(2).sum(dim=1).sqrt()),
    ):
        err = (s - ref).abs()
        bound = 8 * 2.0 ** -9 * mag + 1e-3
        assert bool((err <= bound).all()), f"{name}: worst excess {(err - bound).max().item():.3e}"


def test_no_quadratic_memory():
    """Forward + backward at N = 32768 allocate nothing beyond the inputs,
    outputs, logsumexp and the D workspace (one N x N bf16 matrix of one head
    would be 2 GiB)."""
    w, _, dev = _full(4)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    before = torch.cuda.memory_allocated()
    o, lse = fa.forward(dev["q"], dev["k"], dev["v"], True, 0.0, 0, w.scale)
    g = fa.backward(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, True, 0.0, 0, w.scale)
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - before
    tensor = dev["q"].numel() * 2
    stats = w.B * w.H * w.N * 4
    expected = 4 * tensor + 2 * stats  # o, dq, dk, dv + lse + workspace
    assert peak <= expected + (8 << 20), (peak, expected)
    del g


def test_full_size_deterministic():
    w, _, dev = _full(3)
    res = []
    for _ in range(2):
        o, lse = fa.forward(dev["q"], dev["k"], dev["v"], True, 0.0, 0, w.scale)
        dq, dk, dv = fa.backward(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, True, 0.0, 0, w.scale)
        torch.cuda.synchronize()
        res.append((o, lse, dq, dk, dv))
    for a, b in zip(*res):
        assert torch.equal(a, b)
