"""Full-size workloads on the GPU, in the launch configuration the benchmark
times: sampled outputs against stored oracle values (tests/golden, written by
make_golden.py from the oracle alone), properties that hold at any size, and
the absence of any N x N buffer."""
import hashlib
import os

import numpy as np
import pytest

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
    # each stored value carries up to 2^-9 relative rounding; errors add like a random walk
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
