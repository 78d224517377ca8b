"""GPU parity on seeded random small problems: batch, heads, length, head
dim, mask, dropout and dtype drawn together (numpy Generator seeded 4242),
forward and backward through the C ABI against the fp64 oracle. Lengths
cover single rows, tile-straddling tails and several work-groups.

At one or two keys an output row is a (rescaled) V or dO row rather than an
average, so values reach 3 to 5 and bf16 storage alone misses the exact
value by a mean of up to 1.5e-3 (N = 2, dropout 0.3: measured on the
oracle's values). bf16 results are therefore held to the plain bar above
that storage floor: each element to 2e-2 * max(1, |ref|), the mean to 1e-3
plus the mean |bf16(ref) - ref| of the same tensor. LSE (stored in fp32)
and fp32 results keep the plain bar.

The backward takes D = rowsum(dO * O) from the stored O, so at these
lengths O's storage rounding also moves dQ and dK (a one-key row has
dQ = 0 exactly, and D's error times K otherwise). The backward is
therefore handed the oracle's own O and LSE in their storage types, and
the oracle's backward reads D from that same O (its `o` argument)."""
import numpy as np
import pytest

import oracle
from helpers import assert_close, device_inputs, to_host
from workloads import WORKLOADS, make_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import exact_io_aware_72_amd as fa  # noqa: E402


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _check(name, got, ref, dtype):
    if dtype != "bf16":
        assert_close(name, got, ref, dtype)
        return
    stored = torch.from_numpy(np.asarray(ref)).to(torch.bfloat16).double().numpy()
    floor = float(np.abs(stored - ref).mean()) if ref.size else 0.0
    assert_close(name, got, ref, dtype, tol=(2e-2, 1e-3 + floor), scaled=True)


def _cases(n=24, seed=4242):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype = "f32" if rng.random() < 0.2 else "bf16"
        d = int(rng.choice([64, 80, 128]))
        N = int(rng.choice([1, 2, 31, 33, 63, 65, 127, 129, 255, 257, 300, 511, 513, 700]))
        B = int(rng.integers(1, 4))
        H = int(rng.integers(1, 6))
        causal = bool(rng.random() < 0.6)
        p = float(rng.choice([0.0, 0.0, 0.1, 0.3]))
        base = 1 if dtype == "f32" else 3
        out.append(WORKLOADS[base].with_(B=B, H=H, N=N, d=d, causal=causal, dropout_p=p,
                                         dropout_seed=1000 + i, backward=True))
    return out


CASES = _cases()


@pytest.mark.parametrize("w", CASES, ids=[f"{i}-{w.dtype}-d{w.d}-N{w.N}-B{w.B}H{w.H}-{'c' if w.causal else 'f'}-p{w.dropout_p}"
                                          for i, w in enumerate(CASES)])
def test_random_problem_matches_oracle(w):
    inp = make_inputs(w, with_grad=True)
    dev, val = device_inputs(inp, w.dtype)
    args = (w.causal, w.dropout_p, w.dropout_seed, w.scale)
    o, lse = fa.forward(dev["q"], dev["k"], dev["v"], *args)
    torch.cuda.synchronize()
    o_r, lse_r = oracle.forward(val["q"], val["k"], val["v"], w.scale, w.causal, w.dropout_p,
                                w.dropout_seed)
    _check("O", to_host(o), o_r, w.dtype)
    assert_close("LSE", to_host(lse), lse_r, w.dtype)  # stored in fp32

    # The backward reads D = rowsum(dO * O) from the O it is handed. Both
    # sides get the oracle's O and LSE as stored (O in the input type).
    o_st = torch.from_numpy(o_r).to(dev["q"].dtype).cuda()
    lse_st = torch.from_numpy(lse_r).to(torch.float32).cuda()
    dq, dk, dv = fa.backward(dev["q"], dev["k"], dev["v"], o_st, dev["do"], lse_st, *args)
    torch.cuda.synchronize()
    dq_r, dk_r, dv_r, _ = oracle.backward(val["q"], val["k"], val["v"], val["do"], w.scale, w.causal,
                                          w.dropout_p, w.dropout_seed, o=to_host(o_st))
    _check("dQ", to_host(dq), dq_r, w.dtype)
    _check("dK", to_host(dk), dk_r, w.dtype)
    _check("dV", to_host(dv), dv_r, w.dtype)


def _large_amplitude_cases(n=8, seed=4343):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        out.append(WORKLOADS[3].with_(B=int(rng.integers(1, 3)), H=int(rng.integers(1, 4)),
                                      N=int(rng.choice([1, 2, 65, 127, 129, 300, 513, 700])),
                                      d=int(rng.choice([64, 80, 128])), causal=bool(rng.random() < 0.6),
                                      dropout_p=float(rng.choice([0.0, 0.1])), dropout_seed=2000 + i, amp=8.0))
    return out


LARGE = _large_amplitude_cases()


@pytest.mark.parametrize("w", LARGE, ids=[f"{i}-d{w.d}-N{w.N}-B{w.B}H{w.H}-{'c' if w.causal else 'f'}-p{w.dropout_p}"
                                          for i, w in enumerate(LARGE)])
def test_large_amplitude_forward_matches_oracle(w):
    """Q, K, V at 8 N(0, 1): nearly one-hot rows and V entries up to 30. The
    kernel rounds P to bf16 before P V, so O's error scales with
    m_i = sum_j P~_ij |V_j| (the oracle's forward with |V|), not with |O_i|,
    which can be a small difference of large terms; O is held to
    2e-2 * max(1, m) and a mean of 1e-3 * mean(max(1, m)) plus the measured
    storage floor (the bound is pinned on an emulation of the two bf16
    roundings in test_oracle_fp8.py). LSE (fp32, logits of several hundred)
    takes the plain bar scaled by magnitude above 1."""
    inp = make_inputs(w, with_grad=False)
    dev, val = device_inputs(inp, w.dtype)
    args = (w.causal, w.dropout_p, w.dropout_seed, w.scale)
    o, lse = fa.forward(dev["q"], dev["k"], dev["v"], *args)
    torch.cuda.synchronize()
    o_r, lse_r = oracle.forward(val["q"], val["k"], val["v"], w.scale, w.causal, w.dropout_p, w.dropout_seed)
    mag = np.maximum(1.0, oracle.forward(val["q"], val["k"], np.abs(val["v"]), w.scale, w.causal, w.dropout_p,
                                         w.dropout_seed)[0])
    floor = float(np.abs(torch.from_numpy(o_r).to(torch.bfloat16).double().numpy() - o_r).mean())
    err = np.abs(to_host(o) - o_r)
    worst = float(np.max(err / (2e-2 * mag)))
    assert worst <= 1.0, f"O: max|err|/bound={worst:.3f} (max|err|={err.max():.3e})"
    assert err.mean() <= 1e-3 * mag.mean() + floor, f"O: mean|err|={err.mean():.3e}"
    assert_close("LSE", to_host(lse), lse_r, w.dtype, scaled=True)
