"""fa_backward_noalloc (the backward pass with D in the library's fixed
device array) against fa_backward on the same inputs, through the C ABI: two
calls in a row, the second with a smaller input, each bitwise equal to
fa_backward's gradients (same kernels, same D) and within the bf16 bar of
the oracle."""
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


def _check(w):
    inp = make_inputs(w, with_grad=True)
    dev, val = device_inputs(inp, w.dtype)
    args = (w.causal, w.dropout_p, w.dropout_seed, w.scale)
    o, lse = fa.forward(dev["q"], dev["k"], dev["v"], *args)
    ref = fa.backward(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, *args)
    # outputs pre-filled with garbage: every element must be overwritten
    got = [torch.full_like(dev["q"], 7.0) for _ in range(3)]
    fa.backward_noalloc(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, *got, *args)
    torch.cuda.synchronize()
    for a, b in zip(got, ref):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    g_ref = oracle.backward(val["q"], val["k"], val["v"], val["do"], w.scale, w.causal,
                            w.dropout_p, w.dropout_seed)[:3]
    for name, a, b in zip(("dQ", "dK", "dV"), got, g_ref):
        assert_close(name, to_host(a), b, w.dtype)


def test_noalloc_matches_backward_on_two_calls():
    # larger first, then smaller: the second call reuses the array the first
    # one filled beyond its own extent
    _check(WORKLOADS[3].with_(B=2, H=4, N=1000))
    _check(WORKLOADS[5].with_(B=1, H=2, N=300, d=64))


def test_noalloc_rejects_oversize_before_launch():
    q = torch.zeros((1, 1, 1, 64), dtype=torch.bfloat16, device="cuda")
    L = fa.lib()
    P = q.data_ptr()
    st = L.fa_backward_noalloc(P, P, P, P, P, P, P, P, P, 1, 64, (1 << 16) + 1, 128, 0.1, 1, 0.0,
                               0, None, 1)
    assert st == -2  # FA_ERR_SHAPE: B * H * N above FA_NOALLOC_MAX_ROWS
