"""The library launches kernels on the caller's stream and never allocates,
frees or synchronises, so a forward + backward step can be captured in a HIP
graph. Captured steps (with fa_backward and with fa_backward_noalloc) are
replayed several times, with eager work and synchronisations between the
replays, and every replay must equal the eager step bit for bit."""
import pytest

from helpers import device_inputs
from workloads import WORKLOADS, make_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import exact_io_aware_72_amd as fa  # noqa: E402


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


CASES = [
    WORKLOADS[3].with_(B=2, H=4, N=1000),
    WORKLOADS[5].with_(B=1, H=3, N=777),
    WORKLOADS[4].with_(B=1, H=2, N=513, causal=False),
]


@pytest.mark.parametrize("noalloc", [False, True])
@pytest.mark.parametrize("w", CASES, ids=[f"d{w.d}-N{w.N}-p{w.dropout_p}-{'causal' if w.causal else 'full'}"
                                          for w in CASES])
def test_captured_step_replays_equal_eager(w, noalloc):
    inp = make_inputs(w, with_grad=True)
    dev, _ = device_inputs(inp, w.dtype)
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    args = (w.causal, w.dropout_p, w.dropout_seed, w.scale)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")

    def step():
        fa.forward(q, k, v, *args, out=o, lse=lse)
        if noalloc:
            fa.backward_noalloc(q, k, v, o, do, lse, dq, dk, dv, *args)
        else:
            fa.backward(q, k, v, o, do, lse, *args, dq=dq, dk=dk, dv=dv, workspace=ws)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (o, lse, dq, dk, dv)]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (o, lse, dq, dk, dv):
            t.fill_(float("nan"))  # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, exp in zip(("O", "LSE", "dQ", "dK", "dV"), (o, lse, dq, dk, dv), ref):
            assert torch.equal(got, exp), f"replay {rep}: {name} differs from the eager step"
