"""The largest batch item the kernels address with 32-bit byte offsets: B=1,
H=64, N=131071, d=128 bf16 (N*H*d*2 = 2^31 - 16384 bytes per tensor item;
one more row is rejected at the boundary). Causal forward and backward on
the GPU; O, LSE and dQ checked at sampled rows (the last row included)
against the oracle's formulas on those rows, dK and dV through the exact
column-sum identities."""
import numpy as np
import pytest

from helpers import assert_close
from oracle import attention as A
from workloads import device_normal

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import exact_io_aware_72_amd as fa  # noqa: E402

B, H, N, D = 1, 64, 131071, 128


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.empty_cache()


def test_largest_item_sampled_rows_and_invariants():
    assert N * H * D * 2 < 2 ** 31 <= (N + 1) * H * D * 2
    scale = float(np.float32(1.0 / np.sqrt(D)))
    q, k, v, do = (device_normal((B, N, H, D), 7100 + i) for i in range(4))
    print(f"max-size item: B={B} H={H} N={N} d={D}", flush=True)
    o, lse = fa.forward(q, k, v, True, 0.0, 0, scale)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, True, 0.0, 0, scale)
    torch.cuda.synchronize()
    rows = np.unique(np.r_[0, 1, 127, 128, 65535, 65536, N - 129, N - 2, N - 1,
                           np.random.default_rng(9).integers(0, N, 6)])
    for h in (0, H - 1):
        qh, kh, vh, doh = (x[0, :, h].to(torch.float64).cpu().numpy() for x in (q, k, v, do))
        o_r, l_r, dq_r = [], [], []
        for r in rows:
            s = A.attention_scores(qh[r:r + 1], kh[:r + 1], scale, True, r)
            _, _, l_ = A.softmax_stats(s)
            p = A.attention_probs(s, l_)
            o_row = p @ vh[:r + 1]
            d_row = np.sum(doh[r] * o_row[0])
            dp = doh[r:r + 1] @ vh[:r + 1].T
            dq_r.append((scale * (p * (dp - d_row)) @ kh[:r + 1])[0])
            o_r.append(o_row[0])
            l_r.append(l_[0])
        idx = torch.from_numpy(rows).cuda()
        assert_close(f"O[h={h}]", o[0, idx, h].double().cpu().numpy(), np.array(o_r), "bf16")
        assert_close(f"LSE[h={h}]", lse[0, h, idx].double().cpu().numpy(), np.array(l_r), "bf16")
        assert_close(f"dQ[h={h}]", dq[0, idx, h].double().cpu().numpy(), np.array(dq_r), "bf16")
    # sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i per (h, column), within the
    # random-walk bound of bf16 storage (each value carries 2^-9 relative).
    for name, x, ref in (("sum dK", dk, None), ("sum dV", dv, do)):
        x64 = x[0].to(torch.float64)
        s = x64.sum(dim=0)
        r = torch.zeros_like(s) if ref is None else ref[0].to(torch.float64).sum(dim=0)
        bound = 8 * 2.0 ** -9 * x64.pow(2).sum(dim=0).sqrt() + 1e-3
        err = (s - r).abs()
        assert bool((err <= bound).all()), f"{name}: worst excess {(err - bound).max().item():.3e}"
        del x64
