"""Batch items above 4 GiB: the kernels read rows through buffer resources
based at each block, tile or window start, so no byte offset spans a whole
item. bf16 B=1, H=256, N=66001, d=128 (N*H*d*2 = 4.33e9 bytes per tensor
item, past 2^32): causal forward and backward, O, LSE and dQ checked at
sampled rows (the last row and rows past 2^32 / (H*d*2) = 65536 included)
against the oracle's formulas on those rows, dK and dV through the exact
column-sum identities. fp32 B=1, H=256, N=33001, d=128 (4.33e9 bytes;
the fp32 forward's K/V windows hold 4096 rows at this row size): causal
forward at sampled rows."""
import numpy as np
import pytest

from helpers import assert_close
import oracle
from workloads import device_normal

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import exact_io_aware_72_amd as fa  # noqa: E402


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.empty_cache()


def _rows_reference(q, k, v, do, h, rows, scale):
    """O, LSE and (with do) dQ of the given causal rows of head h: each row
    alone through the oracle (query at key position r, keys 0..r), which is
    exact because a causal row's softmax, O, D and dQ involve only its own
    row of S."""
    qh, kh, vh = (x[0, :, h] for x in (q, k, v))
    H = q.shape[2]
    o_r, l_r, dq_r = [], [], []
    for r in (int(x) for x in rows):
        qr = qh[r:r + 1].to(torch.float64).cpu().numpy()
        kr = kh[:r + 1].to(torch.float64).cpu().numpy()
        vr = vh[:r + 1].to(torch.float64).cpu().numpy()
        o_, l_ = oracle.head_forward(qr, kr, vr, scale, True, 0.0, 0, 0, h, H, row_offset=r, hash_row_offset=r)
        o_r.append(o_[0])
        l_r.append(l_[0])
        if do is not None:
            dor = do[0, r:r + 1, h].to(torch.float64).cpu().numpy()
            dq_, _, _, _ = oracle.head_backward(qr, kr, vr, dor, scale, True, 0.0, 0, 0, h, H,
                                                row_offset=r, hash_row_offset=r)
            dq_r.append(dq_[0])
    return np.array(o_r), np.array(l_r), (np.array(dq_r) if do is not None else None)


def test_bf16_item_over_4gib_sampled_rows_and_invariants():
    B, H, N, D = 1, 256, 66001, 128
    assert N * H * D * 2 > 2 ** 32
    scale = float(np.float32(1.0 / np.sqrt(D)))
    q, k, v, do = (device_normal((B, N, H, D), 7100 + i) for i in range(4))
    print(f"bf16 item over 4 GiB: B={B} H={H} N={N} d={D}", flush=True)
    o, lse = fa.forward(q, k, v, True, 0.0, 0, scale)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, True, 0.0, 0, scale)
    torch.cuda.synchronize()
    rows = np.unique(np.r_[0, 1, 127, 128, 32767, 32768, 65535, 65536, 65537,
                           N - 129, N - 2, N - 1, np.random.default_rng(9).integers(0, N, 6)])
    idx = torch.from_numpy(rows).cuda()
    for h in (0, H - 1):
        o_r, l_r, dq_r = _rows_reference(q, k, v, do, h, rows, scale)
        assert_close(f"O[h={h}]", o[0, idx, h].double().cpu().numpy(), o_r, "bf16")
        assert_close(f"LSE[h={h}]", lse[0, h, idx].double().cpu().numpy(), l_r, "bf16")
        assert_close(f"dQ[h={h}]", dq[0, idx, h].double().cpu().numpy(), dq_r, "bf16")
    # sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i per (h, column), within the
    # random-walk bound of bf16 storage (each value is off by up to 2^-8 of
    # itself, far less on average; 8 * 2^-9 * root-sum-square is several sigma).
    for name, x, ref in (("sum dK", dk, None), ("sum dV", dv, do)):
        x64 = x[0].to(torch.float64)
        s = x64.sum(dim=0)
        r = torch.zeros_like(s) if ref is None else ref[0].to(torch.float64).sum(dim=0)
        bound = 8 * 2.0 ** -9 * x64.pow(2).sum(dim=0).sqrt() + 1e-3
        err = (s - r).abs()
        assert bool((err <= bound).all()), f"{name}: worst excess {(err - bound).max().item():.3e}"
        del x64


def test_f32_item_over_4gib_sampled_rows():
    B, H, N, D = 1, 256, 33001, 128
    assert N * H * D * 4 > 2 ** 32
    scale = float(np.float32(1.0 / np.sqrt(D)))
    q, k, v = (device_normal((B, N, H, D), 7200 + i, dtype="f32") for i in range(3))
    print(f"fp32 item over 4 GiB: B={B} H={H} N={N} d={D}", flush=True)
    o, lse = fa.forward(q, k, v, True, 0.0, 0, scale)
    torch.cuda.synchronize()
    rows = np.unique(np.r_[0, 31, 32, 4095, 4096, 16383, 16384, 32767, 32768, N - 33, N - 2, N - 1,
                           np.random.default_rng(10).integers(0, N, 5)])
    idx = torch.from_numpy(rows).cuda()
    for h in (0, H - 1):
        o_r, l_r, _ = _rows_reference(q, k, v, None, h, rows, scale)
        assert_close(f"O[h={h}]", o[0, idx, h].double().cpu().numpy(), o_r, "f32")
        assert_close(f"LSE[h={h}]", lse[0, h, idx].double().cpu().numpy(), l_r, "f32")
