"""GPU parity for the FP8-score forward: the quantisation kernel's E4M3 codes
and block scales bit for bit against the oracle's fp32 rule, and the forward
against the fp64 oracle on the same quantised inputs (bf16 bar), causal and
full, with ragged tails, for head dims 64, 80 (rows padded to 128 bytes in
LDS) and 128; the full-size N=8192 shape at sampled rows."""
import numpy as np
import pytest

import oracle
from oracle import fp8 as OF
from helpers import assert_close, to_device, to_host
from workloads import WORKLOADS, Workload, make_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import exact_io_aware_72_amd as fa  # noqa: E402


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _decode_table():
    """E4M3 code -> value from the bit layout (bias 7, 3 mantissa bits)."""
    t = np.full(256, np.nan)
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            continue
        x = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
        t[c] = -x if s else x
    return t


@pytest.mark.parametrize("d", [64, 80, 128])
@pytest.mark.parametrize("block_rows", [128, 64])
@pytest.mark.parametrize("amp", [1.0, 1e-3, 300.0])
def test_quantize_matches_oracle_bitwise(d, block_rows, amp):
    w = Workload(60, "q8", 2, 3, 300, d, "bf16", False, 0.0, False, amp=amp)
    inp = make_inputs(w, with_grad=False)
    stored, vals = inp["q"]
    vals = vals.copy()
    vals[1, 128:256, 2] = 0.0  # an all-zero block (128-row) / two (64-row)
    stored = stored.copy()
    stored[1, 128:256, 2] = 0
    x = to_device(stored, "bf16")
    xq, sc = fa.quantize_fp8(x, block_rows)
    torch.cuda.synchronize()
    codes, scales = OF.quantize(vals, block_rows)
    got = _decode_table()[xq.cpu().numpy()]
    np.testing.assert_array_equal(got, codes)
    np.testing.assert_array_equal(sc.cpu().numpy(), scales)


CASES = [(1, 2, 300, True, 128), (2, 1, 77, False, 128), (1, 3, 1000, True, 128),
         (1, 1, 1, True, 128), (1, 2, 513, False, 128), (2, 2, 130, True, 128),
         (1, 2, 300, True, 64), (2, 1, 257, False, 64), (1, 2, 700, True, 80),
         (1, 1, 129, False, 80), (1, 1, 1, True, 80)]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}H{c[1]}N{c[2]}-{'causal' if c[3] else 'full'}-d{c[4]}"
                                             for c in CASES])
def test_forward_fp8_matches_oracle(case):
    B, H, N, causal, d = case
    w = Workload(61, "f8", B, H, N, d, "bf16", causal, 0.0, False)
    inp = make_inputs(w, with_grad=False)
    dev = {k: to_device(v[0], "bf16") for k, v in inp.items()}
    o, lse = fa.forward_fp8(dev["q"], dev["k"], dev["v"], causal, w.scale)
    torch.cuda.synchronize()
    o_r, lse_r = OF.forward_fp8(inp["q"][1], inp["k"][1], inp["v"][1], w.scale, causal)
    assert_close("O", to_host(o), o_r, "bf16")
    assert_close("LSE", to_host(lse), lse_r, "bf16")


def test_forward_fp8_full_size_sampled():
    """The N=8192 causal shape of the headline workload with FP8 scores, in
    the launch configuration the benchmark times, at sampled rows of two
    heads against the oracle on the same quantised inputs."""
    w = WORKLOADS[3]
    inp = make_inputs(w, with_grad=False)
    dev = {k: to_device(v[0], "bf16") for k, v in inp.items()}
    o, lse = fa.forward_fp8(dev["q"], dev["k"], dev["v"], True, w.scale)
    torch.cuda.synchronize()
    cq, sq = OF.quantize(inp["q"][1], OF.Q_BLOCK)
    ck, sk = OF.quantize(inp["k"][1], OF.K_BLOCK)
    qd, kd = OF.dequantize(cq, sq, OF.Q_BLOCK), OF.dequantize(ck, sk, OF.K_BLOCK)
    rows = np.unique(np.r_[0, 1, 127, 128, 4095, 4096, 8190, 8191,
                           np.random.default_rng(4).integers(0, w.N, 12)])
    for b, h in ((0, 0), (1, 15)):
        ref = oracle.sampled_head(qd, kd, inp["v"][1], None, w.scale, True, 0.0, 0, b, h, rows,
                                  rows)
        assert_close(f"O[{b},{h}]", to_host(o[b, torch.from_numpy(rows).cuda(), h]), ref["o"], "bf16")
        assert_close(f"LSE[{b},{h}]", to_host(lse[b, h, torch.from_numpy(rows).cuda()]), ref["lse"],
                     "bf16")
