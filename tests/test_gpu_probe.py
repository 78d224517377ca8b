"""The matrix-core rate probe (fa_probe_mfma_rate) runs the products it
claims: the sum over a wave's lanes of its output equals iters times the sum
of all elements of the 16 products, which for X as the A operand and Y as the
B operand of a 32x32x16 product is sum_k colsum(X)[k] * rowsum(Y)[k]."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import exact_io_aware_72_amd as fa  # noqa: E402


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _bf16(x32):
    """fp32 -> bf16 bits (round to nearest even) and the bf16 values as fp64."""
    u = x32.astype(np.float32).view(np.uint32)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return r, (r.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _k_sums(frag):
    """frag: [64 lanes, 8] values of one fragment. As the A operand lane L
    holds row L % 32, columns 8 (L / 32) + j; as the B operand column L % 32,
    rows 8 (L / 32) + j; either way the sum over the 32-long index for
    contraction index k = 8 h + j is the sum over lanes 32 h .. 32 h + 31."""
    return np.concatenate([frag[:32].sum(axis=0), frag[32:].sum(axis=0)])


def _expected_wave_sum(vals, iters):
    f = vals.reshape(16, 64, 8)
    a, b = f[:8], f[8:]
    tot, mag = 0.0, 0.0
    for i in range(8):
        for x, y in ((a[i], b[i]), (b[i], a[(i + 1) % 8])):
            t = _k_sums(x) * _k_sums(y)
            tot += t.sum()
            mag += np.abs(t).sum()
    return iters * tot, iters * mag


@pytest.mark.parametrize("kind", ["random", "ones"])
def test_probe_sums(kind):
    rng = np.random.default_rng(7)
    x = rng.standard_normal(16 * 64 * 8).astype(np.float32) if kind == "random" \
        else np.ones(16 * 64 * 8, np.float32)
    bits, vals = _bf16(x)
    ops = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    blocks, iters = 3, 5
    out = fa.probe_mfma_rate(ops, blocks, iters)
    torch.cuda.synchronize()
    per_wave = out.double().cpu().numpy().reshape(blocks * 4, 64).sum(axis=1)
    want, mag = _expected_wave_sum(vals, iters)
    if kind == "ones":
        assert want == iters * 16 * 32 * 32 * 16
        np.testing.assert_array_equal(per_wave, want)
    else:
        assert np.all(np.abs(per_wave - want) <= 1e-5 * mag + 1e-3)
