"""GPU parity on seeded random packed batches (numpy Generator seeded 5151):
one to six sequences whose lengths are drawn from empty, single rows,
tile-straddling tails and several work-groups, with the head count, head
dim, mask, dropout rate and dtype drawn with them. Forward and backward
through the C ABI against the packed-batch fp64 oracle.

The bar is the one of the dense random-shape test: sequences of one or two
tokens give output rows that are rescaled V or dO rows (values of 3 to 5),
whose bf16 storage alone misses the exact value by a mean of up to about
1.5e-3; bf16 tensors are held to 2e-2 * max(1, |ref|) and a mean of 1e-3 plus
the mean |bf16(ref) - ref| measured on the oracle's values. The backward is
handed the oracle's O and LSE in their storage types, and the oracle reads D
from that same O."""
import numpy as np
import pytest

from helpers import assert_close, to_device, to_host
from oracle import varlen as OV
from workloads import VarlenWorkload, make_varlen_inputs

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


LENGTHS = [0, 1, 2, 31, 33, 64, 65, 127, 129, 200, 257, 300, 513, 700]


def _cases(n=16, seed=5151):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype = "f32" if rng.random() < 0.2 else "bf16"
        d = int(rng.choice([64, 80, 128]))
        lengths = [int(rng.choice(LENGTHS)) for _ in range(int(rng.integers(1, 7)))]
        if sum(lengths) == 0:
            lengths[0] = 5
        H = int(rng.integers(1, 4))
        causal = bool(rng.random() < 0.6)
        p = float(rng.choice([0.0, 0.0, 0.1, 0.3]))
        out.append(VarlenWorkload(f"rand{i}", len(lengths), H, d, dtype, causal, p, lengths=tuple(lengths),
                                  seed=6000 + i, dropout_seed=7000 + i))
    return out


CASES = _cases()


@pytest.mark.parametrize("w", CASES, ids=[f"{i}-{w.dtype}-d{w.d}-H{w.H}-{'c' if w.causal else 'f'}-p{w.dropout_p}"
                                          f"-L{'_'.join(map(str, w.lengths))}" for i, w in enumerate(CASES)])
def test_random_packed_batch_matches_oracle(w):
    cu, inp = make_varlen_inputs(w)
    cu_d = torch.from_numpy(cu).cuda()
    dev = {k: to_device(v[0], w.dtype) for k, v in inp.items()}
    val = {k: v[1].astype(np.float64) for k, v in inp.items()}
    maxlen = int(max(w.lengths))
    args = (w.causal, w.dropout_p, w.dropout_seed, w.scale)
    o, lse = fa.forward_varlen(dev["q"], dev["k"], dev["v"], cu_d, maxlen, *args)
    torch.cuda.synchronize()
    o_r, lse_r = OV.forward_varlen(val["q"], val["k"], val["v"], cu, w.scale, w.causal, w.dropout_p,
                                   w.dropout_seed)
    _check("O", to_host(o), o_r, w.dtype)
    assert_close("LSE", to_host(lse), lse_r, w.dtype)  # stored in fp32

    o_st = torch.from_numpy(o_r).to(dev["q"].dtype).cuda()
    lse_st = torch.from_numpy(lse_r).to(torch.float32).cuda()
    dq, dk, dv = fa.backward_varlen(dev["q"], dev["k"], dev["v"], o_st, dev["do"], lse_st, cu_d, maxlen, *args)
    torch.cuda.synchronize()
    dq_r, dk_r, dv_r, _ = OV.backward_varlen(val["q"], val["k"], val["v"], val["do"], cu, w.scale, w.causal,
                                             w.dropout_p, w.dropout_seed, o=to_host(o_st))
    _check("dQ", to_host(dq), dq_r, w.dtype)
    _check("dK", to_host(dk), dk_r, w.dtype)
    _check("dV", to_host(dv), dv_r, w.dtype)
