"""GPU parity for packed variable-length batches: the HIP path through the
C ABI against the fp64 packed oracle, element by element, on seeded length
mixes that include empty, length-1 and tile-straddling sequences; plus bit
equality with the fixed-length path at equal lengths and untouched rows
outside every sequence."""
import numpy as np
import pytest

from helpers import assert_close, to_device, to_host
from oracle import varlen as OV
from workloads import VARLEN_WORKLOADS, VarlenWorkload, make_inputs, make_varlen_inputs, Workload

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import exact_io_aware_72_amd as fa  # noqa: E402


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _vw(name, lengths, H, d, dtype, causal, p, amp=1.0, seed=3100):
    return VarlenWorkload(name, len(lengths), H, d, dtype, causal, p, lengths=tuple(lengths),
                          seed=seed, amp=amp)


CASES = [
    _vw("bf16-d128-causal-mix", [1, 0, 130, 257, 64, 500], 2, 128, "bf16", True, 0.0),
    _vw("bf16-d128-full-drop", [128, 256, 3], 2, 128, "bf16", False, 0.2, seed=3101),
    _vw("bf16-d64-full", [300, 17, 129], 2, 64, "bf16", False, 0.0, seed=3102),
    _vw("bf16-d64-causal", [33, 1000, 2], 1, 64, "bf16", True, 0.0, seed=3103),
    _vw("bf16-d80-causal-drop", [200, 1, 333], 2, 80, "bf16", True, 0.1, amp=0.5, seed=3104),
    _vw("bf16-d80-full", [97, 160], 3, 80, "bf16", False, 0.0, amp=0.5, seed=3105),
    _vw("f32-d64-causal", [100, 0, 37, 256], 2, 64, "f32", True, 0.0, seed=3106),
    _vw("f32-d80-full-drop", [70, 130], 1, 80, "f32", False, 0.15, seed=3107),
    _vw("f32-d128-causal", [1, 65, 190], 1, 128, "f32", True, 0.0, seed=3108),
    # longest sequence >= 8192 at d <= 80: the eight-wave forward (256-row
    # work-groups), with sequences shorter than one such group beside it
    _vw("bf16-d64-causal-long", [8300, 0, 300, 1], 1, 64, "bf16", True, 0.0, seed=3109),
    _vw("bf16-d80-full-long-drop", [257, 8200], 1, 80, "bf16", False, 0.1, amp=0.5, seed=3110),
    # a causal grid past what the device holds at once: each work-group takes
    # a pair of one sequence's blocks (the second over descending key tiles);
    # odd and even block counts, empty and one-row sequences
    _vw("bf16-d128-causal-pairs", [1100, 0, 1, 900, 257, 1024, 640, 129, 1000, 3, 768, 512], 32, 128,
        "bf16", True, 0.0, seed=3111),
    _vw("bf16-d64-causal-pairs-drop", [1024, 700, 5, 1100, 300, 999, 1, 64], 48, 64, "bf16", True, 0.1,
        seed=3112),
]


PAIR_CASES = {"bf16-d128-causal-pairs", "bf16-d64-causal-pairs-drop"}


def _device(cu, inp, dtype):
    dev = {k: to_device(v[0], dtype) for k, v in inp.items()}
    val = {k: v[1].astype(np.float64) for k, v in inp.items()}
    return torch.from_numpy(cu).cuda(), dev, val


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_varlen_forward_backward_match_oracle(w):
    cu, inp = make_varlen_inputs(w)
    cu_d, dev, val = _device(cu, inp, w.dtype)
    maxlen = int(max(w.lengths))
    o, lse = fa.forward_varlen(dev["q"], dev["k"], dev["v"], cu_d, maxlen, w.causal, w.dropout_p,
                               w.dropout_seed, w.scale)
    dq, dk, dv = fa.backward_varlen(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, cu_d, maxlen,
                                    w.causal, w.dropout_p, w.dropout_seed, w.scale)
    torch.cuda.synchronize()
    o_r, lse_r = OV.forward_varlen(val["q"], val["k"], val["v"], cu, w.scale, w.causal, w.dropout_p,
                                   w.dropout_seed)
    dq_r, dk_r, dv_r, _ = OV.backward_varlen(val["q"], val["k"], val["v"], val["do"], cu, w.scale,
                                             w.causal, w.dropout_p, w.dropout_seed)
    assert_close("O", to_host(o), o_r, w.dtype)
    assert_close("LSE", to_host(lse), lse_r, w.dtype)
    # The block-pair cases run 32-48 heads: every query sees its sequence's
    # first keys, whose dV then reaches |5| somewhere, where bf16 stores values
    # only to within 0.0156 and the bf16 rounding of P in the dV product adds
    # about 0.01; their gradients take the magnitude-relative bar.
    scaled = w.name in PAIR_CASES
    assert_close("dQ", to_host(dq), dq_r, w.dtype, scaled=scaled)
    assert_close("dK", to_host(dk), dk_r, w.dtype, scaled=scaled)
    assert_close("dV", to_host(dv), dv_r, w.dtype, scaled=scaled)


@pytest.mark.parametrize("dtype,d,causal,p", [("bf16", 128, True, 0.1), ("bf16", 80, False, 0.0),
                                              ("f32", 64, True, 0.0)])
def test_equal_lengths_bitwise_equal_fixed_batch(dtype, d, causal, p):
    B, N, H = 3, 200, 2
    w = Workload(0, "eq", B, H, N, d, dtype, causal, p, True)
    inp = make_inputs(w, with_grad=True)
    dev = {k: to_device(v[0], dtype) for k, v in inp.items()}
    o, lse = fa.forward(dev["q"], dev["k"], dev["v"], causal, p, 5, w.scale)
    dq, dk, dv = fa.backward(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal, p, 5, w.scale)
    pk = {k: t.reshape(B * N, H, d) for k, t in dev.items()}
    cu = torch.arange(0, (B + 1) * N, N, dtype=torch.int32, device="cuda")
    o2, lse2 = fa.forward_varlen(pk["q"], pk["k"], pk["v"], cu, N, causal, p, 5, w.scale)
    dq2, dk2, dv2 = fa.backward_varlen(pk["q"], pk["k"], pk["v"], o2, pk["do"], lse2, cu, N, causal,
                                       p, 5, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o.reshape(B * N, H, d), o2)
    assert torch.equal(lse.permute(1, 0, 2).reshape(H, B * N), lse2)
    for a, b in ((dq, dq2), (dk, dk2), (dv, dv2)):
        assert torch.equal(a.reshape(B * N, H, d), b)


def test_rows_outside_sequences_untouched():
    # Offsets covering rows 10..209 of 230: rows 0..9 and 210..229 belong to no
    # sequence and keep their sentinel values in every output.
    H, d = 2, 64
    total = 230
    g = torch.Generator().manual_seed(0)
    q, k, v, do = (torch.randn(total, H, d, generator=g).to(torch.bfloat16).cuda() for _ in range(4))
    cu = torch.tensor([10, 80, 81, 210], dtype=torch.int32, device="cuda")
    sent = float("nan")
    o = torch.full_like(q, sent)
    lse = torch.full((H, total), sent, dtype=torch.float32, device="cuda")
    fa.forward_varlen(q, k, v, cu, 129, True, out=o, lse=lse)
    dq, dk, dv = (torch.full_like(q, sent) for _ in range(3))
    fa.backward_varlen(q, k, v, o, do, lse, cu, 129, True, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    outside = torch.cat([torch.arange(0, 10), torch.arange(210, total)]).cuda()
    inside = torch.arange(10, 210).cuda()
    for t in (o, dq, dk, dv):
        assert torch.isnan(t[outside]).all()
        assert torch.isfinite(t[inside]).all()
    assert torch.isnan(lse[:, outside]).all() and torch.isfinite(lse[:, inside]).all()


def test_empty_batch_is_a_no_op():
    q = torch.empty((0, 2, 64), dtype=torch.bfloat16, device="cuda")
    cu = torch.zeros(3, dtype=torch.int32, device="cuda")
    o, lse = fa.forward_varlen(q, q, q, cu, 1, True)
    assert o.shape == (0, 2, 64) and lse.shape == (2, 0)


def test_varlen_workload_sampled_rows():
    """The benchmark's packed workload at full size, checked on a sample: the
    shortest sequence in full, and sampled rows/columns of the longest."""
    from oracle import attention as OA
    w = VARLEN_WORKLOADS["varlen16"]
    cu, inp = make_varlen_inputs(w)
    cu_d, dev, val = _device(cu, inp, w.dtype)
    lengths = np.diff(cu)
    maxlen = int(lengths.max())
    o, lse = fa.forward_varlen(dev["q"], dev["k"], dev["v"], cu_d, maxlen, w.causal, w.dropout_p,
                               w.dropout_seed, w.scale)
    dq, dk, dv = fa.backward_varlen(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, cu_d, maxlen,
                                    w.causal, w.dropout_p, w.dropout_seed, w.scale)
    torch.cuda.synchronize()
    got = {n: to_host(t) for n, t in (("o", o), ("dq", dq), ("dk", dk), ("dv", dv))}
    lse_h = to_host(lse)
    H = w.H
    rng = np.random.default_rng(5)
    for s in (int(np.argmin(lengths)), int(np.argmax(lengths))):
        a, e = int(cu[s]), int(cu[s + 1])
        n = e - a
        rows = np.unique(np.r_[0, n - 1, rng.integers(0, n, 14)])
        cols = np.unique(np.r_[0, n - 1, rng.integers(0, n, 14)])
        for h in rng.choice(H, 2, replace=False):
            sl = lambda x: x[None, a:e]  # one sequence as a batch of one
            ref = OA.sampled_head(sl(val["q"]), sl(val["k"]), sl(val["v"]), sl(val["do"]), w.scale,
                                  w.causal, w.dropout_p, w.dropout_seed, 0, int(h), rows, cols)
            assert_close("O", got["o"][a + rows, h], ref["o"], w.dtype)
            assert_close("LSE", lse_h[h, a + rows], ref["lse"], w.dtype)
            assert_close("dQ", got["dq"][a + rows, h], ref["dq"], w.dtype)
            assert_close("dK", got["dk"][a + cols, h], ref["dk"], w.dtype)
            assert_close("dV", got["dv"][a + cols, h], ref["dv"], w.dtype)
