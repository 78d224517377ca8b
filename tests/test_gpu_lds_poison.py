"""Race detection through the library built with -DFA_LDS_POISON
(libfa_poison.so): every LDS stage is filled with all-ones bytes (NaN in bf16
and fp32) between its last read and the next tile's loads, so a read that
runs ahead of its tile's loads, or a stage refilled while still being read,
turns outputs into NaN or changes them. Forward and backward through that
build must equal the regular build bit for bit, for the fixed-length,
packed variable-length, block-sparse (two query groups per dK/dV
work-group), split-KV and FP8-score paths."""
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import exact_io_aware_72_amd as fa  # noqa: E402
from exact_io_aware_72_amd import build as fa_build  # noqa: E402
from workloads import BLOCK, block_mask_random  # noqa: E402


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _rand(shape, seed, dtype=torch.bfloat16):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float32).to(dtype).cuda()


def _both(run, monkeypatch):
    """run() with the regular library, then with the poisoned one."""
    if not os.path.exists(fa_build.POISON_LIB_PATH):
        raise RuntimeError(f"{fa_build.POISON_LIB_PATH} is not built; run __graft_entry__.build()")
    ref = [t.clone() for t in run()]
    torch.cuda.synchronize()
    monkeypatch.setattr(fa, "lib_path", lambda: fa_build.POISON_LIB_PATH)
    monkeypatch.setattr(fa, "_LIB", None)
    got = run()
    torch.cuda.synchronize()
    monkeypatch.undo()
    return ref, got


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _same(ref, got):
    for i, (a, b) in enumerate(zip(ref, got)):
        assert not torch.isnan(b.float()).any(), f"output {i}: NaN (a read ran ahead of its tile)"
        assert torch.equal(_bits(a), _bits(b)), f"output {i} differs from the regular build"


@pytest.mark.parametrize("B,H,N,d,causal,p,dtype", [
    (2, 3, 1000, 128, True, 0.0, torch.bfloat16),
    (1, 2, 777, 80, False, 0.1, torch.bfloat16),
    (2, 2, 300, 64, True, 0.0, torch.bfloat16),
    (1, 1, 8192, 80, True, 0.0, torch.bfloat16),   # eight-wave forward
    (1, 2, 200, 64, True, 0.1, torch.float32),
])
def test_fixed_length(B, H, N, d, causal, p, dtype, monkeypatch):
    q, k, v, do = (_rand((B, N, H, d), 100 + i, dtype) for i in range(4))

    def run():
        o, lse = fa.forward(q, k, v, causal, p, 11)
        dq, dk, dv = fa.backward(q, k, v, o, do, lse, causal, p, 11)
        return o, lse, dq, dk, dv

    _same(*_both(run, monkeypatch))


def test_varlen(monkeypatch):
    lens = [1, 0, 130, 257, 700]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32).cuda()
    T, H, d = sum(lens), 2, 128
    q, k, v, do = (_rand((T, H, d), 200 + i) for i in range(4))

    def run():
        o, lse = fa.forward_varlen(q, k, v, cu, max(lens), True, 0.1, 5)
        dq, dk, dv = fa.backward_varlen(q, k, v, o, do, lse, cu, max(lens), True, 0.1, 5)
        return o, lse, dq, dk, dv

    _same(*_both(run, monkeypatch))


def test_blocksparse(monkeypatch):
    B, H, N, d = 1, 2, 1000, 128
    q, k, v, do = (_rand((B, N, H, d), 300 + i) for i in range(4))
    m = torch.from_numpy(block_mask_random((B, H), N, 0.6, 9)).cuda()
    assert m.shape[-1] == -(-N // BLOCK)

    def run():
        o, lse = fa.forward_blocksparse(q, k, v, m, False, 0.0, 0)
        dq, dk, dv = fa.backward_blocksparse(q, k, v, o, do, lse, m, False, 0.0, 0)
        return o, lse, dq, dk, dv

    _same(*_both(run, monkeypatch))


def test_splitkv_and_fp8(monkeypatch):
    q = _rand((2, 5, 4, 128), 400)
    k, v = _rand((2, 3000, 4, 128), 401), _rand((2, 3000, 4, 128), 402)
    q2, k2, v2 = (_rand((1, 1000, 2, 128), 410 + i) for i in range(3))

    def run():
        o, lse = fa.forward_splitkv(q, k, v, True, 4)
        o8, lse8 = fa.forward_fp8(q2, k2, v2, True)
        return o, lse, o8, lse8

    _same(*_both(run, monkeypatch))


# Launch forms that reuse a work-group's LDS stages across two blocks (block
# pairs per work-group: forward from N = 32768 and for packed batches, the
# eight-wave dQ from N = 32768), the sixteen-wave forward groups, and the
# resident pairs across the work-groups of a CU (a grid the device holds at
# once).
@pytest.mark.parametrize("B,H,N,d,causal,p", [
    (1, 2, 32768, 80, True, 0.0),    # sixteen-wave forward with block pairs; paired eight-wave dQ
    (1, 1, 32800, 128, True, 0.1),   # eight-wave dropout forward with block pairs, ragged last group
    (1, 2, 32768, 64, False, 0.0),   # sixteen-wave forward without the causal mask
    (4, 16, 2048, 64, True, 0.0),    # resident pairs (four work-groups per CU)
])
def test_paired_and_wide_launches(B, H, N, d, causal, p, monkeypatch):
    q, k, v, do = (_rand((B, N, H, d), 500 + i) for i in range(4))

    def run():
        o, lse = fa.forward(q, k, v, causal, p, 13)
        dq, dk, dv = fa.backward(q, k, v, o, do, lse, causal, p, 13)
        return o, lse, dq, dk, dv

    _same(*_both(run, monkeypatch))


def test_varlen_block_pairs(monkeypatch):
    # a causal packed grid larger than the device holds: pairs of one
    # sequence's blocks per work-group, with empty and one-row sequences
    lens = [1100, 0, 1, 900, 257, 1024, 640, 129, 1000, 3, 768, 512]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32).cuda()
    T, H, d = sum(lens), 32, 128
    q, k, v, do = (_rand((T, H, d), 600 + i) for i in range(4))

    def run():
        o, lse = fa.forward_varlen(q, k, v, cu, max(lens), True, 0.0, 5)
        dq, dk, dv = fa.backward_varlen(q, k, v, o, do, lse, cu, max(lens), True, 0.0, 5)
        return o, lse, dq, dk, dv

    _same(*_both(run, monkeypatch))
