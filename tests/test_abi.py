"""The C-ABI library: it loads, exports every symbol include/fa.h declares,
and rejects invalid arguments with the documented status before any HIP call.
CPU only: no call here reaches a kernel launch."""
import ctypes
import os
import re
import subprocess

import pytest

import exact_io_aware_72_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(fa.lib_path()), reason="libfa.so not built")

OK, NULL, SHAPE, HEADDIM, DTYPE, DROPOUT, ALIGN, UNSUP, HIP, ARG = 0, -1, -2, -3, -4, -5, -6, -7, -8, -9
P = 0x10000  # a 16-byte aligned stand-in address; never dereferenced by rejected calls


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_binding_symbols():
    assert _declared() == sorted(fa.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", fa.lib_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in _declared():
        assert name in exported, name
    # nothing but the C ABI is exported from the library's own code
    assert {n for n in exported if n.startswith("fa")} == set(_declared())


def test_clock_library_exports_its_header():
    """libfa_clock.so (benchmark clock stamps) exports what include/fa_clock.h
    declares, and rejects bad arguments before any HIP call."""
    import ctypes
    path = os.path.join(os.path.dirname(fa.lib_path()), "libfa_clock.so")
    text = open(os.path.join(os.path.dirname(HEADER), "fa_clock.h")).read()
    declared = set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", text))
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert declared == {"fa_clock_stamp"} and declared <= exported
    L = ctypes.CDLL(path)
    L.fa_clock_stamp.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    assert L.fa_clock_stamp(None, 8, None) == -1
    assert L.fa_clock_stamp(P + 4, 8, None) == -1
    assert L.fa_clock_stamp(P, 0, None) == -1
    assert L.fa_clock_stamp(P, 1025, None) == -1


def test_version_and_status_strings():
    assert "gfx950" in fa.version()
    L = fa.lib()
    for code in (OK, NULL, SHAPE, HEADDIM, DTYPE, DROPOUT, ALIGN, UNSUP, HIP, ARG, 12345):
        assert isinstance(L.fa_status_string(code), bytes)


def test_workspace_bytes():
    assert fa.workspace_bytes(2, 16, 8192, 128) == 4 * 2 * 16 * 8192
    assert fa.workspace_bytes(0, 16, 8192, 128) == 0
    assert fa.workspace_bytes(1, 1, 1, 63) == 0


def _fwd(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=1, N=16, d=64, scale=0.125, causal=0, p=0.0, seed=0,
             stream=None, dtype=1)
    a.update(kw)
    return fa.lib().fa_forward(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"],
                               a["d"], a["scale"], a["causal"], a["p"], a["seed"], a["stream"],
                               a["dtype"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), NULL), (dict(k=0), NULL), (dict(v=0), NULL), (dict(o=0), NULL), (dict(lse=0), NULL),
    (dict(q=P + 8), ALIGN), (dict(o=P + 2), ALIGN), (dict(lse=P + 4), ALIGN),
    (dict(B=0), SHAPE), (dict(H=-1), SHAPE), (dict(N=0), SHAPE), (dict(B=1 << 20, H=1 << 10, N=1 << 20), SHAPE),
    (dict(N=1 << 30), SHAPE), (dict(N=1 << 30, dtype=0), SHAPE), (dict(H=(1 << 13) + 1, d=128), SHAPE),
    (dict(d=32), HEADDIM), (dict(d=96), HEADDIM), (dict(d=256), HEADDIM),
    (dict(dtype=2), DTYPE), (dict(dtype=-1), DTYPE),
    (dict(p=1.0), DROPOUT), (dict(p=-0.1), DROPOUT), (dict(p=float("nan")), DROPOUT), (dict(p=1.5), DROPOUT),
    # below the 16-bit draws' resolution: nothing would be dropped, yet O rescaled
    (dict(p=1e-6), DROPOUT), (dict(p=2.0 ** -16 * 0.999), DROPOUT), (dict(p=1e-45), DROPOUT),
    (dict(scale=float("inf")), ARG), (dict(scale=float("nan")), ARG), (dict(scale=0.0), ARG),
    (dict(scale=-0.125), ARG),
])
def test_forward_rejects(kw, status):
    assert _fwd(**kw) == status


def test_backward_rejects():
    L = fa.lib()
    args = [P] * 10 + [1, 1, 16, 64, 0.125, 1, 0.0, 0, None, 1]

    def call(**ch):
        a = list(args)
        for idx, val in ch.items():
            a[int(idx[1:])] = val
        return L.fa_backward(*a)

    assert call(a0=0) == NULL
    assert call(a9=0) == NULL  # workspace
    assert call(a9=P + 4) == ALIGN
    assert call(a13=80 + 1) == HEADDIM
    assert call(a12=0) == SHAPE
    assert call(a16=1.0) == DROPOUT
    assert call(a19=7) == DTYPE
    assert call(a14=float("nan")) == ARG
    dk = [P] * 8 + [1, 1, 16, 64, 0.125, 1, 0.0, 0, None, 1]
    dk[6] = 0
    assert L.fa_backward_dkdv(*dk) == NULL
    dq = [P] * 7 + [1, 1, 16, 64, 0.125, 1, 0.0, 0, None, 1]
    dq[10] = 100
    assert L.fa_backward_dq(*dq) == HEADDIM
    assert L.fa_backward_preprocess(P, P, 0, 1, 1, 16, 64, None, 1) == NULL
    assert L.fa_backward_preprocess(P, P + 1, P, 1, 1, 16, 64, None, 1) == ALIGN


@pytest.mark.parametrize("args,status", [
    ((1, 0, 0, 1, 0.1, 0, 0, 4, 4, 0, None), NULL),
    ((1, 0, 0, 1, 1.0, 0, 0, 4, 4, P, None), DROPOUT),
    ((1, 0, 0, 1, 1e-6, 0, 0, 4, 4, P, None), DROPOUT),  # in (0, 2^-16)
    ((1, 0, 1, 1, 0.1, 0, 0, 4, 4, P, None), ARG),      # h >= H
    ((1, -1, 0, 1, 0.1, 0, 0, 4, 4, P, None), ARG),     # b < 0
    ((1, 0, 0, 1, 0.1, -1, 0, 4, 4, P, None), ARG),     # row0 < 0
    ((1, 0, 0, 1, 0.1, 0, 0, 0, 4, P, None), ARG),      # rows < 1
    ((1, 0, 0, 1, 0.1, 0, 0, 65536, 65536, P, None), ARG),  # rows*cols >= 2^31
    ((1, 0, 0, 1, 0.1, 2147483000, 0, 1000, 4, P, None), ARG),  # row0+rows overflows
])
def test_dropout_mask_rejects(args, status):
    assert fa.lib().fa_dropout_mask(*args) == status


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(fa, "_LIB", None)
    monkeypatch.setattr(fa, "lib_path", lambda: str(tmp_path / "absent.so"))
    with pytest.raises(fa.FAError):
        fa.lib()


def _fwd_varlen(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, cu=P, S=2, total=100, maxlen=64, H=2, d=128, scale=0.1,
             causal=1, p=0.0, seed=0, stream=None, dtype=1)
    a.update(kw)
    return fa.lib().fa_forward_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cu"], a["S"],
                                      a["total"], a["maxlen"], a["H"], a["d"], a["scale"],
                                      a["causal"], a["p"], a["seed"], a["stream"], a["dtype"])


@pytest.mark.parametrize("kw,status", [
    (dict(cu=0), NULL), (dict(cu=P + 2), ALIGN), (dict(q=0), NULL), (dict(lse=0), NULL),
    (dict(o=P + 8), ALIGN), (dict(S=0), SHAPE), (dict(maxlen=0), SHAPE), (dict(total=-1), SHAPE),
    (dict(total=1 << 30, H=128), SHAPE), (dict(H=0), SHAPE), (dict(d=96), HEADDIM), (dict(dtype=3), DTYPE),
    (dict(p=1.0), DROPOUT), (dict(scale=float("nan")), ARG),
    # an empty batch passes the argument checks and then touches nothing
    (dict(total=0, q=0, k=0, v=0, o=0, lse=0), OK),
])
def test_forward_varlen_rejects(kw, status):
    assert _fwd_varlen(**kw) == status


def test_backward_varlen_rejects():
    L = fa.lib()
    args = [P] * 11 + [2, 100, 64, 2, 128, 0.1, 1, 0.0, 0, None, 1]

    def call(**ch):
        a = list(args)
        for idx, val in ch.items():
            a[int(idx[1:])] = val
        return L.fa_backward_varlen(*a)

    assert call(a10=0) == NULL        # cu_seqlens
    assert call(a9=0) == NULL         # workspace
    assert call(a9=P + 4) == ALIGN
    assert call(a10=P + 1) == ALIGN
    assert call(a11=0) == SHAPE       # num_seqs
    assert call(a12=-5) == SHAPE      # total
    assert call(a15=80 + 16) == HEADDIM
    assert call(a18=-0.5) == DROPOUT
    assert call(a21=9) == DTYPE
    assert call(a12=0, a0=0) == OK
    assert fa.varlen_workspace_bytes(100, 3, 80) == 4 * 3 * 100
    assert fa.varlen_workspace_bytes(-1, 3, 80) == 0


def _fwd_bs(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, m=P + 1, sb=0, sh=16, B=1, H=2, N=300, d=64, scale=0.1,
             causal=0, p=0.0, seed=0, stream=None, dtype=1)
    a.update(kw)
    return fa.lib().fa_forward_blocksparse(a["q"], a["k"], a["v"], a["o"], a["lse"], a["m"], a["sb"],
                                           a["sh"], a["B"], a["H"], a["N"], a["d"], a["scale"],
                                           a["causal"], a["p"], a["seed"], a["stream"], a["dtype"])


@pytest.mark.parametrize("kw,status", [
    (dict(m=0), NULL), (dict(sb=-1), ARG), (dict(sh=-16), ARG), (dict(N=131073, H=1), SHAPE),
    (dict(q=0), NULL), (dict(o=P + 4), ALIGN), (dict(d=100), HEADDIM), (dict(dtype=5), DTYPE),
    (dict(p=2.0), DROPOUT), (dict(scale=-1.0), ARG), (dict(B=0), SHAPE),
])
def test_forward_blocksparse_rejects(kw, status):
    assert _fwd_bs(**kw) == status


def test_backward_blocksparse_rejects():
    L = fa.lib()
    args = [P] * 10 + [P + 3, 0, 0, 1, 2, 300, 64, 0.1, 1, 0.0, 0, None, 1]

    def call(**ch):
        a = list(args)
        for idx, val in ch.items():
            a[int(idx[1:])] = val
        return L.fa_backward_blocksparse(*a)

    assert call(a10=0) == NULL        # mask
    assert call(a9=0) == NULL         # workspace
    assert call(a11=-1) == ARG
    assert call(a12=-1) == ARG
    assert call(a15=131073, a14=1) == SHAPE
    assert call(a16=96) == HEADDIM
    assert call(a19=1.0) == DROPOUT
    assert call(a22=4) == DTYPE


def test_splitkv_rejects_and_sizes():
    L = fa.lib()
    args = [P] * 6 + [1, 2, 1, 1000, 128, 0.1, 1, 0, None, 1]

    def call(**ch):
        a = list(args)
        for idx, val in ch.items():
            a[int(idx[1:])] = val
        return L.fa_forward_splitkv(*a)

    assert call(a5=0) == NULL            # workspace
    assert call(a5=P + 4) == ALIGN
    assert call(a15=0) == UNSUP          # fp32 is not implemented for split-KV
    assert call(a13=-1) == ARG           # num_splits
    assert call(a13=129) == ARG
    assert call(a8=1001) == SHAPE        # causal with Nk < Nq
    assert call(a9=0) == SHAPE           # Nk
    assert call(a10=96) == HEADDIM
    assert call(a11=float("nan")) == ARG
    assert L.fa_forward_splitkv_workspace_bytes(1, 2, 3, 128, 4) == 4 * 4 * 1 * 2 * 3 * 129
    assert L.fa_forward_splitkv_workspace_bytes(1, 2, 3, 128, 0) == 0
    assert L.fa_splitkv_num_splits(4, 16, 1, 65536, 128) > 1
    assert L.fa_splitkv_num_splits(8, 32, 8192, 8192, 128) == 1
    assert L.fa_splitkv_num_splits(1, 1, 1, 100, 128) == 1   # at least four key tiles per part


def test_fp8_rejects():
    L = fa.lib()
    assert L.fa_quantize_fp8(0, P, P, 1, 16, 1, 128, 128, None) == NULL
    assert L.fa_quantize_fp8(P, P, P, 1, 16, 1, 96, 128, None) == HEADDIM
    assert L.fa_quantize_fp8(P, P, P, 1, 16, 1, 128, 32, None) == ARG
    assert L.fa_quantize_fp8(P, P, P, 1, 0, 1, 128, 128, None) == SHAPE
    args = [P] * 7 + [1, 2, 300, 128, 0.1, 1, None]
    a = list(args); a[5] = 0
    assert L.fa_forward_fp8(*a) == NULL         # q_scale
    a = list(args); a[6] = P + 2
    assert L.fa_forward_fp8(*a) == ALIGN        # k_scale
    a = list(args); a[10] = 96
    assert L.fa_forward_fp8(*a) == HEADDIM      # d not in {64, 80, 128}
    a = list(args); a[11] = 0.0
    assert L.fa_forward_fp8(*a) == ARG          # scale
    a = list(args); a[0] = 0
    assert L.fa_forward_fp8(*a) == NULL


def test_backward_noalloc_rejects_before_any_hip_call():
    L = fa.lib()
    ok = [P] * 9 + [1, 64, 1 << 16, 128, 0.1, 1, 0.0, 0, None, 1]
    big = list(ok); big[11] = (1 << 16) + 1  # B * H * N = 2^22 + 64 > FA_NOALLOC_MAX_ROWS
    assert L.fa_backward_noalloc(*big) == SHAPE
    a = list(ok); a[0] = 0
    assert L.fa_backward_noalloc(*a) == NULL
    a = list(ok); a[8] = P + 2
    assert L.fa_backward_noalloc(*a) == ALIGN
    a = list(ok); a[12] = 96
    assert L.fa_backward_noalloc(*a) == HEADDIM
    a = list(ok); a[15] = 1e-6
    assert L.fa_backward_noalloc(*a) == DROPOUT
    a = list(ok); a[13] = 0.0
    assert L.fa_backward_noalloc(*a) == ARG


def test_shape_products_that_overflow_64_bits_are_rejected():
    # B * N * H of three 2^31 - 1 values exceeds 2^63: rejected before any
    # product is formed.
    L = fa.lib()
    big = 2147483647
    assert L.fa_forward(P, P, P, P, P, big, big, big, 128, 0.1, 0, 0.0, 0, None, 1) == SHAPE
    assert L.fa_backward_workspace_bytes(big, big, big, 128) == 0
    assert L.fa_forward_splitkv_workspace_bytes(big, big, big, 128, 8) == 0
