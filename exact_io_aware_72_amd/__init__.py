"""Exact IO-aware attention for AMD MI355X (gfx950): Python binding.

This module only marshals arguments into libfa.so, the C-ABI library whose
HIP kernels run every step of the forward and backward passes; torch supplies
device memory and the current HIP stream. There is no fallback: if the
library is missing, every call raises.

Usage mirrors the drop-in PyTorch call of "FlashAttention for Efficient
Training", section 4.2: tensors of shape (batch, seq_len, num_heads,
head_dim), `flash_attention(q, k, v)` returns the attention output, and the
autograd backward recomputes attention from the saved logsumexp.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "FAError", "lib", "lib_path", "version", "forward", "backward", "backward_preprocess",
    "backward_dkdv", "backward_dq", "workspace_bytes", "dropout_mask", "FlashAttnFunction",
    "flash_attention", "draw_seed", "forward_varlen", "backward_varlen", "varlen_workspace_bytes",
    "forward_blocksparse", "backward_blocksparse", "BLOCK",
    "forward_splitkv", "splitkv_num_splits", "splitkv_workspace_bytes",
    "quantize_fp8", "forward_fp8", "forward_fp8_quantized", "backward_noalloc", "NOALLOC_MAX_ROWS",
    "EXPORTED_SYMBOLS", "STATUS",
]

FA_F32, FA_BF16 = 0, 1
STATUS = {
    0: "FA_OK", -1: "FA_ERR_NULL", -2: "FA_ERR_SHAPE", -3: "FA_ERR_HEADDIM", -4: "FA_ERR_DTYPE",
    -5: "FA_ERR_DROPOUT", -6: "FA_ERR_ALIGN", -7: "FA_ERR_UNSUPPORTED", -8: "FA_ERR_HIP",
    -9: "FA_ERR_ARG",
}
EXPORTED_SYMBOLS = (
    "fa_forward", "fa_backward", "fa_backward_workspace_bytes", "fa_backward_preprocess",
    "fa_backward_dkdv", "fa_backward_dq", "fa_dropout_mask", "fa_status_string", "fa_version",
    "fa_forward_varlen", "fa_backward_varlen", "fa_backward_varlen_workspace_bytes",
    "fa_forward_blocksparse", "fa_backward_blocksparse",
    "fa_splitkv_num_splits", "fa_forward_splitkv_workspace_bytes", "fa_forward_splitkv",
    "fa_quantize_fp8", "fa_forward_fp8", "fa_backward_noalloc",
)

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


def lib_path() -> str:
    return os.path.join(_HERE, "libfa.so")


class FAError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str = ""):
        self.status = status
        name = STATUS.get(status, str(status))
        super().__init__(f"{where}: {name} ({detail})" if detail else f"{where}: {name}")


_vp, _i, _f, _u64, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_uint64, ctypes.c_size_t
_i64 = ctypes.c_int64
_SIGS = {
    "fa_forward": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _f, _u64, _vp, _i]),
    "fa_backward_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "fa_backward": (_i, [_vp] * 10 + [_i, _i, _i, _i, _f, _i, _f, _u64, _vp, _i]),
    "fa_backward_noalloc": (_i, [_vp] * 9 + [_i, _i, _i, _i, _f, _i, _f, _u64, _vp, _i]),
    "fa_backward_preprocess": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _vp, _i]),
    "fa_backward_dkdv": (_i, [_vp] * 8 + [_i, _i, _i, _i, _f, _i, _f, _u64, _vp, _i]),
    "fa_backward_dq": (_i, [_vp] * 7 + [_i, _i, _i, _i, _f, _i, _f, _u64, _vp, _i]),
    "fa_dropout_mask": (_i, [_u64, _i, _i, _i, _f, _i, _i, _i, _i, _vp, _vp]),
    "fa_forward_varlen": (_i, [_vp] * 6 + [_i, _i, _i, _i, _i, _f, _i, _f, _u64, _vp, _i]),
    "fa_backward_varlen_workspace_bytes": (_sz, [_i, _i, _i]),
    "fa_backward_varlen": (_i, [_vp] * 11 + [_i, _i, _i, _i, _i, _f, _i, _f, _u64, _vp, _i]),
    "fa_forward_blocksparse": (_i, [_vp] * 6 + [_i64, _i64, _i, _i, _i, _i, _f, _i, _f, _u64, _vp, _i]),
    "fa_backward_blocksparse": (_i, [_vp] * 11 + [_i64, _i64, _i, _i, _i, _i, _f, _i, _f, _u64, _vp, _i]),
    "fa_splitkv_num_splits": (_i, [_i, _i, _i, _i, _i]),
    "fa_forward_splitkv_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "fa_forward_splitkv": (_i, [_vp] * 6 + [_i, _i, _i, _i, _i, _f, _i, _i, _vp, _i]),
    "fa_quantize_fp8": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _vp]),
    "fa_forward_fp8": (_i, [_vp] * 7 + [_i, _i, _i, _i, _f, _i, _vp]),
    "fa_status_string": (ctypes.c_char_p, [_i]),
    "fa_version": (ctypes.c_char_p, []),
}


def lib():
    """The loaded libfa.so (ctypes), with argument types set."""
    global _LIB
    if _LIB is None:
        path = lib_path()
        if not os.path.exists(path):
            raise FAError(-7, "load", f"{path} is not built; run __graft_entry__.build() "
                                       "or python -m exact_io_aware_72_amd.build")
        handle = ctypes.CDLL(path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = handle
    return _LIB


def version() -> str:
    return lib().fa_version().decode()


def _check(status: int, where: str):
    if status != 0:
        raise FAError(status, where, lib().fa_status_string(status).decode())


def workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    return int(lib().fa_backward_workspace_bytes(B, H, N, d))


# ---------------------------------------------------------------------------
# torch-facing wrappers
def _torch():
    import torch
    return torch


def _code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float32:
        return FA_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use torch.bfloat16 or torch.float32")


def _shape(q, *others):
    # Checked on every call, so kept cheap: dtype objects are singletons and
    # get_device() is an int (torch.device comparisons cost microseconds).
    if q.dim() != 4:
        raise ValueError("expected tensors of shape (batch, seq_len, num_heads, head_dim)")
    s, dt, dev = q.shape, q.dtype, q.get_device()
    for t in (q,) + others:
        if t.shape != s:
            raise ValueError(f"shape mismatch: {tuple(t.shape)} vs {tuple(s)}")
        if t.dtype is not dt:
            raise TypeError("q, k, v (and o, dout) must share one dtype")
        if not t.is_cuda or t.get_device() != dev:
            raise ValueError("tensors must live on the same GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    B, N, H, d = s
    return B, N, H, d


def _buf(t, shape, dtype, like, name):
    """A caller-supplied buffer: the kernels trust its size, so shape, dtype,
    device and contiguity are checked here."""
    if (t.shape != tuple(shape) or t.dtype is not dtype or not t.is_cuda
            or t.get_device() != like.get_device() or not t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} "
                         f"on {like.device} (got {tuple(t.shape)}, {t.dtype}, {t.device})")
    return t


def _out(t, shape, dtype, like, name):
    """`t` checked as above, or a new tensor if None."""
    if t is None:
        return _torch().empty(tuple(shape), dtype=dtype, device=like.device)
    return _buf(t, shape, dtype, like, name)


def _stream(t):
    """The current HIP stream of t's device, as an integer handle."""
    torch = _torch()
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return raw(t.get_device())
    return torch.cuda.current_stream(t.device).cuda_stream


def _scale(scale, d):
    return float(1.0 / math.sqrt(d)) if scale is None else float(scale)


def forward(q, k, v, causal=False, dropout_p=0.0, seed=0, scale=None, out=None, lse=None):
    """Returns (o, lse): o like q; lse float32 (B, H, N), natural log."""
    torch = _torch()
    B, N, H, d = _shape(q, k, v)
    o = _out(out, q.shape, q.dtype, q, "out")
    lse_t = _out(lse, (B, H, N), torch.float32, q, "lse")
    st = lib().fa_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse_t.data_ptr(),
                          B, H, N, d, _scale(scale, d), int(bool(causal)), float(dropout_p),
                          int(seed), _stream(q), _code(q))
    _check(st, "fa_forward")
    return o, lse_t


def backward(q, k, v, o, dout, lse, causal=False, dropout_p=0.0, seed=0, scale=None,
             dq=None, dk=None, dv=None, workspace=None):
    """Returns (dq, dk, dv) for L = sum(dout * o)."""
    torch = _torch()
    B, N, H, d = _shape(q, k, v, o, dout)
    _buf(lse, (B, H, N), torch.float32, q, "lse")
    dq = _out(dq, q.shape, q.dtype, q, "dq")
    dk = _out(dk, q.shape, q.dtype, q, "dk")
    dv = _out(dv, q.shape, q.dtype, q, "dv")
    ws = _out(workspace, (B, H, N), torch.float32, q, "workspace")
    st = lib().fa_backward(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                           lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                           ws.data_ptr(), B, H, N, d, _scale(scale, d), int(bool(causal)),
                           float(dropout_p), int(seed), _stream(q), _code(q))
    _check(st, "fa_backward")
    return dq, dk, dv


NOALLOC_MAX_ROWS = 1 << 22  # FA_NOALLOC_MAX_ROWS: B * H * N limit of backward_noalloc


def backward_noalloc(q, k, v, o, dout, lse, dq, dk, dv, causal=False, dropout_p=0.0, seed=0,
                     scale=None):
    """fa_backward_noalloc: the backward pass with D in the library's fixed
    device array (no workspace, nothing allocated by the library). The
    caller passes the output buffers; B * H * N <= NOALLOC_MAX_ROWS. Calls
    that overlap on one GPU race on that array."""
    torch = _torch()
    B, N, H, d = _shape(q, k, v, o, dout)
    _buf(lse, (B, H, N), torch.float32, q, "lse")
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _buf(t, q.shape, q.dtype, q, name)
    st = lib().fa_backward_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                   dout.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                   dv.data_ptr(), B, H, N, d, _scale(scale, d), int(bool(causal)),
                                   float(dropout_p), int(seed), _stream(q), _code(q))
    _check(st, "fa_backward_noalloc")
    return dq, dk, dv


def backward_preprocess(o, dout, workspace=None):
    """Step B1 alone: returns D = rowsum(dout * o) as float32 (B, H, N)."""
    torch = _torch()
    B, N, H, d = _shape(o, dout)
    ws = _out(workspace, (B, H, N), torch.float32, o, "workspace")
    st = lib().fa_backward_preprocess(o.data_ptr(), dout.data_ptr(), ws.data_ptr(), B, H, N, d,
                                      _stream(o), _code(o))
    _check(st, "fa_backward_preprocess")
    return ws


def backward_dkdv(q, k, v, dout, lse, workspace, causal=False, dropout_p=0.0, seed=0, scale=None,
                  dk=None, dv=None):
    """Step B2 alone: returns (dk, dv)."""
    torch = _torch()
    B, N, H, d = _shape(q, k, v, dout)
    _buf(lse, (B, H, N), torch.float32, q, "lse")
    _buf(workspace, (B, H, N), torch.float32, q, "workspace")
    dk = _out(dk, q.shape, q.dtype, q, "dk")
    dv = _out(dv, q.shape, q.dtype, q, "dv")
    st = lib().fa_backward_dkdv(q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(),
                                lse.data_ptr(), workspace.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                B, H, N, d, _scale(scale, d), int(bool(causal)), float(dropout_p),
                                int(seed), _stream(q), _code(q))
    _check(st, "fa_backward_dkdv")
    return dk, dv


def backward_dq(q, k, v, dout, lse, workspace, causal=False, dropout_p=0.0, seed=0, scale=None,
                dq=None):
    """Step B3 alone: returns dq."""
    torch = _torch()
    B, N, H, d = _shape(q, k, v, dout)
    _buf(lse, (B, H, N), torch.float32, q, "lse")
    _buf(workspace, (B, H, N), torch.float32, q, "workspace")
    dq = _out(dq, q.shape, q.dtype, q, "dq")
    st = lib().fa_backward_dq(q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(),
                              lse.data_ptr(), workspace.data_ptr(), dq.data_ptr(), B, H, N, d,
                              _scale(scale, d), int(bool(causal)), float(dropout_p), int(seed),
                              _stream(q), _code(q))
    _check(st, "fa_backward_dq")
    return dq


# ---------------------------------------------------------------------------
# Packed variable-length batches: tensors (total, num_heads, head_dim), sequence
# s in rows cu_seqlens[s] .. cu_seqlens[s+1]-1 (cu_seqlens: int32 on the GPU).
def _shape_varlen(q, *others):
    if q.dim() != 3:
        raise ValueError("expected packed tensors of shape (total_tokens, num_heads, head_dim)")
    for t in (q,) + others:
        if t.shape != q.shape:
            raise ValueError(f"shape mismatch: {tuple(t.shape)} vs {tuple(q.shape)}")
        if t.dtype != q.dtype:
            raise TypeError("q, k, v (and o, dout) must share one dtype")
        if t.device != q.device or t.device.type != "cuda":
            raise ValueError("tensors must live on the same GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    return q.shape


def _cu(cu_seqlens, q):
    torch = _torch()
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be a 1-D int32 tensor of num_seqs + 1 offsets")
    if cu_seqlens.device != q.device or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous tensor on the tensors' GPU")
    return cu_seqlens.numel() - 1


def varlen_workspace_bytes(total: int, H: int, d: int) -> int:
    return int(lib().fa_backward_varlen_workspace_bytes(total, H, d))


def forward_varlen(q, k, v, cu_seqlens, max_seqlen, causal=False, dropout_p=0.0, seed=0,
                   scale=None, out=None, lse=None):
    """Returns (o, lse): o like q; lse float32 (H, total), natural log."""
    torch = _torch()
    total, H, d = _shape_varlen(q, k, v)
    nseq = _cu(cu_seqlens, q)
    o = _out(out, q.shape, q.dtype, q, "out")
    lse_t = _out(lse, (H, total), torch.float32, q, "lse")
    st = lib().fa_forward_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                 lse_t.data_ptr(), cu_seqlens.data_ptr(), nseq, total,
                                 int(max_seqlen), H, d, _scale(scale, d), int(bool(causal)),
                                 float(dropout_p), int(seed), _stream(q), _code(q))
    _check(st, "fa_forward_varlen")
    return o, lse_t


def backward_varlen(q, k, v, o, dout, lse, cu_seqlens, max_seqlen, causal=False, dropout_p=0.0,
                    seed=0, scale=None, dq=None, dk=None, dv=None, workspace=None):
    """Returns (dq, dk, dv) for L = sum(dout * o) over a packed batch."""
    torch = _torch()
    total, H, d = _shape_varlen(q, k, v, o, dout)
    nseq = _cu(cu_seqlens, q)
    _buf(lse, (H, total), torch.float32, q, "lse")
    dq = _out(dq, q.shape, q.dtype, q, "dq")
    dk = _out(dk, q.shape, q.dtype, q, "dk")
    dv = _out(dv, q.shape, q.dtype, q, "dv")
    ws = _out(workspace, (H, total), torch.float32, q, "workspace")
    st = lib().fa_backward_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                  dout.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                  dv.data_ptr(), ws.data_ptr(), cu_seqlens.data_ptr(), nseq, total,
                                  int(max_seqlen), H, d, _scale(scale, d), int(bool(causal)),
                                  float(dropout_p), int(seed), _stream(q), _code(q))
    _check(st, "fa_backward_varlen")
    return dq, dk, dv


# ---------------------------------------------------------------------------
# Block-sparse masks over 128 x 128 blocks of the score matrix.
BLOCK = 128


def _mask_args(mask, q, B, H, N):
    """(pointer, batch stride, head stride) of a uint8 GPU mask shaped
    (nb, nb), (H, nb, nb) or (B, H, nb, nb), nb = ceil(N / 128); the last two
    dimensions must be contiguous, the others may be broadcast (stride 0)."""
    torch = _torch()
    nb = -(-N // BLOCK)
    if mask.dtype != torch.uint8 or mask.device != q.device:
        raise ValueError("block mask must be a uint8 tensor on the tensors' GPU")
    if tuple(mask.shape[-2:]) != (nb, nb) or mask.stride(-1) != 1 or mask.stride(-2) != nb:
        raise ValueError(f"block mask must end in a contiguous ({nb}, {nb}) grid")
    if mask.dim() == 2:
        return mask.data_ptr(), 0, 0
    if mask.dim() == 3 and mask.shape[0] == H:
        return mask.data_ptr(), 0, mask.stride(0)
    if mask.dim() == 4 and tuple(mask.shape[:2]) == (B, H):
        return mask.data_ptr(), mask.stride(0), mask.stride(1)
    raise ValueError("block mask must be (nb, nb), (H, nb, nb) or (B, H, nb, nb)")


def forward_blocksparse(q, k, v, block_mask, causal=False, dropout_p=0.0, seed=0, scale=None,
                        out=None, lse=None):
    """Returns (o, lse) computing only the blocks where block_mask != 0."""
    torch = _torch()
    B, N, H, d = _shape(q, k, v)
    mp, sb, sh = _mask_args(block_mask, q, B, H, N)
    o = _out(out, q.shape, q.dtype, q, "out")
    lse_t = _out(lse, (B, H, N), torch.float32, q, "lse")
    st = lib().fa_forward_blocksparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                      lse_t.data_ptr(), mp, sb, sh, B, H, N, d, _scale(scale, d),
                                      int(bool(causal)), float(dropout_p), int(seed), _stream(q),
                                      _code(q))
    _check(st, "fa_forward_blocksparse")
    return o, lse_t


def backward_blocksparse(q, k, v, o, dout, lse, block_mask, causal=False, dropout_p=0.0, seed=0,
                         scale=None, dq=None, dk=None, dv=None, workspace=None):
    """Returns (dq, dk, dv) for L = sum(dout * o) under the same block mask."""
    torch = _torch()
    B, N, H, d = _shape(q, k, v, o, dout)
    mp, sb, sh = _mask_args(block_mask, q, B, H, N)
    _buf(lse, (B, H, N), torch.float32, q, "lse")
    dq = _out(dq, q.shape, q.dtype, q, "dq")
    dk = _out(dk, q.shape, q.dtype, q, "dk")
    dv = _out(dv, q.shape, q.dtype, q, "dv")
    ws = _out(workspace, (B, H, N), torch.float32, q, "workspace")
    st = lib().fa_backward_blocksparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                       dout.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                       dv.data_ptr(), ws.data_ptr(), mp, sb, sh, B, H, N, d,
                                       _scale(scale, d), int(bool(causal)), float(dropout_p),
                                       int(seed), _stream(q), _code(q))
    _check(st, "fa_backward_blocksparse")
    return dq, dk, dv


# ---------------------------------------------------------------------------
# Split-KV forward: queries (B, Nq, H, d) against keys/values (B, Nk, H, d).
def splitkv_num_splits(B, H, Nq, Nk, d) -> int:
    return int(lib().fa_splitkv_num_splits(B, H, Nq, Nk, d))


def splitkv_workspace_bytes(B, H, Nq, d, num_splits) -> int:
    return int(lib().fa_forward_splitkv_workspace_bytes(B, H, Nq, d, num_splits))


def forward_splitkv(q, k, v, causal=False, num_splits=0, scale=None, out=None, lse=None,
                    workspace=None):
    """Returns (o, lse) with o like q and lse float32 (B, H, Nq). Causal
    queries are the last Nq positions of the Nk keys. num_splits = 0 picks the
    count with splitkv_num_splits."""
    torch = _torch()
    B, Nq, H, d = _shape(q)
    Bk, Nk, Hk, dk = _shape(k, v)
    if (Bk, Hk, dk) != (B, H, d) or k.dtype != q.dtype or k.device != q.device:
        raise ValueError("k, v must be (B, Nk, H, d) like q on the same GPU")
    ns = int(num_splits) if num_splits else splitkv_num_splits(B, H, Nq, Nk, d)
    if ns < 1:
        raise FAError(-2, "fa_forward_splitkv", "invalid shape")
    o = _out(out, q.shape, q.dtype, q, "out")
    lse_t = _out(lse, (B, H, Nq), torch.float32, q, "lse")
    nbytes = splitkv_workspace_bytes(B, H, Nq, d, ns)
    if workspace is None:
        workspace = torch.empty(nbytes // 4, dtype=torch.float32, device=q.device)
    elif (workspace.dtype != torch.float32 or workspace.device != q.device
          or not workspace.is_contiguous() or workspace.numel() * 4 < nbytes):
        raise ValueError(f"workspace must be a contiguous float32 GPU tensor of >= {nbytes} bytes")
    st = lib().fa_forward_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                  lse_t.data_ptr(), workspace.data_ptr(), B, H, Nq, Nk, d,
                                  _scale(scale, d), int(bool(causal)), ns, _stream(q), _code(q))
    _check(st, "fa_forward_splitkv")
    return o, lse_t


# ---------------------------------------------------------------------------
# FP8 scores: per-block quantised Q and K (OCP E4M3 bytes) with fp32 scales.
def quantize_fp8(x, block_rows, out=None, scales=None):
    """x bf16 (B, N, H, d) -> (uint8 codes like x, float32 scales (B, H, nblk))."""
    torch = _torch()
    B, N, H, d = _shape(x)
    xq = _out(out, x.shape, torch.uint8, x, "out")
    nblk = -(-N // int(block_rows))
    sc = _out(scales, (B, H, nblk), torch.float32, x, "scales")
    st = lib().fa_quantize_fp8(x.data_ptr(), xq.data_ptr(), sc.data_ptr(), B, N, H, d,
                               int(block_rows), _stream(x))
    _check(st, "fa_quantize_fp8")
    return xq, sc


def forward_fp8_quantized(q8, k8, v, q_scale, k_scale, causal=False, scale=None, out=None, lse=None):
    """Forward with FP8 scores from pre-quantised q8 (128-row blocks) and k8
    (64-row blocks); v bf16 (B, N, H, d). Returns (o, lse)."""
    torch = _torch()
    B, N, H, d = _shape(v)
    _buf(q8, v.shape, torch.uint8, v, "q8")
    _buf(k8, v.shape, torch.uint8, v, "k8")
    _buf(q_scale, (B, H, -(-N // 128)), torch.float32, v, "q_scale")
    _buf(k_scale, (B, H, -(-N // 64)), torch.float32, v, "k_scale")
    o = _out(out, v.shape, v.dtype, v, "out")
    lse_t = _out(lse, (B, H, N), torch.float32, v, "lse")
    st = lib().fa_forward_fp8(q8.data_ptr(), k8.data_ptr(), v.data_ptr(), o.data_ptr(),
                              lse_t.data_ptr(), q_scale.data_ptr(), k_scale.data_ptr(), B, H, N, d,
                              _scale(scale, d), int(bool(causal)), _stream(v))
    _check(st, "fa_forward_fp8")
    return o, lse_t


def forward_fp8(q, k, v, causal=False, scale=None):
    """Quantises q (per 128 rows) and k (per 64 rows) and runs the FP8-score
    forward. Returns (o, lse)."""
    q8, qs = quantize_fp8(q, 128)
    k8, ks = quantize_fp8(k, 64)
    return forward_fp8_quantized(q8, k8, v, qs, ks, causal, scale)


def dropout_mask(seed, b, h, H, dropout_p, row0, col0, rows, cols, device="cuda"):
    """Keep mask (uint8, rows x cols) of head (b, h), from the kernels' hash."""
    torch = _torch()
    out = torch.empty((rows, cols), dtype=torch.uint8, device=device)
    st = lib().fa_dropout_mask(int(seed), b, h, H, float(dropout_p), row0, col0, rows, cols,
                               out.data_ptr(), _stream(out))
    _check(st, "fa_dropout_mask")
    return out


def _autograd_function():
    torch = _torch()

    class FlashAttnFunction(torch.autograd.Function):
        """Autograd wrapper: forward saves (q, k, v, o, lse); backward
        recomputes the attention probabilities from them. With dropout and
        seed=None, each forward call draws a fresh seed (draw_seed), so
        every call gets a new keep mask; the seed is kept on the autograd
        node (its `seed` attribute) and the backward pass regenerates the
        same mask from it."""

        @staticmethod
        def forward(ctx, q, k, v, causal=False, dropout_p=0.0, seed=None, scale=None):
            q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
            if seed is None:
                seed = draw_seed() if dropout_p > 0 else 0
            o, lse = forward(q, k, v, causal, dropout_p, seed, scale)
            ctx.save_for_backward(q, k, v, o, lse)
            ctx.args = (causal, dropout_p, seed, scale)
            ctx.seed = seed
            return o

        @staticmethod
        def backward(ctx, do):
            q, k, v, o, lse = ctx.saved_tensors
            causal, dropout_p, seed, scale = ctx.args
            dq, dk, dv = backward(q, k, v, o, do.contiguous(), lse, causal, dropout_p, seed, scale)
            return dq, dk, dv, None, None, None, None

    return FlashAttnFunction


class _Lazy:
    _fn = None

    def __get__(self, obj, owner):
        if _Lazy._fn is None:
            _Lazy._fn = _autograd_function()
        return _Lazy._fn


class _Namespace:
    FlashAttnFunction = _Lazy()


def __getattr__(name):
    if name == "FlashAttnFunction":
        return _Namespace.FlashAttnFunction
    raise AttributeError(name)


def draw_seed():
    """A dropout seed in [0, 2^63) drawn from torch's default CPU generator
    (reproducible under torch.manual_seed)."""
    torch = _torch()
    return int(torch.randint(0, 2 ** 63 - 1, (1,), dtype=torch.int64).item())


def flash_attention(q, k, v, causal=False, dropout_p=0.0, seed=None, scale=None):
    """O = softmax(q k^T * scale) v over (batch, seq_len, num_heads, head_dim)
    tensors, differentiable through FlashAttnFunction. With dropout and
    seed=None every call draws a fresh seed (see FlashAttnFunction); pass a
    seed to fix the keep mask."""
    return _Namespace.FlashAttnFunction.apply(q, k, v, causal, dropout_p, seed, scale)
