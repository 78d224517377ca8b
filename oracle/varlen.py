"""Plain fp64 attention over packed batches of sequences of different lengths.

Test infrastructure only (see the package docstring).

"FlashAttention for Efficient Training", section 5.2 "Handling Variable
Sequence Lengths", defines the scores of a padded batch: a query of a sequence
of length L scores the keys j < L (0-based) as usual and every later key as
-inf. Those -inf scores contribute nothing to the softmax, so each sequence's
outputs are plain attention over that sequence alone, which is what this
module computes; padded query rows are not outputs. Sequences are packed back
to back without padding: sequence s owns rows cu_seqlens[s] .. cu_seqlens[s+1]-1
of [total, H, d] arrays, and its positions restart at 0 (causal masking and the
dropout hash use positions within the sequence, with the sequence index s in
the hash's batch slot). Statistics (LSE, D) are returned as [H, total].
"""
from __future__ import annotations

import numpy as np

from .attention import head_backward, head_forward


def _spans(cu_seqlens):
    cu = np.asarray(cu_seqlens, np.int64)
    if cu.ndim != 1 or cu.size < 1 or cu[0] != 0 or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must start at 0 and not decrease")
    return [(s, int(cu[s]), int(cu[s + 1])) for s in range(cu.size - 1)]


def forward_varlen(q, k, v, cu_seqlens, scale, causal, dropout_p=0.0, seed=0):
    """q, k, v: [total, H, d]. Returns (O [total, H, d], LSE [H, total]), float64."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    total, H, _ = q.shape
    o = np.zeros((total, H, v.shape[2]), np.float64)
    lse = np.zeros((H, total), np.float64)
    for s, a, e in _spans(cu_seqlens):
        if e == a:
            continue
        for h in range(H):
            o[a:e, h], lse[h, a:e] = head_forward(q[a:e, h], k[a:e, h], v[a:e, h], scale, causal,
                                                  dropout_p, seed, s, h, H)
    return o, lse


def backward_varlen(q, k, v, do, cu_seqlens, scale, causal, dropout_p=0.0, seed=0, o=None):
    """Returns (dQ, dK, dV [total, H, d], D [H, total]) for L = sum(dO * O).
    With o ([total, H, d], the forward output as a backward is handed it), D
    is rowsum(dO * o), as in attention.backward."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    o = None if o is None else np.asarray(o, np.float64)
    total, H, _ = q.shape
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dd = np.zeros((H, total), np.float64)
    for s, a, e in _spans(cu_seqlens):
        if e == a:
            continue
        for h in range(H):
            dq[a:e, h], dk[a:e, h], dv[a:e, h], dd[h, a:e] = head_backward(
                q[a:e, h], k[a:e, h], v[a:e, h], do[a:e, h], scale, causal, dropout_p, seed, s, h,
                H, oh=None if o is None else o[a:e, h])
    return dq, dk, dv, dd
