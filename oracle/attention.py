"""Plain fp64 exact attention, forward and backward, on the CPU.

Test infrastructure only (see the package docstring). This is the standard
(unfused) attention the pages compare against, written out: it materialises the score
matrix S and the probability matrix P (as described in "How FlashAttention
Optimizes GPU Memory for Fast AI Training", section "The Flaw in Standard
Attention"), row panel by row panel so that long sequences fit in host memory.
Softmax acts row by row, so a row panel is exactly the rows of the full
matrices; sums over rows (dK, dV) are split across panels and added.

Definitions followed ("FlashAttention for Efficient Training" unless noted):
  * O = softmax(Q K^T / sqrt(d_k)) V                    (section 1.1, section 3.1)
  * S_ij = scale * Q_i . K_j, with scale = 1/sqrt(d_k)  (section 3.1, "Tiling and
    Memory Hierarchy"); the kernel's fp32 scale value is used as given
  * causal: S_ij = -inf where the key j lies after the query i; masked scores
    contribute nothing (the -inf masking of section 5.2 "Handling Variable
    Sequence Lengths"; causal use in section 5.1 "Memory-Efficient Backward
    Pass"). Queries and keys share positions 0..N-1 (top-left aligned).
  * block-sparse: with a mask over 128 x 128 blocks of S, the scores of a
    zero block are -inf and take no part in the softmax; the page computes
    only the nonzero blocks (section 3.2 "Block-Sparse Attention Support").
    A row left with no finite score gets P = 0, O = 0 and LSE = -inf
  * queries against a longer key sequence (forward_cross): under the causal
    mask the Nq queries are the last Nq of the Nk positions (a reading; the
    pages only use queries and keys of one length)
  * numerically stable softmax: subtract the row max before exp (section 6.2
    "Hardware-Specific Optimizations")
  * per-row logsumexp LSE_i = log sum_j exp(S_ij), natural log (section 3.2,
    "Precision Handling and Numerical Stability", log_softmax = x - logsumexp)
  * dropout on P (section 3.1 "Fused Kernel Design"): P~ = P * Z / (1 - p),
    with Z the keep mask of dropout_hash.py; the row statistics use the
    undropped P
  * dV = P~^T dO (section 3.2 "Integration with Autograd Engines"); dQ and dK
    follow from the chain rule, which the same section leaves to the reader:
        dP~ = dO V^T,  dP = dP~ * Z / (1 - p),  D_i = sum_j P_ij dP_ij,
        dS = P * (dP - D),  dQ = scale * dS K,  dK = scale * dS^T Q.
    D_i also equals sum_c dO_ic O_ic; both are computed and must agree.
    A recompute backward that is handed the forward's output reads D from
    that stored O, not from P * dP; with backward(..., o=stored), D_i is
    sum_c dO_ic o_ic of the given o, and dQ, dK (linear in D) are what that
    backward computes exactly. dV does not depend on D.
    (The explicit dQ formulas printed in sections 2.1, 2.2, 4.1 and 5.1 of
    that page drop the D term and the K factor and are not used.)

Arrays use the (batch, seq_len, num_heads, head_dim) layout of the page's
PyTorch usage example (section 4.2); LSE is returned as [B, H, N].
"""
from __future__ import annotations

import numpy as np

from .dropout_hash import keep_mask

_PANEL = 256


def attention_scores(q, k, scale, causal, row0=0):
    """S = scale * q k^T for query rows row0.. (q: R x d, k: M x d), with the
    causal mask applied as -inf where key index > query index."""
    s = float(scale) * (np.asarray(q, np.float64) @ np.asarray(k, np.float64).T)
    if causal:
        qi = row0 + np.arange(s.shape[0])[:, None]
        kj = np.arange(s.shape[1])[None, :]
        s = np.where(kj > qi, -np.inf, s)
    return s


BLOCK = 128  # side of a block-sparse mask block


def apply_block_mask(s, bmask, rows, cols):
    """Block-sparse attention ("FlashAttention for Efficient Training",
    section 3.2 "Block-Sparse Attention Support"): scores of query i and key j
    whose block bmask[i // 128][j // 128] is zero are -inf, i.e. not part of
    the softmax. `rows`, `cols` are the positions of s's rows and columns."""
    if bmask is None:
        return s
    keep = np.asarray(bmask, bool)[np.asarray(rows) // BLOCK][:, np.asarray(cols) // BLOCK]
    return np.where(keep, s, -np.inf)


def softmax_stats(s):
    """Row max m, row sum l = sum exp(s - m), and LSE = m + log(l).
    A row with no unmasked entry gets LSE = -inf."""
    m = np.max(s, axis=1)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    l = np.sum(np.exp(s - m_safe[:, None]), axis=1)
    with np.errstate(divide="ignore"):
        lse = np.where(finite, m_safe + np.log(l), -np.inf)
    return m, l, lse


def attention_probs(s, lse):
    """P = exp(S - LSE) row by row; fully masked rows give zeros."""
    lse_safe = np.where(np.isfinite(lse), lse, 0.0)
    p = np.exp(s - lse_safe[:, None])
    return np.where(np.isfinite(lse)[:, None], p, 0.0)


def _heads(B, H, heads):
    return [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)


def _panel_cols(causal, r1, N):
    # Under the causal mask, rows < r1 see only keys < r1; later columns are
    # all -inf and contribute exactly zero, so they are left out.
    return min(r1, N) if causal else N


def _dropped(p_mat, seed, b, h, H, dropout_p, rows, cols):
    if dropout_p == 0.0:
        return p_mat
    z = keep_mask(seed, b, h, H, dropout_p, rows, cols)
    r = 1.0 / (1.0 - float(np.float32(dropout_p)))
    return p_mat * z * r


def head_forward(qh, kh, vh, scale, causal, dropout_p, seed, b, h, H, panel=_PANEL, bmask=None,
                 row_offset=0, hash_row_offset=0):
    """One head of one sequence: qh is [n, d], kh, vh are [m, d] float64
    arrays, (b, h, H) key the dropout hash, bmask is this head's block mask or
    None. Query i sits at key position row_offset + i for the causal mask,
    and is row hash_row_offset + i of the dropout hash and the block mask (a
    panel of rows cut from a larger square problem passes its first row as
    both offsets).
    Returns (O [n, d], LSE [n]); rows with no unmasked key get O = 0,
    LSE = -inf."""
    n = qh.shape[0]
    o = np.zeros((n, vh.shape[1]), np.float64)
    lse = np.zeros(n, np.float64)
    for r0 in range(0, n, panel):
        r1 = min(r0 + panel, n)
        nc = _panel_cols(causal, row_offset + r1, kh.shape[0])
        s = attention_scores(qh[r0:r1], kh[:nc], scale, causal, row_offset + r0)
        rows = np.arange(hash_row_offset + r0, hash_row_offset + r1)
        s = apply_block_mask(s, bmask, rows, np.arange(nc))
        _, _, l_ = softmax_stats(s)
        p = attention_probs(s, l_)
        pt = _dropped(p, seed, b, h, H, dropout_p, rows, np.arange(nc))
        o[r0:r1] = pt @ vh[:nc]
        lse[r0:r1] = l_
    return o, lse


def head_backward(qh, kh, vh, doh, scale, causal, dropout_p, seed, b, h, H, panel=_PANEL,
                  check_d=True, bmask=None, oh=None, row_offset=0, hash_row_offset=0):
    """One head of one sequence (qh, doh [n, d], kh, vh [m, d] float64
    arrays). Returns (dQ, dK, dV, D) with D = rowsum(P * dP) of length n, or,
    with a given output oh [n, d], D = rowsum(dO * oh). Query i sits at key
    position row_offset + i and is row hash_row_offset + i of the dropout
    hash and the block mask, as in head_forward: a panel of rows cut from a
    larger problem gets its own rows of dQ and D exactly, and those rows'
    share of dK and dV."""
    n = qh.shape[0]
    dq = np.zeros_like(qh)
    dk = np.zeros_like(kh)
    dv = np.zeros_like(vh)
    dd = np.zeros(n, np.float64)
    keep_r = 1.0 / (1.0 - float(np.float32(dropout_p)))
    for r0 in range(0, n, panel):
        r1 = min(r0 + panel, n)
        rows = np.arange(hash_row_offset + r0, hash_row_offset + r1)
        nc = _panel_cols(causal, row_offset + r1, kh.shape[0])
        cols = np.arange(nc)
        s = attention_scores(qh[r0:r1], kh[:nc], scale, causal, row_offset + r0)
        s = apply_block_mask(s, bmask, rows, cols)
        _, _, l_ = softmax_stats(s)
        p = attention_probs(s, l_)
        if dropout_p != 0.0:
            z = keep_mask(seed, b, h, H, dropout_p, rows, cols)
            pt = p * z * keep_r
        else:
            z = None
            pt = p
        dv[:nc] += pt.T @ doh[r0:r1]
        dpt = doh[r0:r1] @ vh[:nc].T
        dp = dpt * z * keep_r if z is not None else dpt
        d_row = np.sum(p * dp, axis=1)
        if oh is not None:
            d_row = np.sum(doh[r0:r1] * oh[r0:r1], axis=1)
        elif check_d:
            o_rows = pt @ vh[:nc]
            d_alt = np.sum(doh[r0:r1] * o_rows, axis=1)
            if not np.allclose(d_row, d_alt, rtol=1e-9, atol=1e-9):
                raise AssertionError("rowsum(P*dP) != rowsum(dO*O)")
        ds = p * (dp - d_row[:, None])
        dq[r0:r1] = float(scale) * (ds @ kh[:nc])
        dk[:nc] += float(scale) * (ds.T @ qh[r0:r1])
        dd[r0:r1] = d_row
    return dq, dk, dv, dd


def forward(q, k, v, scale, causal, dropout_p=0.0, seed=0, heads=None, panel=_PANEL,
            block_mask=None):
    """Returns (O [B,N,H,d] float64, LSE [B,H,N] float64).
    Only the (b, h) pairs in `heads` are computed (others are left zero).
    block_mask: None, or [B,H,nb,nb] (nb = ceil(N/128)), nonzero = computed."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, N, H, d = q.shape
    o = np.zeros((B, N, H, v.shape[3]), np.float64)
    lse = np.zeros((B, H, N), np.float64)
    for b, h in _heads(B, H, heads):
        o[b, :, h, :], lse[b, h, :] = head_forward(
            q[b, :, h, :], k[b, :, h, :], v[b, :, h, :], scale, causal, dropout_p, seed, b, h, H,
            panel, None if block_mask is None else block_mask[b][h])
    return o, lse


def forward_cross(q, k, v, scale, causal, panel=_PANEL):
    """Queries [B, Nq, H, d] against keys and values [B, Nk, H, d]. Under the
    causal mask the queries are the last Nq of the Nk positions (query i at
    position Nk - Nq + i), so query i sees keys j <= i + Nk - Nq; with
    Nq = Nk this is forward(). Returns (O [B, Nq, H, d], LSE [B, H, Nq])."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, Nq, H, _ = q.shape
    Nk = k.shape[1]
    off = Nk - Nq if causal else 0
    o = np.zeros((B, Nq, H, v.shape[3]), np.float64)
    lse = np.zeros((B, H, Nq), np.float64)
    for b in range(B):
        for h in range(H):
            o[b, :, h, :], lse[b, h, :] = head_forward(q[b, :, h, :], k[b, :, h, :], v[b, :, h, :],
                                                       scale, causal, 0.0, 0, b, h, H, panel,
                                                       None, off)
    return o, lse


def backward(q, k, v, do, scale, causal, dropout_p=0.0, seed=0, heads=None, panel=_PANEL,
             check_d=True, block_mask=None, o=None):
    """Returns (dQ, dK, dV, D) for L = sum(dO * O), float64.
    D is [B,H,N] = rowsum(P * dP). With check_d, also checks D against
    rowsum(dO * O) computed from this module's own forward output. With o
    ([B,N,H,d], e.g. the forward output as stored in a narrower type), D is
    rowsum(dO * o) instead and the check is skipped."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    B, N, H, d = q.shape
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dd = np.zeros((B, H, N), np.float64)
    o = None if o is None else np.asarray(o, np.float64)
    for b, h in _heads(B, H, heads):
        dq[b, :, h, :], dk[b, :, h, :], dv[b, :, h, :], dd[b, h, :] = head_backward(
            q[b, :, h, :], k[b, :, h, :], v[b, :, h, :], do[b, :, h, :], scale, causal,
            dropout_p, seed, b, h, H, panel, check_d,
            None if block_mask is None else block_mask[b][h],
            None if o is None else o[b, :, h, :])
    return dq, dk, dv, dd


def sampled_head(q, k, v, do, scale, causal, dropout_p, seed, b, h, rows, cols, panel=_PANEL,
                 bmask=None):
    """Oracle values for one head (b, h) at selected query rows and key columns.

    Computes LSE and O for every row of the head (needed by any key column),
    then O, LSE and dQ at `rows`, and dK and dV at `cols`, from the same
    definitions as forward()/backward(). Returns a dict of float64 arrays:
      o[rows, d], lse[rows], dq[rows, d], dk[cols, d], dv[cols, d], D[rows].
    q, k, v, do are [B, N, H, d] arrays (any float dtype); bmask is this
    head's block mask or None.
    """
    H = q.shape[2]
    qh = np.asarray(q[b, :, h, :], np.float64)
    kh = np.asarray(k[b, :, h, :], np.float64)
    vh = np.asarray(v[b, :, h, :], np.float64)
    doh = np.asarray(do[b, :, h, :], np.float64) if do is not None else None
    N = qh.shape[0]
    rows = np.asarray(rows, np.int64)
    cols = np.asarray(cols, np.int64)
    keep_r = 1.0 / (1.0 - float(np.float32(dropout_p)))

    # Full-head statistics: LSE and O for all rows, D for all rows.
    lse_all = np.zeros(N)
    o_all = np.zeros((N, vh.shape[1]))
    for r0 in range(0, N, panel):
        r1 = min(r0 + panel, N)
        nc = _panel_cols(causal, r1, N)
        s = attention_scores(qh[r0:r1], kh[:nc], scale, causal, r0)
        s = apply_block_mask(s, bmask, np.arange(r0, r1), np.arange(nc))
        _, _, l_ = softmax_stats(s)
        p = attention_probs(s, l_)
        pt = _dropped(p, seed, b, h, H, dropout_p, np.arange(r0, r1), np.arange(nc))
        o_all[r0:r1] = pt @ vh[:nc]
        lse_all[r0:r1] = l_
    out = {"o": o_all[rows], "lse": lse_all[rows]}
    if doh is None:
        return out
    d_all = np.sum(doh * o_all, axis=1)  # D_i = sum_c dO_ic O_ic

    # dQ at the sampled rows: one row of S, P, dP, dS each.
    s = attention_scores(qh[rows], kh, scale, False)
    if causal:
        s = np.where(np.arange(N)[None, :] > rows[:, None], -np.inf, s)
    s = apply_block_mask(s, bmask, rows, np.arange(N))
    p = attention_probs(s, lse_all[rows])
    dpt = doh[rows] @ vh.T
    if dropout_p != 0.0:
        z = keep_mask(seed, b, h, H, dropout_p, rows, np.arange(N))
        dp = dpt * z * keep_r
    else:
        dp = dpt
    d_rows = np.sum(p * dp, axis=1)
    ds = p * (dp - d_rows[:, None])
    out["dq"] = float(scale) * (ds @ kh)
    out["D"] = d_rows

    # dK, dV at the sampled columns: one column of S, P, dP, dS each.
    st = attention_scores(kh[cols], qh, scale, False).T  # [N, len(cols)] = scale q k^T
    if causal:
        st = np.where(cols[None, :] > np.arange(N)[:, None], -np.inf, st)
    st = apply_block_mask(st, bmask, np.arange(N), cols)
    pc = attention_probs(st, lse_all)
    dpct = doh @ vh[cols].T
    if dropout_p != 0.0:
        zc = keep_mask(seed, b, h, H, dropout_p, np.arange(N), cols)
        ptc = pc * zc * keep_r
        dpc = dpct * zc * keep_r
    else:
        ptc = pc
        dpc = dpct
    dsc = pc * (dpc - d_all[:, None])
    out["dv"] = ptc.T @ doh
    out["dk"] = float(scale) * (dsc.T @ qh)
    return out
