"""FP8 (OCP E4M3) per-block quantisation and attention with quantised
scores, in fp64 on the CPU. Test infrastructure only (see the package
docstring).

"FlashAttention for Efficient Training", section 6.2 "Quantization and
Mixed-Precision Approaches", writes the scores of quantised attention as
Q K^T ~ S_Q * Qh * Kh^T * S_K, with quantised queries and keys Qh, Kh and
their scaling factors. Readings fixed here (the page names neither format
nor granularity):
  * format: OCP 8-bit floating point E4M3 (Open Compute Project "OCP 8-bit
    Floating Point Specification (OFP8)"): 1 sign bit, 4 exponent bits with
    bias 7, 3 mantissa bits; largest finite value 448, subnormals down to
    2^-9; rounding to nearest, ties to even;
  * scales: one per (b, h) and block of rows -- 128 query rows, 64 key
    rows -- set from the block's largest magnitude: scale = amax / 448,
    codes = E4M3(x * (448 / amax)), each step in fp32; an all-zero block
    has scale 1 and zero codes;
  * the scores are then exact products of the dequantised values
    (code * scale), and everything after the scores is the plain attention
    of attention.py.
"""
from __future__ import annotations

import numpy as np

from .attention import forward

E4M3_MAX = 448.0
Q_BLOCK = 128
K_BLOCK = 64


def e4m3_round(y):
    """Round to the nearest E4M3 value, ties to even; magnitudes above 448
    (possible here only as fp32 overshoot of 448 by an ulp) give 448."""
    y = np.asarray(y, np.float64)
    a = np.abs(y)
    # exponent of the binade; subnormals share the spacing of the 2^-6 binade
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.clip(e, -6, 8)
    step = np.exp2(e - 3)  # 3 mantissa bits
    r = np.round(a / step) * step  # numpy rounds halves to even
    return np.sign(y) * np.minimum(r, E4M3_MAX)


def quantize(x, block_rows):
    """x: [B, N, H, d] values (float32-exact). Returns (codes as float64 E4M3
    values [B, N, H, d], scales float32 [B, H, ceil(N / block_rows)])."""
    x = np.asarray(x, np.float32)
    B, N, H, d = x.shape
    nblk = -(-N // block_rows)
    codes = np.zeros(x.shape, np.float64)
    scales = np.ones((B, H, nblk), np.float32)
    for b in range(B):
        for h in range(H):
            for j in range(nblk):
                rows = slice(j * block_rows, min(N, (j + 1) * block_rows))
                blk = x[b, rows, h, :]
                amax = np.float32(np.max(np.abs(blk)))
                if amax == 0:
                    continue
                inv = np.float32(E4M3_MAX) / amax  # fp32 division
                codes[b, rows, h, :] = e4m3_round(blk * inv)  # fp32 product, then rounding
                scales[b, h, j] = amax / np.float32(E4M3_MAX)
    return codes, scales


def dequantize(codes, scales, block_rows):
    """codes * scale of each row's block, in fp64 (exact)."""
    rep = np.repeat(np.asarray(scales, np.float64), block_rows, axis=2)[:, :, :codes.shape[1]]
    return np.asarray(codes, np.float64) * rep.transpose(0, 2, 1)[:, :, :, None]


def forward_fp8(q, k, v, scale, causal):
    """Attention with scores from per-block E4M3 queries (128-row blocks) and
    keys (64-row blocks); v as given. Returns (O [B,N,H,d], LSE [B,H,N])."""
    cq, sq = quantize(q, Q_BLOCK)
    ck, sk = quantize(k, K_BLOCK)
    return forward(dequantize(cq, sq, Q_BLOCK), dequantize(ck, sk, K_BLOCK), v, scale, causal)
