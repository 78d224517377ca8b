"""Dropout keep mask as a counter hash of (seed, b, h, row, col).

The pages fuse dropout on the attention probabilities into the kernel
("FlashAttention for Efficient Training" section 3.1 "Fused Kernel Design";
"How FlashAttention Optimizes GPU Memory for Fast AI Training", section
"3. Kernel Fusion") but name no random generator. The generator used here is
a reading, fixed so that the forward and the backward pass regenerate the
same mask from a seed instead of storing N x N bits:

  G         = 0x9E3779B97F4A7C15                (odd, floor(2^64 / golden ratio))
  mix64(z)  = SplitMix64 output function (Steele, Lea, Flood, "Fast Splittable
              Pseudorandom Number Generators", OOPSLA 2014), arithmetic mod 2^64:
                z ^= z >> 30; z *= 0xBF58476D1CE4E5B9
                z ^= z >> 27; z *= 0x94D049BB133111EB
                z ^= z >> 31
  fmix32(x) = MurmurHash3 32-bit finalizer (A. Appleby, public domain), mod 2^32:
                x ^= x >> 16; x *= 0x85EBCA6B
                x ^= x >> 13; x *= 0xC2B2AE35
                x ^= x >> 16
  K_bh      = mix64(seed + G * (1 + b*H + h))
  A_i       = low 32 bits of mix64(K_bh + G * (2*i + 1))     (one per query row)
  B_j       = low 32 bits of mix64(K_bh + G * (2*j + 2))     (one per key column)
  w_ij      = fmix32(A_i XOR B_j)
  T         = floor(p * 2^32), p taken as the float32 value the kernel receives
  keep_ij   = (w_ij >= T)

The keep probability is exactly 1 - T / 2^32. Kept probabilities are scaled
by 1 / (1 - p).
"""
from __future__ import annotations

import numpy as np

MASK64 = (1 << 64) - 1
GOLDEN_GAMMA = 0x9E3779B97F4A7C15
_SM_M1 = np.uint64(0xBF58476D1CE4E5B9)
_SM_M2 = np.uint64(0x94D049BB133111EB)
_MM_C1 = np.uint32(0x85EBCA6B)
_MM_C2 = np.uint32(0xC2B2AE35)


def mix64(z):
    """SplitMix64 output function on uint64 values (wraps mod 2^64)."""
    z = np.asarray(z, dtype=np.uint64).copy()
    with np.errstate(over="ignore"):
        z ^= z >> np.uint64(30)
        z *= _SM_M1
        z ^= z >> np.uint64(27)
        z *= _SM_M2
        z ^= z >> np.uint64(31)
    return z


def fmix32(x):
    """MurmurHash3 fmix32 on uint32 values (wraps mod 2^32)."""
    x = np.asarray(x, dtype=np.uint32).copy()
    with np.errstate(over="ignore"):
        x ^= x >> np.uint32(16)
        x *= _MM_C1
        x ^= x >> np.uint32(13)
        x *= _MM_C2
        x ^= x >> np.uint32(16)
    return x


def head_key(seed: int, b: int, h: int, H: int) -> int:
    """K_bh = mix64(seed + G * (1 + b*H + h)) as a Python int."""
    z = (int(seed) + GOLDEN_GAMMA * (1 + b * H + h)) & MASK64
    return int(mix64(np.array([z], dtype=np.uint64))[0])


def _keyed(key: int, idx, odd: int):
    idx = np.asarray(idx, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(key) + np.uint64(GOLDEN_GAMMA) * (np.uint64(2) * idx + np.uint64(odd))
    return (mix64(z) & np.uint64(0xFFFFFFFF)).astype(np.uint32)


def row_keys(key: int, rows):
    """A_i = lo32(mix64(K_bh + G*(2i+1)))."""
    return _keyed(key, rows, 1)


def col_keys(key: int, cols):
    """B_j = lo32(mix64(K_bh + G*(2j+2)))."""
    return _keyed(key, cols, 2)


def keep_threshold(p: float) -> int:
    """T = floor(p_f32 * 2^32), exact in float64."""
    pf = float(np.float32(p))
    if not (0.0 <= pf < 1.0):
        raise ValueError("dropout probability must lie in [0, 1)")
    return int(np.floor(pf * 4294967296.0))


def keep_mask(seed: int, b: int, h: int, H: int, p: float, rows, cols):
    """Boolean keep mask, shape (len(rows), len(cols)), for head (b, h)."""
    key = head_key(seed, b, h, H)
    a = row_keys(key, rows)
    c = col_keys(key, cols)
    w = fmix32(a[:, None] ^ c[None, :])
    return w >= np.uint32(keep_threshold(p))
