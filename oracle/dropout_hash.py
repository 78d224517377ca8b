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
  B_c       = low 32 bits of mix64(K_bh + G * (2*c + 2))     (one per pair of key
              columns j = 2c, 2c + 1)
  w_ic      = fmix32(A_i XOR B_c)
  u_ij      = low 16 bits of w_ic for even j, high 16 bits for odd j
  T         = floor(p * 2^16), p taken as the float32 value the kernel receives
  keep_ij   = (u_ij >= T)

One hash thus gives the draws of two neighbouring keys of a row, each a
16-bit uniform; the keep probability is exactly 1 - T / 2^16, within 2^-16 of
1 - p. Kept probabilities are scaled by 1 / (1 - p).
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


def pair_keys(key: int, pairs):
    """B_c = lo32(mix64(K_bh + G*(2c+2))), c indexing pairs of key columns."""
    return _keyed(key, pairs, 2)


def keep_threshold(p: float) -> int:
    """T = floor(p_f32 * 2^16), exact in float64. A p in (0, 2^-16) would
    give T = 0 (nothing dropped, yet kept values rescaled) and is rejected."""
    pf = float(np.float32(p))
    if not (0.0 <= pf < 1.0):
        raise ValueError("dropout probability must lie in [0, 1)")
    if 0.0 < pf < 2.0 ** -16:
        raise ValueError("dropout probability below 2^-16, the draws' resolution")
    return int(np.floor(pf * 65536.0))


def uniforms16(seed: int, b: int, h: int, H: int, rows, cols):
    """The 16-bit draws u_ij, shape (len(rows), len(cols)), for head (b, h)."""
    key = head_key(seed, b, h, H)
    cols = np.asarray(cols, dtype=np.int64)
    a = row_keys(key, rows)
    c = pair_keys(key, cols // 2)
    w = fmix32(a[:, None] ^ c[None, :])
    odd = (cols % 2 == 1)[None, :]
    return np.where(odd, w >> np.uint32(16), w & np.uint32(0xFFFF)).astype(np.uint32)


def keep_mask(seed: int, b: int, h: int, H: int, p: float, rows, cols):
    """Boolean keep mask, shape (len(rows), len(cols)), for head (b, h)."""
    return uniforms16(seed, b, h, H, rows, cols) >= np.uint32(keep_threshold(p))
