"""Seeded synthetic inputs for exact attention, shared by the oracle tests,
the GPU parity tests and the benchmark.

This module holds no attention arithmetic. It only draws Gaussian tensors,
rounds them to the stored dtype and names the workloads.

The workloads follow the attention shapes the pages discuss: the
(batch, seq_len, num_heads, head_dim) tensor layout of the PyTorch usage
example ("FlashAttention for Efficient Training", section 4.2 "Integration
with Popular Frameworks"), long-context causal training (section 4.1, and the
"Impact on Long-Context AI Training" section of "How FlashAttention Optimizes
GPU Memory for Fast AI Training"), and attention dropout fused into the
kernel (section 3.1 "Fused Kernel Design"). No dataset or trained weights are
involved: Q, K, V and the upstream gradient dO are i.i.d. normal draws.

Recipe (fixed; the parity tests and stored expected values depend on it):
  rng = numpy.random.default_rng(1000 + config_id)
  q, k, v, do = four draws of rng.standard_normal([B, N, H, d], float32),
                in that order, each multiplied by `amp` in float32
  bf16 configs: each tensor rounded to bfloat16, round-to-nearest-even.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "workload",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "make_inputs",
    "make_tensor",
    "counted_flops",
    "VarlenWorkload",
    "VARLEN_WORKLOADS",
    "varlen_lengths",
    "make_varlen_inputs",
    "counted_flops_varlen",
    "BLOCK",
    "block_mask_local_global",
    "block_mask_random",
    "SPARSE_WORKLOADS",
    "SplitKVWorkload",
    "SPLITKV_WORKLOADS",
    "make_cross_inputs",
    "device_normal",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention problem: shapes, dtype, mask, dropout and the seed recipe."""

    config_id: int
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str  # "f32" or "bf16"
    causal: bool
    dropout_p: float  # stored as fp32 by the kernels and the oracle alike
    backward: bool  # whether the workload includes the backward pass
    amp: float = 1.0
    dropout_seed: int = 2026

    @property
    def scale(self) -> float:
        """1/sqrt(d) rounded to fp32, the value both sides receive."""
        return float(np.float32(1.0 / math.sqrt(self.d)))

    @property
    def seed(self) -> int:
        return 1000 + self.config_id

    @property
    def shape(self) -> tuple:
        return (self.B, self.N, self.H, self.d)

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    1: Workload(1, "f32_B1_H1_N256_d64_full_fwd", 1, 1, 256, 64, "f32", False, 0.0, False),
    2: Workload(2, "bf16_B4_H16_N2048_d64_causal_fwd", 4, 16, 2048, 64, "bf16", True, 0.0, False),
    3: Workload(3, "bf16_B2_H16_N8192_d128_causal_fwdbwd", 2, 16, 8192, 128, "bf16", True, 0.0, True),
    4: Workload(4, "bf16_B1_H16_N32768_d80_causal_fwdbwd_amp0.5", 1, 16, 32768, 80, "bf16", True, 0.0, True,
                amp=0.5),
    5: Workload(5, "bf16_B1_H8_N65536_d128_causal_dropout0.1_fwdbwd", 1, 8, 65536, 128, "bf16", True, 0.1, True),
}


def workload(config_id: int) -> Workload:
    return WORKLOADS[config_id]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16. NaN stays NaN (quiet bit set).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint32)
    nan = np.isnan(x)
    if nan.any():
        r = np.where(nan, ((u >> 16) | 0x40).astype(np.uint32), r)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def make_tensor(rng: np.random.Generator, shape, amp: float, dtype: str):
    """One Gaussian tensor in the stored dtype.

    Returns (stored, values): `stored` is float32 (f32) or uint16 bf16 bit
    patterns (bf16); `values` is the exact float32 value of each stored
    element, which is what the oracle upcasts.
    """
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if amp != 1.0:
        x = (x * np.float32(amp)).astype(np.float32)
    if dtype == "f32":
        return x, x
    if dtype == "bf16":
        bits = f32_to_bf16_bits(x)
        return bits, bf16_bits_to_f32(bits)
    raise ValueError(f"unknown dtype {dtype!r}")


def make_inputs(w: Workload, with_grad: bool | None = None, N: int | None = None):
    """Draw q, k, v (and dO) for workload `w`.

    Returns a dict with keys 'q', 'k', 'v' (and 'do'), each a pair
    (stored, values) as in `make_tensor`. `N` overrides the sequence length
    (same seed recipe, smaller problem) for tests that need a short variant.
    """
    if with_grad is None:
        with_grad = w.backward
    shape = (w.B, N if N is not None else w.N, w.H, w.d)
    rng = np.random.default_rng(w.seed)
    out = {}
    for name in ("q", "k", "v") + (("do",) if with_grad else ()):
        out[name] = make_tensor(rng, shape, w.amp, w.dtype)
    return out


def counted_flops(B: int, H: int, N: int, d: int, causal: bool, backward: bool) -> tuple:
    """FLOP convention of the headline metric: forward 4*B*H*N^2*d, halved
    when causal; backward 2.5x forward. Returns (forward, backward)."""
    fwd = 4.0 * B * H * N * N * d
    if causal:
        fwd /= 2.0
    return fwd, (2.5 * fwd if backward else 0.0)


# ---------------------------------------------------------------------------
# Packed batches of sequences of different lengths ("FlashAttention for
# Efficient Training", section 5.2 "Handling Variable Sequence Lengths").
#
# Recipe (fixed): rng = numpy.random.default_rng(seed);
#   lengths = rng.integers(min_len, max_len + 1, size=num_seqs) unless the
#   workload lists them explicitly; cu_seqlens = [0, cumsum(lengths)] (int32);
#   then q, k, v, do drawn as for fixed-length batches with shape
#   [total, H, d] from the same rng, after the lengths.
@dataclasses.dataclass(frozen=True)
class VarlenWorkload:
    name: str
    num_seqs: int
    H: int
    d: int
    dtype: str
    causal: bool
    dropout_p: float
    min_len: int = 1
    max_len: int = 1
    lengths: tuple = ()
    seed: int = 3000
    amp: float = 1.0
    dropout_seed: int = 2027

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.d)))

    def with_(self, **kw) -> "VarlenWorkload":
        return dataclasses.replace(self, **kw)


VARLEN_WORKLOADS = {
    # Sixteen causal sequences of 512..8192 tokens (mean about 4.3k), the
    # length spread the pages' padding-versus-packing comparison is about.
    "varlen16": VarlenWorkload("bf16_varlen16_H16_len512-8192_d128_causal_fwdbwd", 16, 16, 128,
                               "bf16", True, 0.0, min_len=512, max_len=8192, seed=3006),
}


def varlen_lengths(w: VarlenWorkload) -> np.ndarray:
    """Sequence lengths of `w` (int64), drawn first from the workload's rng."""
    if w.lengths:
        return np.asarray(w.lengths, np.int64)
    rng = np.random.default_rng(w.seed)
    return rng.integers(w.min_len, w.max_len + 1, size=w.num_seqs).astype(np.int64)


def make_varlen_inputs(w: VarlenWorkload, with_grad: bool = True):
    """Returns (cu_seqlens int32 [num_seqs + 1], dict name -> (stored, values))
    with tensors of shape [total, H, d]."""
    rng = np.random.default_rng(w.seed)
    if w.lengths:
        lengths = np.asarray(w.lengths, np.int64)
    else:
        lengths = rng.integers(w.min_len, w.max_len + 1, size=w.num_seqs).astype(np.int64)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    shape = (int(cu[-1]), w.H, w.d)
    out = {}
    for name in ("q", "k", "v") + (("do",) if with_grad else ()):
        out[name] = make_tensor(rng, shape, w.amp, w.dtype)
    return cu, out


def counted_flops_varlen(lengths, H: int, d: int, causal: bool, backward: bool) -> tuple:
    """counted_flops summed over the sequences of a packed batch."""
    fwd = sum(counted_flops(1, H, int(n), d, causal, False)[0] for n in lengths)
    return fwd, (2.5 * fwd if backward else 0.0)


# ---------------------------------------------------------------------------
# Block-sparse masks over 128 x 128 blocks of the score matrix ("FlashAttention
# for Efficient Training", section 3.2 "Block-Sparse Attention Support", for
# sequences beyond 16K tokens). Structure only: uint8 arrays, 1 = computed.
BLOCK = 128


def block_mask_local_global(N: int, window: int, n_global: int) -> np.ndarray:
    """[nb, nb] mask: query block i sees key blocks |i - j| <= window (a
    sliding window) and the first n_global key blocks (global tokens)."""
    nb = -(-N // BLOCK)
    i = np.arange(nb)[:, None]
    j = np.arange(nb)[None, :]
    return ((np.abs(i - j) <= window) | (j < n_global)).astype(np.uint8)


def block_mask_random(shape, N: int, density: float, seed: int) -> np.ndarray:
    """[..., nb, nb] Bernoulli(density) mask from default_rng(seed)."""
    nb = -(-N // BLOCK)
    rng = np.random.default_rng(seed)
    return (rng.random(tuple(shape) + (nb, nb)) < density).astype(np.uint8)


# Long-sequence block-sparse workload: local window of +-8 blocks plus two
# global key blocks, shared by all heads; inputs drawn as for fixed-length
# workloads with seed 1000 + config_id.
SPARSE_WORKLOADS = {
    "local_global": (Workload(6, "bf16_B1_H16_N32768_d128_full_blocksparse_w8g2_fwdbwd", 1, 16, 32768, 128,
                              "bf16", False, 0.0, True), dict(window=8, n_global=2)),
}


# ---------------------------------------------------------------------------
# Queries against a longer key sequence (split-KV forward): decoding (one new
# query per sequence against its cached keys) and short-batch prefill, the
# low-parallelism shapes of "FlashAttention for Efficient Training", section
# 6.1 "Limited Parallelism for Small Batch Sizes".
#
# Recipe (fixed): rng = default_rng(seed); q = standard_normal([B, Nq, H, d]),
# then k, v = standard_normal([B, Nk, H, d]) each, float32, rounded to bf16.
@dataclasses.dataclass(frozen=True)
class SplitKVWorkload:
    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    causal: bool
    seed: int
    dtype: str = "bf16"

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.d)))


SPLITKV_WORKLOADS = {
    "decode": SplitKVWorkload("bf16_decode_B4_H16_Nq1_Nk65536_d128", 4, 16, 1, 65536, 128, True, 3100),
    "prefill_small": SplitKVWorkload("bf16_B1_H8_N4096_d128_causal_fwd", 1, 8, 4096, 4096, 128, True, 3101),
}


def make_cross_inputs(B: int, H: int, Nq: int, Nk: int, d: int, dtype: str, seed: int, amp: float = 1.0):
    """dict name -> (stored, values) for q [B, Nq, H, d] and k, v [B, Nk, H, d]."""
    rng = np.random.default_rng(seed)
    out = {"q": make_tensor(rng, (B, Nq, H, d), amp, dtype)}
    for name in ("k", "v"):
        out[name] = make_tensor(rng, (B, Nk, H, d), amp, dtype)
    return out


def device_normal(shape, seed: int, dtype: str = "bf16", device: str = "cuda"):
    """A standard normal tensor drawn on the device by torch's Philox
    generator seeded with `seed` (float32 draws, then rounded to bf16 with
    round-to-nearest-even), for shapes too large to draw on the host. The
    same seed gives the same tensor on any run of the same torch build."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    return x.to(torch.bfloat16) if dtype == "bf16" else x
