"""CPU fp64 oracle for exact attention — TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check in __graft_entry__ and the CPU-baseline
leg of bench.py may import this package. The library under
exact_io_aware_72_amd/ never imports, calls or links it, and it shares no
code with that library: the two meet only through the seeded inputs of the
separate `workloads` module.

Contents:
  attention.py     plain fp64 forward / backward that materialise S and P
  dropout_hash.py  the dropout keep-mask counter hash, from the published
                   SplitMix64 and MurmurHash3 finalizers
  varlen.py        the same attention over packed batches of sequences of
                   different lengths
  fp8.py           OCP E4M3 per-block quantisation and attention with
                   quantised scores

Parity status: every function here is pinned by tests under tests/ against
closed forms, invariants, brute force and finite differences, except the
choice of dropout generator, which the pages do not specify (the generator
itself is pinned to published test vectors; which generator to use is a
reading, not a fact of the pages).
"""
from .attention import (  # noqa: F401
    attention_scores,
    softmax_stats,
    attention_probs,
    forward,
    forward_cross,
    head_forward,
    head_backward,
    backward,
    sampled_head,
)
from .dropout_hash import (  # noqa: F401
    mix64,
    fmix32,
    head_key,
    row_keys,
    pair_keys,
    uniforms16,
    keep_threshold,
    keep_mask,
)
