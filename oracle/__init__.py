"""CPU fp64 oracle for fused scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import or call anything in this package.  The product path (the HIP library
and its Python binding) never imports it, and this package imports nothing from the product.

Contents:

* ``attention.attention_fp64``  -- the plain definition: matmul, scale, causal mask, softmax,
  matmul, plus the logsumexp of the scaled masked scores.
* ``attention.attention_rows_fp64`` -- the same definition for a chosen subset of query rows
  (for sampled checks of problems too large to evaluate whole).
* ``attention.splitkv_partials_fp64`` / ``attention.combine_fp64`` -- the split-KV decode model:
  per-split locally normalised partial outputs with (max, sum) metadata, and their combine.
* ``attention.flash2_tiled_fp64`` -- the FlashAttention-2 online-softmax recurrence over Q and K/V
  blocks, run in fp64 as a CPU model of the algorithm (not of any kernel).

Every function is pinned by ``tests/test_oracle.py`` against closed forms, invariants, a library
routine (scipy) and brute force; none is "parity unpinned".
"""
from .attention import (  # noqa: F401
    attention_fp64,
    attention_probs_fp64,
    attention_rows_fp64,
    combine_fp64,
    flash2_tiled_fp64,
    splitkv_partials_fp64,
    visible_mask,
)
