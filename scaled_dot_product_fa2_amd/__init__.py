"""MI355X (gfx950) fused scaled-dot-product attention.

``softmax(scale * Q Kᵀ + causal mask) V`` and its logsumexp, computed by hand-written HIP kernels
behind a small C ABI (``include/sdpa_fa2.h``):

* ``attn_fwd``      -- FlashAttention-2-style prefill forward, bf16 in/out, fp32 accumulation;
* ``attn_fwd_f32``  -- the same on fp32 tensors;
* ``attn_decode_splitkv`` -- split-KV decode: per-split partials with (max, sum) metadata, then a
  combine kernel.

The Python functions here only marshal torch tensors into the C ABI (``binding.py``).
"""
from .binding import (  # noqa: F401
    AttentionError,
    attn_decode_splitkv,
    attn_decode_workspace_bytes,
    attn_fwd,
    attn_fwd_f32,
    load,
    status_string,
)
