"""MI355X (gfx950) fused scaled-dot-product attention.

``softmax(scale * Q Kᵀ + bias + causal mask) V`` and its logsumexp, computed by hand-written HIP
kernels behind a small C ABI (``include/sdpa_fa2.h``):

* ``attn_fwd``      -- FlashAttention-2-style prefill forward, bf16 in/out, fp32 accumulation;
* ``attn_fwd_f32``  -- the same on fp32 tensors;
* ``attn_decode_splitkv`` -- split-KV decode: per-split partials with (max, sum) metadata, then a
  combine kernel;
* ``attn_fwd_ex`` / ``attn_decode_splitkv_ex`` -- the bf16 paths with per-batch key lengths
  (``seqlens_k``) and an additive bias;
* ``attn_forward`` -- one entry for any query length: split-KV below 32 query rows, prefill
  otherwise;
* ``attn_bwd`` -- the gradients dq, dk, dv of the forward (head dims 64 and 128), also of the
  forward with key lengths and a bias (the bias itself gets no gradient).

The Python functions here only marshal torch tensors into the C ABI (``binding.py``).
"""
from .binding import (  # noqa: F401
    AttentionError,
    attn_bwd,
    attn_bwd_workspace_bytes,
    attn_decode_num_splits,
    attn_decode_splitkv,
    attn_decode_splitkv_ex,
    attn_decode_workspace_bytes,
    attn_forward,
    attn_forward_workspace_bytes,
    attn_fwd,
    attn_fwd_ex,
    attn_fwd_f32,
    load,
    status_string,
)
