"""Seeded synthetic inputs for the attention workloads, shared by tests, bench and smoke.

This module draws and encodes numbers; it performs none of the attention arithmetic, so both the
HIP path and the CPU oracle may consume what it produces without sharing any of the method.

Inputs are i.i.d. N(0, 1) draws (numpy PCG64 ``standard_normal`` in float32), drawn in the order
Q, K, V from one generator seeded per workload, then either kept as float32 or rounded to bfloat16
with round-to-nearest-even.  The rounded values are what both sides consume, so the rounding of
the inputs is not part of any error budget.

The layouts are the native ``[batch, heads, seq, head_dim]`` tensors of the profiling article
("PyTorch 어텐션 프로파일링 Flash, cuDNN, Math 백엔드 완벽 비교", section 1, and the cuDNN backend note
in section 2); grouped-query K/V carry fewer heads than Q ("FlashAttention-2: Faster Attention with
Better Parallelism and Work Partitioning", code example ``fa2_with_gqa``).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r = r.copy()
        r[nan] = np.uint16(0x7FC0)
    return r


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns exactly to float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class QKV:
    """Host copies of one workload's inputs in their storage encoding.

    ``dtype`` is ``"bf16"`` (arrays hold uint16 bit patterns) or ``"f32"`` (arrays hold float32).
    """

    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    dtype: str

    def widened(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        if self.dtype == "bf16":
            return bf16_bits_to_f32(a).astype(np.float64)
        return a.astype(np.float64)

    def as_f64(self):
        return self.widened("q"), self.widened("k"), self.widened("v")


def draw_qkv(seed: int, B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int,
             dtype: str = "bf16") -> QKV:
    """Draw Q [B,Hq,Nq,d], K and V [B,Hkv,Nk,d] ~ N(0,1) in that order from one seeded PCG64."""
    if dtype not in ("bf16", "f32"):
        raise ValueError(f"dtype must be 'bf16' or 'f32', got {dtype!r}")
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, Nq, d), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, Nk, d), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, Nk, d), dtype=np.float32)
    if dtype == "bf16":
        q, k, v = bf16_bits_from_f32(q), bf16_bits_from_f32(k), bf16_bits_from_f32(v)
    return QKV(q=q, k=k, v=v, dtype=dtype)


def draw_grad(seed: int, shape) -> np.ndarray:
    """An output gradient (the dO of a backward pass): i.i.d. N(0, 1) from a seeded PCG64,
    rounded to bfloat16 bits."""
    rng = np.random.default_rng(seed)
    return bf16_bits_from_f32(rng.standard_normal(tuple(shape), dtype=np.float32))


def draw_seqlens(seed: int, B: int, Nk: int, edges: bool = True) -> np.ndarray:
    """Per-batch key lengths, int32 [B]: uniform in [1, Nk] from a seeded PCG64.  With ``edges``
    the first entries become Nk, 0 and 1 (all keys, none, a single key), as far as B allows."""
    rng = np.random.default_rng(seed)
    L = rng.integers(1, max(Nk, 1) + 1, size=B).astype(np.int32) if Nk > 0 else np.zeros(B, np.int32)
    if edges:
        for i, val in enumerate((Nk, 0, min(1, Nk))[:B]):
            L[i] = val
    return L


def draw_bias(seed: int, Bb: int, Hb: int, Nq: int, Nk: int, kind: str = "normal",
              std: float = 1.0, masked_frac: float = 0.0) -> np.ndarray:
    """An additive attention bias [Bb, Hb, Nq, Nk] as bfloat16 bits.

    ``kind``: ``"normal"`` -- i.i.d. N(0, std^2) from a seeded PCG64; ``"alibi"`` -- a linear
    distance penalty -slope_h * |i + (Nk - Nq) - j| with slopes 2^(-8 (h + 1) / Hb), the usual
    position bias of decoder models.  ``masked_frac`` then sets that fraction of the entries,
    chosen by the same generator, to -inf (a padding-style mask).
    """
    rng = np.random.default_rng(seed)
    if kind == "normal":
        b = rng.standard_normal((Bb, Hb, Nq, Nk), dtype=np.float32) * np.float32(std)
    elif kind == "alibi":
        slopes = np.exp2(-8.0 * (np.arange(Hb) + 1) / Hb).astype(np.float32)
        dist = np.abs(np.arange(Nq)[:, None] + (Nk - Nq) - np.arange(Nk)[None, :]).astype(np.float32)
        b = np.broadcast_to(-slopes[None, :, None, None] * dist[None, None], (Bb, Hb, Nq, Nk))
    else:
        raise ValueError(f"unknown bias kind {kind!r}")
    b = np.array(b, dtype=np.float32)
    if masked_frac > 0:
        b[rng.random(b.shape) < masked_frac] = -np.inf
    return bf16_bits_from_f32(b)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    dtype: str
    causal: bool
    seed: int
    n_splits: Optional[int] = None  # set for the split-KV decode workloads

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def draw(self) -> QKV:
        return draw_qkv(self.seed, self.B, self.Hq, self.Hkv, self.Nq, self.Nk, self.d, self.dtype)

    def flops(self) -> float:
        """Convention 4*B*H*Nq*Nk*d, halved when causal (square prefill)."""
        f = 4.0 * self.B * self.Hq * self.Nq * self.Nk * self.d
        return f / 2 if self.causal and self.Nq == self.Nk else f


def _sweep() -> Dict[str, Workload]:
    out = {}
    for i, (n, b) in enumerate(((512, 32), (1024, 16), (2048, 8), (4096, 4))):
        for causal in (False, True):
            name = f"sweep_n{n}_b{b}_{'causal' if causal else 'noncausal'}"
            out[name] = Workload(name, b, 16, 16, n, n, 128, "bf16", causal, 30 + i)
    return out


WORKLOADS: Dict[str, Workload] = {
    "tiny_causal_f32": Workload("tiny_causal_f32", 1, 2, 2, 128, 128, 64, "f32", True, 1),
    "prefill_causal_b2h16n2048": Workload("prefill_causal_b2h16n2048", 2, 16, 16, 2048, 2048, 128,
                                          "bf16", True, 2),
    **_sweep(),
    "long_causal_b1h8n16384": Workload("long_causal_b1h8n16384", 1, 8, 8, 16384, 16384, 128,
                                       "bf16", True, 4),
    "decode_gqa_nq1": Workload("decode_gqa_nq1", 8, 32, 8, 1, 8192, 128, "bf16", True, 5, 16),
    "decode_gqa_nq4": Workload("decode_gqa_nq4", 8, 32, 8, 4, 8192, 128, "bf16", True, 5, 16),
}


def to_device(a: np.ndarray, dtype: str, device="cuda"):
    """Upload a host array (bf16 bits or float32) as a contiguous torch tensor of that dtype."""
    import torch

    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device).contiguous()
