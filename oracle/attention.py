"""Plain fp64 CPU attention: the definition the fused kernels must reproduce.

Test infrastructure only (see the package docstring): never imported by the product path.

Sources (page title, then section):

* "PyTorch 어텐션 프로파일링 Flash, cuDNN, Math 백엔드 완벽 비교", section 1 (naive attention): scores =
  q·kᵀ, times scale, causal positions filled with -inf, row softmax, times v.
* "FlashAttention-2: Faster Attention with Better Parallelism and Work Partitioning", section
  "방법론 / 알고리즘 개요" (the forward recurrence over K/V blocks with running max m, running sum l,
  deferred 1/l) and "인과적 마스킹 최적화" (blocks above the diagonal skipped), plus the code example's
  ``standard_attention`` (divide by √d, ``tril`` mask) and ``fa2_with_gqa`` (K/V heads broadcast).
* "[onnxruntime] WebGPU FlashAttention 최적화: 커널 퓨전과 가변 시퀀스 길이 지원으로 성능 극대화", section
  "1. 커널 퓨전" (each split emits a locally normalised partial output plus (local max, local sum);
  the reduce step rescales partials into the exact softmax-weighted V), and section "2." (the
  default scale is 1/√head_size when the given scale is 0).

Readings where the pages are silent (each applied identically everywhere):

* Causal visibility is bottom-right aligned: key j is visible to query i iff j <= i + (Nk - Nq).
  It is the square ``tril`` mask when Nq == Nk.
* A row with no visible key has output 0 and logsumexp -inf; a split with no visible key has
  m = -inf, l = 0, partial 0 and contributes nothing to the combine.
* Logsumexp is the natural log of the sum of exp over the scaled, masked scores of a row.
* GQA: query head hq reads K/V head hq // (Hq / Hkv).
* Splits are contiguous key chunks of ceil(Nk / n_splits) keys; the last ones may be short/empty.
* Variable key lengths (``seqlens_k``, the "가변 시퀀스 길이" of the onnxruntime page, whose decode
  kernel reads the KV length on the GPU): ``seqlens_k[b]`` is the number of valid keys of batch
  element b (0 <= L_b <= Nk, the capacity of the K/V tensors).  Keys at or past L_b do not exist
  for that element, and causal visibility uses its own length: j <= i + (L_b - Nq).  Split
  chunks stay those of the capacity Nk, clipped to L_b.
* Attention bias (the same page, section "1. 커널 퓨전": the fused decode kernel applies the
  attention bias and the causal mask after QKᵀ, with bias dimensions 0 and 1 broadcast): a
  tensor [Bb, Hb, Nq, Nk] with Bb in {1, B} and Hb in {1, Hq} is added to the scaled scores
  before masking: s = scale·q·kᵀ + bias.  A -inf entry masks its key exactly as the causal fill
  does (section 1 of the PyTorch page writes masked positions as -inf), so a row whose every
  key is masked this way is a row with no visible key.

* Backward (``attention_backward_fp64``): not on the pages.  The gradients of the scalar
  L = Σ dO ∘ O are the chain rule through the same five steps, written out as the definition:
  dV = Pᵀ·dO, dP = dO·Vᵀ, dS = P ∘ (dP − Σ_k P_ik dP_ik) (the softmax Jacobian), dQ = scale·dS·K,
  dK = scale·dSᵀ·Q; K/V heads shared by several query heads (GQA) receive the sum over those
  heads.  Masked positions have P = 0 and pass no gradient.

All arithmetic is numpy float64; the matrix product (``@``) is the only library primitive.
"""
from __future__ import annotations

import math
from typing import Tuple

import numpy as np

NEG_INF = -np.inf


def _check(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if v.shape != k.shape or Bk != B or dk != d:
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape}")
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    return B, Hq, Hkv, Nq, Nk, d


def visible_mask(rows: np.ndarray, Nq: int, Nk: int, causal: bool) -> np.ndarray:
    """[len(rows), Nk] boolean: True where key j may be attended by query row i."""
    cols = np.arange(Nk)
    if not causal:
        return np.ones((len(rows), Nk), dtype=bool)
    return cols[None, :] <= (rows[:, None] + (Nk - Nq))


def _scores(qrows: np.ndarray, kh: np.ndarray, scale: float) -> np.ndarray:
    """Step 1-2 of the naive definition: q·kᵀ, then multiply by the scale."""
    return (qrows @ kh.T) * scale


def _masked_softmax(s: np.ndarray, vis: np.ndarray):
    """Steps 3-4: fill invisible scores with -inf, then row softmax.

    Returns (P, m, l) with m the row max over visible scores and l = sum exp(s - m); rows with no
    visible key get P = 0, m = -inf, l = 0.  A score that is already -inf (a -inf bias entry) is
    a masked key like any other, so a row whose every score is -inf has no visible key.
    """
    s = np.where(vis, s, NEG_INF)
    live = vis & ~np.isneginf(s)
    any_vis = live.any(axis=1)
    m = np.where(any_vis, s.max(axis=1, initial=NEG_INF), NEG_INF)
    shifted = np.where(live, s - np.where(any_vis, m, 0.0)[:, None], NEG_INF)
    e = np.exp(shifted)  # exp(-inf) = 0 for invisible entries
    l = e.sum(axis=1)
    p = np.divide(e, l[:, None], out=np.zeros_like(e), where=(l[:, None] > 0))
    return p, m, l


def _weighted_values(p: np.ndarray, vh: np.ndarray) -> np.ndarray:
    """Step 5: probabilities times V."""
    return p @ vh


def _kv_head(hq: int, Hq: int, Hkv: int) -> int:
    """GQA: contiguous groups of Hq / Hkv query heads share one K/V head."""
    return hq // (Hq // Hkv)


def _row_lse(m: np.ndarray, l: np.ndarray) -> np.ndarray:
    """ln Σ exp(score) = m + ln l; -inf for rows with no visible key."""
    ok = l > 0
    return np.where(ok, m + np.log(np.where(ok, l, 1.0)), NEG_INF)


def _resolve_scale(scale: float, d: int) -> float:
    return 1.0 / math.sqrt(d) if scale == 0 else float(scale)


def _key_lengths(seqlens_k, B: int, Nk: int) -> np.ndarray:
    """Valid keys per batch element: all Nk, or ``seqlens_k[b]`` (checked to lie in [0, Nk])."""
    if seqlens_k is None:
        return np.full(B, Nk, dtype=np.int64)
    L = np.asarray(seqlens_k, dtype=np.int64).reshape(-1)
    if L.shape != (B,) or (L < 0).any() or (L > Nk).any():
        raise ValueError(f"seqlens_k must be {B} lengths in [0, {Nk}]")
    return L


def _bias_view(bias, B: int, Hq: int, Nq: int, Nk: int):
    """Callable (b, hq) -> the [Nq, Nk] bias slice, broadcasting a size-1 batch or head dim."""
    if bias is None:
        return None
    bias = np.asarray(bias, dtype=np.float64)
    Bb, Hb = bias.shape[0], bias.shape[1]
    if bias.ndim != 4 or Bb not in (1, B) or Hb not in (1, Hq) or bias.shape[2:] != (Nq, Nk):
        raise ValueError(f"bias must be [1 or {B}, 1 or {Hq}, {Nq}, {Nk}], got {bias.shape}")
    return lambda b, hq: bias[b if Bb == B else 0, hq if Hb == Hq else 0]


def _row_scores(qrows, kh, scale, bias_rows):
    """Scaled scores of some query rows against the keys ``kh``, plus the bias rows if any."""
    s = _scores(qrows, kh, scale)
    return s if bias_rows is None else s + bias_rows


def attention_fp64(q, k, v, scale: float, causal: bool, row_block: int = 1024, bias=None,
                   seqlens_k=None) -> Tuple[np.ndarray, np.ndarray]:
    """O [B,Hq,Nq,d] and LSE [B,Hq,Nq] of softmax(scale·q·kᵀ + bias + causal mask)·v, in fp64.

    ``scale`` is the float the GPU receives (0 selects 1/√d); it is widened to fp64 unchanged.
    ``bias`` and ``seqlens_k`` are optional (see the module docstring for their readings).
    Rows are processed ``row_block`` at a time only to bound memory; rows are independent.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Hkv, Nq, Nk, d = _check(q, k, v)
    scale = _resolve_scale(scale, d)
    L = _key_lengths(seqlens_k, B, Nk)
    bview = _bias_view(bias, B, Hq, Nq, Nk)
    out = np.zeros((B, Hq, Nq, d), dtype=np.float64)
    lse = np.full((B, Hq, Nq), NEG_INF, dtype=np.float64)
    for b in range(B):
        Lb = int(L[b])
        if Lb == 0:
            continue  # no key at all: O = 0, LSE = -inf
        for hq in range(Hq):
            hkv = _kv_head(hq, Hq, Hkv)
            for i0 in range(0, Nq, row_block):
                rows = np.arange(i0, min(Nq, i0 + row_block))
                brows = None if bview is None else bview(b, hq)[rows, :Lb]
                s = _row_scores(q[b, hq, rows], k[b, hkv, :Lb], scale, brows)
                vis = visible_mask(rows, Nq, Lb, causal)
                p, m, l = _masked_softmax(s, vis)
                out[b, hq, rows] = _weighted_values(p, v[b, hkv, :Lb])
                lse[b, hq, rows] = _row_lse(m, l)
    return out, lse


def attention_rows_fp64(q, k, v, scale: float, causal: bool, rows, bias=None, seqlens_k=None
                        ) -> Tuple[np.ndarray, np.ndarray]:
    """Only the query rows ``rows`` (positions in 0..Nq-1, same for every batch and head) of
    ``attention_fp64``: O [B,Hq,len(rows),d], LSE [B,Hq,len(rows)].  The causal mask uses each
    row's true position, so sampled rows of a large problem are exact rows of the full result."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Hkv, Nq, Nk, d = _check(q, k, v)
    scale = _resolve_scale(scale, d)
    L = _key_lengths(seqlens_k, B, Nk)
    bview = _bias_view(bias, B, Hq, Nq, Nk)
    rows = np.asarray(rows, dtype=np.int64)
    if rows.ndim != 1 or (len(rows) and (rows.min() < 0 or rows.max() >= Nq)):
        raise ValueError("rows must be positions in [0, Nq)")
    out = np.zeros((B, Hq, len(rows), d))
    lse = np.full((B, Hq, len(rows)), NEG_INF)
    for b in range(B):
        Lb = int(L[b])
        if Lb == 0:
            continue
        for hq in range(Hq):
            hkv = _kv_head(hq, Hq, Hkv)
            brows = None if bview is None else bview(b, hq)[rows, :Lb]
            s = _row_scores(q[b, hq, rows], k[b, hkv, :Lb], scale, brows)
            p, m, l = _masked_softmax(s, visible_mask(rows, Nq, Lb, causal))
            out[b, hq] = _weighted_values(p, v[b, hkv, :Lb])
            lse[b, hq] = _row_lse(m, l)
    return out, lse


def attention_probs_fp64(q, k, scale: float, causal: bool) -> np.ndarray:
    """The probability matrix P [B,Hq,Nq,Nk] of the definition (small inputs only)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, Hq, Hkv, Nq, Nk, d = _check(q, k, k)
    scale = _resolve_scale(scale, d)
    P = np.zeros((B, Hq, Nq, Nk))
    rows = np.arange(Nq)
    vis = visible_mask(rows, Nq, Nk, causal)
    for b in range(B):
        for hq in range(Hq):
            P[b, hq] = _masked_softmax(_scores(q[b, hq], k[b, _kv_head(hq, Hq, Hkv)], scale),
                                       vis)[0]
    return P


def split_bounds(Nk: int, n_splits: int):
    """[(start, end)] of the contiguous key chunks; chunk length ceil(Nk / n_splits)."""
    if n_splits < 1:
        raise ValueError("n_splits must be >= 1")
    L = -(-Nk // n_splits)
    return [(min(s * L, Nk), min((s + 1) * L, Nk)) for s in range(n_splits)]


def splitkv_partials_fp64(q, k, v, scale: float, causal: bool, n_splits: int, bias=None,
                          seqlens_k=None):
    """Per-split partials of the decode model.

    Returns (O_s [B,Hq,Nq,S,d], m_s [B,Hq,Nq,S], l_s [B,Hq,Nq,S]): for split s and row i,
    m_s is the max scaled visible score in the chunk, l_s = Σ exp(score - m_s) over the chunk, and
    O_s = Σ exp(score - m_s)·v / l_s (locally normalised).  Empty or fully masked chunks give
    m_s = -inf, l_s = 0, O_s = 0.  Chunks are those of the capacity Nk, clipped to each batch
    element's key length when ``seqlens_k`` is given.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Hkv, Nq, Nk, d = _check(q, k, v)
    scale = _resolve_scale(scale, d)
    L = _key_lengths(seqlens_k, B, Nk)
    bview = _bias_view(bias, B, Hq, Nq, Nk)
    bounds = split_bounds(Nk, n_splits)
    S = len(bounds)
    O_s = np.zeros((B, Hq, Nq, S, d))
    m_s = np.full((B, Hq, Nq, S), NEG_INF)
    l_s = np.zeros((B, Hq, Nq, S))
    rows = np.arange(Nq)
    for b in range(B):
        Lb = int(L[b])
        vis_all = visible_mask(rows, Nq, Lb, causal)
        for hq in range(Hq):
            hkv = _kv_head(hq, Hq, Hkv)
            for si, (c0, c1) in enumerate(bounds):
                k0, k1 = min(c0, Lb), min(c1, Lb)
                if k1 <= k0:
                    continue
                brows = None if bview is None else bview(b, hq)[:, k0:k1]
                s = _row_scores(q[b, hq], k[b, hkv, k0:k1], scale, brows)
                p, m, l = _masked_softmax(s, vis_all[:, k0:k1])
                O_s[b, hq, :, si] = _weighted_values(p, v[b, hkv, k0:k1])
                m_s[b, hq, :, si] = m
                l_s[b, hq, :, si] = l
    return O_s, m_s, l_s


def combine_fp64(O_s, m_s, l_s):
    """Reduce split partials: M = max m_s, w_s = l_s·exp(m_s - M), O = Σ w_s·O_s / Σ w_s,
    LSE = M + ln Σ w_s.  Rows whose splits are all empty give O = 0, LSE = -inf."""
    O_s = np.asarray(O_s, dtype=np.float64)
    m_s = np.asarray(m_s, dtype=np.float64)
    l_s = np.asarray(l_s, dtype=np.float64)
    M = m_s.max(axis=-1)
    finite = np.isfinite(M)
    Msafe = np.where(finite, M, 0.0)
    with np.errstate(invalid="ignore"):
        w = np.where(l_s > 0, l_s * np.exp(m_s - Msafe[..., None]), 0.0)
    W = w.sum(axis=-1)
    num = (w[..., None] * O_s).sum(axis=-2)
    O = np.divide(num, W[..., None], out=np.zeros_like(num), where=(W[..., None] > 0))
    return O, _row_lse(Msafe, W)


def _online_step(m, l, O, S, vblk):
    """One K/V block of the FA2 recurrence: m_new = max(m, rowmax S), P = exp(S - m_new),
    l = exp(m - m_new)·l + rowsum P, O = exp(m - m_new)·O + P·v.  Rows whose max is still -inf
    (nothing visible yet) keep P = 0, l = 0, O = 0."""
    m_new = np.maximum(m, S.max(axis=1))
    ref = np.where(np.isfinite(m_new), m_new, 0.0)
    P = np.exp(S - ref[:, None])
    alpha = np.exp(m - ref)
    return m_new, alpha * l + P.sum(axis=1), alpha[:, None] * O + P @ vblk


def flash2_tiled_fp64(q, k, v, scale: float, causal: bool, Br: int, Bc: int,
                      skip_masked_blocks: bool = True):
    """The FA2 forward recurrence in fp64, over Q blocks of Br rows and K/V blocks of Bc keys.

    For each Q block: O = 0, l = 0, m = -inf; for each K/V block: S = scale·q·kᵀ (masked),
    m_new = max(m, rowmax S), P = exp(S - m_new), l = exp(m - m_new)·l + rowsum P,
    O = exp(m - m_new)·O + P·v, m = m_new; finally O / l.  With ``skip_masked_blocks`` the blocks
    lying entirely above the causal diagonal are not visited.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Hkv, Nq, Nk, d = _check(q, k, v)
    scale = _resolve_scale(scale, d)
    out = np.zeros((B, Hq, Nq, d))
    lse = np.full((B, Hq, Nq), NEG_INF)
    off = Nk - Nq
    for b in range(B):
        for hq in range(Hq):
            hkv = _kv_head(hq, Hq, Hkv)
            for i0 in range(0, Nq, Br):
                i1 = min(Nq, i0 + Br)
                rows = np.arange(i0, i1)
                qi = q[b, hq, i0:i1]
                O = np.zeros((i1 - i0, d))
                l = np.zeros(i1 - i0)
                m = np.full(i1 - i0, NEG_INF)
                for j0 in range(0, Nk, Bc):
                    j1 = min(Nk, j0 + Bc)
                    if causal and skip_masked_blocks and j0 > (i1 - 1) + off:
                        break  # every later block is above the diagonal too
                    S = (qi @ k[b, hkv, j0:j1].T) * scale
                    vis = visible_mask(rows, Nq, Nk, causal)[:, j0:j1]
                    S = np.where(vis, S, NEG_INF)
                    m, l, O = _online_step(m, l, O, S, v[b, hkv, j0:j1])
                ok = l > 0
                out[b, hq, i0:i1] = np.divide(O, l[:, None], out=np.zeros_like(O),
                                              where=ok[:, None])
                lse[b, hq, i0:i1] = _row_lse(m, l)
    return out, lse


def _softmax_backward(p: np.ndarray, dp: np.ndarray) -> np.ndarray:
    """Gradient w.r.t. the scores of a row softmax: dS_ij = P_ij (dP_ij − Σ_k P_ik dP_ik)."""
    return p * (dp - (p * dp).sum(axis=1, keepdims=True))


def _accumulate(acc: np.ndarray, x: np.ndarray) -> np.ndarray:
    """Sum over the query heads that share one K/V head."""
    return acc + x


def attention_backward_fp64(q, k, v, dout, scale: float, causal: bool, seqlens_k=None,
                            bias=None):
    """(dq [B,Hq,Nq,d], dk [B,Hkv,Nk,d], dv [B,Hkv,Nk,d]): the gradients of L = Σ dout ∘ O for
    O = softmax(scale·q·kᵀ + bias + causal mask)·v, in fp64, from the definition (see the module
    docstring).  With ``seqlens_k`` (the reading of ``attention_fp64``) element b has only its
    first seqlens_k[b] keys: the causal mask is aligned to the end of those, and the keys past
    them, which do not take part in O, get zero gradients.  ``bias`` (as in ``attention_fp64``) is
    a constant: it shifts the scores, so it enters P, and no gradient is taken for it.  Small and
    medium inputs only: every (batch, head) keeps its [Nq, Nk] matrices."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    B, Hq, Hkv, Nq, Nk, d = _check(q, k, v)
    if dout.shape != q.shape:
        raise ValueError(f"dout must have the shape of q {q.shape}, got {dout.shape}")
    scale = _resolve_scale(scale, d)
    L = _key_lengths(seqlens_k, B, Nk)
    bview = _bias_view(bias, B, Hq, Nq, Nk)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    rows = np.arange(Nq)
    for b in range(B):
        Lb = int(L[b])
        if Lb == 0:
            continue  # no key: O = 0 whatever the inputs, every gradient is zero
        vis = visible_mask(rows, Nq, Lb, causal)
        for hq in range(Hq):
            hkv = _kv_head(hq, Hq, Hkv)
            kh, vh, qh, doh = k[b, hkv, :Lb], v[b, hkv, :Lb], q[b, hq], dout[b, hq]
            brows = None if bview is None else bview(b, hq)[:, :Lb]
            p, _, _ = _masked_softmax(_row_scores(qh, kh, scale, brows), vis)
            dp = doh @ vh.T
            ds = _softmax_backward(p, dp)
            dq[b, hq] = scale * (ds @ kh)
            dk[b, hkv, :Lb] = _accumulate(dk[b, hkv, :Lb], scale * (ds.T @ qh))
            dv[b, hkv, :Lb] = _accumulate(dv[b, hkv, :Lb], p.T @ doh)
    return dq, dk, dv
