"""Pins of the CPU oracle to facts other than itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with a closed form, an
invariant of softmax attention, a library routine (scipy), brute force, or the hand-derived
fixture under ``tests/golden/``.  ``test_oracle.py`` runs every pin; ``test_oracle_mutants.py``
plants plausible mistakes in the oracle's steps and checks that some pin fails for each.

All expected values here come from the mathematics, never from the oracle under test.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import scipy.special

from oracle import attention as A

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def _tril_visible(Nq, Nk, causal):
    """Independent construction of the end-aligned causal mask through numpy's tril."""
    if not causal:
        return np.ones((Nq, Nk), dtype=bool)
    return np.tril(np.ones((Nq, Nk), dtype=bool), k=Nk - Nq)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    same_inf = (np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b)))
    with np.errstate(invalid="ignore"):
        err = np.where(same_inf, 0.0, np.abs(a - b))
    assert np.all(np.isfinite(err)) and err.max(initial=0.0) <= tol, \
        f"{what}: max err {err.max(initial=0.0)} > {tol}"


# ---- closed forms and invariants ----------------------------------------------------------

def pin_probs_rows_sum_to_one():
    for causal in (False, True):
        for Nq, Nk in ((7, 7), (3, 11), (11, 11), (5, 2)):
            q = _rand(1, 1, 4, Nq, 8)
            k = _rand(2, 1, 2, Nk, 8)
            P = A.attention_probs_fp64(q, k, 0.3, causal)
            vis = _tril_visible(Nq, Nk, causal)
            has = vis.any(axis=1)
            sums = P.sum(axis=-1)
            _close(sums[..., has], np.ones_like(sums[..., has]), 1e-14, "row sums")
            _close(sums[..., ~has], np.zeros_like(sums[..., ~has]), 0.0, "empty-row sums")
            assert np.all(P[..., ~vis] == 0.0), "probability on a masked position"
            assert np.all(P[..., vis] > 0.0), "zero probability on a visible position"


def pin_constant_values():
    for causal in (False, True):
        for Nq, Nk in ((9, 9), (4, 13)):
            q = _rand(3, 2, 4, Nq, 8)
            k = _rand(4, 2, 2, Nk, 8)
            c = _rand(5, 8)
            v = np.broadcast_to(c, (2, 2, Nk, 8)).copy()
            O, _ = A.attention_fp64(q, k, v, 0.5, causal)
            _close(O, np.broadcast_to(c, O.shape), 1e-14, "constant V")


def pin_identical_keys_prefix_mean():
    for causal in (False, True):
        for Nq, Nk in ((12, 12), (5, 12)):
            d = 8
            q = _rand(6, 1, 3, Nq, d)
            kappa = _rand(7, d)
            k = np.broadcast_to(kappa, (1, 3, Nk, d)).copy()
            v = _rand(8, 1, 3, Nk, d)
            scale = 0.7
            O, lse = A.attention_fp64(q, k, v, scale, causal)
            for h in range(3):
                for i in range(Nq):
                    n = min(Nk, i + (Nk - Nq) + 1) if causal else Nk
                    _close(O[0, h, i], v[0, h, :n].mean(axis=0), 1e-14, "prefix mean")
                    expect = scale * float(q[0, h, i] @ kappa) + math.log(n)
                    _close(lse[0, h, i], expect, 1e-13, "prefix lse")


def pin_causal_row_zero():
    N, d = 10, 16
    q = _rand(9, 2, 2, N, d)
    k = _rand(10, 2, 2, N, d)
    v = _rand(11, 2, 2, N, d)
    O, lse = A.attention_fp64(q, k, v, 0.25, True)
    _close(O[:, :, 0], v[:, :, 0], 0.0, "causal row 0 equals v_0")
    _close(lse[:, :, 0], 0.25 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]), 1e-15,
           "causal row 0 lse")


def pin_gqa_equals_repeated_heads():
    q = _rand(12, 2, 8, 6, 8)
    k = _rand(13, 2, 2, 9, 8)
    v = _rand(14, 2, 2, 9, 8)
    for causal in (False, True):
        O, lse = A.attention_fp64(q, k, v, 0.4, causal)
        O2, lse2 = A.attention_fp64(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), 0.4,
                                    causal)
        _close(O, O2, 0.0, "GQA vs repeated heads")
        _close(lse, lse2, 0.0, "GQA lse vs repeated heads")


def pin_key_shift_invariance():
    q = _rand(15, 1, 2, 7, 8)
    k = _rand(16, 1, 2, 7, 8)
    v = _rand(17, 1, 2, 7, 8)
    u = _rand(18, 8)
    for causal in (False, True):
        O, lse = A.attention_fp64(q, k, v, 0.6, causal)
        O2, lse2 = A.attention_fp64(q, k + u, v, 0.6, causal)
        _close(O2, O, 1e-13, "key shift: O")
        _close(lse2, lse + 0.6 * (q @ u), 1e-13, "key shift: lse")


def pin_permutation_invariance():
    q = _rand(19, 1, 2, 6, 8)
    k = _rand(20, 1, 2, 11, 8)
    v = _rand(21, 1, 2, 11, 8)
    perm = np.random.default_rng(22).permutation(11)
    O, lse = A.attention_fp64(q, k, v, 0.5, False)
    O2, lse2 = A.attention_fp64(q, k[:, :, perm], v[:, :, perm], 0.5, False)
    _close(O2, O, 1e-14, "permutation: O")
    _close(lse2, lse, 1e-14, "permutation: lse")


def pin_dominant_key():
    # Query i aligns with key j*(i); every other score is >= 50 lower, so the softmax bound
    # |O_i - v_j*| <= 2 (Nk - 1) e^-50 max|v| holds.
    Nk, d = 16, 16
    k = np.zeros((1, 1, Nk, d))
    for j in range(Nk):
        k[0, 0, j, j] = 1.0
    q = np.zeros((1, 1, 4, d))
    targets = [3, 0, 15, 7]
    for i, j in enumerate(targets):
        q[0, 0, i, j] = 100.0
    v = _rand(23, 1, 1, Nk, d)
    O, lse = A.attention_fp64(q, k, v, 0.5, False)
    bound = 2 * (Nk - 1) * math.exp(-50) * np.abs(v).max()
    for i, j in enumerate(targets):
        _close(O[0, 0, i], v[0, 0, j], bound, "dominant key")
        assert abs(lse[0, 0, i] - 50.0) <= (Nk - 1) * math.exp(-50) + 1e-14


def pin_fully_masked_rows():
    q = _rand(24, 1, 2, 6, 8)
    k = _rand(25, 1, 2, 2, 8)
    v = _rand(26, 1, 2, 2, 8)
    O, lse = A.attention_fp64(q, k, v, 0.5, True)  # rows 0..3 see no key (j <= i - 4)
    assert np.all(O[:, :, :4] == 0.0) and np.all(np.isneginf(lse[:, :, :4]))
    assert np.all(np.isfinite(lse[:, :, 4:]))
    _close(O[:, :, 4], v[:, :, 0], 0.0, "first visible row sees only key 0")
    O0, lse0 = A.attention_fp64(q, k[:, :, :0], v[:, :, :0], 0.5, False)
    assert np.all(O0 == 0.0) and np.all(np.isneginf(lse0)), "Nk = 0 gives empty rows"


def pin_default_scale():
    q = _rand(27, 1, 2, 5, 16)
    k = _rand(28, 1, 2, 5, 16)
    v = _rand(29, 1, 2, 5, 16)
    O, lse = A.attention_fp64(q, k, v, 0.0, True)
    O2, lse2 = A.attention_fp64(q, k, v, 0.25, True)
    _close(O, O2, 0.0, "scale 0 means 1/sqrt(d)")
    _close(lse, lse2, 0.0, "scale 0 means 1/sqrt(d)")


# ---- brute force and a library routine -----------------------------------------------------

def _brute(q, k, v, scale, causal):
    """Scalar Python: O_i = Σ exp(s_ij) v_j / Σ exp(s_ij), lse_i = ln Σ exp(s_ij), no max shift."""
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    O = np.zeros((B, Hq, Nq, d))
    lse = np.full((B, Hq, Nq), -np.inf)
    for b in range(B):
        for h in range(Hq):
            hk = h // (Hq // Hkv)
            for i in range(Nq):
                w = []
                for j in range(Nk):
                    if causal and j > i + (Nk - Nq):
                        continue
                    s = scale * math.fsum(float(q[b, h, i, t]) * float(k[b, hk, j, t])
                                          for t in range(d))
                    w.append((math.exp(s), j))
                if not w:
                    continue
                z = math.fsum(e for e, _ in w)
                lse[b, h, i] = math.log(z)
                for t in range(d):
                    O[b, h, i, t] = math.fsum(e * float(v[b, hk, j, t]) for e, j in w) / z
    return O, lse


def pin_brute_force_small():
    cases = [(1, 2, 2, 5, 5, 4, True), (2, 4, 2, 3, 9, 8, True), (1, 3, 1, 8, 8, 8, False),
             (1, 2, 1, 16, 16, 8, True), (1, 2, 2, 6, 3, 4, True)]
    for n, (B, Hq, Hkv, Nq, Nk, d, causal) in enumerate(cases):
        q = _rand(100 + n, B, Hq, Nq, d)
        k = _rand(200 + n, B, Hkv, Nk, d)
        v = _rand(300 + n, B, Hkv, Nk, d)
        O, lse = A.attention_fp64(q, k, v, 0.45, causal)
        Ob, lseb = _brute(q, k, v, 0.45, causal)
        _close(O, Ob, 1e-12, f"brute force O case {n}")
        _close(lse, lseb, 1e-12, f"brute force lse case {n}")


def pin_scipy_softmax():
    B, Hq, Hkv, Nq, Nk, d = 2, 4, 2, 24, 40, 32
    q = _rand(30, B, Hq, Nq, d)
    k = _rand(31, B, Hkv, Nk, d)
    v = _rand(32, B, Hkv, Nk, d)
    for causal in (False, True):
        O, lse = A.attention_fp64(q, k, v, 0.2, causal)
        vis = _tril_visible(Nq, Nk, causal)
        for b in range(B):
            for h in range(Hq):
                hk = h // (Hq // Hkv)
                s = 0.2 * np.einsum("id,jd->ij", q[b, h], k[b, hk])
                s = np.where(vis, s, -np.inf)
                _close(O[b, h], np.einsum("ij,jd->id", scipy.special.softmax(s, axis=1),
                                          v[b, hk]), 1e-13, "scipy softmax O")
                _close(lse[b, h], scipy.special.logsumexp(s, axis=1), 1e-13, "scipy lse")


def pin_golden_closed_form():
    with open(os.path.join(GOLDEN, "closed_form_small.json")) as f:
        g = json.load(f)
    q = np.array(g["q"])[None, None]
    k = np.array(g["k"])[None, None]
    v = np.array(g["v"])[None, None]
    for case in g["cases"]:
        O, lse = A.attention_fp64(q, k, v, g["scale"], case["causal"])
        _close(O[0, 0], np.array(case["out"]), g["tolerance"], "golden O")
        _close(lse[0, 0], np.array(case["lse"]), g["tolerance"], "golden lse")


# ---- the split-KV model and the FA2 recurrence ---------------------------------------------

def pin_split_combine_equals_single_pass():
    B, Hq, Hkv, d = 2, 8, 2, 16
    for Nq, Nk, causal in ((1, 37, True), (4, 16, True), (4, 33, False), (6, 5, True)):
        q = _rand(40, B, Hq, Nq, d)
        k = _rand(41, B, Hkv, Nk, d)
        v = _rand(42, B, Hkv, Nk, d)
        O, lse = A.attention_fp64(q, k, v, 0.3, causal)
        for S in sorted({1, 2, 3, min(16, Nk), Nk}):
            O_s, m_s, l_s = A.splitkv_partials_fp64(q, k, v, 0.3, causal, S)
            Oc, lsec = A.combine_fp64(O_s, m_s, l_s)
            _close(Oc, O, 1e-12, f"split combine O (S={S})")
            _close(lsec, lse, 1e-12, f"split combine lse (S={S})")
            # partials are locally normalised softmax outputs of their own key chunk
            L = -(-Nk // S)
            for s in range(S):
                k0, k1 = min(s * L, Nk), min((s + 1) * L, Nk)
                vis = _tril_visible(Nq, Nk, causal)[:, k0:k1]
                has = vis.any(axis=1)
                if not causal and k1 > k0:
                    # a non-causal chunk's partial is plain attention over that chunk alone
                    Osub, lsub = A.attention_fp64(q, k[:, :, k0:k1], v[:, :, k0:k1], 0.3, False)
                    _close(O_s[:, :, :, s], Osub, 1e-12, "partial = chunk softmax")
                    _close(m_s[:, :, :, s] + np.log(l_s[:, :, :, s]), lsub, 1e-12,
                           "chunk logsumexp")
                assert np.all(l_s[:, :, ~has, s] == 0) and np.all(np.isneginf(m_s[:, :, ~has, s]))
                assert np.all(l_s[:, :, has, s] >= 1.0 - 1e-15), "local sum includes exp(0)"


def pin_tiled_recurrence_equals_definition():
    B, Hq, Hkv, d = 1, 4, 2, 8
    for Nq, Nk in ((19, 19), (7, 23), (23, 7)):
        q = _rand(50, B, Hq, Nq, d)
        k = _rand(51, B, Hkv, Nk, d)
        v = _rand(52, B, Hkv, Nk, d)
        for causal in (False, True):
            O, lse = A.attention_fp64(q, k, v, 0.5, causal)
            for Br, Bc in ((1, 1), (3, 5), (8, 8), (64, 4), (5, 64)):
                for skip in (False, True):
                    Ot, lset = A.flash2_tiled_fp64(q, k, v, 0.5, causal, Br, Bc, skip)
                    _close(Ot, O, 1e-12, f"tiled O Br={Br} Bc={Bc}")
                    _close(lset, lse, 1e-12, f"tiled lse Br={Br} Bc={Bc}")


def pin_decode_rows_equal_prefill_rows():
    B, Hq, Hkv, Nk, d = 1, 4, 2, 20, 8
    k = _rand(60, B, Hkv, Nk, d)
    v = _rand(61, B, Hkv, Nk, d)
    qfull = _rand(62, B, Hq, Nk, d)
    Ofull, lsefull = A.attention_fp64(qfull, k, v, 0.35, True)
    for Nq in (1, 4):
        O, lse = A.attention_fp64(qfull[:, :, Nk - Nq:], k, v, 0.35, True)
        _close(O, Ofull[:, :, Nk - Nq:], 1e-15, "decode rows = last prefill rows")
        _close(lse, lsefull[:, :, Nk - Nq:], 1e-15, "decode lse = last prefill lse")


def pin_row_subset_equals_full_rows():
    B, Hq, Hkv, Nq, Nk, d = 2, 4, 2, 37, 53, 8
    q = _rand(70, B, Hq, Nq, d)
    k = _rand(71, B, Hkv, Nk, d)
    v = _rand(72, B, Hkv, Nk, d)
    rows = np.array([0, 1, 17, 36, 5])
    for causal in (False, True):
        O, lse = A.attention_fp64(q, k, v, 0.3, causal)
        Or, lser = A.attention_rows_fp64(q, k, v, 0.3, causal, rows)
        _close(Or, O[:, :, rows], 1e-15, "row subset O")
        _close(lser, lse[:, :, rows], 1e-15, "row subset lse")
    # a row's result depends on its position only through the mask: identical keys give the
    # prefix mean of the visible values for each sampled position
    kappa = _rand(73, d)
    kk = np.broadcast_to(kappa, (B, Hkv, Nk, d)).copy()
    Or, _ = A.attention_rows_fp64(q, kk, v, 0.3, True, rows)
    for n, i in enumerate(rows):
        _close(Or[:, :, n], np.repeat(v[:, :, :i + (Nk - Nq) + 1].mean(axis=2), 2, axis=1),
               1e-14, "row subset prefix mean")


# ---- per-batch key lengths and attention bias -----------------------------------------------

def _brute_general(q, k, v, scale, causal, lengths=None, bias=None):
    """Scalar Python with per-batch key lengths L_b (keys j < L_b exist, causal visibility
    j <= i + L_b - Nq) and an additive bias bias[b|0, h|0, i, j] on the scaled score."""
    B, Hq, Nq, d = q.shape
    Hkv, Nk, dv = k.shape[1], k.shape[2], v.shape[3]
    O = np.zeros((B, Hq, Nq, dv))
    lse = np.full((B, Hq, Nq), -np.inf)
    for b in range(B):
        Lb = Nk if lengths is None else int(lengths[b])
        for h in range(Hq):
            hk = h // (Hq // Hkv)
            for i in range(Nq):
                w = []
                for j in range(Lb):
                    if causal and j > i + (Lb - Nq):
                        continue
                    sc = scale * math.fsum(float(q[b, h, i, t]) * float(k[b, hk, j, t])
                                           for t in range(d))
                    if bias is not None:
                        sc += float(bias[b if bias.shape[0] > 1 else 0,
                                         h if bias.shape[1] > 1 else 0, i, j])
                    w.append((math.exp(sc), j))
                if not w:
                    continue
                z = math.fsum(e for e, _ in w)
                lse[b, h, i] = math.log(z)
                for t in range(dv):
                    O[b, h, i, t] = math.fsum(e * float(v[b, hk, j, t]) for e, j in w) / z
    return O, lse


def pin_varlen_brute_force():
    B, Hq, Hkv, Nq, Nk, d = 4, 2, 1, 3, 6, 4
    q, k, v = _rand(600, B, Hq, Nq, d), _rand(601, B, Hkv, Nk, d), _rand(602, B, Hkv, Nk, d)
    L = np.array([6, 2, 0, 4])
    for causal in (False, True):
        O, lse = A.attention_fp64(q, k, v, 0.5, causal, seqlens_k=L)
        Ob, lseb = _brute_general(q, k, v, 0.5, causal, lengths=L)
        _close(O, Ob, 1e-12, "varlen brute force O")
        _close(lse, lseb, 1e-12, "varlen brute force lse")
        rows = np.array([0, 2])
        Or, lr = A.attention_rows_fp64(q, k, v, 0.5, causal, rows, seqlens_k=L)
        _close(Or, Ob[:, :, rows], 1e-12, "varlen rows O")
        _close(lr, lseb[:, :, rows], 1e-12, "varlen rows lse")


def pin_varlen_ignores_keys_past_length():
    """Keys at or past L_b do not exist: replacing them by anything changes nothing."""
    B, Hq, Hkv, Nq, Nk, d = 3, 4, 2, 5, 9, 8
    q, k, v = _rand(610, B, Hq, Nq, d), _rand(611, B, Hkv, Nk, d), _rand(612, B, Hkv, Nk, d)
    L = np.array([9, 5, 7])
    k2, v2 = k.copy(), v.copy()
    for b in range(B):
        k2[b, :, L[b]:] = 1e3 * _rand(613 + b, Hkv, Nk - L[b], d)
        v2[b, :, L[b]:] = -7.0
    for causal in (False, True):
        O1, l1 = A.attention_fp64(q, k, v, 0.3, causal, seqlens_k=L)
        O2, l2 = A.attention_fp64(q, k2, v2, 0.3, causal, seqlens_k=L)
        _close(O1, O2, 0.0, "varlen past-length O")
        _close(l1, l2, 0.0, "varlen past-length lse")


def pin_varlen_closed_forms():
    """L_b = 0: O = 0, LSE = -inf.  L_b = 1: every row sees key 0 only (non-causal, or causal
    rows i >= Nq - 1), so O = v_0 and LSE = scale·q·k_0; the other causal rows see nothing."""
    B, Hq, Hkv, Nq, Nk, d = 2, 2, 2, 4, 6, 8
    q, k, v = _rand(620, B, Hq, Nq, d), _rand(621, B, Hkv, Nk, d), _rand(622, B, Hkv, Nk, d)
    L = np.array([0, 1])
    for causal in (False, True):
        O, lse = A.attention_fp64(q, k, v, 0.7, causal, seqlens_k=L)
        assert np.all(O[0] == 0) and np.all(np.isneginf(lse[0])), "L = 0 row not empty"
        for h in range(Hq):
            for i in range(Nq):
                if causal and i < Nq - 1:
                    assert np.all(O[1, h, i] == 0) and np.isneginf(lse[1, h, i])
                    continue
                _close(O[1, h, i], v[1, h, 0], 1e-15, "L = 1 output")
                _close(lse[1, h, i], 0.7 * float(q[1, h, i] @ k[1, h, 0]), 1e-13, "L = 1 lse")


def pin_varlen_split_combine():
    B, Hq, Hkv, Nq, Nk, d = 3, 4, 2, 4, 37, 8
    q, k, v = _rand(630, B, Hq, Nq, d), _rand(631, B, Hkv, Nk, d), _rand(632, B, Hkv, Nk, d)
    L = np.array([37, 11, 0])
    for causal in (False, True):
        for S in (1, 3, 5, 37):
            O_s, m_s, l_s = A.splitkv_partials_fp64(q, k, v, 0.4, causal, S, seqlens_k=L)
            Oc, lc = A.combine_fp64(O_s, m_s, l_s)
            Ob, lb = _brute_general(q, k, v, 0.4, causal, lengths=L)
            _close(Oc, Ob, 1e-12, f"varlen split/combine O S={S}")
            _close(lc, lb, 1e-12, f"varlen split/combine lse S={S}")


def pin_bias_brute_force():
    B, Hq, Hkv, Nq, Nk, d = 2, 4, 2, 3, 5, 4
    q, k, v = _rand(640, B, Hq, Nq, d), _rand(641, B, Hkv, Nk, d), _rand(642, B, Hkv, Nk, d)
    L = np.array([5, 3])
    for shape in ((1, 1), (B, 1), (1, Hq), (B, Hq)):
        bias = _rand(643 + shape[0] + 3 * shape[1], shape[0], shape[1], Nq, Nk)
        for causal in (False, True):
            for lengths in (None, L):
                O, lse = A.attention_fp64(q, k, v, 0.6, causal, bias=bias, seqlens_k=lengths)
                Ob, lseb = _brute_general(q, k, v, 0.6, causal, lengths=lengths, bias=bias)
                _close(O, Ob, 1e-12, f"bias brute force O {shape}")
                _close(lse, lseb, 1e-12, f"bias brute force lse {shape}")
                O_s, m_s, l_s = A.splitkv_partials_fp64(q, k, v, 0.6, causal, 2, bias=bias,
                                                        seqlens_k=lengths)
                Oc, lc = A.combine_fp64(O_s, m_s, l_s)
                _close(Oc, Ob, 1e-12, f"bias split/combine O {shape}")
                _close(lc, lseb, 1e-12, f"bias split/combine lse {shape}")


def pin_bias_row_shift():
    """Adding c_i to every bias entry of row i leaves O unchanged and adds c_i to LSE."""
    B, Hq, Hkv, Nq, Nk, d = 2, 2, 1, 6, 10, 8
    q, k, v = _rand(650, B, Hq, Nq, d), _rand(651, B, Hkv, Nk, d), _rand(652, B, Hkv, Nk, d)
    bias = _rand(653, B, Hq, Nq, Nk)
    c = 3.0 * _rand(654, B, Hq, Nq)
    for causal in (False, True):
        O1, l1 = A.attention_fp64(q, k, v, 0.25, causal, bias=bias)
        O2, l2 = A.attention_fp64(q, k, v, 0.25, causal, bias=bias + c[..., None])
        _close(O1, O2, 1e-12, "bias row shift O")
        _close(l1 + c, l2, 1e-12, "bias row shift lse")


def pin_bias_rank_one_is_extra_head_dim():
    """A bias scale·u_i·w_j equals one more head dimension (q_i, u_i)·(k_j, w_j) at the same
    scale, with no bias."""
    B, Hq, Hkv, Nq, Nk, d = 1, 2, 2, 5, 7, 6
    q, k, v = _rand(660, B, Hq, Nq, d), _rand(661, B, Hkv, Nk, d), _rand(662, B, Hkv, Nk, d)
    u, w = _rand(663, B, Hq, Nq), _rand(664, B, Hkv, Nk)
    bias = 0.35 * u[..., :, None] * w[..., None, :]
    qa = np.concatenate([q, u[..., None]], axis=-1)
    ka = np.concatenate([k, w[..., None]], axis=-1)
    va = v
    for causal in (False, True):
        O1, l1 = A.attention_fp64(q, k, v, 0.35, causal, bias=bias)
        Ob, lb = _brute_general(qa, ka, va, 0.35, causal)
        _close(O1, Ob, 1e-12, "rank-one bias O")
        _close(l1, lb, 1e-12, "rank-one bias lse")


def pin_bias_neg_inf_is_mask():
    """A bias that is -inf exactly where the causal mask hides a key and 0 elsewhere gives the
    causal result with no bias; a row biased to -inf everywhere has no visible key."""
    B, Hq, Hkv, Nq, Nk, d = 2, 3, 1, 5, 9, 4
    q, k, v = _rand(670, B, Hq, Nq, d), _rand(671, B, Hkv, Nk, d), _rand(672, B, Hkv, Nk, d)
    rows, cols = np.arange(Nq)[:, None], np.arange(Nk)[None, :]
    bias = np.where(cols <= rows + (Nk - Nq), 0.0, -np.inf)[None, None]
    Oc, lc = A.attention_fp64(q, k, v, 0.5, True)
    Ob, lb = A.attention_fp64(q, k, v, 0.5, False, bias=bias)
    _close(Ob, Oc, 1e-12, "-inf bias as causal mask O")
    _close(lb, lc, 1e-12, "-inf bias as causal mask lse")
    O_s, m_s, l_s = A.splitkv_partials_fp64(q, k, v, 0.5, False, 3, bias=bias)
    Os, ls = A.combine_fp64(O_s, m_s, l_s)
    _close(Os, Oc, 1e-12, "-inf bias as causal mask, split O")
    _close(ls, lc, 1e-12, "-inf bias as causal mask, split lse")
    full = np.zeros((1, Hq, Nq, Nk))
    full[0, 1, 2, :] = -np.inf
    O, lse = A.attention_fp64(q, k, v, 0.5, False, bias=full)
    assert np.all(O[:, 1, 2] == 0.0) and np.all(lse[:, 1, 2] == -np.inf), "all -inf row"
    assert np.isfinite(O).sum() == O.size and np.isfinite(lse).sum() == lse.size - B
    O_s, m_s, l_s = A.splitkv_partials_fp64(q, k, v, 0.5, False, 2, bias=full)
    assert np.all(l_s[:, 1, 2] == 0.0) and np.all(m_s[:, 1, 2] == -np.inf), "all -inf split"


# ---- backward ------------------------------------------------------------------------------

def _loss(q, k, v, g, scale, causal):
    O, _ = A.attention_fp64(q, k, v, scale, causal)
    return float((O * g).sum())


def pin_bwd_finite_differences():
    """Every gradient element against a central difference of L = Σ g ∘ O through the forward
    oracle (itself pinned above), with GQA, causal and non-causal, rows without keys."""
    h = 1e-6
    for causal, (Nq, Nk) in ((False, (4, 5)), (True, (4, 5)), (True, (5, 3))):
        B, Hq, Hkv, d = 1, 2, 1, 3
        q, k, v = _rand(700, B, Hq, Nq, d), _rand(701, B, Hkv, Nk, d), _rand(702, B, Hkv, Nk, d)
        g = _rand(703, B, Hq, Nq, d)
        grads = A.attention_backward_fp64(q, k, v, g, 0.7, causal)
        for t, (x, gx) in enumerate(zip((q, k, v), grads)):
            num = np.zeros_like(x)
            for idx in np.ndindex(*x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p = [q, k, v]
                args_m = [q, k, v]
                args_p[t], args_m[t] = xp, xm
                num[idx] = (_loss(*args_p, g, 0.7, causal) - _loss(*args_m, g, 0.7, causal)) / (2 * h)
            _close(gx, num, 1e-7, f"finite differences causal={causal} tensor {'qkv'[t]}")


def pin_bwd_varlen_finite_differences():
    """With per-element key lengths (0, 1, a ragged 3 and all 5 keys), every gradient element
    against a central difference of L = Σ g ∘ O through the forward oracle with those lengths
    (pinned above): keys past an element's length do not move O, so their gradients are zero,
    and the causal mask follows the length."""
    h = 1e-6
    L = [0, 1, 3, 5]
    for causal, Nq in ((False, 4), (True, 4), (True, 2)):
        B, Hq, Hkv, Nk, d = 4, 2, 1, 5, 3
        q, k, v = _rand(730, B, Hq, Nq, d), _rand(731, B, Hkv, Nk, d), _rand(732, B, Hkv, Nk, d)
        g = _rand(733, B, Hq, Nq, d)

        def loss(q_, k_, v_):
            O, _ = A.attention_fp64(q_, k_, v_, 0.6, causal, seqlens_k=L)
            return float((O * g).sum())

        grads = A.attention_backward_fp64(q, k, v, g, 0.6, causal, seqlens_k=L)
        for t, (x, gx) in enumerate(zip((q, k, v), grads)):
            num = np.zeros_like(x)
            for idx in np.ndindex(*x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p, args_m = [q, k, v], [q, k, v]
                args_p[t], args_m[t] = xp, xm
                num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
            _close(gx, num, 1e-7, f"varlen finite differences causal={causal} tensor {'qkv'[t]}")
        for b, Lb in enumerate(L):
            assert np.all(grads[1][b, :, Lb:] == 0) and np.all(grads[2][b, :, Lb:] == 0)
        assert np.all(grads[0][0] == 0), "no key: dq = 0"


def pin_bwd_bias_finite_differences():
    """With an additive bias (a per-(batch, head) one with -inf entries and a broadcast one, with
    and without key lengths), every gradient element against a central difference of
    L = Σ g ∘ O through the forward oracle with that bias (pinned above)."""
    h = 1e-6
    B, Hq, Hkv, Nq, Nk, d = 2, 2, 1, 3, 4, 3
    q, k, v = _rand(740, B, Hq, Nq, d), _rand(741, B, Hkv, Nk, d), _rand(742, B, Hkv, Nk, d)
    g = _rand(743, B, Hq, Nq, d)
    full = _rand(744, B, Hq, Nq, Nk) * 2.0
    full[0, 1, 2, 1] = -np.inf
    full[1, 0, 0, :] = -np.inf  # a row with every key masked
    shared = _rand(745, 1, 1, Nq, Nk)
    for bias, causal, L in ((full, False, None), (full, True, None), (shared, True, [2, 4])):
        def loss(q_, k_, v_):
            O, _ = A.attention_fp64(q_, k_, v_, 0.8, causal, bias=bias, seqlens_k=L)
            return float((O * g).sum())

        grads = A.attention_backward_fp64(q, k, v, g, 0.8, causal, seqlens_k=L, bias=bias)
        for t, (x, gx) in enumerate(zip((q, k, v), grads)):
            num = np.zeros_like(x)
            for idx in np.ndindex(*x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p, args_m = [q, k, v], [q, k, v]
                args_p[t], args_m[t] = xp, xm
                num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
            _close(gx, num, 1e-7, f"bias finite differences causal={causal} tensor {'qkv'[t]}")


def pin_bwd_shift_invariances():
    """Shifting every key by c leaves O unchanged (a row-constant score change), so Σ_j dK_j = 0;
    shifting every value by c shifts O by c on rows with a visible key, so Σ_j dV_j = Σ dO over
    those rows; scaling q and scaling k by α change the scores alike, so Σ q∘dq = Σ k∘dk."""
    B, Hq, Hkv, Nq, Nk, d = 2, 4, 2, 6, 9, 5
    for causal, Nq_ in ((False, Nq), (True, Nq), (True, 12)):
        q, k, v = _rand(710, B, Hq, Nq_, d), _rand(711, B, Hkv, Nk, d), _rand(712, B, Hkv, Nk, d)
        g = _rand(713, B, Hq, Nq_, d)
        dq, dk, dv = A.attention_backward_fp64(q, k, v, g, 0.4, causal)
        _close(dk.sum(axis=2), np.zeros((B, Hkv, d)), 1e-12, "sum of dK")
        has = _tril_visible(Nq_, Nk, causal).any(axis=1)
        G = Hq // Hkv
        want = g[:, :, has].sum(axis=2).reshape(B, Hkv, G, d).sum(axis=2)
        _close(dv.sum(axis=2), want, 1e-12, "sum of dV")
        lhs = (q * dq).reshape(B, Hkv, G, Nq_, d).sum(axis=(2, 3, 4))
        rhs = (k * dk).sum(axis=(2, 3))
        _close(lhs, rhs, 1e-12, "q.dq = k.dk")


def pin_bwd_gqa_equals_repeated_heads():
    """With K/V shared by G query heads, dK and dV are the sums over those heads of the
    gradients computed with K/V repeated per head (plain multi-head attention)."""
    B, Hq, Hkv, Nq, Nk, d = 1, 6, 2, 5, 7, 4
    q, k, v = _rand(720, B, Hq, Nq, d), _rand(721, B, Hkv, Nk, d), _rand(722, B, Hkv, Nk, d)
    g = _rand(723, B, Hq, Nq, d)
    G = Hq // Hkv
    kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    for causal in (False, True):
        dq, dk, dv = A.attention_backward_fp64(q, k, v, g, 0.5, causal)
        dq1, dk1, dv1 = A.attention_backward_fp64(q, kr, vr, g, 0.5, causal)
        _close(dq, dq1, 1e-12, "GQA dq")
        _close(dk, dk1.reshape(B, Hkv, G, Nk, d).sum(axis=2), 1e-12, "GQA dk")
        _close(dv, dv1.reshape(B, Hkv, G, Nk, d).sum(axis=2), 1e-12, "GQA dv")


ALL_PINS = [
    pin_probs_rows_sum_to_one,
    pin_constant_values,
    pin_identical_keys_prefix_mean,
    pin_causal_row_zero,
    pin_gqa_equals_repeated_heads,
    pin_key_shift_invariance,
    pin_permutation_invariance,
    pin_dominant_key,
    pin_fully_masked_rows,
    pin_default_scale,
    pin_brute_force_small,
    pin_scipy_softmax,
    pin_golden_closed_form,
    pin_split_combine_equals_single_pass,
    pin_tiled_recurrence_equals_definition,
    pin_decode_rows_equal_prefill_rows,
    pin_row_subset_equals_full_rows,
    pin_varlen_brute_force,
    pin_varlen_ignores_keys_past_length,
    pin_varlen_closed_forms,
    pin_varlen_split_combine,
    pin_bias_brute_force,
    pin_bias_row_shift,
    pin_bias_rank_one_is_extra_head_dim,
    pin_bias_neg_inf_is_mask,
    pin_bwd_finite_differences,
    pin_bwd_varlen_finite_differences,
    pin_bwd_bias_finite_differences,
    pin_bwd_shift_invariances,
    pin_bwd_gqa_equals_repeated_heads,
]
