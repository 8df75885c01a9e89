"""Plant plausible mistakes in the oracle's steps (on the CPU) and check that the pin suite
catches every one of them.  This is what makes the pins meaningful: a dropped term, a wrong sign
or index, or a transposed operand anywhere in the oracle fails at least one pin."""
import numpy as np
import pytest

import oracle_pins
from oracle import attention as A

NEG_INF = -np.inf


def _softmax_cols(s, vis):
    p, m, l = _ORIG["_masked_softmax"](s, vis)
    e = np.where(vis, np.exp(np.where(vis, s, 0.0) - np.where(np.isfinite(m), m, 0.0)[:, None]), 0)
    cs = e.sum(axis=0, keepdims=True)
    return np.divide(e, cs, out=np.zeros_like(e), where=cs > 0), m, l


def _softmax_unnormalised(s, vis):
    p, m, l = _ORIG["_masked_softmax"](s, vis)
    return p * l[:, None], m, l


def _softmax_no_max_in_m(s, vis):
    p, m, l = _ORIG["_masked_softmax"](s, vis)
    return p, np.where(np.isfinite(m), 0.0, m), l


def _online_no_rescale_O(m, l, O, S, vblk):
    m_new = np.maximum(m, S.max(axis=1))
    ref = np.where(np.isfinite(m_new), m_new, 0.0)
    P = np.exp(S - ref[:, None])
    alpha = np.exp(m - ref)
    return m_new, alpha * l + P.sum(axis=1), O + P @ vblk


def _online_no_rescale_l(m, l, O, S, vblk):
    m_new = np.maximum(m, S.max(axis=1))
    ref = np.where(np.isfinite(m_new), m_new, 0.0)
    P = np.exp(S - ref[:, None])
    alpha = np.exp(m - ref)
    return m_new, l + P.sum(axis=1), alpha[:, None] * O + P @ vblk


def _combine_no_exp(O_s, m_s, l_s):
    return _ORIG["combine_fp64"](O_s, np.where(np.isfinite(m_s), 0.0, m_s), l_s)


def _partials_unnormalised(q, k, v, scale, causal, n_splits, **kw):
    O_s, m_s, l_s = _ORIG["splitkv_partials_fp64"](q, k, v, scale, causal, n_splits, **kw)
    return O_s * l_s[..., None], m_s, l_s


def _bias_scaled(qrows, kh, scale, bias_rows):
    s = _ORIG["_scores"](qrows, kh, scale)
    return s if bias_rows is None else s + scale * bias_rows


def _key_lengths_capacity(seqlens_k, B, Nk):
    return np.full(B, Nk, dtype=np.int64)


def _key_lengths_minus_one(seqlens_k, B, Nk):
    L = _ORIG["_key_lengths"](seqlens_k, B, Nk)
    return L if seqlens_k is None else np.maximum(L - 1, 0)


def _bias_transposed_heads(bias, B, Hq, Nq, Nk):
    view = _ORIG["_bias_view"](bias, B, Hq, Nq, Nk)
    if view is None:
        return None
    bias = np.asarray(bias, dtype=np.float64)
    return lambda b, hq: bias[0 if bias.shape[0] == 1 else b, 0 if bias.shape[1] == 1 else
                              (Hq - 1 - hq)]


MUTANTS = {
    "scale_dropped": ("_scores", lambda qr, kh, scale: qr @ kh.T),
    "scale_divides": ("_scores", lambda qr, kh, scale: (qr @ kh.T) / scale),
    "scale_squared": ("_scores", lambda qr, kh, scale: (qr @ kh.T) * scale * scale),
    "keys_reversed": ("_scores", lambda qr, kh, scale: (qr @ kh[::-1].T) * scale),
    "mask_reversed": ("visible_mask", lambda rows, Nq, Nk, causal: np.ones((len(rows), Nk), bool)
                      if not causal else np.arange(Nk)[None, :] >= rows[:, None] + (Nk - Nq)),
    "mask_top_left": ("visible_mask", lambda rows, Nq, Nk, causal: np.ones((len(rows), Nk), bool)
                      if not causal else np.arange(Nk)[None, :] <= rows[:, None]),
    "mask_off_by_one": ("visible_mask", lambda rows, Nq, Nk, causal:
                        np.ones((len(rows), Nk), bool)
                        if not causal else np.arange(Nk)[None, :] < rows[:, None] + (Nk - Nq)),
    "mask_ignored": ("visible_mask", lambda rows, Nq, Nk, causal: np.ones((len(rows), Nk), bool)),
    "mask_ignores_row_position": ("visible_mask", lambda rows, Nq, Nk, causal:
                                  np.ones((len(rows), Nk), bool) if not causal else
                                  np.arange(Nk)[None, :] <= np.arange(len(rows))[:, None]
                                  + (Nk - Nq)),
    "softmax_over_columns": ("_masked_softmax", _softmax_cols),
    "softmax_unnormalised": ("_masked_softmax", _softmax_unnormalised),
    "lse_without_max": ("_masked_softmax", _softmax_no_max_in_m),
    "values_reversed": ("_weighted_values", lambda p, vh: p @ vh[::-1]),
    "values_shifted": ("_weighted_values", lambda p, vh: p @ np.roll(vh, 1, axis=0)),
    "gqa_modulo": ("_kv_head", lambda hq, Hq, Hkv: hq % Hkv),
    "lse_natural_log_dropped": ("_row_lse", lambda m, l: np.where(l > 0, m + l, NEG_INF)),
    "lse_log2": ("_row_lse", lambda m, l: np.where(l > 0, m + np.log2(np.where(l > 0, l, 1)),
                                                   NEG_INF)),
    "online_O_not_rescaled": ("_online_step", _online_no_rescale_O),
    "online_l_not_rescaled": ("_online_step", _online_no_rescale_l),
    "combine_without_exp": ("combine_fp64", _combine_no_exp),
    "partials_unnormalised": ("splitkv_partials_fp64", _partials_unnormalised),
    "bias_dropped": ("_row_scores", lambda qr, kh, scale, br: _ORIG["_scores"](qr, kh, scale)),
    "bias_scaled": ("_row_scores", _bias_scaled),
    "bias_subtracted": ("_row_scores", lambda qr, kh, scale, br: _ORIG["_scores"](qr, kh, scale)
                        if br is None else _ORIG["_scores"](qr, kh, scale) - br),
    "bias_heads_reversed": ("_bias_view", _bias_transposed_heads),
    "seqlens_ignored": ("_key_lengths", _key_lengths_capacity),
    "seqlens_off_by_one": ("_key_lengths", _key_lengths_minus_one),
    "bwd_softmax_not_centred": ("_softmax_backward", lambda p, dp: p * dp),
    "bwd_softmax_sign": ("_softmax_backward",
                         lambda p, dp: p * ((p * dp).sum(axis=1, keepdims=True) - dp)),
    "bwd_softmax_centred_on_mean": ("_softmax_backward",
                                    lambda p, dp: p * (dp - dp.mean(axis=1, keepdims=True))),
    "bwd_gqa_last_head_only": ("_accumulate", lambda acc, x: x),
    "bwd_gqa_average": ("_accumulate", lambda acc, x: 0.5 * (acc + x)),
}

_ORIG = {name: getattr(A, name) for name, _ in MUTANTS.values()}


def _failing_pins():
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            failed.append(pin.__name__)
    return failed


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_mutant_is_caught(mutant, monkeypatch):
    name, fn = MUTANTS[mutant]
    monkeypatch.setattr(A, name, fn)
    failed = _failing_pins()
    assert failed, f"no pin caught the planted mistake {mutant!r}"


def test_unmutated_oracle_passes_every_pin():
    assert _failing_pins() == []
