"""CPU-only: the pins are strong enough.  Each test plants one plausible
mistake in the oracle (a dropped term, a wrong sign, an off-by-one, a wrong
index, a transposed operand) and requires that at least one pin fails."""

import numpy as np
import pytest

import oracle
import oracle.sdpa as oa
from tests import oracle_checks as oc

_real_probabilities = oa.probabilities
_real_allowed = oa.allowed_mask
_real_rowpos = oa.row_positions


def _mask_causal_strict(nq, nk, valid_len, causal, window, rows=None, **kw):
    if rows is None:
        rows = np.arange(nq)
    rows = np.asarray(rows)
    live, off = _real_rowpos(nq, nk, valid_len)
    pos = rows + off
    j = np.arange(nk)[None, :]
    ok = (rows[:, None] < live) & (j < valid_len)
    if causal:
        ok &= j < pos[:, None]          # planted: excludes the token itself
    if window > 0:
        ok &= (pos[:, None] - j) < window
    return ok & _optional_terms(pos, j, causal, window, kw)


def _mask_window_wide(nq, nk, valid_len, causal, window, rows=None, **kw):
    if rows is None:
        rows = np.arange(nq)
    rows = np.asarray(rows)
    live, off = _real_rowpos(nq, nk, valid_len)
    pos = rows + off
    j = np.arange(nk)[None, :]
    ok = (rows[:, None] < live) & (j < valid_len)
    if causal:
        ok &= j <= pos[:, None]
    if window > 0:
        ok &= (pos[:, None] - j) <= window   # planted: one key too many
    return ok & _optional_terms(pos, j, causal, window, kw)


def _mask_no_padding(nq, nk, valid_len, causal, window, rows=None, **kw):
    return _real_allowed(nq, nk, nk, causal, window, rows, **kw)  # planted


def _optional_terms(pos, j, causal, window, kw):
    """The two-sided window and sink terms as the real oracle has them, so
    that a planted mistake elsewhere stays the only difference.  Returns the
    keys the window condition removes unless a sink brings them back."""
    wr = kw.get("window_right", 0)
    sk = kw.get("sinks", 0)
    keep = np.ones((pos.shape[0], j.shape[1]), dtype=bool)
    if wr > 0:
        keep &= (j - pos[:, None]) < wr
    if sk > 0:
        sink = j < sk
        if causal:
            sink = sink & (j <= pos[:, None])
        keep |= sink
    return keep


def _mask_sinks_past_causal(nq, nk, valid_len, causal, window, rows=None,
                            window_right=0, sinks=0):
    ok = _real_allowed(nq, nk, valid_len, causal, window, rows,
                       window_right=window_right, sinks=sinks)
    if sinks > 0:
        if rows is None:
            rows = np.arange(nq)
        rows = np.asarray(rows)
        live, _ = _real_rowpos(nq, nk, valid_len)
        j = np.arange(nk)[None, :]
        ok |= (rows[:, None] < live) & (j < min(sinks, valid_len))  # planted:
    return ok                                     # sinks seen past causal


def _mask_right_wide(nq, nk, valid_len, causal, window, rows=None,
                     window_right=0, sinks=0):
    return _real_allowed(nq, nk, valid_len, causal, window, rows,
                         window_right=window_right + 1 if window_right > 0
                         else 0, sinks=sinks)     # planted: one key too many


def _rowpos_top_left(nq, nk, valid_len):
    live = valid_len if nq == nk else nq
    return live, 0                       # planted: decode query at position 0


def _rowpos_chunk_at_end(nq, nk, valid_len):
    live = valid_len if nq == nk else nq
    return live, valid_len - 1           # planted: right for one new token,
                                         # every chunk row past the end


def _probs_no_scale(q_rows, k_rows, scale, mask):
    return _real_probabilities(q_rows, k_rows, 1.0, mask)  # planted


def _probs_sign(q_rows, k_rows, scale, mask):
    return _real_probabilities(q_rows, k_rows, -scale, mask)  # planted


def _probs_lse_log2(q_rows, k_rows, scale, mask):
    p, lse = _real_probabilities(q_rows, k_rows, scale, mask)
    return p, lse / np.log(2.0)          # planted: log base 2


def _probs_mask_after_softmax(q_rows, k_rows, scale, mask):
    full = np.ones_like(mask)
    p, lse = _real_probabilities(q_rows, k_rows, scale, full)
    return np.where(mask, p, 0.0), lse   # planted: not renormalised


def _probs_no_max_shift_rounding(q_rows, k_rows, scale, mask):
    q64 = np.asarray(q_rows, dtype=np.float64)
    k64 = np.asarray(k_rows, dtype=np.float64)
    s = scale * (q64 @ k64.T)
    e = np.where(mask, np.exp(s), 0.0)
    l = e.sum(axis=1, keepdims=True)
    p = e / np.where(l > 0, l, 1.0)
    lse = np.where(mask.any(axis=1), np.log(l[:, 0] + 1e-300), -np.inf)
    return p, lse + 1e-9                 # planted: tiny lse offset


def _head_map_mod(hq, hkv):
    return [h % hkv for h in range(hq)]  # planted: interleaved groups


MUTANTS = {
    "causal_excludes_self": ("allowed_mask", _mask_causal_strict),
    "window_one_too_wide": ("allowed_mask", _mask_window_wide),
    "padding_ignored": ("allowed_mask", _mask_no_padding),
    "decode_top_left": ("row_positions", _rowpos_top_left),
    "chunk_at_end": ("row_positions", _rowpos_chunk_at_end),
    "sinks_past_causal": ("allowed_mask", _mask_sinks_past_causal),
    "window_right_wide": ("allowed_mask", _mask_right_wide),
    "scale_dropped": ("probabilities", _probs_no_scale),
    "score_sign_flipped": ("probabilities", _probs_sign),
    "lse_log2": ("probabilities", _probs_lse_log2),
    "mask_after_softmax": ("probabilities", _probs_mask_after_softmax),
    "lse_offset": ("probabilities", _probs_no_max_shift_rounding),
    "gqa_interleaved": ("_head_map", _head_map_mod),
}


def _run_checks(attn):
    failed = []
    for check in oc.ALL_CHECKS:
        try:
            check(attn)
        except AssertionError:
            failed.append(check.__name__)
    return failed


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(oa, attr, fn)
    failed = _run_checks(oa.attention)
    assert failed, f"no pin catches the planted mistake {name!r}"


def test_swapped_operand_is_caught():
    def attn_k_for_v(q, k, v, **kw):
        return oracle.attention(q, k, k, **kw)  # planted: K used as V
    assert _run_checks(attn_k_for_v)


def test_real_oracle_passes_all():
    assert _run_checks(oracle.attention) == []
