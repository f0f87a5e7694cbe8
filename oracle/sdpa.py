"""fp64 reference of masked multi-head scaled dot-product attention.

Test infrastructure only (see the package docstring).  Plain NumPy; one matrix
product per (batch, head, chunk of query rows) is the only library primitive
used besides elementwise exp/log/max/sum.  The mask is built explicitly over
every key, never from range shortcuts.

Layouts follow the [batch, heads, n, d] convention of the PyTorch SDPA call in
the O(n^2) tutorial page (Example 2) and of its Linformer example (Example 3):
    q: [B, Hq, Nq, d]     k, v: [B, Hkv, Nk, d]
    o: [B, Hq, Nq, d]     lse:  [B, Hq, Nq]
"""

import numpy as np

_ROW_CHUNK = 512  # query rows per dense score block (bounds memory at N=16384)


def row_positions(nq, nk, valid_len):
    """Number of live query rows and the position offset of query row 0.

    Reading of the pages (they only describe the square self-attention case and
    the one-token generation step):
      * Nq == Nk (self-attention over a padded batch): the first `valid_len`
        rows are live and query i sits at position i.
      * Nq != Nk (here: one new token against a KV cache, as in the SpAtten
        review's Background section on the generation stage, where the current
        token's K and V are appended to the cache): all Nq rows are live and
        they are the LAST Nq positions of the sequence, so query i sits at
        position valid_len - Nq + i ("bottom-right" alignment).
    Returns (live_rows, offset).
    """
    live = valid_len if nq == nk else nq
    return live, valid_len - live


def allowed_mask(nq, nk, valid_len, causal, window, rows=None, *,
                 window_right=0, sinks=0):
    """Boolean [len(rows), nk] matrix: may query row i attend to key j?

    allowed(i, j) holds iff all of
      * i is a live query row and j < valid_len: padding tokens neither give
        nor receive attention (explainer page, "Padding Masking"; tutorial page
        Example 7, pad tokens skipped);
      * causal => j <= pos(i): each token attends only to itself and earlier
        tokens (explainer page, "Look-Ahead Masking");
      * window > 0 => pos(i) - j < window: a one-sided look-back window that
        includes the token itself, i.e. the token and the previous window-1
        keys (tutorial page, "Local Window Attention": each token looks only at
        its neighbours; reading: one-sided, causal direction).
    Two further options (the tutorial page's local window read as a
    neighbourhood on both sides, and its strategy list's global tokens / the
    explainer page's attention sink read as keys every query sees):
      * window_right > 0 => j - pos(i) < window_right (the right limit of a
        two-sided window; with `window` as the left limit the neighbourhood
        is pos - window < j < pos + window_right);
      * sinks > 0: keys j < sinks are allowed whatever the window says (the
        causal and padding conditions still apply).
    window <= 0 means no window.  The explainer page sets masked scores to a
    "very small negative value (-inf)"; the reading taken here is exact
    exclusion (-inf), never a finite large negative number.
    """
    if rows is None:
        rows = np.arange(nq)
    rows = np.asarray(rows, dtype=np.int64)
    live, off = row_positions(nq, nk, valid_len)
    pos = rows + off
    j = np.arange(nk, dtype=np.int64)[None, :]
    ok = (rows[:, None] < live) & (j < valid_len)
    if causal:
        ok &= j <= pos[:, None]
    win = np.ones_like(ok)
    if window > 0:
        win &= (pos[:, None] - j) < window
    if window_right > 0:
        win &= (j - pos[:, None]) < window_right
    if sinks > 0:
        win |= j < sinks
    return ok & win


def probabilities(q_rows, k_rows, scale, mask):
    """Softmax probabilities for one head, straight from the definition.

    q_rows: [n, d], k_rows: [m, d], mask: bool [n, m].
    Score s_ij = scale * q_i . k_j (SpAtten review, Background - Attention
    Mechanism, the score Q K^T / sqrt(D); the explainer page's scaled
    dot-product divides by sqrt(d_k); here `scale` is the caller's factor,
    1/sqrt(d) by default).  Probability p_ij = exp(s_ij) / sum_j exp(s_ij)
    over allowed j (SpAtten review, D. Progressive Quantization, the
    attention-probability equation), evaluated as exp(s_ij - m_i) / l_i with
    m_i the row maximum, which is the same value.
    Returns (P [n, m], lse [n]).  A row with no allowed key has P = 0 and
    lse = -inf.
    """
    q64 = np.asarray(q_rows, dtype=np.float64)
    k64 = np.asarray(k_rows, dtype=np.float64)
    s = scale * (q64 @ k64.T)
    s = np.where(mask, s, -np.inf)
    any_allowed = mask.any(axis=1)
    m = np.where(any_allowed, s.max(axis=1, initial=-np.inf), 0.0)
    e = np.where(mask, np.exp(s - m[:, None]), 0.0)
    l = e.sum(axis=1)
    safe_l = np.where(any_allowed, l, 1.0)
    p = e / safe_l[:, None]
    with np.errstate(divide="ignore"):
        lse = np.where(any_allowed, m + np.log(safe_l), -np.inf)
    return p, lse


def _head_map(hq, hkv):
    """Query head h reads K/V head h // (Hq/Hkv).

    Grouped-query attention is only named on the pages ("Attentions Under the
    Microscope", Methodology, the list of variants); the reading taken is
    contiguous groups: Hkv == Hq is multi-head attention, Hkv == 1 is
    multi-query attention.
    """
    if hq % hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    g = hq // hkv
    return [h // g for h in range(hq)]


def _extra(window_right, sinks):
    """Keyword arguments for the two optional mask terms, only when used."""
    kw = {}
    if window_right > 0:
        kw["window_right"] = window_right
    if sinks > 0:
        kw["sinks"] = sinks
    return kw


def _valid_len(seqlens, b, nk):
    if seqlens is None:
        return nk
    return int(min(max(int(seqlens[b]), 0), nk))


def attention(q, k, v, *, scale=None, causal=False, window=0, seqlens=None,
              window_right=0, sinks=0):
    """Full fp64 attention output and log-sum-exp.

    Each head is an independent attention (explainer page, "Multi-Head
    Attention": parallel heads, each its own scaled dot-product attention);
    the output row is O_i = sum_j p_ij v_j (explainer page, softmax
    normalisation and weighted sum; SpAtten review, Softmax(score) V).
    lse_i = log sum_{allowed j} exp(s_ij), natural log, scale applied (not on
    the pages; reading).  Rows with no allowed key: O_i = 0, lse_i = -inf.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    b_, hq, nq, d = q.shape
    _, hkv, nk, _ = k.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    heads = _head_map(hq, hkv)
    o = np.zeros((b_, hq, nq, d), dtype=np.float64)
    lse = np.full((b_, hq, nq), -np.inf, dtype=np.float64)
    for b in range(b_):
        vlen = _valid_len(seqlens, b, nk)
        for h in range(hq):
            hk = heads[h]
            k64 = k[b, hk].astype(np.float64)
            v64 = v[b, hk].astype(np.float64)
            for r0 in range(0, nq, _ROW_CHUNK):
                rows = np.arange(r0, min(nq, r0 + _ROW_CHUNK))
                mask = allowed_mask(nq, nk, vlen, causal, window, rows,
                                    **_extra(window_right, sinks))
                p, l_ = probabilities(q[b, h, rows], k64, scale, mask)
                # keys at or beyond the valid length are never allowed, so
                # their probabilities are exactly 0; leave those V rows out of
                # the sum so padded contents (even NaN) cannot leak in.
                o[b, h, rows] = p[:, :vlen] @ v64[:vlen]
                lse[b, h, rows] = l_
    return o, lse


def attention_rows(q, k, v, picks, *, scale=None, causal=False, window=0,
                   seqlens=None, window_right=0, sinks=0):
    """Oracle values for selected output rows only.

    picks: iterable of (b, h, i).  Returns (o [n, d] fp64, lse [n] fp64) in
    the order given.  Same definition as `attention`; used to check sampled
    rows of full-size workloads where the dense oracle would be slow.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    _, hq, nq, d = q.shape
    _, hkv, nk, _ = k.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    heads = _head_map(hq, hkv)
    picks = list(picks)
    o = np.zeros((len(picks), d), dtype=np.float64)
    lse = np.full((len(picks),), -np.inf, dtype=np.float64)
    for n, (b, h, i) in enumerate(picks):
        hk = heads[h]
        vlen = _valid_len(seqlens, b, nk)
        mask = allowed_mask(nq, nk, vlen, causal, window, [i],
                            **_extra(window_right, sinks))
        p, l_ = probabilities(q[b, h, [i]], k[b, hk], scale, mask)
        o[n] = p[0, :vlen] @ v[b, hk, :vlen].astype(np.float64)
        lse[n] = l_[0]
    return o, lse
