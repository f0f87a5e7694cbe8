"""Pins for the fp64 oracle: each check compares an attention callable with
something fixed independently of it (brute-force loops, a closed form, an
invariant of the definition, a value derived from a page's worked example, or
an independent library routine).

Every check takes `attn`, a callable with the signature of
`oracle.attention(q, k, v, *, scale, causal, window, seqlens) -> (o, lse)`, and
raises AssertionError on a mismatch.  The pin tests run them on the real
oracle; the mutation tests run them on deliberately broken copies and require
that at least one check fails for each planted mistake.
"""

import json
import math
import os

import numpy as np

from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _tolist(a):
    return np.asarray(a, dtype=np.float64).tolist()


# --------------------------------------------------------------------------
# brute force on tiny inputs

BRUTE_CASES = [
    # (B, Hq, Hkv, Nq, Nk, d, causal, window, padded)
    (1, 1, 1, 5, 5, 3, False, 0, False),
    (2, 2, 1, 7, 7, 4, True, 0, False),
    (2, 3, 3, 6, 6, 2, True, 2, True),
    (1, 4, 2, 9, 9, 5, True, 3, True),
    (2, 6, 3, 8, 8, 3, False, 0, True),
    (2, 4, 1, 1, 9, 4, True, 0, True),    # one-token decode, MQA
    (3, 4, 2, 1, 7, 3, True, 3, True),    # decode with window
    (2, 2, 2, 1, 6, 2, False, 0, False),  # decode without mask
    (1, 2, 1, 4, 4, 5, True, 1, False),   # window of one: self only
    (3, 4, 2, 5, 12, 3, True, 0, True),   # chunk of 5 against a cache
    (2, 3, 1, 4, 10, 2, True, 3, True),   # chunk with a window
    (2, 2, 1, 6, 9, 4, False, 0, True),   # cross-attention, key padding
]


def check_brute(attn, seed=0):
    rng = np.random.default_rng(seed)
    for (B, Hq, Hkv, Nq, Nk, d, causal, window, padded) in BRUTE_CASES:
        q = _rand(rng, B, Hq, Nq, d)
        k = _rand(rng, B, Hkv, Nk, d)
        v = _rand(rng, B, Hkv, Nk, d)
        seqlens = rng.integers(0, Nk + 1, size=B) if padded else None
        scale = float(rng.uniform(0.2, 1.5))
        o, lse = attn(q, k, v, scale=scale, causal=causal, window=window,
                      seqlens=seqlens)
        ob, lb = brute.attention_loops(_tolist(q), _tolist(k), _tolist(v),
                                       scale=scale, causal=causal,
                                       window=window, seqlens=seqlens)
        ob = np.array(ob)
        lb = np.array(lb)
        assert np.array_equal(np.isinf(lse), np.isinf(lb)), "empty rows differ"
        fin = np.isfinite(lb)
        np.testing.assert_allclose(lse[fin], lb[fin], rtol=0, atol=1e-12)
        np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# worked examples printed on the FlashAttention-3 review page

def load_worked_examples():
    with open(os.path.join(GOLDEN, "fa3_review_worked_examples.json")) as f:
        return json.load(f)["examples"]


def _softmax_closed_form(scores):
    m = max(scores)
    w = [math.exp(s - m) for s in scores]
    t = math.fsum(w)
    return [x / t for x in w], m + math.log(t)


def check_worked_examples(attn):
    for ex in load_worked_examples():
        Q = np.array(ex["Q"], dtype=np.float64)
        K = np.array(ex["K"], dtype=np.float64)
        V = np.array(ex["V"], dtype=np.float64)
        n = Q.shape[0]
        o, lse = attn(Q[None, None], K[None, None], V[None, None], scale=1.0,
                      causal=False, window=0, seqlens=None)
        for i in range(n):
            # dot products written out by hand from the printed entries
            scores = [Q[i, 0] * K[j, 0] + Q[i, 1] * K[j, 1] for j in range(n)]
            p, l_ = _softmax_closed_form(scores)
            want = [math.fsum(p[j] * V[j, c] for j in range(n))
                    for c in range(V.shape[1])]
            np.testing.assert_allclose(o[0, 0, i], want, rtol=1e-14,
                                       atol=1e-15)
            assert abs(lse[0, 0, i] - l_) <= 1e-13 * abs(l_)
        cons = ex.get("printed_consistent", {})
        if "S_row0" in cons:
            p, l_ = _softmax_closed_form([float(s) for s in cons["S_row0"]])
            want = [math.fsum(p[j] * V[j, c] for j in range(n))
                    for c in range(V.shape[1])]
            np.testing.assert_allclose(o[0, 0, 0], want, rtol=1e-14,
                                       atol=1e-15)
            assert abs(lse[0, 0, 0] - l_) <= 1e-13 * abs(l_)


def check_fa1_example_closed_form(attn):
    """Q=[[1,2],[3,4]], K=[[2,1],[4,3]], V=I: scores [[4,10],[10,24]], so
    row 0 weights are (1, e^6)/(1+e^6) and row 1 weights (1, e^14)/(1+e^14);
    at scale 1/sqrt(2) row 0 weights are (1, e^(6/sqrt 2)) normalised."""
    Q = np.array([[1.0, 2.0], [3.0, 4.0]])[None, None]
    K = np.array([[2.0, 1.0], [4.0, 3.0]])[None, None]
    V = np.eye(2)[None, None]
    o, lse = attn(Q, K, V, scale=1.0, causal=False, window=0, seqlens=None)
    def sig(x):
        return 1.0 / (1.0 + math.exp(-x))
    np.testing.assert_allclose(o[0, 0, 0], [sig(-6.0), sig(6.0)], rtol=1e-14)
    np.testing.assert_allclose(o[0, 0, 1], [sig(-14.0), sig(14.0)],
                               rtol=1e-13)
    np.testing.assert_allclose(
        lse[0, 0], [10 + math.log1p(math.exp(-6)),
                    24 + math.log1p(math.exp(-14))], rtol=1e-15)
    s = 1 / math.sqrt(2)
    o, _ = attn(Q, K, V, scale=s, causal=False, window=0, seqlens=None)
    np.testing.assert_allclose(o[0, 0, 0], [sig(-6.0 * s), sig(6.0 * s)],
                               rtol=1e-14)


# --------------------------------------------------------------------------
# closed forms

def _valid(seqlens, b, nk):
    return nk if seqlens is None else int(min(max(seqlens[b], 0), nk))


def check_scale_zero_means(attn, seed=1):
    """scale = 0 makes every allowed key equally likely, so each output row is
    the plain mean of V over its allowed keys and lse = ln(#allowed).  The
    allowed sets are written here as index ranges (prefix, sliding window,
    valid length), independently of the oracle's explicit mask."""
    rng = np.random.default_rng(seed)
    B, H, N, d = 3, 2, 23, 4
    k = _rand(rng, B, H, N, d)
    v = _rand(rng, B, H, N, d)
    q = _rand(rng, B, H, N, d)
    seqlens = np.array([23, 11, 0])
    for causal, window in [(False, 0), (True, 0), (True, 5), (True, 1)]:
        o, lse = attn(q, k, v, scale=0.0, causal=causal, window=window,
                      seqlens=seqlens)
        for b in range(B):
            L = _valid(seqlens, b, N)
            for i in range(N):
                if i >= L:
                    assert np.all(o[b, :, i] == 0) and np.all(
                        np.isneginf(lse[b, :, i]))
                    continue
                hi = i + 1 if causal else L
                lo = max(0, i - window + 1) if window > 0 else 0
                want = v[b, :, lo:hi].mean(axis=1)
                np.testing.assert_allclose(o[b, :, i], want, rtol=1e-13,
                                           atol=1e-14)
                np.testing.assert_allclose(lse[b, :, i], math.log(hi - lo),
                                           rtol=1e-15, atol=1e-15)
    # decode row: sees the last `window` valid keys, or all of them
    qd = _rand(rng, B, H, 1, d)
    for window in (0, 4):
        o, lse = attn(qd, k, v, scale=0.0, causal=True, window=window,
                      seqlens=seqlens)
        for b in range(B):
            L = _valid(seqlens, b, N)
            if L == 0:
                assert np.all(o[b] == 0) and np.all(np.isneginf(lse[b]))
                continue
            lo = max(0, L - window) if window > 0 else 0
            np.testing.assert_allclose(o[b, :, 0], v[b, :, lo:L].mean(axis=1),
                                       rtol=1e-13, atol=1e-14)
            np.testing.assert_allclose(lse[b, :, 0], math.log(L - lo),
                                       rtol=1e-15)


def check_one_and_two_keys(attn, seed=2):
    """L = 1 gives o = v0 and lse = s0; L = 2 gives
    o = sigma(s0 - s1) v0 + sigma(s1 - s0) v1 and
    lse = max(s0, s1) + log(1 + exp(-|s0 - s1|))."""
    rng = np.random.default_rng(seed)
    d = 6
    for _ in range(5):
        q = _rand(rng, 1, 1, 1, d)
        k = _rand(rng, 1, 1, 2, d)
        v = _rand(rng, 1, 1, 2, d)
        sc = float(rng.uniform(0.1, 2.0))
        s = [sc * math.fsum(q[0, 0, 0, c] * k[0, 0, j, c] for c in range(d))
             for j in range(2)]
        o, lse = attn(q, k[:, :, :1], v[:, :, :1], scale=sc, causal=False,
                      window=0, seqlens=None)
        np.testing.assert_allclose(o[0, 0, 0], v[0, 0, 0], rtol=1e-15)
        np.testing.assert_allclose(lse[0, 0, 0], s[0], rtol=1e-14)
        o, lse = attn(q, k, v, scale=sc, causal=False, window=0, seqlens=None)
        sig = 1.0 / (1.0 + math.exp(-(s[0] - s[1])))
        want = sig * v[0, 0, 0] + (1 - sig) * v[0, 0, 1]
        np.testing.assert_allclose(o[0, 0, 0], want, rtol=1e-13, atol=1e-15)
        wl = max(s) + math.log1p(math.exp(-abs(s[0] - s[1])))
        np.testing.assert_allclose(lse[0, 0, 0], wl, rtol=1e-14)


def check_causal_row0(attn, seed=3):
    """Under the look-ahead mask row 0 sees only key 0: o_0 = v_0 and
    lse_0 = scale * q_0 . k_0."""
    rng = np.random.default_rng(seed)
    B, H, N, d = 2, 3, 17, 8
    q, k, v = (_rand(rng, B, H, N, d) for _ in range(3))
    o, lse = attn(q, k, v, scale=0.3, causal=True, window=0, seqlens=None)
    np.testing.assert_allclose(o[:, :, 0], v[:, :, 0], rtol=1e-15)
    want = 0.3 * np.einsum("bhc,bhc->bh", q[:, :, 0], k[:, :, 0])
    np.testing.assert_allclose(lse[:, :, 0], want, rtol=1e-13, atol=1e-15)


# --------------------------------------------------------------------------
# invariants

def check_rows_sum_to_one(attn, seed=4):
    """V = 1 gives O = 1 on every row with an allowed key, because softmax
    weights sum to one."""
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, N, d = 2, 4, 2, 19, 5
    q = _rand(rng, B, Hq, N, d) * 3
    k = _rand(rng, B, Hkv, N, d) * 3
    v = np.ones((B, Hkv, N, d))
    seqlens = np.array([19, 7])
    for causal, window in [(False, 0), (True, 0), (True, 4)]:
        o, lse = attn(q, k, v, scale=1.0, causal=causal, window=window,
                      seqlens=seqlens)
        live = np.isfinite(lse)
        np.testing.assert_allclose(o[live], 1.0, rtol=0, atol=1e-14)
        assert np.all(o[~live] == 0)


def check_identical_keys(attn, seed=5):
    """All keys equal: every allowed key gets the same weight, so O is the
    mean of V over the allowed keys (a flat distribution)."""
    rng = np.random.default_rng(seed)
    B, H, N, d = 1, 2, 13, 4
    q = _rand(rng, B, H, N, d)
    k = np.broadcast_to(_rand(rng, B, H, 1, d), (B, H, N, d)).copy()
    v = _rand(rng, B, H, N, d)
    o, _ = attn(q, k, v, scale=0.7, causal=True, window=0, seqlens=None)
    for i in range(N):
        np.testing.assert_allclose(o[0, :, i], v[0, :, :i + 1].mean(axis=1),
                                   rtol=1e-13, atol=1e-14)


def check_dominant_logit(attn, seed=6):
    """One score exceeding all others by >= 40 puts all but ~e^-40 of the mass
    on that key, so the output is that V row."""
    rng = np.random.default_rng(seed)
    N, d = 16, 8
    q = _rand(rng, 1, 1, 1, d)
    k = _rand(rng, 1, 1, N, d) * 0.1
    v = _rand(rng, 1, 1, N, d)
    jstar = 11
    scale = 0.25
    qn = q[0, 0, 0] / np.dot(q[0, 0, 0], q[0, 0, 0])
    k[0, 0, jstar] += (60.0 / scale) * qn
    o, _ = attn(q, k, v, scale=scale, causal=False, window=0, seqlens=None)
    np.testing.assert_allclose(o[0, 0, 0], v[0, 0, jstar], rtol=1e-14,
                               atol=1e-14)


def check_window_n_equals_causal(attn, seed=7):
    rng = np.random.default_rng(seed)
    B, H, N, d = 2, 2, 21, 4
    q, k, v = (_rand(rng, B, H, N, d) for _ in range(3))
    seqlens = np.array([21, 9])
    oc, lc = attn(q, k, v, scale=0.5, causal=True, window=0, seqlens=seqlens)
    for w in (N, N + 5):
        ow, lw = attn(q, k, v, scale=0.5, causal=True, window=w,
                      seqlens=seqlens)
        assert np.array_equal(oc, ow) and np.array_equal(lc, lw)
    ow, _ = attn(q, k, v, scale=0.5, causal=True, window=N - 1,
                 seqlens=None)
    oc, _ = attn(q, k, v, scale=0.5, causal=True, window=0, seqlens=None)
    assert not np.allclose(ow[:, :, -1], oc[:, :, -1])


def check_gqa_equals_repeated_mha(attn, seed=8):
    """GQA(Hq, Hkv) equals MHA with each K/V head repeated Hq/Hkv times
    (contiguous groups); Hkv == Hq is plain MHA."""
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, N, d = 2, 6, 2, 11, 3
    q = _rand(rng, B, Hq, N, d)
    k = _rand(rng, B, Hkv, N, d)
    v = _rand(rng, B, Hkv, N, d)
    g = Hq // Hkv
    kr = np.repeat(k, g, axis=1)
    vr = np.repeat(v, g, axis=1)
    for causal in (False, True):
        og, lg = attn(q, k, v, scale=0.4, causal=causal, window=0,
                      seqlens=None)
        om, lm = attn(q, kr, vr, scale=0.4, causal=causal, window=0,
                      seqlens=None)
        np.testing.assert_allclose(og, om, rtol=0, atol=1e-15)
        np.testing.assert_allclose(lg, lm, rtol=0, atol=1e-15)


def check_linearity_and_permutation(attn, seed=9):
    rng = np.random.default_rng(seed)
    B, H, N, d = 1, 2, 12, 5
    q, k, v1, v2 = (_rand(rng, B, H, N, d) for _ in range(4))
    a, b = 0.7, -1.3
    o1, _ = attn(q, k, v1, scale=0.5, causal=True, window=0, seqlens=None)
    o2, _ = attn(q, k, v2, scale=0.5, causal=True, window=0, seqlens=None)
    o12, _ = attn(q, k, a * v1 + b * v2, scale=0.5, causal=True, window=0,
                  seqlens=None)
    np.testing.assert_allclose(o12, a * o1 + b * o2, rtol=1e-12, atol=1e-13)
    perm = rng.permutation(N)
    o, l_ = attn(q, k, v1, scale=0.5, causal=False, window=0, seqlens=None)
    op, lp = attn(q, k[:, :, perm], v1[:, :, perm], scale=0.5, causal=False,
                  window=0, seqlens=None)
    np.testing.assert_allclose(op, o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lp, l_, rtol=1e-13)


def check_decode_is_last_row(attn, seed=10):
    """A one-token query against a cache of valid length L gives the same row
    as the last live row of causal self-attention over those L tokens."""
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, N, d = 3, 4, 2, 14, 4
    q = _rand(rng, B, Hq, N, d)
    k = _rand(rng, B, Hkv, N, d)
    v = _rand(rng, B, Hkv, N, d)
    seqlens = np.array([14, 6, 1])
    of, lf = attn(q, k, v, scale=0.6, causal=True, window=3, seqlens=seqlens)
    qd = np.stack([q[b, :, seqlens[b] - 1] for b in range(B)])[:, :, None]
    od, ld = attn(qd, k, v, scale=0.6, causal=True, window=3,
                  seqlens=seqlens)
    for b in range(B):
        np.testing.assert_allclose(od[b, :, 0], of[b, :, seqlens[b] - 1],
                                   rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(ld[b, :, 0], lf[b, :, seqlens[b] - 1],
                                   rtol=1e-14)


def check_chunk_is_tail_of_prefill(attn, seed=13):
    """A chunk of Nq new query rows against a cache of valid length L gives,
    row for row, causal self-attention over the L tokens at positions
    L - Nq .. L - 1; a chunk row whose position is negative (L < Nq) sees no
    key.  Generalises the one-token case."""
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, N, d, nq = 4, 4, 2, 15, 4, 5
    q = _rand(rng, B, Hq, N, d)
    k = _rand(rng, B, Hkv, N, d)
    v = _rand(rng, B, Hkv, N, d)
    seqlens = np.array([15, 9, 5, 3])
    for window in (0, 4):
        of, lf = attn(q, k, v, scale=0.7, causal=True, window=window,
                      seqlens=seqlens)
        qc = np.zeros((B, Hq, nq, d))
        for b in range(B):
            for i in range(nq):
                pos = seqlens[b] - nq + i
                if pos >= 0:
                    qc[b, :, i] = q[b, :, pos]
        oc, lc = attn(qc, k, v, scale=0.7, causal=True, window=window,
                      seqlens=seqlens)
        for b in range(B):
            for i in range(nq):
                pos = seqlens[b] - nq + i
                if pos >= 0:
                    np.testing.assert_allclose(oc[b, :, i], of[b, :, pos],
                                               rtol=1e-13, atol=1e-14)
                    np.testing.assert_allclose(lc[b, :, i], lf[b, :, pos],
                                               rtol=1e-14)
                else:
                    assert np.all(oc[b, :, i] == 0)
                    assert np.all(np.isneginf(lc[b, :, i]))


def check_cross_attention_against_torch(attn, seed=14):
    """Cross-attention (decoder queries against encoder keys and values, no
    causal mask, Nq != Nk; explainer page, encoder-decoder attention) with
    key padding equals PyTorch's CPU float64 scaled dot-product attention
    with a boolean key mask."""
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, nq, nk, d = 3, 4, 2, 11, 23, 8
    q = _rand(rng, B, Hq, nq, d)
    k = _rand(rng, B, Hkv, nk, d)
    v = _rand(rng, B, Hkv, nk, d)
    seqlens = np.array([23, 7, 16])
    o, lse = attn(q, k, v, scale=0.3, causal=False, window=0,
                  seqlens=seqlens)
    mask = np.zeros((B, 1, nq, nk), dtype=bool)
    for b in range(B):
        mask[b, 0, :, :seqlens[b]] = True
    kr = torch.from_numpy(np.repeat(k, Hq // Hkv, axis=1))
    vr = torch.from_numpy(np.repeat(v, Hq // Hkv, axis=1))
    ref = F.scaled_dot_product_attention(
        torch.from_numpy(q), kr, vr, attn_mask=torch.from_numpy(mask),
        scale=0.3).numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-11, atol=1e-12)


# --------------------------------------------------------------------------
# two-sided windows and sink keys

MASK_CASES = [
    # (B, Hq, Hkv, Nq, Nk, d, causal, window, window_right, sinks, padded)
    (2, 2, 1, 9, 9, 3, False, 3, 3, 0, False),   # two-sided neighbourhood
    (2, 4, 2, 11, 11, 4, False, 2, 4, 2, True),  # asymmetric, sinks, padding
    (1, 2, 2, 10, 10, 2, True, 3, 0, 2, True),   # causal window + sinks
    (2, 2, 1, 4, 12, 3, True, 3, 0, 3, True),    # chunk, window + sinks
    (3, 2, 1, 1, 13, 4, True, 4, 0, 2, True),    # decode, window + sinks
    (1, 3, 1, 8, 8, 2, False, 0, 2, 1, False),   # right limit only
]


def check_brute_masks(attn, seed=15):
    rng = np.random.default_rng(seed)
    for (B, Hq, Hkv, Nq, Nk, d, causal, wl, wr, sk, padded) in MASK_CASES:
        q = _rand(rng, B, Hq, Nq, d)
        k = _rand(rng, B, Hkv, Nk, d)
        v = _rand(rng, B, Hkv, Nk, d)
        seqlens = rng.integers(0, Nk + 1, size=B) if padded else None
        scale = float(rng.uniform(0.2, 1.5))
        o, lse = attn(q, k, v, scale=scale, causal=causal, window=wl,
                      seqlens=seqlens, window_right=wr, sinks=sk)
        ob, lb = brute.attention_loops(_tolist(q), _tolist(k), _tolist(v),
                                       scale=scale, causal=causal, window=wl,
                                       seqlens=seqlens, window_right=wr,
                                       sinks=sk)
        ob = np.array(ob)
        lb = np.array(lb)
        assert np.array_equal(np.isinf(lse), np.isinf(lb)), "empty rows differ"
        fin = np.isfinite(lb)
        np.testing.assert_allclose(lse[fin], lb[fin], rtol=0, atol=1e-12)
        np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)


def check_masks_scale_zero(attn, seed=16):
    """scale = 0: every allowed key weighs the same, so O_i is the mean of V
    over the allowed set and lse_i = ln |allowed(i)|; the set is the window
    [pos-wl+1, pos+wr-1] joined with the sinks [0, s), cut to [0, L) and, if
    causal, to j <= pos."""
    rng = np.random.default_rng(seed)
    B, H, N, d = 2, 2, 14, 3
    v = _rand(rng, B, H, N, d)
    q = _rand(rng, B, H, N, d)
    k = _rand(rng, B, H, N, d)
    seqlens = np.array([14, 9])
    for causal, wl, wr, sk in [(False, 3, 2, 2), (True, 4, 0, 3),
                               (False, 0, 3, 1), (True, 2, 0, 20)]:
        o, lse = attn(q, k, v, scale=0.0, causal=causal, window=wl,
                      seqlens=seqlens, window_right=wr, sinks=sk)
        for b in range(B):
            L = seqlens[b]
            for i in range(N):
                if i >= L:
                    assert np.all(o[b, :, i] == 0)
                    continue
                lo = i - wl + 1 if wl > 0 else 0
                hi = i + wr if wr > 0 else N
                keys = set(range(max(lo, 0), min(hi, L)))
                keys |= set(range(min(sk, L)))
                if causal:
                    keys = {j for j in keys if j <= i}
                js = sorted(keys)
                np.testing.assert_allclose(o[b, :, i], v[b][:, js].mean(axis=1),
                                           rtol=1e-13, atol=1e-14)
                np.testing.assert_allclose(lse[b, :, i], math.log(len(js)),
                                           rtol=1e-14)


def check_masks_extremes(attn, seed=17):
    """A two-sided window of at least N on both sides equals no window; sinks
    covering every key equal no window; zero sinks change nothing."""
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, N, d = 2, 4, 2, 13, 4
    q = _rand(rng, B, Hq, N, d)
    k = _rand(rng, B, Hkv, N, d)
    v = _rand(rng, B, Hkv, N, d)
    seqlens = np.array([13, 8])
    o0, l0 = attn(q, k, v, scale=0.5, causal=False, window=0,
                  seqlens=seqlens)
    o1, l1 = attn(q, k, v, scale=0.5, causal=False, window=N, seqlens=seqlens,
                  window_right=N)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
    o2, l2 = attn(q, k, v, scale=0.5, causal=False, window=2, seqlens=seqlens,
                  window_right=2, sinks=N)
    assert np.array_equal(o0, o2) and np.array_equal(l0, l2)
    o3, l3 = attn(q, k, v, scale=0.5, causal=True, window=3, seqlens=seqlens)
    o4, l4 = attn(q, k, v, scale=0.5, causal=True, window=3, seqlens=seqlens,
                  sinks=0, window_right=0)
    assert np.array_equal(o3, o4) and np.array_equal(l3, l4)
    o5, l5 = attn(q, k, v, scale=0.5, causal=False, window=2, seqlens=seqlens,
                  window_right=2)
    assert not np.allclose(o0, o5)


def check_masks_against_torch(attn, seed=18):
    """Two-sided windows and sinks against PyTorch's CPU float64 SDPA with a
    boolean mask built here from index ranges."""
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, N, d = 2, 4, 2, 31, 8
    q = _rand(rng, B, Hq, N, d)
    k = _rand(rng, B, Hkv, N, d)
    v = _rand(rng, B, Hkv, N, d)
    seqlens = np.array([31, 17])
    for causal, wl, wr, sk in [(False, 5, 5, 0), (False, 4, 2, 3),
                               (True, 6, 0, 2)]:
        o, lse = attn(q, k, v, scale=0.4, causal=causal, window=wl,
                      seqlens=seqlens, window_right=wr, sinks=sk)
        mask = np.zeros((B, 1, N, N), dtype=bool)
        for b in range(B):
            L = seqlens[b]
            for i in range(L):
                lo = max(0, i - wl + 1) if wl > 0 else 0
                hi = min(L, i + wr) if wr > 0 else L
                mask[b, 0, i, lo:hi] = True
                mask[b, 0, i, :min(sk, L)] = True
                if causal:
                    mask[b, 0, i, i + 1:] = False
        kr = torch.from_numpy(np.repeat(k, Hq // Hkv, axis=1))
        vr = torch.from_numpy(np.repeat(v, Hq // Hkv, axis=1))
        ref = F.scaled_dot_product_attention(
            torch.from_numpy(q), kr, vr, attn_mask=torch.from_numpy(mask),
            scale=0.4).numpy()
        live = mask[:, 0].any(axis=-1)
        for b in range(B):
            np.testing.assert_allclose(o[b][:, live[b]], ref[b][:, live[b]],
                                       rtol=1e-11, atol=1e-12)


def check_split_combine(attn, seed=11):
    """Splitting the keys into chunks, attending to each chunk alone and
    merging the (o_c, lse_c) pairs with weights exp(lse_c - lse),
    lse = log sum_c exp(lse_c), reproduces attention over all keys.  This
    holds only if lse is the natural-log normaliser with the scale applied."""
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, N, d = 2, 4, 2, 29, 6
    q = _rand(rng, B, Hq, 1, d)
    k = _rand(rng, B, Hkv, N, d) * 2
    v = _rand(rng, B, Hkv, N, d)
    o_all, l_all = attn(q, k, v, scale=0.8, causal=False, window=0,
                        seqlens=None)
    for bounds in ([0, 29], [0, 10, 29], [0, 8, 16, 24, 29], [0, 1, 28, 29]):
        os_, ls_ = [], []
        for a, b in zip(bounds[:-1], bounds[1:]):
            oc, lc = attn(q, k[:, :, a:b], v[:, :, a:b], scale=0.8,
                          causal=False, window=0, seqlens=None)
            os_.append(oc)
            ls_.append(lc)
        ls_ = np.stack(ls_)
        mx = ls_.max(axis=0)
        lse = mx + np.log(np.exp(ls_ - mx).sum(axis=0))
        o = sum(np.exp(lc - lse)[..., None] * oc for oc, lc in zip(os_, ls_))
        np.testing.assert_allclose(lse, l_all, rtol=1e-14)
        np.testing.assert_allclose(o, o_all, rtol=1e-12, atol=1e-13)


def check_against_torch_sdpa(attn, seed=12):
    """Independent library routine: PyTorch's CPU float64 scaled dot-product
    attention (the call the O(n^2) tutorial page shows in Example 2) with an
    explicit boolean mask built here from index ranges and K/V repeated per
    group.  Rows with no allowed key are excluded (the library returns NaN
    there by its own convention)."""
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, N, d = 2, 6, 3, 37, 16
    q = _rand(rng, B, Hq, N, d)
    k = _rand(rng, B, Hkv, N, d)
    v = _rand(rng, B, Hkv, N, d)
    seqlens = np.array([37, 20])
    for causal, window in [(False, 0), (True, 0), (True, 7)]:
        o, lse = attn(q, k, v, scale=0.25, causal=causal, window=window,
                      seqlens=seqlens)
        mask = np.zeros((B, 1, N, N), dtype=bool)
        for b in range(B):
            L = seqlens[b]
            for i in range(L):
                lo = max(0, i - window + 1) if window > 0 else 0
                hi = i + 1 if causal else L
                mask[b, 0, i, lo:hi] = True
        kr = torch.from_numpy(np.repeat(k, Hq // Hkv, axis=1))
        vr = torch.from_numpy(np.repeat(v, Hq // Hkv, axis=1))
        ref = F.scaled_dot_product_attention(
            torch.from_numpy(q), kr, vr, attn_mask=torch.from_numpy(mask),
            scale=0.25).numpy()
        live = mask[:, 0].any(axis=-1)
        for b in range(B):
            np.testing.assert_allclose(o[b][:, live[b]], ref[b][:, live[b]],
                                       rtol=1e-11, atol=1e-12)


ALL_CHECKS = [
    check_brute,
    check_worked_examples,
    check_fa1_example_closed_form,
    check_scale_zero_means,
    check_one_and_two_keys,
    check_causal_row0,
    check_rows_sum_to_one,
    check_identical_keys,
    check_dominant_logit,
    check_window_n_equals_causal,
    check_gqa_equals_repeated_mha,
    check_linearity_and_permutation,
    check_decode_is_last_row,
    check_chunk_is_tail_of_prefill,
    check_cross_attention_against_torch,
    check_brute_masks,
    check_masks_scale_zero,
    check_masks_extremes,
    check_masks_against_torch,
    check_split_combine,
    check_against_torch_sdpa,
]
