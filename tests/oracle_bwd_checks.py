"""Pins for the fp64 backward oracle (`oracle.attention_backward`).

Every check takes `bwd`, a callable with the signature of
`oracle.attention_backward(q, k, v, do, *, scale, causal, window, seqlens,
window_right, sinks) -> (dq, dk, dv)`, and raises AssertionError on a
mismatch.  What each is pinned to is fixed independently of the chain-rule
derivation in the oracle:

  * central finite differences of the (separately pinned) forward oracle;
  * PyTorch's CPU float64 autograd through its own SDPA, with a boolean mask
    built here from index ranges;
  * closed forms (scale 0, a window of one key, two keys);
  * invariants of the definition (sum of dK over keys is 0, sum of dV over
    keys is the sum of dO over rows that see a key, GQA equals MHA with K/V
    repeated, a chunk's gradients equal the tail of full self-attention's,
    linearity in dO).
"""

import math

import numpy as np

import oracle


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _valid(seqlens, b, nk):
    return nk if seqlens is None else int(min(max(seqlens[b], 0), nk))


def _live_and_off(nq, nk, L):
    """Live rows and the position of row 0, restated from the boundary's
    semantics: Nq == Nk -> the first L rows at positions 0.., otherwise all
    Nq rows as the last Nq positions."""
    live = L if nq == nk else nq
    return live, L - live


def _allowed_ranges(pos, L, causal, wl, wr, sk):
    """Allowed keys of a row at position pos, as a boolean vector over
    0..L-1, written from index ranges."""
    ok = np.zeros(max(L, 0), dtype=bool)
    lo = max(0, pos - wl + 1) if wl > 0 else 0
    hi = min(L, pos + wr) if wr > 0 else L
    if hi > lo:
        ok[lo:hi] = True
    ok[:min(sk, L)] = True
    if causal:
        ok[max(0, pos + 1):] = False
    return ok


# --------------------------------------------------------------------------
# finite differences of the forward oracle

FD_CASES = [
    # (B, Hq, Hkv, Nq, Nk, d, causal, wl, wr, sinks, padded)
    (1, 2, 1, 5, 5, 3, True, 0, 0, 0, False),    # GQA, causal
    (2, 2, 2, 6, 6, 2, False, 0, 0, 0, True),    # no causal mask, padding
    (1, 3, 1, 6, 6, 3, True, 3, 0, 2, True),     # window + sinks, padding
    (2, 2, 1, 3, 7, 2, True, 0, 0, 0, True),     # chunk against a cache
    (1, 2, 1, 1, 6, 3, True, 2, 0, 1, True),     # decode, window + sinks
    (1, 2, 2, 7, 7, 2, False, 2, 3, 0, False),   # two-sided window
    (2, 2, 1, 4, 8, 3, False, 0, 0, 0, True),    # cross-attention, padding
]


def check_bwd_finite_differences(bwd, seed=40, h=1e-5):
    """Every element of dq, dk, dv against the central difference
    (L(x + h) - L(x - h)) / 2h of L = sum(dO * O), O from the forward
    oracle.  Truncation error is O(h^2) ~ 1e-10 here."""
    rng = np.random.default_rng(seed)
    for (B, Hq, Hkv, Nq, Nk, d, causal, wl, wr, sk, padded) in FD_CASES:
        q = _rand(rng, B, Hq, Nq, d)
        k = _rand(rng, B, Hkv, Nk, d)
        v = _rand(rng, B, Hkv, Nk, d)
        do = _rand(rng, B, Hq, Nq, d)
        seqlens = rng.integers(0, Nk + 1, size=B) if padded else None
        scale = float(rng.uniform(0.3, 1.2))
        kw = dict(scale=scale, causal=causal, window=wl, seqlens=seqlens,
                  window_right=wr, sinks=sk)
        dq, dk, dv = bwd(q, k, v, do, **kw)

        def loss(qq, kk, vv):
            o, _ = oracle.attention(qq, kk, vv, **kw)
            return float((o * do).sum())

        for name, x, got in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            fd = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                keep = x[idx]
                x[idx] = keep + h
                lp = loss(q, k, v)
                x[idx] = keep - h
                lm = loss(q, k, v)
                x[idx] = keep
                fd[idx] = (lp - lm) / (2 * h)
            np.testing.assert_allclose(
                got, fd, rtol=1e-6, atol=1e-7,
                err_msg=f"d{name} vs finite differences, case "
                        f"{(B, Hq, Hkv, Nq, Nk, d, causal, wl, wr, sk)}")


# --------------------------------------------------------------------------
# an independent library: torch autograd through its SDPA

def check_bwd_against_torch_autograd(bwd, seed=41):
    """PyTorch CPU float64 autograd of F.scaled_dot_product_attention with an
    explicit boolean mask; K/V repeated per group by indexing, so their
    gradients are summed over the group by autograd.  Every live row of the
    cases below sees at least one key (torch gives NaN for an empty row)."""
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(seed)
    cases = [
        # (B, Hq, Hkv, Nq, Nk, d, causal, wl, wr, sinks, seqlens)
        (2, 4, 2, 19, 19, 5, True, 0, 0, 0, [19, 11]),
        (1, 3, 1, 23, 23, 4, False, 4, 6, 2, None),
        (2, 2, 1, 17, 17, 3, True, 5, 0, 3, [17, 9]),
        (2, 4, 4, 6, 21, 4, True, 0, 0, 0, [21, 8]),     # chunk, L >= Nq
        (2, 2, 1, 9, 15, 3, False, 0, 0, 0, [15, 4]),    # cross-attention
    ]
    for (B, Hq, Hkv, Nq, Nk, d, causal, wl, wr, sk, sl) in cases:
        q = _rand(rng, B, Hq, Nq, d)
        k = _rand(rng, B, Hkv, Nk, d)
        v = _rand(rng, B, Hkv, Nk, d)
        do = _rand(rng, B, Hq, Nq, d)
        seqlens = None if sl is None else np.array(sl)
        scale = 0.45
        dq, dk, dv = bwd(q, k, v, do, scale=scale, causal=causal, window=wl,
                         seqlens=seqlens, window_right=wr, sinks=sk)
        G = Hq // Hkv
        for b in range(B):
            L = _valid(seqlens, b, Nk)
            live, off = _live_and_off(Nq, Nk, L)
            mask = np.zeros((live, L), dtype=bool)
            for i in range(live):
                mask[i] = _allowed_ranges(i + off, L, causal, wl, wr, sk)
            assert mask.any(axis=1).all()
            tq = torch.tensor(q[b, :, :live], requires_grad=True)
            tk = torch.tensor(k[b, :, :L], requires_grad=True)
            tv = torch.tensor(v[b, :, :L], requires_grad=True)
            heads = torch.tensor([h // G for h in range(Hq)])
            o = F.scaled_dot_product_attention(
                tq, tk[heads], tv[heads], attn_mask=torch.from_numpy(mask),
                scale=scale)
            o.backward(torch.from_numpy(do[b, :, :live]))
            np.testing.assert_allclose(dq[b, :, :live], tq.grad.numpy(),
                                       rtol=1e-10, atol=1e-11)
            np.testing.assert_allclose(dk[b, :, :L], tk.grad.numpy(),
                                       rtol=1e-10, atol=1e-11)
            np.testing.assert_allclose(dv[b, :, :L], tv.grad.numpy(),
                                       rtol=1e-10, atol=1e-11)
            assert np.all(dq[b, :, live:] == 0)
            assert np.all(dk[b, :, L:] == 0) and np.all(dv[b, :, L:] == 0)


# --------------------------------------------------------------------------
# closed forms

def check_bwd_scale_zero(bwd, seed=42):
    """scale = 0: the scores are constant, so dQ = dK = 0 exactly, and every
    allowed key of row i has p = 1/n_i: dV_j = sum over rows i allowed to
    see j of dO_i / n_i (allowed sets from index ranges)."""
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, d = 2, 4, 2, 3
    G = Hq // Hkv
    for (Nq, Nk, causal, wl, wr, sk, sl) in [
            (13, 13, True, 0, 0, 0, [13, 6]),
            (13, 13, True, 4, 0, 2, [13, 9]),
            (11, 11, False, 3, 2, 1, [11, 0]),
            (4, 12, True, 0, 0, 0, [12, 2]),
            (1, 9, True, 3, 0, 2, [9, 5])]:
        q = _rand(rng, B, Hq, Nq, d)
        k = _rand(rng, B, Hkv, Nk, d)
        v = _rand(rng, B, Hkv, Nk, d)
        do = _rand(rng, B, Hq, Nq, d)
        seqlens = np.array(sl)
        dq, dk, dv = bwd(q, k, v, do, scale=0.0, causal=causal, window=wl,
                         seqlens=seqlens, window_right=wr, sinks=sk)
        assert np.all(dq == 0) and np.all(dk == 0)
        want = np.zeros_like(dv)
        for b in range(B):
            L = _valid(seqlens, b, Nk)
            live, off = _live_and_off(Nq, Nk, L)
            for h in range(Hq):
                for i in range(live):
                    ok = _allowed_ranges(i + off, L, causal, wl, wr, sk)
                    n = int(ok.sum())
                    if n:
                        want[b, h // G, :L][ok] += do[b, h, i] / n
        np.testing.assert_allclose(dv, want, rtol=1e-13, atol=1e-14)


def check_bwd_self_only(bwd, seed=43):
    """A causal window of one key: each live row attends only to itself
    (p = 1), so O_i = V_i, dV_j = sum over the group's heads of dO_j, and
    the softmax gradient is exactly zero: dQ = dK = 0."""
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, N, d = 2, 6, 2, 9, 4
    q = _rand(rng, B, Hq, N, d)
    k = _rand(rng, B, Hkv, N, d)
    v = _rand(rng, B, Hkv, N, d)
    do = _rand(rng, B, Hq, N, d)
    seqlens = np.array([9, 5])
    dq, dk, dv = bwd(q, k, v, do, scale=0.7, causal=True, window=1,
                     seqlens=seqlens)
    assert np.all(dq == 0) and np.all(dk == 0)
    want = np.zeros_like(dv)
    for b in range(B):
        L = seqlens[b]
        want[b, :, :L] = do[b, :, :L].reshape(Hkv, Hq // Hkv, L, d).sum(1)
    np.testing.assert_allclose(dv, want, rtol=1e-14, atol=1e-15)


def check_bwd_two_keys(bwd, seed=44):
    """One query row, two keys: O = s v0 + (1 - s) v1 with
    s = sigmoid(a), a = scale q.(k0 - k1).  Then, with g = dO.(v0 - v1):
    dq = scale s(1-s) g (k0 - k1), dk0 = -dk1 = scale s(1-s) g q,
    dv0 = s dO, dv1 = (1 - s) dO; K/V gradients summed over the group."""
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, d = 3, 4, 2, 5
    G = Hq // Hkv
    q = _rand(rng, B, Hq, 1, d)
    k = _rand(rng, B, Hkv, 2, d)
    v = _rand(rng, B, Hkv, 2, d)
    do = _rand(rng, B, Hq, 1, d)
    scale = 0.6
    dq, dk, dv = bwd(q, k, v, do, scale=scale, causal=True)
    for b in range(B):
        wk = np.zeros((Hkv, 2, d))
        wv = np.zeros((Hkv, 2, d))
        for h in range(Hq):
            hk = h // G
            qq, k0, k1 = q[b, h, 0], k[b, hk, 0], k[b, hk, 1]
            a = scale * float(qq @ (k0 - k1))
            s = 1.0 / (1.0 + math.exp(-a))
            g = float(do[b, h, 0] @ (v[b, hk, 0] - v[b, hk, 1]))
            c = scale * s * (1 - s) * g
            np.testing.assert_allclose(dq[b, h, 0], c * (k0 - k1),
                                       rtol=1e-12, atol=1e-14)
            wk[hk, 0] += c * qq
            wk[hk, 1] -= c * qq
            wv[hk, 0] += s * do[b, h, 0]
            wv[hk, 1] += (1 - s) * do[b, h, 0]
        np.testing.assert_allclose(dk[b], wk, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(dv[b], wv, rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------------------
# invariants

def check_bwd_sums(bwd, seed=45):
    """Each softmax row's gradient sums to zero over its keys, so
    sum_j dK_j = scale * sum_i (sum_j dS_ij) q_i = 0; and each row's
    probabilities sum to one, so sum_j dV_j = sum of dO_i over the rows
    that see at least one key (summed over the group)."""
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, d = 2, 6, 3, 4
    G = Hq // Hkv
    for (Nq, Nk, causal, wl, wr, sk, sl) in [
            (15, 15, True, 0, 0, 0, [15, 7]),
            (15, 15, False, 3, 4, 2, [15, 12]),
            (5, 14, True, 4, 0, 1, [14, 3]),
            (1, 11, True, 0, 0, 0, [11, 0])]:
        q = _rand(rng, B, Hq, Nq, d)
        k = _rand(rng, B, Hkv, Nk, d)
        v = _rand(rng, B, Hkv, Nk, d)
        do = _rand(rng, B, Hq, Nq, d)
        seqlens = np.array(sl)
        dq, dk, dv = bwd(q, k, v, do, scale=0.8, causal=causal, window=wl,
                         seqlens=seqlens, window_right=wr, sinks=sk)
        np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
        for b in range(B):
            L = _valid(seqlens, b, Nk)
            live, off = _live_and_off(Nq, Nk, L)
            want = np.zeros((Hkv, d))
            for h in range(Hq):
                for i in range(live):
                    if _allowed_ranges(i + off, L, causal, wl, wr, sk).any():
                        want[h // G] += do[b, h, i]
            np.testing.assert_allclose(dv[b].sum(axis=1), want, rtol=1e-12,
                                       atol=1e-12)


def check_bwd_gqa_equals_repeated_mha(bwd, seed=46):
    """GQA gradients equal MHA gradients with every K/V head repeated for its
    group, dK/dV then summed over the group's copies."""
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, N, d = 2, 6, 2, 10, 3
    G = Hq // Hkv
    q = _rand(rng, B, Hq, N, d)
    k = _rand(rng, B, Hkv, N, d)
    v = _rand(rng, B, Hkv, N, d)
    do = _rand(rng, B, Hq, N, d)
    seqlens = np.array([10, 6])
    kw = dict(scale=0.5, causal=True, window=4, seqlens=seqlens, sinks=1)
    dq, dk, dv = bwd(q, k, v, do, **kw)
    dq2, dk2, dv2 = bwd(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1),
                        do, **kw)
    np.testing.assert_allclose(dq, dq2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(dk, dk2.reshape(B, Hkv, G, N, d).sum(2),
                               rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dv, dv2.reshape(B, Hkv, G, N, d).sum(2),
                               rtol=1e-12, atol=1e-13)


def check_bwd_chunk_is_tail(bwd, seed=47):
    """A chunk of Nq rows against L keys is the last Nq rows of causal
    self-attention over L tokens: with dO zero on the earlier rows, full
    self-attention's dK, dV and its last Nq rows of dQ equal the chunk's."""
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, Nq, Nk, d = 2, 4, 2, 5, 13, 3
    q = _rand(rng, B, Hq, Nq, d)
    k = _rand(rng, B, Hkv, Nk, d)
    v = _rand(rng, B, Hkv, Nk, d)
    do = _rand(rng, B, Hq, Nq, d)
    seqlens = np.array([13, 8])
    for wl, sk in [(0, 0), (4, 2)]:
        dq, dk, dv = bwd(q, k, v, do, scale=0.6, causal=True, window=wl,
                         seqlens=seqlens, sinks=sk)
        for b in range(B):
            L = seqlens[b]
            qf = np.zeros((1, Hq, L, d))
            dof = np.zeros((1, Hq, L, d))
            qf[0, :, L - Nq:] = q[b]
            dof[0, :, L - Nq:] = do[b]
            dqf, dkf, dvf = bwd(qf, k[b:b + 1, :, :L], v[b:b + 1, :, :L],
                                dof, scale=0.6, causal=True, window=wl,
                                sinks=sk)
            np.testing.assert_allclose(dq[b], dqf[0, :, L - Nq:], rtol=1e-12,
                                       atol=1e-13)
            np.testing.assert_allclose(dk[b, :, :L], dkf[0], rtol=1e-12,
                                       atol=1e-13)
            np.testing.assert_allclose(dv[b, :, :L], dvf[0], rtol=1e-12,
                                       atol=1e-13)


def check_bwd_linear_in_do(bwd, seed=48):
    """The gradients are linear in dO."""
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, N, d = 1, 2, 1, 8, 3
    q = _rand(rng, B, Hq, N, d)
    k = _rand(rng, B, Hkv, N, d)
    v = _rand(rng, B, Hkv, N, d)
    d1 = _rand(rng, B, Hq, N, d)
    d2 = _rand(rng, B, Hq, N, d)
    kw = dict(scale=0.9, causal=True)
    a = bwd(q, k, v, d1, **kw)
    b_ = bwd(q, k, v, d2, **kw)
    c = bwd(q, k, v, d1 - 2.5 * d2, **kw)
    for x, y, z in zip(a, b_, c):
        np.testing.assert_allclose(z, x - 2.5 * y, rtol=1e-12, atol=1e-13)


BWD_CHECKS = [
    check_bwd_finite_differences,
    check_bwd_against_torch_autograd,
    check_bwd_scale_zero,
    check_bwd_self_only,
    check_bwd_two_keys,
    check_bwd_sums,
    check_bwd_gqa_equals_repeated_mha,
    check_bwd_chunk_is_tail,
    check_bwd_linear_in_do,
]
