"""fp64 gradients of masked multi-head scaled dot-product attention.

Test infrastructure only (see the package docstring).

The pages name the backward pass and its outputs, dQ, dK and dV, only by its
cost: the FlashAttention-3 review counts it at about 2.5 times the forward
FLOPs and compares FA2 and FA3 on it. None of them prints its equations. What
it computes is nevertheless fixed by the forward definition: the exact
gradient, with respect to Q, K and V, of a scalar loss whose gradient with
respect to the output O is dO. This module writes that gradient out by the
chain rule through the forward pass's steps, in their order:

    S' = scale * Q K^T with masked entries at -inf, P = row softmax(S')
    O = P V

    dV   = P^T dO                      (O = P V, linear in V)
    dP   = dO V^T                      (O = P V, linear in P)
    dS'_ij = p_ij (dP_ij - sum_k p_ik dP_ik)
                                       (Jacobian of one softmax row:
                                        d p_ik / d s_ij = p_ik (delta_jk - p_ij))
    dQ   = scale * dS' K,   dK = scale * dS'^T Q
                                       (S' = scale * Q K^T)

A masked entry has p = 0, so its score gets no gradient; a row with no
allowed key contributes nothing, and its dQ row is 0.  Padding keys (j at or
beyond the valid length) get dK = dV = 0.  Grouped-query attention: a K/V head
is read by several query heads, so its gradient is the sum over them.

Plain NumPy, float64; the matrix product is the only library primitive.  Each
(batch, head) is processed over chunks of query rows; the chunks only bound
memory (every product is summed over all rows of the head).
"""

import numpy as np

from . import sdpa as _fwd

_ROW_CHUNK = 512


def softmax_backward(p, dp):
    """Gradient of the scores of each softmax row: p * (dp - rowsum(p * dp)).

    p, dp: [n, m] for one head.  Masked entries have p = 0 and get 0.
    """
    return p * (dp - (p * dp).sum(axis=1, keepdims=True))


def head_gradients(p, q_rows, k_valid, v_valid, do_rows, scale):
    """Gradients of one head over a block of query rows.

    p: [n, m] probabilities over the m valid keys; q_rows, do_rows: [n, d];
    k_valid, v_valid: [m, d].  Returns (dq_rows [n, d], dk_part [m, d],
    dv_part [m, d]); dk_part and dv_part are this block's share of the key
    gradients.
    """
    dv_part = p.T @ do_rows
    dp = do_rows @ v_valid.T
    ds = softmax_backward(p, dp)
    dq_rows = scale * (ds @ k_valid)
    dk_part = scale * (ds.T @ q_rows)
    return dq_rows, dk_part, dv_part


def accumulate(total, part):
    """Key gradients of a K/V head: the sum over the query heads (and query
    row blocks) that read it."""
    return total + part


def attention_backward(q, k, v, do, *, scale=None, causal=False, window=0,
                       seqlens=None, window_right=0, sinks=0):
    """fp64 (dq, dk, dv) of O = softmax(scale Q K^T + mask) V given dO.

    q, do: [B, Hq, Nq, d]; k, v: [B, Hkv, Nk, d]; the mask, the row positions
    and the head map are the forward oracle's (`oracle.sdpa`).  Returns
    dq [B, Hq, Nq, d], dk and dv [B, Hkv, Nk, d], all float64.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    do = np.asarray(do)
    b_, hq, nq, d = q.shape
    _, hkv, nk, _ = k.shape
    if do.shape != q.shape:
        raise ValueError("do must have the shape of q")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    heads = _fwd._head_map(hq, hkv)
    extra = _fwd._extra(window_right, sinks)
    dq = np.zeros((b_, hq, nq, d), dtype=np.float64)
    dk = np.zeros((b_, hkv, nk, d), dtype=np.float64)
    dv = np.zeros((b_, hkv, nk, d), dtype=np.float64)
    for b in range(b_):
        vlen = _fwd._valid_len(seqlens, b, nk)
        live, _ = _fwd.row_positions(nq, nk, vlen)
        for h in range(hq):
            hk = heads[h]
            k64 = k[b, hk, :vlen].astype(np.float64)
            v64 = v[b, hk, :vlen].astype(np.float64)
            for r0 in range(0, min(live, nq), _ROW_CHUNK):
                rows = np.arange(r0, min(live, nq, r0 + _ROW_CHUNK))
                mask = _fwd.allowed_mask(nq, nk, vlen, causal, window, rows,
                                         **extra)
                # keys at or beyond the valid length are never allowed, and
                # dead rows are never visited: padded contents (even NaN)
                # cannot reach a gradient
                p, _ = _fwd.probabilities(q[b, h, rows], k64, scale,
                                          mask[:, :vlen])
                q64 = q[b, h, rows].astype(np.float64)
                do64 = do[b, h, rows].astype(np.float64)
                dq_r, dk_p, dv_p = head_gradients(p, q64, k64, v64, do64,
                                                  scale)
                dq[b, h, rows] = dq_r
                dk[b, hk, :vlen] = accumulate(dk[b, hk, :vlen], dk_p)
                dv[b, hk, :vlen] = accumulate(dv[b, hk, :vlen], dv_p)
    return dq, dk, dv
