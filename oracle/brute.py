"""Scalar-loop attention for tiny inputs: the second, independent statement of
the definition that the NumPy oracle is checked against.

Test infrastructure only.  Pure Python floats (IEEE double), `math.fsum` for
every sum, `math.exp`/`math.log`, nested lists, no NumPy arithmetic and no code
shared with `oracle.sdpa` (the mask predicate is restated here on
purpose).  Meant for N <= ~16, d <= ~8.

Definition followed (see `oracle.sdpa` for the page citations):
  s_ij = scale * sum_c q[i][c] * k[j][c]
  allowed(i, j): live query row, j < valid length, causal => j <= pos(i),
                 window > 0 => pos(i) - j < window
  p_ij = exp(s_ij) / sum_{allowed j'} exp(s_ij')
  o_i  = sum_{allowed j} p_ij * v_j,  lse_i = log sum_{allowed j} exp(s_ij)
Rows with no allowed key give o_i = 0 and lse_i = -inf.
"""

import math


def _allowed(i, j, nq, nk, valid_len, causal, window, window_right=0,
             sinks=0):
    if nq == nk:
        live, pos = valid_len, i
    else:
        live, pos = nq, valid_len - nq + i
    if i >= live or j >= valid_len:
        return False
    if causal and j > pos:
        return False
    if j < sinks:
        return True
    if window > 0 and pos - j >= window:
        return False
    if window_right > 0 and j - pos >= window_right:
        return False
    return True


def attention_loops(q, k, v, *, scale, causal=False, window=0, seqlens=None,
                    window_right=0, sinks=0):
    """q: nested lists [B][Hq][Nq][d]; k, v: [B][Hkv][Nk][d].

    Returns (o [B][Hq][Nq][d], lse [B][Hq][Nq]) as nested lists of floats.
    """
    b_n = len(q)
    hq = len(q[0])
    nq = len(q[0][0])
    d = len(q[0][0][0])
    hkv = len(k[0])
    nk = len(k[0][0])
    group = hq // hkv
    o = []
    lse = []
    for b in range(b_n):
        vlen = nk if seqlens is None else min(max(int(seqlens[b]), 0), nk)
        ob, lb = [], []
        for h in range(hq):
            hk = h // group
            oh, lh = [], []
            for i in range(nq):
                scores = {}
                for j in range(nk):
                    if _allowed(i, j, nq, nk, vlen, causal, window,
                                window_right, sinks):
                        dot = math.fsum(q[b][h][i][c] * k[b][hk][j][c]
                                        for c in range(d))
                        scores[j] = scale * dot
                if not scores:
                    oh.append([0.0] * d)
                    lh.append(-math.inf)
                    continue
                m = max(scores.values())
                w = {j: math.exp(s - m) for j, s in scores.items()}
                total = math.fsum(w.values())
                row = [math.fsum(w[j] * v[b][hk][j][c] for j in w) / total
                       for c in range(d)]
                oh.append(row)
                lh.append(m + math.log(total))
            ob.append(oh)
            lb.append(lh)
        o.append(ob)
        lse.append(lb)
    return o, lse
