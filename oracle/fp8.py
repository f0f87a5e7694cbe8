"""FP8 block quantization with incoherent processing, and attention on the
quantized operands: the reference for the FP8 path.

Test infrastructure only (see the package docstring).

What the FlashAttention-3 review page describes (its FP8 sections, the
"Block Quantization" and "Incoherent Processing" passages), restated:
  * FP8 is E4M3: 1 sign, 4 exponent and 3 mantissa bits.
  * Block quantization: Q, K and V are cut into blocks of rows; each block
    keeps its own scale, set from the block's range, the block is scaled
    and then rounded to FP8.
  * Incoherent processing: before quantization Q and K are multiplied by a
    random orthogonal matrix M, a Hadamard matrix times a random diagonal of
    +-1, Q' = Q M and K' = K M; Q' K'^T = Q K^T, so attention is unchanged
    while outliers in a few channels are spread over all of them.
  * The measure: the RMSE of FP8 attention against the exact result, which
    the page reports 2.6 times lower than with one scale per tensor.
Readings taken where the page leaves a step open:
  * E4M3 is the OCP "fn" variant: exponent bias 7, subnormals, no
    infinities, S.1111.111 is NaN, largest finite value 448.  Rounding is to
    nearest, ties to even; a value whose rounding would pass 448 (|x| > 464)
    becomes NaN.  The quantizer never produces one (below).
  * Scale from the range: s = amax / 448 with amax = max |x| over the
    block's valid rows (padding rows are left out and encode as 0); a value
    is encoded as E4M3(x * (448 / amax)), computed in float32; a block with
    amax = 0 has s = 0 and all codes 0.  These are the decisions that fix a
    code, so they are taken in float32, like the kernel that makes them.
  * Blocks are 64 rows of one (batch, head): the kernels' tile height.
  * M = D H with D = diag(signs), H the Sylvester Hadamard matrix (entries
    +-1, H H^T = d I), applied unnormalised: Q'' = Q D H, K'' = K D H, and
    Q'' K''^T = d Q K^T, so the softmax scale is divided by d.  x D H is
    evaluated by the fast Walsh-Hadamard transform in float32, butterfly
    stages of width 1, 2, 4, ..., d/2 in that order (the kernel does the
    same, so both produce the same float32 values).  V is not rotated.
  * One scale per tensor (the baseline): the same steps with a single block
    spanning every valid row of the tensor, no rotation.
"""

import numpy as np

from . import sdpa as _fwd

E4M3_MAX = 448.0
BLOCK = 64


def e4m3_table():
    """Value of each of the 256 E4M3 codes (NaN for the two NaN codes)."""
    vals = np.zeros(256, dtype=np.float64)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = sign * (m / 8.0) * 2.0 ** -6       # subnormal
        else:
            vals[c] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_TABLE = e4m3_table()
_POS = _TABLE[:0x7F]  # codes 0x00 .. 0x7E: the non-negative finite values


def e4m3_encode(x):
    """Round to the nearest E4M3 value, ties to the even code; |x| > 464
    (past the midpoint between 448 and the next step, 480, which has no
    code) and NaN give the NaN code; 464 itself is a tie and goes to 448.
    x: array of float64 or float32 (values are taken exactly).  Returns
    uint8 codes of x's shape."""
    x = np.asarray(x, dtype=np.float64)
    flat = x.reshape(-1)
    out = np.zeros(flat.shape, dtype=np.uint8)
    neg = np.signbit(flat)
    a = np.abs(flat)
    nan = ~np.isfinite(a) | (a > 464.0)
    ok = ~nan
    j = np.searchsorted(_POS, np.where(ok, a, 0.0))  # _POS[j-1] < a <= _POS[j]
    j = np.minimum(j, len(_POS) - 1)
    exact = _POS[j] == a
    lo = np.maximum(j - 1, 0)
    dl = a - _POS[lo]
    dh = _POS[j] - a
    pick = np.where(dl < dh, lo, np.where(dh < dl, j, np.where(lo % 2 == 0,
                                                                lo, j)))
    code = np.where(exact, j, pick)
    # values at or above 448 that round to 448 (448 <= a <= 464)
    code = np.where(a >= E4M3_MAX, 0x7E, code)
    out[ok] = code[ok].astype(np.uint8)
    out[nan] = 0x7F
    out |= np.where(neg, 0x80, 0).astype(np.uint8)
    return out.reshape(x.shape)


def e4m3_decode(codes):
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def hadamard(d):
    """Sylvester Hadamard matrix of order d (a power of two), entries +-1."""
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    if h.shape[0] != d:
        raise ValueError("d must be a power of two")
    return h


def fwht_f32(x):
    """x H along the last axis, in float32, by butterflies: stage h = 1, 2,
    4, ..., d/2 replaces each pair (x_j, x_{j+h}) of every block of 2h by
    (x_j + x_{j+h}, x_j - x_{j+h})."""
    y = np.array(x, dtype=np.float32, copy=True)
    d = y.shape[-1]
    h = 1
    while h < d:
        y = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
        a = y[..., 0, :].copy()
        b = y[..., 1, :].copy()
        y[..., 0, :] = a + b
        y[..., 1, :] = a - b
        y = y.reshape(y.shape[:-3] + (d,))
        h *= 2
    return y


def rotate(x, signs):
    """x D H (float32): signs multiply each channel (exact), then the
    unnormalised Hadamard transform."""
    s = np.asarray(signs, dtype=np.float32)
    return fwht_f32(np.asarray(x, dtype=np.float32) * s)


def _block_scale(amax):
    """(scale, multiplier) of a block from its amax, in float32."""
    amax = np.float32(amax)
    if amax == 0:
        return np.float32(0.0), np.float32(0.0)
    return (np.float32(amax / np.float32(E4M3_MAX)),
            np.float32(np.float32(E4M3_MAX) / amax))


def quantize(x, valid, *, signs=None, per_tensor=False):
    """Quantize a [B, H, N, d] tensor to E4M3 codes in blocks of 64 rows.

    valid[b]: number of valid rows of batch b (rows at or past it are
    padding: excluded from amax, encoded as 0).  Returns (codes uint8
    [B, H, N, d], scales float32 [B, H, ceil(N/64)]), both in the natural
    row order (the kernels' storage layouts are a permutation of these).
    """
    x = np.asarray(x, dtype=np.float32)
    b_, h_, n, d = x.shape
    nb = (n + BLOCK - 1) // BLOCK
    xr = rotate(x, signs) if signs is not None else x.copy()
    rows = np.arange(n)
    live = rows[None, :] < np.asarray(valid)[:, None]          # [B, N]
    xr = np.where(live[:, None, :, None], xr, np.float32(0.0))
    codes = np.zeros(x.shape, dtype=np.uint8)
    scales = np.zeros((b_, h_, nb), dtype=np.float32)
    if per_tensor:
        s, mul = _block_scale(np.abs(xr).max() if xr.size else 0.0)
        codes = e4m3_encode(np.float32(xr * mul))
        scales[:] = s
        return codes, scales
    for b in range(b_):
        for h in range(h_):
            for blk in range(nb):
                sl = slice(blk * BLOCK, min(n, (blk + 1) * BLOCK))
                s, mul = _block_scale(np.abs(xr[b, h, sl]).max())
                codes[b, h, sl] = e4m3_encode(
                    (xr[b, h, sl] * mul).astype(np.float32))
                scales[b, h, blk] = s
    return codes, scales


def dequantize(codes, scales):
    """codes [B, H, N, d], scales [B, H, ceil(N/64)] -> float64 values."""
    n = codes.shape[2]
    per_row = np.repeat(scales.astype(np.float64), BLOCK, axis=2)[:, :, :n]
    return e4m3_decode(codes) * per_row[..., None]


def quantize_all(q, k, v, seqlens, *, signs=None, per_tensor=False):
    """The FP8 path's quantization step for one attention problem: Q and K
    rotated when signs are given, V never; valid rows from the boundary's
    semantics (Q: the live rows; K, V: the valid length)."""
    b_, _, nq, _ = np.shape(q)
    nk = np.shape(k)[2]
    lk = np.array([_fwd._valid_len(seqlens, b, nk) for b in range(b_)])
    lq = np.array([_fwd.row_positions(nq, nk, int(lk[b]))[0]
                   for b in range(b_)])
    out = {}
    out["q"] = quantize(q, lq, signs=signs, per_tensor=per_tensor)
    out["k"] = quantize(k, lk, signs=signs, per_tensor=per_tensor)
    out["v"] = quantize(v, lk, per_tensor=per_tensor)
    return out


def attention_quantized(qz, kz, vz, *, scale, rotated, causal=False,
                        window=0, seqlens=None, window_right=0, sinks=0):
    """Exact (fp64) attention of the dequantized operands: the function the
    FP8 kernel approximates.  With rotated operands Q'' K''^T = d Q K^T, so
    the softmax scale is divided by d."""
    qd = dequantize(*qz)
    kd = dequantize(*kz)
    vd = dequantize(*vz)
    d = qd.shape[-1]
    sc = scale / d if rotated else scale
    return _fwd.attention(qd, kd, vd, scale=sc, causal=causal, window=window,
                          seqlens=seqlens, window_right=window_right,
                          sinks=sinks)


def rmse(a, b, live):
    """Root mean squared difference over the rows where `live` is True."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    diff = (a - b)[live]
    return float(np.sqrt(np.mean(diff * diff))) if diff.size else 0.0
