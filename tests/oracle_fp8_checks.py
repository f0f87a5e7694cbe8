"""Pins for the FP8 reference (`oracle.fp8`).

Every check takes `fp8`, a module-like object with the functions of
`oracle.fp8` (e4m3_table, e4m3_encode, e4m3_decode, hadamard, fwht_f32,
rotate, quantize, dequantize, attention_quantized), and raises AssertionError
on a mismatch.  They are pinned to the E4M3 format's definition (4 exponent
bits with bias 7, 3 mantissa bits, subnormals, 448 the largest finite value),
to brute force over all codes, to the algebra of Hadamard matrices, and to
properties that block quantization must have whatever its implementation.
"""

import math

import numpy as np

import oracle


def check_e4m3_format(fp8):
    t = fp8.e4m3_table()
    assert t.shape == (256,)
    fixed = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 / 8 * 2.0 ** -6,
             0x08: 2.0 ** -6, 0x38: 1.0, 0x39: 1.125, 0x40: 2.0,
             0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0}
    for c, v in fixed.items():
        assert t[c] == v, (hex(c), t[c], v)
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert t[0x80] == 0 and np.signbit(t[0x80])
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0), "codes 0x00..0x7E increase"
    assert np.array_equal(t[0x80:0xFF], -pos)
    # 3 mantissa bits: within a binade the step is 2^(e-7)/8
    for e in range(1, 15):
        vals = pos[8 * e: 8 * e + 8]
        assert np.allclose(np.diff(vals), 2.0 ** (e - 7) / 8)


def check_e4m3_encode(fp8, seed=60):
    t = fp8.e4m3_table()
    finite = [c for c in range(256) if not np.isnan(t[c])]
    # every finite code round-trips (including -0)
    got = fp8.e4m3_encode(t[finite])
    assert list(got) == finite
    # nearest value by brute force over all codes, ties to the even code
    rng = np.random.default_rng(seed)
    x = np.concatenate([rng.standard_normal(3000) *
                        rng.choice([1e-3, 0.05, 1.0, 30.0, 200.0], 3000),
                        rng.uniform(-447.9, 447.9, 1000)])
    x = x[np.abs(x) < 464.0]  # beyond, the result is NaN (checked below)
    codes = fp8.e4m3_encode(x)
    fin = np.array(finite)
    tv = t[fin]
    for xi, ci in zip(x, codes):
        d = np.abs(tv - xi)
        best = d.min()
        cands = [int(c) for c in fin[d == best] if not (t[c] == 0 and
                 np.signbit(t[c]) != np.signbit(xi))]
        assert int(ci) in cands, (xi, hex(ci), [hex(c) for c in cands])
        if len(cands) > 1:   # a tie between neighbours: the even mantissa
            assert int(ci) % 2 == 0
    # midpoints between neighbouring codes go to the even one
    pos = t[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2
    mc = fp8.e4m3_encode(mids)
    assert np.all(mc % 2 == 0)
    # range end: 448 up to the midpoint 464 rounds to 448, beyond is NaN
    assert list(fp8.e4m3_encode([447.0, 455.9, 463.99, 464.0])) == \
        [0x7E] * 4
    assert list(fp8.e4m3_encode([464.5, 1e6, -500.0])) == [0x7F, 0x7F, 0xFF]
    # below half the smallest subnormal: zero of the same sign
    assert list(fp8.e4m3_encode([2.0 ** -11, -2.0 ** -11, 2.0 ** -10])) == \
        [0x00, 0x80, 0x00]


def check_hadamard_algebra(fp8, seed=61):
    for d in (2, 8, 64, 128):
        h = fp8.hadamard(d)
        assert np.array_equal(np.abs(h), np.ones((d, d)))
        assert np.array_equal(h @ h.T, d * np.eye(d))
    rng = np.random.default_rng(seed)
    d = 128
    h = fp8.hadamard(d)
    x = rng.integers(-8, 9, size=(5, d)).astype(np.float32)
    assert np.array_equal(fp8.fwht_f32(x).astype(np.float64),
                          x.astype(np.float64) @ h)
    # rotate(e_i) = row i of D H: the signs act before the transform
    s = rng.choice([-1.0, 1.0], d)
    for i in (0, 1, 77):
        e = np.zeros(d, dtype=np.float32)
        e[i] = 1
        assert np.array_equal(fp8.rotate(e[None], s)[0], s[i] * h[i])
    # (x D H)(y D H)^T = d x y^T for integer x, y (exact in float32)
    y = rng.integers(-8, 9, size=(7, d)).astype(np.float32)
    xr = fp8.rotate(x, s).astype(np.float64)
    yr = fp8.rotate(y, s).astype(np.float64)
    assert np.array_equal(xr @ yr.T, d * (x.astype(np.float64) @
                                          y.astype(np.float64).T))


def check_quantize_blocks(fp8, seed=62):
    rng = np.random.default_rng(seed)
    B, H, N, d = 2, 2, 150, 16
    x = rng.standard_normal((B, H, N, d)).astype(np.float32)
    x[0, 1, 70, 3] = 9.0          # an outlier in block 1 of (0, 1)
    valid = np.array([150, 100])
    x[1, :, 100:] = 1e6           # padding: never enters a scale
    codes, scales = fp8.quantize(x, valid)
    assert codes.dtype == np.uint8 and scales.shape == (B, H, 3)
    assert np.all(codes[1, :, 100:] == 0)
    t = fp8.e4m3_table()
    for b in range(B):
        for h in range(H):
            for blk in range(3):
                rows = slice(64 * blk, min(N, 64 * blk + 64, valid[b]))
                xb = x[b, h, rows]
                if xb.size == 0:
                    assert scales[b, h, blk] == 0
                    continue
                amax = np.float32(np.abs(xb).max())
                assert scales[b, h, blk] == np.float32(amax / np.float32(448))
                # the largest element maps to +-448 exactly
                cb = codes[b, h, rows]
                assert np.abs(t[cb]).max() == 448.0
                # each value is within half a step of its dequantized value
                dq = t[cb] * np.float64(scales[b, h, blk])
                err = np.abs(dq - xb)
                bound = np.maximum(np.abs(xb) * 2.0 ** -4,
                                   2.0 ** -10 * scales[b, h, blk])
                assert np.all(err <= bound * (1 + 1e-6))
    # blocks are independent: scaling one block by 2^5 changes its scale
    # by 2^5 and nothing else
    x2 = x.copy()
    x2[0, 0, 64:128] *= 32
    c2, s2 = fp8.quantize(x2, valid)
    assert np.array_equal(c2, codes)
    assert s2[0, 0, 1] == 32 * scales[0, 0, 1]
    s2[0, 0, 1] = scales[0, 0, 1]
    assert np.array_equal(s2, scales)
    # one scale per tensor: every block shares the tensor's amax
    ct, st = fp8.quantize(x, valid, per_tensor=True)
    live = np.arange(N)[None, :] < valid[:, None]
    amax = np.float32(np.abs(x[np.broadcast_to(live[:, None, :, None],
                                               x.shape)]).max())
    assert np.all(st == np.float32(amax / np.float32(448)))
    assert np.all(ct[1, :, 100:] == 0)


def check_rotation_preserves_attention(fp8, seed=63):
    """Attention of the rotated operands with the softmax scale divided by d
    equals attention of the originals (integer inputs: the rotation is exact
    in float32), so incoherent processing changes nothing before rounding."""
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, N, d = 2, 4, 2, 37, 32
    q = rng.integers(-3, 4, size=(B, Hq, N, d)).astype(np.float32)
    k = rng.integers(-3, 4, size=(B, Hkv, N, d)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, N, d))
    s = rng.choice([-1.0, 1.0], d)
    sl = np.array([37, 20])
    o, lse = oracle.attention(q, k, v, scale=0.05, causal=True, seqlens=sl)
    o2, lse2 = oracle.attention(fp8.rotate(q, s), fp8.rotate(k, s), v,
                                scale=0.05 / d, causal=True, seqlens=sl)
    np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-13)
    fin = np.isfinite(lse)
    np.testing.assert_allclose(lse2[fin], lse[fin], rtol=1e-12, atol=1e-12)


def check_attention_quantized(fp8, seed=64):
    """attention_quantized is attention of the dequantized operands; with
    the rotation its scale is divided by d; and block quantization with the
    rotation tracks the exact result more closely than one scale per tensor
    when a few channels carry outliers (the page's claim, as an ordering)."""
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, N, d = 2, 2, 1, 160, 64
    q = rng.standard_normal((B, Hq, N, d)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, N, d)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, N, d)).astype(np.float32)
    q[..., 5] *= 25
    k[..., 5] *= 25
    k[:, :, :, 40] *= 15
    s = rng.choice([-1.0, 1.0], d)
    sl = np.array([160, 90])
    scale = 1 / math.sqrt(d)
    kw = dict(causal=True, seqlens=sl)
    qz = fp8.quantize(q, sl, signs=s)
    kz = fp8.quantize(k, sl, signs=s)
    vz = fp8.quantize(v, sl)
    o, _ = fp8.attention_quantized(qz, kz, vz, scale=scale, rotated=True,
                                   **kw)
    o_ref, _ = oracle.attention(fp8.dequantize(*qz), fp8.dequantize(*kz),
                                fp8.dequantize(*vz), scale=scale / d, **kw)
    assert np.array_equal(o, o_ref)
    exact, lse = oracle.attention(q, k, v, scale=scale, **kw)
    live = np.isfinite(lse)
    err_blk = fp8.rmse(o, exact, live)
    qt = fp8.quantize(q, sl, per_tensor=True)
    kt = fp8.quantize(k, sl, per_tensor=True)
    vt = fp8.quantize(v, sl, per_tensor=True)
    ot, _ = fp8.attention_quantized(qt, kt, vt, scale=scale, rotated=False,
                                    **kw)
    err_t = fp8.rmse(ot, exact, live)
    assert err_blk < err_t, (err_blk, err_t)


def check_quantize_all(fp8, seed=65):
    """The problem-level step: Q and K rotated with the signs, V never;
    valid rows from the boundary's semantics (a chunk's Q rows are all
    live); the attention of the result tracks the exact one within FP8
    error."""
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, Nq, Nk, d = 2, 2, 1, 40, 100, 32
    q = rng.standard_normal((B, Hq, Nq, d)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, Nk, d)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, Nk, d)).astype(np.float32)
    s = rng.choice([-1.0, 1.0], d)
    sl = np.array([100, 70])
    z = fp8.quantize_all(q, k, v, sl, signs=s)
    np.testing.assert_array_equal(z["q"][0], fp8.quantize(q, [40, 40],
                                                          signs=s)[0])
    np.testing.assert_array_equal(z["k"][0], fp8.quantize(k, sl, signs=s)[0])
    np.testing.assert_array_equal(z["v"][0], fp8.quantize(v, sl)[0])
    o, _ = fp8.attention_quantized(z["q"], z["k"], z["v"],
                                   scale=1 / math.sqrt(d), rotated=True,
                                   causal=True, seqlens=sl)
    exact, lse = oracle.attention(q, k, v, scale=1 / math.sqrt(d),
                                  causal=True, seqlens=sl)
    live = np.isfinite(lse)
    err = np.abs(o - exact)[live]
    assert err.max() < 0.1 and err.mean() < 0.02, (err.max(), err.mean())


def _bf16(x):
    """float32 values rounded to bfloat16 (nearest even), kept in float32."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(
        torch.bfloat16).to(torch.float32).numpy()


def check_fwht_f32_against_exact_rotation(fp8, seed=66):
    """The float32 butterflies against the exact rotation, independently of
    any kernel.

    Exact: for bfloat16 inputs (8 significant bits) at d <= 128, x D H is a
    sum of at most 128 signed bf16 values; scaled by a power of two they are
    integers far below 2^53, so a float64 matrix product holds them exactly
    (checked here against an int64 product).
    Error bound: the float32 transform runs log2(d) butterfly stages, each
    rounding once (unit roundoff u = 2^-24) a value bounded by sum_i |x_i|,
    so |fwht_f32(x) - x H| <= log2(d) u sum_i |x_i| (to first order).
    Code decisions: with the float32 path's block multiplier, a code of the
    float32 value may differ from the code of the exact value only where the
    exact scaled value lies within that error (plus the float32 product's
    own rounding) of a midpoint between two E4M3 values.  Such codes are
    counted and bounded.  On these inputs the float32 values carry any
    rounding in 1-3% of elements, at most 0.14 of the bound, and no code of
    the 786432 differs from the exact rotation's."""
    rng = np.random.default_rng(seed)
    mids = (fp8._POS[:-1] + fp8._POS[1:]) / 2.0
    u = 2.0 ** -24
    changed_total = 0
    codes_total = 0
    for d in (64, 128):
        n = 4096
        x = rng.standard_normal((n, d)).astype(np.float32)
        x[:, rng.choice(d, 4, replace=False)] *= 20.0  # outlier channels
        x = _bf16(x)
        s = rng.choice([-1.0, 1.0], d)
        h = fp8.hadamard(d)
        xs = x.astype(np.float64) * s
        exact = xs @ h
        # the float64 product is exact: compare with integers
        _, e = np.frexp(xs[xs != 0])
        k = int(8 - e.min())  # 2^k x is an integer for every element
        xi = np.rint(np.ldexp(xs, k)).astype(np.int64)
        assert np.array_equal(np.ldexp(xi.astype(np.float64), -k), xs)
        yi = xi @ h.astype(np.int64)
        assert np.abs(yi).max() < 2 ** 53
        assert np.array_equal(np.ldexp(yi.astype(np.float64), -k), exact)
        # the float32 butterflies stay within their error bound
        y32 = fp8.rotate(x, s).astype(np.float64)
        bound = 1.01 * math.log2(d) * u * np.abs(x).astype(np.float64).sum(
            axis=1, keepdims=True)
        err = np.abs(y32 - exact)
        assert np.all(err <= bound), float((err / bound).max())
        assert err.max() > 0  # the inputs do exercise the rounding
        # code decisions, 64-row blocks, the float32 path's multiplier
        for b0 in range(0, n, 64):
            blk32 = y32[b0:b0 + 64].astype(np.float32)
            _, mul = fp8._block_scale(np.abs(blk32).max())
            c32 = fp8.e4m3_encode(np.float32(blk32 * mul))
            z = exact[b0:b0 + 64] * np.float64(mul)
            c64 = fp8.e4m3_encode(z)
            diff = c32 != c64
            codes_total += diff.size
            if not diff.any():
                continue
            a = np.abs(z[diff])
            j = np.clip(np.searchsorted(mids, a), 1, len(mids) - 1)
            dist = np.minimum(np.abs(a - mids[j - 1]), np.abs(a - mids[j]))
            tol = (bound[b0:b0 + 64] * np.ones_like(z))[diff] * float(mul) \
                + 2.0 * u * a
            assert np.all(dist <= tol), float((dist / tol).max())
            changed_total += int(diff.sum())
    assert changed_total <= 5e-4 * codes_total, (changed_total, codes_total)


FP8_CHECKS = [
    check_e4m3_format,
    check_e4m3_encode,
    check_hadamard_algebra,
    check_fwht_f32_against_exact_rotation,
    check_quantize_blocks,
    check_rotation_preserves_attention,
    check_attention_quantized,
    check_quantize_all,
]
