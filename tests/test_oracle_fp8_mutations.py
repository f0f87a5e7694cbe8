"""CPU-only: the FP8 reference's pins are strong enough.  Each test plants
one plausible mistake (truncation instead of rounding, ties away from zero,
the wrong largest value, padding inside a scale, the signs applied after the
transform, the scale not divided by d, V rotated too, blocks of 32 rows) and
requires that at least one pin fails."""

import numpy as np
import pytest

import oracle.fp8 as real
from tests import oracle_fp8_checks as ofc


class Mutant:
    """oracle.fp8 with one function replaced; the others are the real ones
    but see the replacement (they are re-bound here)."""

    def __init__(self, **over):
        self.__dict__.update(over)

    def __getattr__(self, name):
        return getattr(real, name)


def _encode_trunc(x):
    x = np.asarray(x, dtype=np.float64)
    t = real._POS
    a = np.abs(x).reshape(-1)
    j = np.clip(np.searchsorted(t, a, side="right") - 1, 0, len(t) - 1)
    out = j.astype(np.uint8) | np.where(np.signbit(x.reshape(-1)), 0x80,
                                        0).astype(np.uint8)
    return out.reshape(x.shape)  # planted: round toward zero


def _encode_ties_away(x):
    x = np.asarray(x, dtype=np.float64)
    t = real._POS
    a = np.abs(x).reshape(-1)
    j = np.clip(np.searchsorted(t, a), 1, len(t) - 1)
    lo = j - 1
    pick = np.where(a - t[lo] < t[j] - a, lo, j)  # planted: ties go up
    pick = np.where(t[j] == a, j, pick)
    pick = np.where(a == 0, 0, pick)
    out = pick.astype(np.uint8) | np.where(np.signbit(x.reshape(-1)), 0x80,
                                           0).astype(np.uint8)
    return out.reshape(x.shape)


def _quantize_with(**kw):
    def quantize(x, valid, *, signs=None, per_tensor=False):
        x = np.asarray(x, dtype=np.float32)
        b_, h_, n, d = x.shape
        blk = kw.get("block", 64)
        mx = np.float32(kw.get("emax", 448.0))
        nb = (n + 63) // 64
        if signs is not None:
            if kw.get("signs_after"):
                xr = real.fwht_f32(x) * np.asarray(signs, np.float32)
            else:
                xr = real.rotate(x, signs)
        else:
            xr = x.copy()
        live = np.arange(n)[None, :] < np.asarray(valid)[:, None]
        if not kw.get("padding_in_scale"):
            xr = np.where(live[:, None, :, None], xr, np.float32(0))
        codes = np.zeros(x.shape, np.uint8)
        scales = np.zeros((b_, h_, nb), np.float32)
        for b in range(b_):
            for h in range(h_):
                for s0 in range(0, n, blk):
                    sl = slice(s0, min(n, s0 + blk))
                    amax = np.float32(np.abs(xr[b, h, sl]).max())
                    if amax == 0:
                        continue
                    codes[b, h, sl] = real.e4m3_encode(
                        (xr[b, h, sl] * (mx / amax)).astype(np.float32))
                    scales[b, h, s0 // 64] = np.float32(amax / mx)
        if kw.get("padding_in_scale"):
            codes = np.where(live[:, None, :, None], codes, 0).astype(np.uint8)
        return codes, scales
    return quantize


def _attn_unscaled(qz, kz, vz, *, scale, rotated, **kw):
    return real.attention_quantized(qz, kz, vz, scale=scale, rotated=False,
                                    **kw)  # planted: scale not divided by d


def _quantize_all_v_rotated(q, k, v, seqlens, *, signs=None,
                            per_tensor=False):
    out = real.quantize_all(q, k, v, seqlens, signs=signs,
                            per_tensor=per_tensor)
    if signs is not None:  # planted: V rotated as well
        lk = [int(seqlens[b]) for b in range(np.shape(v)[0])]
        out["v"] = real.quantize(v, lk, signs=signs, per_tensor=per_tensor)
    return out


def _fwht_with(round_stage=None, swap=False):
    def fwht(x):
        y = np.array(x, dtype=np.float32, copy=True)
        d = y.shape[-1]
        h = 1
        while h < d:
            y = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
            a = y[..., 0, :].copy()
            b = y[..., 1, :].copy()
            y[..., 0, :] = a + b
            y[..., 1, :] = (b - a) if swap else (a - b)  # planted: sign
            if round_stage:
                y = round_stage(y)  # planted: a stage kept in low precision
            y = y.reshape(y.shape[:-3] + (d,))
            h *= 2
        return y
    return dict(fwht_f32=fwht,
                rotate=lambda x, s: fwht(np.asarray(x, np.float32) *
                                         np.asarray(s, np.float32)))


def _to_bf16(y):
    from tests.oracle_fp8_checks import _bf16
    return _bf16(y).reshape(y.shape)


MUTANTS = {
    "fwht_in_bf16": _fwht_with(round_stage=_to_bf16),
    "fwht_butterfly_sign": _fwht_with(swap=True),
    "v_rotated_too": dict(quantize_all=_quantize_all_v_rotated),
    "encode_truncates": dict(e4m3_encode=_encode_trunc),
    "encode_ties_away": dict(e4m3_encode=_encode_ties_away),
    "scale_from_240": dict(quantize=_quantize_with(emax=240.0)),
    "padding_in_scale": dict(quantize=_quantize_with(padding_in_scale=True)),
    "signs_after_transform": dict(
        quantize=_quantize_with(signs_after=True),
        rotate=lambda x, s: real.fwht_f32(x) * np.asarray(s, np.float32)),
    "rotation_scale_not_divided": dict(attention_quantized=_attn_unscaled),
    "blocks_of_32": dict(quantize=_quantize_with(block=32)),
}


def _run(mod):
    failed = []
    for check in ofc.FP8_CHECKS:
        try:
            check(mod)
        except AssertionError:
            failed.append(check.__name__)
    return failed


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_fp8_mistake_is_caught(name):
    assert _run(Mutant(**MUTANTS[name])), f"no pin catches {name!r}"


def test_real_fp8_reference_passes_all():
    assert _run(real) == []
