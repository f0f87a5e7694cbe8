"""GPU parity on a seeded sweep of shapes and masks drawn at random, every
row against the oracle: head dimension, dtype, group size, Nq (= Nk, 1, or
in between), Nk, causal or not, left and right window limits, sink keys,
valid lengths and amplitude.  The draws come from one fixed generator, so
the sweep is the same on every run; each case prints its shape first.
Sizes are capped so that the whole sweep's oracle work stays within
seconds.
"""

import numpy as np
import pytest

import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

N_CASES = 192


def _draw_cases(seed=20261204, n=N_CASES):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        d = int(rng.choice([64, 128]))
        dtype = "fp32" if rng.random() < 0.15 else "bf16"
        hkv = int(rng.choice([1, 2, 3]))
        g = int(rng.choice([1, 2, 3, 4, 7, 8]))
        nk = int(rng.integers(1, 700))
        kind = rng.random()
        nq = nk if kind < 0.55 else (1 if kind < 0.75 else
                                    int(rng.integers(1, nk + 1)))
        b = int(rng.integers(1, 4))
        if b * hkv * g * nq * nk * d > 1.5e8:  # oracle time
            continue
        causal = bool(rng.random() < 0.6)
        window = int(rng.integers(1, nk + 40)) if rng.random() < 0.35 else 0
        wr = int(rng.integers(1, nk + 40)) if rng.random() < 0.2 else 0
        sinks = int(rng.integers(1, 80)) if rng.random() < 0.2 else 0
        padded = rng.random() < 0.5
        lo = int(rng.integers(0, nk + 1)) if padded else 0
        amp = float(rng.choice([0.5, 1.0, 1.0, 2.0]))
        name = f"rand{len(cases):02d}"
        cases.append(synth.Workload(
            name, B=b, Hq=hkv * g, Hkv=hkv, Nq=nq, Nk=nk, d=d, dtype=dtype,
            causal=causal, window=window, window_right=wr, sinks=sinks,
            len_lo=lo if padded else 0, len_hi=nk if padded else 0,
            amp=amp))
    return cases


CASES = _draw_cases()


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_random_shape(w):
    gu.check_full(w.name, w, 1000 + int(w.name[4:]))


# ---- the backward pass on a seeded sweep -----------------------------------
# Rows that see a single key have gradients that vanish only by cancellation
# (their exact value is 0, the bf16 path leaves an fp32 residue), so the
# sweep keeps every sequence at 8 keys or more and windows of 8 or more; a
# tensor's bounds are stated against its own scale, as in the backward
# tests.

N_BWD_CASES = 48


def _draw_bwd_cases(seed=20261205, n=N_BWD_CASES):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        d = int(rng.choice([64, 128]))
        hkv = int(rng.choice([1, 2]))
        g = int(rng.choice([1, 2, 3, 4, 7]))
        nk = int(rng.integers(16, 600))
        kind = rng.random()
        nq = nk if kind < 0.6 else (1 if kind < 0.7 else
                                   int(rng.integers(2, nk + 1)))
        b = int(rng.integers(1, 4))
        if b * hkv * g * nq * nk * d > 1.0e8:
            continue
        causal = bool(rng.random() < 0.6)
        window = int(rng.integers(8, nk + 40)) if rng.random() < 0.3 else 0
        wr = int(rng.integers(8, nk + 40)) if rng.random() < 0.2 else 0
        sinks = int(rng.integers(1, 40)) if rng.random() < 0.2 else 0
        padded = rng.random() < 0.5
        lo = int(rng.integers(8, nk + 1)) if padded else 0
        cases.append(synth.Workload(
            f"bwdrand{len(cases):02d}", B=b, Hq=hkv * g, Hkv=hkv, Nq=nq,
            Nk=nk, d=d, dtype="bf16", causal=causal, window=window,
            window_right=wr, sinks=sinks, len_lo=lo if padded else 0,
            len_hi=nk if padded else 0))
    return cases


BWD_CASES = _draw_bwd_cases()


@pytest.mark.parametrize("w", BWD_CASES, ids=lambda w: w.name)
def test_random_shape_backward(w):
    from tests.test_gpu_backward import check_bwd_full
    check_bwd_full(w.name, w, 2000 + int(w.name[7:]))


# ---- the FP8 path on a seeded sweep ----------------------------------------
# Each case: codes and scales bit for bit against the FP8 reference, then the
# forward against the exact attention of the dequantized operands (the
# checks and tolerances of the FP8 tests).

N_FP8_CASES = 32


def _draw_fp8_cases(seed=20261206, n=N_FP8_CASES):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        d = int(rng.choice([64, 128]))
        hkv = int(rng.choice([1, 2]))
        g = int(rng.choice([1, 2, 4, 7]))
        nk = int(rng.integers(1, 700))
        kind = rng.random()
        nq = nk if kind < 0.6 else (1 if kind < 0.7 else
                                   int(rng.integers(1, nk + 1)))
        b = int(rng.integers(1, 4))
        if b * hkv * g * nq * nk * d > 1.0e8:
            continue
        causal = bool(rng.random() < 0.6)
        window = int(rng.integers(1, nk + 40)) if rng.random() < 0.3 else 0
        wr = int(rng.integers(1, nk + 40)) if rng.random() < 0.2 else 0
        sinks = int(rng.integers(1, 40)) if rng.random() < 0.2 else 0
        padded = rng.random() < 0.5
        lo = int(rng.integers(0, nk + 1)) if padded else 0
        rot = bool(rng.random() < 0.7)
        pt = bool(rng.random() < 0.2)
        cases.append((synth.Workload(
            f"fp8rand{len(cases):02d}", B=b, Hq=hkv * g, Hkv=hkv, Nq=nq,
            Nk=nk, d=d, dtype="bf16", causal=causal, window=window,
            window_right=wr, sinks=sinks, len_lo=lo if padded else 0,
            len_hi=nk if padded else 0), rot, pt))
    return cases


FP8_CASES = _draw_fp8_cases()


@pytest.mark.parametrize("w,rot,pt", FP8_CASES,
                         ids=lambda c: getattr(c, "name", str(c)))
def test_random_shape_fp8(w, rot, pt):
    from tests.test_gpu_fp8 import (test_fp8_forward_matches_oracle,
                                    test_fp8_quantize_bit_exact)
    test_fp8_quantize_bit_exact(w, rot, pt)
    test_fp8_forward_matches_oracle(w, rot, pt)


# ---- medium sizes, sampled rows ---------------------------------------------
# Launches of several rounds of the chip's workgroup slots (block orders with
# and without bands, groups that do and do not divide over the XCDs, the
# run-time causal tail), each checked on sampled rows (tile edges, the
# valid-length boundary, random rows) computed by the oracle one by one.

N_MEDIUM_CASES = 16


def _draw_medium_cases(seed=20261207, n=N_MEDIUM_CASES):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        d = int(rng.choice([64, 128]))
        hkv = int(rng.choice([1, 2, 4, 8]))
        g = int(rng.choice([1, 2, 4, 7]))
        nk = int(rng.integers(1024, 8193))
        nq = nk if rng.random() < 0.8 else int(rng.integers(2, nk + 1))
        b = int(rng.integers(1, 5))
        if b * hkv * g * nq * nk * d > 6e10:  # GPU time and memory
            continue
        causal = bool(rng.random() < 0.75)
        window = int(rng.integers(64, nk)) if rng.random() < 0.25 else 0
        sinks = int(rng.integers(1, 100)) if rng.random() < 0.15 else 0
        padded = rng.random() < 0.4
        lo = int(rng.integers(1, nk + 1)) if padded else 0
        cases.append(synth.Workload(
            f"medrand{len(cases):02d}", B=b, Hq=hkv * g, Hkv=hkv, Nq=nq,
            Nk=nk, d=d, dtype="bf16", causal=causal or window > 0,
            window=window, sinks=sinks, len_lo=lo if padded else 0,
            len_hi=nk if padded else 0))
    return cases


MEDIUM_CASES = _draw_medium_cases()


@pytest.mark.parametrize("w", MEDIUM_CASES, ids=lambda w: w.name)
def test_random_medium_shape_sampled(w):
    gu.check_sampled(w.name, w, 3000 + int(w.name[7:]))
