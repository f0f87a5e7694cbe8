"""CPU-only: the fp64 oracle pinned to brute force, closed forms, invariants,
the pages' worked examples and an independent library routine."""

import math

import numpy as np
import pytest

import oracle
from tests import oracle_bwd_checks as obc
from tests import oracle_fp8_checks as ofc
from tests import oracle_checks as oc


@pytest.mark.parametrize("check", oc.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(oracle.attention)


def test_printed_numbers_are_inconsistent_with_printed_inputs():
    """Documents why the review page's printed S/P/O numbers are not used as
    expected values: they do not follow from the printed Q and K."""
    for ex in oc.load_worked_examples():
        Q = np.array(ex["Q"], dtype=np.float64)
        K = np.array(ex["K"], dtype=np.float64)
        S = Q @ K.T
        bad = ex.get("printed_inconsistent", {})
        if "S" in bad:
            printed = np.array(bad["S"], dtype=np.float64)
            assert printed.shape != S.shape or not np.array_equal(printed, S)
        if "S_row1" in bad:
            assert not np.array_equal(np.array(bad["S_row1"]), S[1])
        good = ex.get("printed_consistent", {})
        if "S_row0" in good:
            assert np.array_equal(np.array(good["S_row0"]), S[0])
        if "P_row0" in bad:
            for sc in (1.0, 1 / math.sqrt(2)):
                p, _ = oracle.probabilities(Q[:1], K, sc,
                                            np.ones((1, 4), dtype=bool))
                assert not np.allclose(p[0, :2], bad["P_row0"], atol=5e-3)


def test_perturbation_bound_progressive_quantization():
    """SpAtten review, D. Progressive Quantization: an error ds on one score
    changes the probabilities by sum_i |dp_i| ~= 2 ds p0 (1 - p0) <= ds / 2.
    The perturbation is made through the oracle's public inputs (moving key 0
    along q so that exactly s_0 shifts by ds)."""
    rng = np.random.default_rng(21)
    for trial in range(20):
        n, d = int(rng.integers(2, 40)), 8
        q = rng.standard_normal((1, d))
        k = rng.standard_normal((n, d)) * rng.uniform(0.2, 3)
        scale = 0.5
        mask = np.ones((1, n), dtype=bool)
        p, _ = oracle.probabilities(q, k, scale, mask)
        ds = 1e-6
        k2 = k.copy()
        k2[0] += (ds / scale) * q[0] / np.dot(q[0], q[0])
        p2, _ = oracle.probabilities(q, k2, scale, mask)
        err = np.abs(p2 - p).sum()
        p0 = p[0, 0]
        want = 2 * ds * p0 * (1 - p0)
        assert err <= ds / 2 + 1e-15
        assert abs(err - want) <= 1e-3 * want + 1e-15


def test_probabilities_rows_sum_to_one():
    rng = np.random.default_rng(22)
    q = rng.standard_normal((9, 4)) * 4
    k = rng.standard_normal((13, 4)) * 4
    mask = oracle.allowed_mask(13, 13, 13, True, 0, np.arange(9))
    p, lse = oracle.probabilities(q, k, 1.0, mask)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    assert np.all(p[~mask] == 0)


def test_rows_api_matches_full():
    rng = np.random.default_rng(23)
    B, Hq, Hkv, N, d = 2, 4, 2, 40, 8
    q = rng.standard_normal((B, Hq, N, d))
    k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d))
    sl = np.array([40, 17])
    o, lse = oracle.attention(q, k, v, scale=0.3, causal=True, window=9,
                              seqlens=sl)
    picks = [(0, 0, 0), (1, 3, 16), (1, 2, 30), (0, 1, 39)]
    orow, lrow = oracle.attention_rows(q, k, v, picks, scale=0.3,
                                       causal=True, window=9, seqlens=sl)
    for n, (b, h, i) in enumerate(picks):
        np.testing.assert_allclose(orow[n], o[b, h, i], rtol=1e-14,
                                   atol=1e-15)
        assert lrow[n] == lse[b, h, i] or (np.isneginf(lrow[n])
                                           and np.isneginf(lse[b, h, i]))


def test_padding_contents_never_read():
    """NaN in padded K/V rows and padded query rows leaves every output equal
    to the run with ordinary numbers there."""
    import synth
    w = synth.Workload("t", B=3, Hq=4, Hkv=2, Nq=33, Nk=33, d=8,
                       dtype="fp32", causal=True, len_lo=1, len_hi=33)
    a = synth.make_inputs(w, 5, pad_fill="draw")
    b = synth.make_inputs(w, 5, pad_fill="nan")
    assert np.isnan(b["k32"]).any()
    oa, la = oracle.attention(a["q32"], a["k32"], a["v32"], scale=w.scale,
                              causal=True, seqlens=a["seqlens"])
    ob, lb = oracle.attention(b["q32"], b["k32"], b["v32"], scale=w.scale,
                              causal=True, seqlens=b["seqlens"])
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)


@pytest.mark.parametrize("check", obc.BWD_CHECKS, ids=lambda c: c.__name__)
def test_backward_oracle_pin(check):
    check(oracle.attention_backward)


@pytest.mark.parametrize("check", ofc.FP8_CHECKS, ids=lambda c: c.__name__)
def test_fp8_oracle_pin(check):
    check(oracle.fp8)
