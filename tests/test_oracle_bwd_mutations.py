"""CPU-only: the backward oracle's pins are strong enough.  Each test plants
one plausible mistake in the chain rule (a dropped or sign-flipped term, the
wrong operand or axis, a missing scale, a group not summed) and requires that
at least one pin fails."""

import numpy as np
import pytest

import oracle
import oracle.sdpa_bwd as ob
from tests import oracle_bwd_checks as obc


def _drop_rowsum(p, dp):
    return p * dp  # planted: softmax Jacobian without its row-sum term


def _rowsum_sign(p, dp):
    return p * (dp + (p * dp).sum(axis=1, keepdims=True))  # planted: sign


def _rowsum_axis(p, dp):
    return p * (dp - (p * dp).sum(axis=0, keepdims=True))  # planted: axis


def _grads(dv_from_ds=False, dk_from_dp=False, dq_from_v=False,
           dk_unscaled=False, dq_unscaled=False):
    def head_gradients(p, q_rows, k_valid, v_valid, do_rows, scale):
        dp = do_rows @ v_valid.T
        ds = ob.softmax_backward(p, dp)
        dv_part = (ds if dv_from_ds else p).T @ do_rows
        dq_rows = (1.0 if dq_unscaled else scale) * (
            ds @ (v_valid if dq_from_v else k_valid))
        dk_part = (1.0 if dk_unscaled else scale) * (
            (dp if dk_from_dp else ds).T @ q_rows)
        return dq_rows, dk_part, dv_part
    return head_gradients


def _overwrite(total, part):
    return part  # planted: a K/V head keeps only its last query head's share


MUTANTS = {
    "drop_rowsum_term": ("softmax_backward", _drop_rowsum),
    "rowsum_sign": ("softmax_backward", _rowsum_sign),
    "rowsum_over_rows": ("softmax_backward", _rowsum_axis),
    "dv_from_ds": ("head_gradients", _grads(dv_from_ds=True)),
    "dk_from_dp": ("head_gradients", _grads(dk_from_dp=True)),
    "dq_from_v": ("head_gradients", _grads(dq_from_v=True)),
    "dk_unscaled": ("head_gradients", _grads(dk_unscaled=True)),
    "dq_unscaled": ("head_gradients", _grads(dq_unscaled=True)),
    "group_not_summed": ("accumulate", _overwrite),
}


def _run_checks(bwd):
    failed = []
    for check in obc.BWD_CHECKS:
        try:
            check(bwd)
        except AssertionError:
            failed.append(check.__name__)
    return failed


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_backward_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(ob, attr, fn)
    failed = _run_checks(ob.attention_backward)
    assert failed, f"no pin catches the planted mistake {name!r}"


def test_swapped_gradients_are_caught():
    def bwd_swapped(q, k, v, do, **kw):
        dq, dk, dv = oracle.attention_backward(q, k, v, do, **kw)
        return dq, dv, dk  # planted: dK and dV exchanged
    assert _run_checks(bwd_swapped)


def test_real_backward_oracle_passes_all():
    assert _run_checks(oracle.attention_backward) == []
