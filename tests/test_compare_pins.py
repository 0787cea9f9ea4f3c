"""Pins of the parity metric ``oracle.compare.errors`` (CPU).

Every GPU parity assertion passes through ``errors``, so it is checked here
against values worked out by hand, not against another call of itself:

* max_abs = max |O - O*| over every element (a largest error of either sign),
* rel_l2  = ||O - O*||_F / ||O*||_F, normalised by the reference (O*) side,
* lse_max = max |L - L*| over every row (one bad row is enough).

The tolerance metrics are the ones the parity gate states: maximum absolute
error, relative L2 error over the whole tensor, and the largest logsumexp
error.  Copies of ``errors`` with a planted mistake (no absolute value in the
O or L check, the candidate's norm as the denominator, a mean where a maximum
belongs, a squared ratio, a dropped element) must fail at least one of the
hand-computed cases.
"""

import math

import numpy as np
import pytest

from oracle.compare import errors
from gpu_util import TOL, check

# (o, o_ref, lse, lse_ref, expected errors) -- every figure worked out by hand
CASES = [
    # one positive and one negative error; the negative one is the larger
    (np.array([[1.0, -5.0], [3.0, 0.5]]), np.array([[0.5, -2.0], [3.0, 0.5]]),
     np.array([0.0, 0.0]), np.array([0.0, 0.0]),
     {"max_abs": 3.0, "rel_l2": math.sqrt(0.25 + 9.0) / math.sqrt(0.25 + 4.0 + 9.0 + 0.25), "lse_max": 0.0}),
    # candidate norm far from the reference norm: rel_l2 = 1 / ||O*||
    (np.array([10.0, 0.0, 0.0]), np.array([9.0, 0.0, 0.0]),
     np.array([0.0, 0.0, 0.5, 0.0]), np.array([0.0, 0.0, 0.0, 0.0]),
     {"max_abs": 1.0, "rel_l2": 1.0 / 9.0, "lse_max": 0.5}),
    # lse wrong at one row only, below the reference there
    (np.array([1.0, 2.0]), np.array([1.0, 2.0]),
     np.array([3.0, 2.3, 1.0]), np.array([3.0, 3.0, 1.0]),
     {"max_abs": 0.0, "rel_l2": 0.0, "lse_max": 0.7}),
    # a single bad element among many good ones
    (np.concatenate([np.ones(99), [1.25]]), np.ones(100),
     np.zeros(5), np.zeros(5),
     {"max_abs": 0.25, "rel_l2": 0.25 / 10.0, "lse_max": 0.0}),
]


def _close(a, b):
    return math.isclose(a, b, rel_tol=1e-12, abs_tol=1e-15)


@pytest.mark.parametrize("case", range(len(CASES)))
def test_hand_computed(case):
    o, o_ref, lse, lse_ref, want = CASES[case]
    got = errors(o, o_ref, lse, lse_ref)
    for k, v in want.items():
        assert _close(got[k], v), f"case {case}: {k} = {got[k]}, by hand {v}"


def test_without_lse_reports_output_metrics_only():
    got = errors(np.array([1.0, 3.0]), np.array([1.0, 1.0]))
    assert set(got) == {"max_abs", "rel_l2"}
    assert _close(got["max_abs"], 2.0) and _close(got["rel_l2"], 2.0 / math.sqrt(2.0))


def test_inputs_taken_in_float64():
    # bf16-sized values given as float32 must not be compared in float32
    o = np.array([1.0 + 2.0 ** -30], dtype=np.float64)       # rounds to 1.0 in float32
    got = errors(o, np.array([1.0], dtype=np.float32))
    assert _close(got["max_abs"], 2.0 ** -30)


def test_nan_never_passes():
    # a NaN produced by a kernel must fail the tolerance check, not vanish
    e = errors(np.array([1.0, np.nan]), np.array([1.0, 1.0]), np.array([0.0]), np.array([0.0]))
    with pytest.raises(AssertionError):
        check(e, "bf16", "nan in O")
    e = errors(np.array([1.0]), np.array([1.0]), np.array([np.nan]), np.array([0.0]))
    with pytest.raises(AssertionError):
        check(e, "bf16", "nan in L")


def test_tolerance_check_boundaries():
    tol = TOL["bf16"]
    check(dict(tol), "bf16", "exactly at the limits")
    for k in tol:
        worse = dict(tol)
        worse[k] = tol[k] * (1 + 1e-9)
        with pytest.raises(AssertionError):
            check(worse, "bf16", f"{k} just over")


# ---------------------------------------------------------------- planted mistakes

def _mut_no_abs(o, o_ref, lse=None, lse_ref=None):
    d = np.asarray(o, float) - np.asarray(o_ref, float)
    out = {"max_abs": float(np.max(d)), "rel_l2": float(np.linalg.norm(d) / np.linalg.norm(o_ref))}
    if lse is not None:
        out["lse_max"] = float(np.max(np.asarray(lse, float) - np.asarray(lse_ref, float)))
    return out


def _mut_candidate_norm(o, o_ref, lse=None, lse_ref=None):
    out = errors(o, o_ref, lse, lse_ref)
    d = np.asarray(o, float) - np.asarray(o_ref, float)
    out["rel_l2"] = float(np.linalg.norm(d) / np.linalg.norm(o))
    return out


def _mut_mean_lse(o, o_ref, lse=None, lse_ref=None):
    out = errors(o, o_ref)
    if lse is not None:
        out["lse_max"] = float(np.mean(np.abs(np.asarray(lse, float) - np.asarray(lse_ref, float))))
    return out


def _mut_mean_abs(o, o_ref, lse=None, lse_ref=None):
    out = errors(o, o_ref, lse, lse_ref)
    out["max_abs"] = float(np.mean(np.abs(np.asarray(o, float) - np.asarray(o_ref, float))))
    return out


def _mut_drop_last(o, o_ref, lse=None, lse_ref=None):
    o, o_ref = np.ravel(o)[:-1], np.ravel(o_ref)[:-1]
    return errors(o, o_ref, lse, lse_ref)


def _mut_rel_sq(o, o_ref, lse=None, lse_ref=None):
    out = errors(o, o_ref, lse, lse_ref)
    d = np.asarray(o, float) - np.asarray(o_ref, float)
    out["rel_l2"] = float(np.sum(d * d) / np.sum(np.asarray(o_ref, float) ** 2))
    return out


MUTANTS = [_mut_no_abs, _mut_candidate_norm, _mut_mean_lse, _mut_mean_abs, _mut_drop_last, _mut_rel_sq]


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda f: f.__name__)
def test_planted_mistakes_are_caught(mutant):
    caught = False
    for o, o_ref, lse, lse_ref, want in CASES:
        got = mutant(o, o_ref, lse, lse_ref)
        if any(not _close(got[k], v) for k, v in want.items()):
            caught = True
            break
    assert caught, f"{mutant.__name__} passes every hand-computed case"
