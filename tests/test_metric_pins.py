"""Pins of the acceptance metric itself: normalised error = max |dW - dW_ref| / den.

The weight-gradient parity tests all decide pass or fail through
``oracle.normalised_error`` and the denominator ``WgradAccumulator.den``
(the largest sum of |dY|*|X| over one dW element).  Both are pinned here on
hand-worked values, and planted mistakes in copies of their source (the
absolute value dropped, a sum or mean instead of a max, NaN passed through, a
zero denominator read as a pass) must each fail a pin.  CPU only.
"""
from __future__ import annotations

import inspect
import textwrap

import numpy as np
import pytest

import oracle


def pin_metric_hand_values(fn):
    # diffs 0, -0.5, +1.0 -> max |diff| = 1.0; den 4 -> 0.25
    assert fn([1.0, 2.0, 3.0], np.array([1.0, 2.5, 2.0]), 4.0) == 0.25
    # the largest deviation is negative: |-3| = 3 -> 1.5
    assert fn([0.0, -3.0, 1.0], np.array([0.0, 0.0, 0.0]), 2.0) == 1.5
    # several elements off: the max, not the sum or the mean, of |diff|
    assert fn([1.0, 1.0, 1.0, 1.0], np.zeros(4), 8.0) == 0.125
    # 2-D arrays (the [K, R, S, Cg] results are compared flat)
    got = fn(np.array([[1.0, -2.0], [0.5, 4.0]]), np.array([[1.0, -1.0], [0.0, 4.0]]), 0.5)
    assert got == 2.0, got


def pin_metric_exact_match(fn):
    ref = np.array([3.0, -7.0, 0.0])
    assert fn(ref.copy(), ref, 10.0) == 0.0
    assert fn(np.array([], np.float64), np.array([], np.float64), 1.0) == 0.0


def pin_metric_non_finite(fn):
    ref = np.zeros(3)
    for bad in (np.nan, np.inf, -np.inf):
        t = np.array([0.0, bad, 0.0])
        assert fn(t, ref, 1.0) == float("inf"), bad


def pin_metric_zero_denominator(fn):
    # den = 0 happens only when every |dY||X| sum is zero, i.e. dW_ref is all zero
    assert fn(np.zeros(3), np.zeros(3), 0.0) == 0.0
    assert fn(np.array([0.0, 1e-30, 0.0]), np.zeros(3), 0.0) == float("inf")


def pin_metric_float32_input(fn):
    # GPU results arrive as float32: the difference is taken in float64
    t = np.array([1.0 + 2.0 ** -20], np.float32)
    got = fn(t, np.array([1.0]), 1.0)
    assert got == 2.0 ** -20, got


def pin_denominator_is_max(acc_cls):
    """den = max over dW elements of sum |dY||X|, on a 1x1 case worked by hand.

    X [1,1,2,2]: pixel 0 holds channels (1, -2), pixel 1 (3, -4); dY [1,1,2,1]
    = (1, -1).  dW = (1 - 3, -2 + 4) = (-2, 2); sum |dY||X| is 1 + 3 = 4 for
    c0 and 2 + 4 = 6 for c1 -> den 6 (the sum over elements would be 10, the
    mean 5, the largest |dW| 2)."""
    x = np.array([[[[1.0, -2.0], [3.0, -4.0]]]], np.float32)
    dy = np.array([[[[1.0], [-1.0]]]], np.float32)
    acc = acc_cls(2, 1, 2, 1, 1, 1, nthreads=1)
    acc.add(x, dy)
    assert acc.den == 6.0, acc.den
    assert np.array_equal(acc.dw[:, 0, 0, :], [[-2.0, 2.0]]), acc.dw


METRIC_PINS = [pin_metric_hand_values, pin_metric_exact_match, pin_metric_non_finite,
               pin_metric_zero_denominator, pin_metric_float32_input]


@pytest.mark.parametrize("pin", METRIC_PINS, ids=lambda f: f.__name__)
def test_metric_pin(pin):
    pin(oracle.normalised_error)


def test_denominator_pin():
    pin_denominator_is_max(oracle.WgradAccumulator)


def _mutated_function(obj, old, new):
    """Compile a copy of obj's source with one textual edit (the edit must hit once)."""
    src = textwrap.dedent(inspect.getsource(obj))
    assert src.count(old) == 1, (obj, old)
    ns = {"np": np, "oracle": oracle, "float": float}
    ns.update(vars(oracle))
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    return ns[obj.__name__]


METRIC_MUTANTS = {
    "abs_dropped": ("np.max(np.abs(dw_test - dw_ref))", "np.max(dw_test - dw_ref)"),
    "sum_of_diffs": ("np.max(np.abs(dw_test - dw_ref))", "np.sum(np.abs(dw_test - dw_ref))"),
    "mean_of_diffs": ("np.max(np.abs(dw_test - dw_ref))", "np.mean(np.abs(dw_test - dw_ref))"),
    "nan_passes": ("if not np.all(np.isfinite(dw_test)):", "if False:"),
    "zero_den_passes": ('return 0.0 if diff == 0.0 else float("inf")', "return 0.0"),
    "float16_diff": ("dw_test = np.asarray(dw_test, dtype=np.float64)",
                     "dw_test = np.asarray(dw_test, dtype=np.float16)"),
    "multiplied_by_den": ("return diff / den", "return diff * den"),
}


@pytest.mark.parametrize("name", sorted(METRIC_MUTANTS))
def test_metric_mutant_is_caught(name):
    old, new = METRIC_MUTANTS[name]
    fn = _mutated_function(oracle.normalised_error, old, new)
    for pin in METRIC_PINS:
        try:
            pin(fn)
        except (AssertionError, ValueError, TypeError):
            return
    pytest.fail("metric mutant %s passed every pin" % name)


DEN_MUTANTS = {
    "sum_not_max": ("float(self._abs.max())", "float(self._abs.sum())"),
    "mean_not_max": ("float(self._abs.max())", "float(self._abs.mean())"),
    "signed_dw_max": ("float(self._abs.max())", "float(np.abs(self._dw).max())"),
}


@pytest.mark.parametrize("name", sorted(DEN_MUTANTS))
def test_denominator_mutant_is_caught(name):
    old, new = DEN_MUTANTS[name]
    src = textwrap.dedent(inspect.getsource(oracle.WgradAccumulator))
    assert src.count(old) == 1
    ns = dict(vars(oracle))
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    with pytest.raises(AssertionError):
        pin_denominator_is_max(ns["WgradAccumulator"])
