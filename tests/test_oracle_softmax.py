"""Pins of oracle.softmax (the processed distributions softmax(logits / T))
against closed forms and exact special cases, not against itself."""
import math

import numpy as np
import pytest

from oracle.softmax import softmax_rows


def test_two_logits_follow_the_logistic_function():
    # softmax of (a, b) at T is (1 / (1 + e^((b-a)/T)), 1 / (1 + e^((a-b)/T)))
    rng = np.random.default_rng(5)
    for _ in range(20):
        a, b = (float(np.float32(v)) for v in rng.normal(0, 4, size=2))
        T = float(rng.choice([0.3, 0.7, 1.0, 2.5]))
        p = softmax_rows(np.array([[a, b]], dtype=np.float32), T)[0]
        assert p[0] == pytest.approx(1.0 / (1.0 + math.exp((b - a) / T)), rel=1e-14)
        assert p[1] == pytest.approx(1.0 / (1.0 + math.exp((a - b) / T)), rel=1e-14)


def test_ratios_are_exponentials_of_logit_differences():
    rng = np.random.default_rng(6)
    x = rng.normal(0, 3, size=(3, 257)).astype(np.float32)
    T = 0.7
    p = softmax_rows(x, T)
    xd = x.astype(np.float64)
    for r in range(3):
        i, j = rng.integers(0, 257, size=2)
        assert p[r, i] / p[r, j] == pytest.approx(math.exp((xd[r, i] - xd[r, j]) / T), rel=1e-12)


def test_hand_worked_row():
    # logits (0, ln 2, ln 3) at T = 1: weights 1 : 2 : 3 (up to the fp32
    # rounding of ln 2 and ln 3, a relative 1e-7)
    x = np.array([[0.0, math.log(2.0), math.log(3.0)]], dtype=np.float32)
    p = softmax_rows(x, 1.0)[0]
    np.testing.assert_allclose(p, [1 / 6, 2 / 6, 3 / 6], rtol=1e-7)
    # the same row at T = 0.5 squares the weights: 1 : 4 : 9
    np.testing.assert_allclose(softmax_rows(x, 0.5)[0], [1 / 14, 4 / 14, 9 / 14], rtol=2e-7)


def test_uniform_row_is_one_over_V():
    for V in (1, 7, 1000):
        p = softmax_rows(np.full((2, V), 3.25, dtype=np.float32), 0.9)
        np.testing.assert_allclose(p, 1.0 / V, rtol=1e-15)


def test_shift_invariance_and_temperature_scaling():
    rng = np.random.default_rng(7)
    # logits on a 2^-16 grid within (-64, 64), so that adding 64 is exact in fp32
    x = (np.round(np.clip(rng.normal(0, 3, size=(4, 300)), -63, 63) * 65536) / 65536).astype(np.float32)
    base = softmax_rows(x, 1.0)
    xs = x + np.float32(64.0)
    assert np.array_equal(xs.astype(np.float64) - 64.0, x.astype(np.float64))
    np.testing.assert_allclose(softmax_rows(xs, 1.0), base, rtol=1e-12)
    # scaling the logits by 2 (exact in fp32) equals halving the temperature
    np.testing.assert_allclose(softmax_rows(x * np.float32(2.0), 1.0), softmax_rows(x, 0.5), rtol=1e-12)


def test_large_logits_do_not_overflow():
    # without the max subtraction exp(1000) overflows
    x = np.array([[1000.0, 999.0, 998.0]], dtype=np.float32)
    p = softmax_rows(x, 1.0)[0]
    w = np.exp([0.0, -1.0, -2.0])
    np.testing.assert_allclose(p, w / w.sum(), rtol=1e-14)


def test_masked_entries_get_zero_and_the_rest_renormalise():
    rng = np.random.default_rng(8)
    x = rng.normal(0, 3, size=(1, 50)).astype(np.float32)
    keep = rng.random(50) < 0.6
    xm = np.where(keep, x, -np.inf).astype(np.float32)
    p = softmax_rows(xm, 0.8)[0]
    assert (p[~keep] == 0.0).all()
    np.testing.assert_allclose(p[keep], softmax_rows(x[:, keep], 0.8)[0], rtol=1e-14)


def test_rows_are_independent_and_sum_to_one():
    rng = np.random.default_rng(9)
    x = rng.normal(0, 3, size=(2, 3, 4096)).astype(np.float32)
    p = softmax_rows(x, 0.7)
    assert p.shape == x.shape
    np.testing.assert_allclose(p.sum(axis=-1), 1.0, rtol=1e-13)
    np.testing.assert_allclose(p[1, 2], softmax_rows(x[1, 2][None], 0.7)[0], rtol=1e-15)
    assert (p > 0).all()


def test_processed_rows_of_the_workloads_are_this_function_rounded_to_fp32():
    import workloads
    rng = np.random.default_rng(10)
    x = rng.normal(0, 3, size=(3, 5000)).astype(np.float32)
    np.testing.assert_array_equal(workloads.softmax_rows(x, 0.7), softmax_rows(x, 0.7).astype(np.float32))


def test_rejects_bad_input():
    x = np.zeros((1, 4), dtype=np.float32)
    for T in (0.0, -1.0, float("inf"), float("nan")):
        with pytest.raises(ValueError):
            softmax_rows(x, T)
    with pytest.raises(ValueError):
        softmax_rows(np.full((1, 4), -np.inf, dtype=np.float32))
    with pytest.raises(ValueError):
        softmax_rows(np.array([[0.0, np.nan]], dtype=np.float32))
