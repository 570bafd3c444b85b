"""Pins of the ALP predictor oracle (oracle/alp.py).

Features checked on hand-computed batches; the weighted ridge solution
checked against noise-free recovery, numpy's least squares (the lam = 1,
delta -> infinity special case) and hand-solved one- and two-observation
examples, including one that fixes the forgetting weights.
"""
import numpy as np
import pytest

from oracle import alp as A


def test_features_by_hand():
    # one 16384-token chunk after 49152 cached tokens
    assert A.features([16384], [65536]) == [1.0, 49152 * 16384 / 1e6, 16384 ** 2 / 1e6, 0.0]
    # two decodes (contexts 5000 and 20000) and an empty sequence
    assert A.features([1, 1, 0], [5000, 20000, 7]) == [1.0, 0.0, 0.0, 25.0]
    # a prefill from scratch has no past term
    assert A.features([3], [3]) == [1.0, 0.0, 9e-6, 0.0]
    with pytest.raises(ValueError):
        A.features([5], [4])


def test_noise_free_recovery():
    rng = np.random.default_rng(1)
    theta = np.array([0.05, 0.9, 0.45, 0.002])
    xs = np.column_stack([np.ones(40), rng.uniform(0, 2000, 40), rng.uniform(0, 300, 40), rng.uniform(0, 5000, 40)])
    for lam in (1.0, 0.98, 0.9):
        got = A.weighted_ridge(xs, xs @ theta, lam, 1e14)
        assert np.allclose(got, theta, rtol=1e-7, atol=1e-9)


def test_equals_least_squares_without_forgetting():
    rng = np.random.default_rng(2)
    xs = np.column_stack([np.ones(60), rng.uniform(0, 50, 60), rng.uniform(0, 9, 60), rng.uniform(0, 30, 60)])
    ys = xs @ np.array([0.3, 0.02, 0.5, 0.01]) * rng.uniform(0.9, 1.1, 60)
    ref, *_ = np.linalg.lstsq(xs, ys, rcond=None)
    assert np.allclose(A.weighted_ridge(xs, ys, 1.0, 1e14), ref, rtol=1e-7, atol=1e-10)


def test_hand_solved_examples():
    x = [[1.0, 0.0, 0.0, 0.0]]
    # one observation y = 2 with P0 = delta I: theta0 = y / (1 + 1/delta)
    assert A.weighted_ridge(x, [2.0], 1.0, 1.0)[0] == pytest.approx(1.0)
    assert A.weighted_ridge(x, [2.0], 1.0, 3.0)[0] == pytest.approx(1.5)
    # with forgetting the prior decays too: theta0 = 2 / (1 + 0.5 / 1)
    assert A.weighted_ridge(x, [2.0], 0.5, 1.0)[0] == pytest.approx(4.0 / 3.0)
    # two observations of the constant, y = 1 then 3, lam = 0.5, delta = inf:
    # weights 0.5 (older) and 1 -> (0.5 * 1 + 3) / 1.5
    assert A.weighted_ridge(x * 2, [1.0, 3.0], 0.5, 1e15)[0] == pytest.approx(3.5 / 1.5)


def test_forgetting_tracks_a_change():
    rng = np.random.default_rng(3)
    xs = np.column_stack([np.ones(80), rng.uniform(0, 10, 80), np.zeros(80), np.zeros(80)])
    ys = np.where(np.arange(80) < 40, xs @ [1.0, 1.0, 0, 0], xs @ [1.0, 2.0, 0, 0])
    slow = A.weighted_ridge(xs, ys, 1.0, 1e9)[1]
    fast = A.weighted_ridge(xs, ys, 0.8, 1e9)[1]
    assert abs(fast - 2.0) < 1e-2 and abs(slow - 2.0) > 0.2


def test_mape():
    assert A.mape([1.1, 0.9], [1.0, 1.0]) == pytest.approx(0.1)
