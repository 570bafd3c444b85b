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
    # one 16384-token chunk after 49152 cached tokens, 64 q / 8 KV heads: 16384 / 32 x 8 = 4096 workgroups,
    # exactly 16 rounds of 256, so no fill term
    assert A.features([16384], [65536], 64, 8) == [1.0, 49152 * 16384 / 1e6, 16384 ** 2 / 1e6, 0.0, 0.0]
    # two decodes (contexts 5000 and 20000) and an empty sequence
    assert A.features([1, 1, 0], [5000, 20000, 7], 64, 8) == [1.0, 0.0, 0.0, 25.0, 0.0]
    # a prefill from scratch has no past term; 3 tokens x group 8 = 24 rows per KV head take the decode path
    assert A.features([3], [3], 64, 8) == [1.0, 0.0, 9e-6, 0.0, 0.0]
    # 512 tokens: 16 x 8 = 128 workgroups fill half of one round: idle fraction 1, pairs 1000*512 + 512*513/2
    assert A.features([512], [1512], 64, 8)[4] == (1000 * 512 + 512 * 513 / 2) / 1e6
    # 1056 tokens: 33 x 8 = 264 workgroups, two rounds: idle 512/264 - 1
    assert A.features([1056], [1056], 64, 8)[4] == (512 / 264 - 1) * (1056 * 1057 / 2) / 1e6
    # group 6 (48 q / 8 KV heads): 2 heads per workgroup, 128 tokens: 1000 tokens -> 8 x 24 = 192 workgroups
    assert A.features([1000], [1000], 48, 8)[4] == (256 / 192 - 1) * (1000 * 1001 / 2) / 1e6
    with pytest.raises(ValueError):
        A.features([5], [4], 64, 8)
    with pytest.raises(ValueError):
        A.features([5], [5], 64, 7)


def test_noise_free_recovery():
    rng = np.random.default_rng(1)
    theta = np.array([0.05, 0.9, 0.45, 0.002, 0.3])
    xs = np.column_stack([np.ones(40), rng.uniform(0, 2000, 40), rng.uniform(0, 300, 40), rng.uniform(0, 5000, 40),
                          rng.uniform(0, 50, 40)])
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
