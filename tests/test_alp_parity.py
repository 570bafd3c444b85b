"""The library's ALP predictor (host code behind the C ABI: features and the
recursive least-squares update) against the oracle's closed-form weighted
ridge solution (oracle/alp.py), which shares no code with it.

The recursion and the closed form agree up to rounding.  The bar is on
predictions (every observed batch, 1e-9 relative): the coefficients themselves
agree only to ~1e-4 of their scale along the direction the data barely
constrains (mostly the constant term), which moves no prediction.
"""
import numpy as np
import pytest

from chunked_prefill_causal_amd import _lib as L
from oracle import alp as A


def random_batch(rng):
    n = int(rng.integers(1, 6))
    q, kv = [], []
    for _ in range(n):
        kind = rng.integers(0, 3)
        if kind == 0:                                   # decode
            q.append(1); kv.append(int(rng.integers(1, 40000)))
        elif kind == 1:                                 # prefill chunk
            c = int(rng.integers(2, 16385)); q.append(c); kv.append(c + int(rng.integers(0, 114689)))
        else:                                           # empty entry
            q.append(0); kv.append(int(rng.integers(0, 100)))
    return q, kv


def test_features_match():
    rng = np.random.default_rng(4)
    for _ in range(500):
        q, kv = random_batch(rng)
        for heads, kv_heads in ((64, 8), (32, 8), (48, 8), (16, 16)):
            assert list(L.chunkattn_alp_features(q, kv, heads, kv_heads)) == A.features(q, kv, heads, kv_heads)


@pytest.mark.parametrize("lam,delta", [(1.0, 1e6), (0.99, 1e6), (0.9, 1e3), (1.0, 1e2)])
def test_rls_matches_closed_form(lam, delta):
    rng = np.random.default_rng(int(lam * 1000) + int(delta))
    theta_true = np.array([0.08, 0.011, 0.0055, 0.0021, 0.004])
    p = L.AlpPredictor(lam, delta)
    xs, ys = [], []
    for i in range(120):
        q, kv = random_batch(rng)
        x = A.features(q, kv, 64, 8)
        y = float(np.dot(theta_true, x)) * float(rng.uniform(0.95, 1.05))
        before = p.predict(x)
        err = p.update(x, y)
        assert err == pytest.approx(y - before, rel=1e-12, abs=1e-15)
        xs.append(x); ys.append(y)
        if i % 17 == 0 or i == 119:
            ref = A.weighted_ridge(xs, ys, lam, delta)
            pred_ref = np.asarray(xs) @ ref
            pred_lib = np.asarray(xs) @ np.asarray(p.theta)
            assert np.max(np.abs(pred_lib - pred_ref) / np.abs(pred_ref)) < 1e-9, i
            assert np.max(np.abs(np.asarray(p.theta) - ref)) < 1e-3 * np.abs(ref).max(), i
    assert p.state.n_obs == 120


def test_rejections():
    with pytest.raises(L.ChunkAttnError):
        L.chunkattn_alp_features([5], [4], 64, 8)
    with pytest.raises(L.ChunkAttnError):
        L.chunkattn_alp_features([5], [5], 64, 0)
    with pytest.raises(L.ChunkAttnError):
        L.AlpPredictor(1.5, 1e6)
    with pytest.raises(L.ChunkAttnError):
        L.AlpPredictor(1.0, 0.0)
    p = L.AlpPredictor()
    with pytest.raises(L.ChunkAttnError):
        p.update([1.0, np.nan, 0, 0, 0], 1.0)
    assert p.state.n_obs == 0
