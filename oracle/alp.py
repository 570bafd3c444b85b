"""TEST INFRASTRUCTURE ONLY — plain reference of the ALP-style attention
latency predictor.

Only ``tests/`` may import this module; the library never does.

"Revisiting Pipeline Parallelism for LLM Serving" paper notes, §2.3: the
attention time of an iteration is modelled as linear in three features
summed over the batch — new prefill tokens against the existing context
(L_past * L_pre), the new chunk against itself (L_pre^2) and decode requests
reading their context (L_dec) — and the coefficients are adapted online by
recursive least squares (RLS) with a forgetting factor.  The notes' formula
itself is lost in the extracted text; only the feature names survive.

Readings (also in the design notes):

* For the attention kernel alone a constant term stands in for the notes'
  offline token-linear part, and features are scaled to millions (the two
  quadratic terms) and thousands (decode context) of tokens.
* A sequence with q_len > 1 is a prefill chunk (L_pre = q_len, L_past =
  kv_len - q_len); one with q_len == 1 is a decode (L_dec = kv_len).
* RLS starts from theta = 0 and covariance delta * I.  Exponentially weighted
  RLS is an exact recursion for the weighted ridge solution

      theta_n = (sum_i lam^(n-i) x_i x_i' + lam^n / delta I)^-1  sum_i lam^(n-i) x_i y_i

  so that solution, written out, is the reference here (not the recursion).
* Fifth feature (this library's addition, not the notes'): the fill of the
  batch's prefill launch.  The varlen entry sends a sequence to its prefill
  kernel when q_len x (heads / kv_heads) > 32; that kernel runs 256 query
  rows per workgroup — h consecutive heads of one KV group (h = the largest
  of 8, 4, 2, 1 dividing the group) times 256 / h tokens — one workgroup per
  CU on 256 CUs.  With W its workgroups, fill = (ceil(W / 256) * 256 / W - 1)
  x its causal pairs (L_past L_pre + L_pre (L_pre + 1) / 2) / 1e6.
"""
from __future__ import annotations

import numpy as np


CUS, ROWS_PER_WORKGROUP = 256, 256


def prefill_workgroups(q: int, heads: int, kv_heads: int) -> int:
    """Workgroups of one sequence's prefill-path launch (0 when it takes the decode path)."""
    group = heads // kv_heads
    if q < 1 or q * group <= 32:
        return 0
    h = next(h for h in (8, 4, 2, 1) if group % h == 0)
    tokens = ROWS_PER_WORKGROUP // h
    return -(-q // tokens) * (heads // h)


def features(q_lens, kv_lens, heads: int, kv_heads: int) -> list[float]:
    if heads <= 0 or kv_heads <= 0 or heads % kv_heads:
        raise ValueError("heads must be a positive multiple of kv_heads")
    past_pre = pre_sq = dec = fill_pairs = 0.0
    wgs = 0
    for q, kv in zip(q_lens, kv_lens):
        q, kv = int(q), int(kv)
        if q < 0 or kv < q:
            raise ValueError("need kv_len >= q_len >= 0")
        if q == 1:
            dec += kv
        elif q > 1:
            past_pre += (kv - q) * q
            pre_sq += q * q
        w = prefill_workgroups(q, heads, kv_heads)
        if w:
            wgs += w
            fill_pairs += (kv - q) * q + q * (q + 1) / 2
    idle = (-(-wgs // CUS) * CUS) / wgs - 1.0 if wgs else 0.0
    return [1.0, past_pre / 1e6, pre_sq / 1e6, dec / 1e3, idle * fill_pairs / 1e6]


def weighted_ridge(xs, ys, lam: float = 1.0, delta: float = 1e6) -> np.ndarray:
    """theta after n observations of exponentially weighted RLS (closed form, fp64)."""
    xs = np.asarray(xs, dtype=np.float64)
    ys = np.asarray(ys, dtype=np.float64)
    n, f = xs.shape
    w = lam ** np.arange(n - 1, -1, -1, dtype=np.float64)        # lam^(n-i), i = 1..n
    a = (xs * w[:, None]).T @ xs + (lam ** n / delta) * np.eye(f)
    b = (xs * w[:, None]).T @ ys
    return np.linalg.solve(a, b)


def predict(theta, x) -> float:
    return float(np.dot(theta, x))


def mape(pred, meas) -> float:
    pred = np.asarray(pred, dtype=np.float64)
    meas = np.asarray(meas, dtype=np.float64)
    return float(np.mean(np.abs(pred - meas) / np.abs(meas)))
