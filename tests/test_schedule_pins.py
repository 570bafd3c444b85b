"""Pins of the schedule oracle (oracle/schedule.py) to the VPP technical review.

The values the pages print for their worked examples (§4.2 Eq. (3b) at k = 3,
the C_0 boundary case, §4.7 Eq. (4a)), the drain window (N + 1) t of §4.5, and
closed forms that follow from the model (makespans, hidden hand-offs), so
that a swapped issue order, a wrong stage-to-rank map, an off-by-one in the
packing rule or a lost hand-off delay each fails at least one test.
"""
import math
import random

import pytest

from oracle import schedule as S


def test_eq3b_worked_example_k3():
    # VPP review §4.2: t = 1, k = 3 -> pp1 spends 2 tau_3 = 8 on C_3's middle
    # stages while pp0 runs s3/C_2 (3) and s0/C_4 (5): 3 + 5 = 8 = 2 * 4.
    r = S.simulate(S.VPP, S.tau_linear(8, 1.0))
    assert (r["start"][(3, 1)], r["end"][(3, 2)]) == (13.0, 21.0)
    assert (r["start"][(2, 3)], r["end"][(2, 3)]) == (13.0, 16.0)
    assert (r["start"][(4, 0)], r["end"][(4, 0)]) == (16.0, 21.0)


def test_c0_boundary_case():
    # While pp1 runs C_0's middle stages (2 tau_0 = 2t), pp0 has only s0/C_1,
    # whose latency tau_1 = 2t fills the window exactly.
    for t in (1.0, 0.25, 3.0):
        r = S.simulate(S.VPP, S.tau_linear(5, t))
        assert (r["start"][(0, 1)], r["end"][(0, 2)]) == (t, 3 * t)
        assert (r["start"][(1, 0)], r["end"][(1, 0)]) == (t, 3 * t)


@pytest.mark.parametrize("kind", [S.VPP, S.VPP_ASYNC])
def test_linear_tau_keeps_pp1_busy(kind):
    # Eq. (3b) holds for any tau_k = a + b k, so after the first step pp1 never
    # waits.  At the C_0 step pp0 runs s0/C_1 (a + b) against pp1's 2a: pp1
    # waits max(0, b - a) once (b = a under Eq. (2), the pages' "coincidence").
    rng = random.Random(3)
    for _ in range(40):
        a, b, n = rng.uniform(0.5, 3), rng.uniform(0, 4), rng.randint(3, 12)
        tau = [a + b * k for k in range(n)]
        r = S.simulate(kind, tau)
        gaps = [r["start"][(k, 1)] - r["end"][(k - 1, 2)] for k in range(1, n)]
        assert gaps[0] == pytest.approx(max(0.0, b - a), abs=1e-9)
        assert max(abs(g) for g in gaps[1:]) < 1e-9


def test_drain_window_is_n_plus_one_t():
    # §4.5: pp0 idles (N + 1) t while pp1 runs the last chunk's middle stages
    # (2 tau_{N-1} - tau_{N-2} = 2Nt - (N-1)t).
    for n, t in ((8, 1.0), (4, 2.5), (16, 0.5)):
        r = S.simulate(S.VPP, S.tau_linear(n, t))
        window = r["end"][(n - 1, 2)] - r["start"][(n - 1, 1)]
        busy = r["end"][(n - 2, 3)] - r["start"][(n - 2, 3)]
        assert r["start"][(n - 2, 3)] == r["start"][(n - 1, 1)]
        assert window - busy == pytest.approx((n + 1) * t)
        assert S.drain_window(n, t) == pytest.approx((n + 1) * t)


def test_eq4a_packing_example():
    # §4.7: N = 8, t = 1 -> window 9; 1 + 2 + 3 = 6 <= 9 packs three chunks and
    # tau'_3 = 4 > 3 left stops the loop.
    assert S.drain_pack(8, 1.0, S.tau_linear(8, 1.0)) == (3, 3.0)


def test_packing_boundary_is_inclusive():
    assert S.drain_pack(2, 1.0, [1.0, 2.0, 0.5]) == (2, 0.0)     # exact fit packs
    assert S.drain_pack(2, 1.0, [4.0, 0.1]) == (0, 3.0)          # first misfit stops


def test_cpp_closed_form():
    # Conventional layout, non-decreasing tau, hand-off delay c: pp1 always
    # waits for pp0, so the span is 2 sum(tau) + c + 2 tau_{N-1}.
    rng = random.Random(5)
    for _ in range(20):
        n = rng.randint(1, 10)
        tau = sorted(rng.uniform(0.1, 5) for _ in range(n))
        c = rng.choice([0.0, rng.uniform(0, 2)])
        r = S.simulate(S.CPP, tau, comm=c)
        assert r["makespan"] == pytest.approx(2 * sum(tau) + c + 2 * tau[-1])
        assert r["busy"] == [pytest.approx(2 * sum(tau))] * 2


def test_vpp_closed_form():
    # V layout, linear tau, no hand-off delay: pp1 runs without a gap from
    # tau_0 on, then pp0's last exit stage: tau_0 + 2 sum(tau) + tau_{N-1}.
    for n, t in ((8, 1.0), (3, 2.0), (12, 0.75)):
        tau = S.tau_linear(n, t)
        for kind in (S.VPP, S.VPP_ASYNC):
            assert S.simulate(kind, tau)["makespan"] == pytest.approx(tau[0] + 2 * sum(tau) + tau[-1])
    # the eight-chunk example: 81 vs 88 under the conventional layout
    assert S.simulate(S.VPP, S.tau_linear(8, 1.0))["makespan"] == 81.0
    assert S.simulate(S.CPP, S.tau_linear(8, 1.0))["makespan"] == 88.0


def test_async_hides_hand_offs():
    # §4.4: issuing s0 of chunk k+1 before s3 of chunk k-1 lets each hand-off
    # to pp1 overlap pp0's compute; with c <= tau_0 only the first hand-off
    # in and the last one out stay exposed.  The synchronous order exposes
    # more of them.
    for n, t, c in ((8, 1.0, 0.5), (6, 2.0, 1.0), (10, 1.0, 1.0)):
        tau = S.tau_linear(n, t)
        base = tau[0] + 2 * sum(tau) + tau[-1]
        assert S.simulate(S.VPP_ASYNC, tau, comm=c)["makespan"] == pytest.approx(base + 2 * c)
        assert S.simulate(S.VPP, tau, comm=c)["makespan"] > base + 2 * c + 1e-9


def test_schedule_invariants():
    rng = random.Random(11)
    for _ in range(60):
        n = rng.randint(1, 9)
        tau = [rng.uniform(0, 4) for _ in range(n)]
        req = sorted(rng.randint(0, 2) for _ in range(n))
        kind, c, pack = rng.choice([S.CPP, S.VPP, S.VPP_ASYNC]), rng.uniform(0, 1), rng.random() < 0.5
        r = S.simulate(kind, tau, comm=c, request=req, pack=pack)
        ranks = S.RANK_OF_STAGE[kind]
        for rank in (0, 1):           # a rank runs one stage at a time
            iv = sorted((r["start"][ks], r["end"][ks]) for ks in r["start"] if ranks[ks[1]] == rank)
            for (a0, a1), (b0, b1) in zip(iv, iv[1:]):
                assert b0 >= a1 - 1e-12
        for k in range(n):            # stages of a chunk in order, hand-offs delayed
            for s in range(1, 4):
                gap = c if ranks[s] != ranks[s - 1] else 0.0
                assert r["start"][(k, s)] >= r["end"][(k, s - 1)] + gap - 1e-12
        assert sum(r["busy"]) == pytest.approx(4 * sum(tau))
        assert r["makespan"] >= max(r["busy"]) - 1e-12


def test_requests_without_packing_run_back_to_back():
    a, b = S.tau_linear(5, 1.0), [0.5, 2.0, 1.0]
    for kind in (S.CPP, S.VPP, S.VPP_ASYNC):
        whole = S.simulate(kind, a + b, request=[0] * 5 + [1] * 3, pack=False)["makespan"]
        assert whole == pytest.approx(S.simulate(kind, a)["makespan"] + S.simulate(kind, b)["makespan"])


def test_packing_fills_the_drain_slot():
    # §4.5: the next request's first j entry stages (Alg. 2) run on pp0 between
    # the current request's last two exit stages, and packing shortens the span.
    n = 8
    tau = S.tau_linear(n, 1.0) * 2
    req = [0] * n + [1] * n
    j, _ = S.drain_pack(n, 1.0, tau[n:])
    for kind in (S.VPP, S.VPP_ASYNC):
        packed = S.simulate(kind, tau, request=req, pack=True)
        plain = S.simulate(kind, tau, request=req, pack=False)
        assert packed["makespan"] < plain["makespan"]
        slot = (packed["end"][(n - 2, 3)], packed["start"][(n - 1, 3)])
        for i in range(j):
            assert slot[0] <= packed["start"][(n + i, 0)] and packed["end"][(n + i, 0)] <= slot[1] + 1e-12
        assert packed["start"][(n + j, 0)] >= packed["end"][(n - 1, 3)]
