"""The library's schedule simulator (host code behind the C ABI) against the
plain oracle (oracle/schedule.py), which shares no code with it.

The two compute the timing differently: the library walks the ranks' op
orders as an event loop, the oracle builds the precedence graph (rank order,
stage hand-offs, request barriers) and takes longest paths in topological
order.  Every stage time comes from the same additions (end + hand-off) and
maxima either way, so the comparison is exact; busy times are sums taken in
different orders and are compared to 1e-12 relative.  Host-only calls: no GPU
is involved.
"""
import math
import random

import numpy as np
import pytest

from chunked_prefill_causal_amd import _lib as L
from oracle import schedule as S

KINDS = [(L.CA_SCHED_CPP, S.CPP), (L.CA_SCHED_VPP, S.VPP), (L.CA_SCHED_VPP_ASYNC, S.VPP_ASYNC)]


def compare(kind_lib, kind_orc, tau, comm=0.0, request=None, pack=True):
    got = L.chunkattn_sched_simulate(kind_lib, tau, comm=comm, request=request, pack=pack)
    ref = S.simulate(kind_orc, list(tau), comm=comm, request=request, pack=pack)
    n = len(tau)
    for k in range(n):
        for s in range(4):
            assert got["start"][k, s] == ref["start"][(k, s)], (k, s)
            assert got["end"][k, s] == ref["end"][(k, s)], (k, s)
    assert got["makespan"] == ref["makespan"]
    for rank in (0, 1):
        assert got["busy"][rank] == pytest.approx(ref["busy"][rank], rel=1e-12, abs=1e-12)


@pytest.mark.parametrize("kind_lib,kind_orc", KINDS)
def test_random_single_requests(kind_lib, kind_orc):
    rng = random.Random(kind_lib * 100 + 1)
    for _ in range(200):
        n = rng.randint(1, 40)
        shape = rng.choice(["linear", "noisy", "random", "measured"])
        if shape == "linear":
            tau = S.tau_linear(n, rng.uniform(0.1, 5))
        elif shape == "noisy":
            a, b = rng.uniform(0.5, 4), rng.uniform(0, 8)
            tau = [(a + b * k) * rng.uniform(0.97, 1.03) for k in range(n)]
        elif shape == "measured":    # the 128K prompt's per-chunk kernel times, ms
            tau = [3.709, 10.821, 17.991, 25.16, 32.307, 39.441, 46.551, 53.722][:n] + [60.0] * max(0, n - 8)
        else:
            tau = [rng.uniform(0, 10) for _ in range(n)]
        compare(kind_lib, kind_orc, tau, comm=rng.choice([0.0, rng.uniform(0, 3)]))


@pytest.mark.parametrize("kind_lib,kind_orc", KINDS)
def test_random_request_streams(kind_lib, kind_orc):
    rng = random.Random(kind_lib * 100 + 2)
    for _ in range(150):
        n_req = rng.randint(1, 5)
        tau, req = [], []
        for r in range(n_req):
            n = rng.randint(1, 12)
            t = rng.uniform(0.2, 3)
            tau += [(k + 1) * t * rng.uniform(0.9, 1.1) for k in range(n)]
            req += [r * 3] * n                  # ids need only be non-decreasing
        compare(kind_lib, kind_orc, tau, comm=rng.uniform(0, 1), request=req, pack=rng.random() < 0.5)


def test_edge_cases():
    for kl, ko in KINDS:
        compare(kl, ko, [])
        compare(kl, ko, [2.5])
        compare(kl, ko, [0.0, 0.0, 0.0])
        compare(kl, ko, [1.0, 2.0, 3.0], request=[0, 1, 2], pack=True)
        compare(kl, ko, [1.0, 2.0, 3.0], request=[0, 1, 2], pack=False)
        compare(kl, ko, [5.0, 1.0, 9.0, 0.5], comm=2.0)


def test_drain_pack_matches_oracle():
    rng = random.Random(9)
    assert L.chunkattn_sched_drain_pack(8, 1.0, S.tau_linear(8, 1.0)) == (3, 3.0)
    for _ in range(300):
        n, t = rng.randint(0, 30), rng.uniform(0, 4)
        nxt = [rng.choice([rng.uniform(0, 5), float(rng.randint(0, 5))]) for _ in range(rng.randint(0, 12))]
        j, left = L.chunkattn_sched_drain_pack(n, t, nxt)
        rj, rleft = S.drain_pack(n, t, nxt)
        assert j == rj and left == rleft


def test_rejections():
    lib = L.lib()
    with pytest.raises(L.ChunkAttnError):
        L.chunkattn_sched_simulate(7, [1.0])
    with pytest.raises(L.ChunkAttnError):
        L.chunkattn_sched_simulate(L.CA_SCHED_VPP, [1.0, -2.0])
    with pytest.raises(L.ChunkAttnError):
        L.chunkattn_sched_simulate(L.CA_SCHED_VPP, [1.0, math.inf])
    with pytest.raises(L.ChunkAttnError):
        L.chunkattn_sched_simulate(L.CA_SCHED_VPP, [1.0, 2.0], comm=-1.0)
    with pytest.raises(L.ChunkAttnError):
        L.chunkattn_sched_simulate(L.CA_SCHED_VPP, [1.0, 2.0], request=[1, 0])
    assert lib.chunkattn_sched_simulate(1, 2, None, None, 0.0, 1, None, None, None, None) == L.CA_EINVAL
    with pytest.raises(L.ChunkAttnError):
        L.chunkattn_sched_drain_pack(-1, 1.0, [1.0])
    with pytest.raises(L.ChunkAttnError):
        L.chunkattn_sched_drain_pack(4, 1.0, [np.nan])
    assert lib.chunkattn_last_error().decode()
