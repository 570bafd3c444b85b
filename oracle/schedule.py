"""TEST INFRASTRUCTURE ONLY — plain reference of the two-rank pipeline schedules
that chunked prefill feeds (CPP, VPP's V-shaped fold-back, VPP-Async) and of
the drain-window packing rule.

Only ``tests/`` may import this module; the library never does.

What is computed follows the VPP technical review (English edition):

* §4.1, Eq. (2): with attention dominating, the per-stage latency of chunk k
  grows linearly, ``tau_k = (k + 1) t``.
* §4.2, Alg. 1 and Eq. (3a)/(3b): two physical ranks, four virtual stages.
  The V-shaped layout puts s0 and s3 on pp0 and s1, s2 on pp1; a chunk runs
  s0 (pp0) -> s1, s2 (pp1) -> s3 (pp0).  While pp1 runs chunk k's middle
  stages, pp0 runs s3 of chunk k-1 and s0 of chunk k+1 (in that order).
* §4.4 (VPP-Async): pp0 issues those two the other way round, s0 of chunk
  k+1 first, so its hand-off to pp1 overlaps pp0's own compute.
* §2.4 / §4.2 (conventional layout, "CPP"): stage i on rank i // 2, so pp0
  runs s0, s1 and pp1 runs s2, s3 of every chunk, one chunk after another.
* §4.5, Alg. 2 and Eq. (4a): the drain window of a request of N chunks is
  estimated as (N + 1) t, and the next request's leading chunks are packed
  into it greedily, cheapest (earliest) first.

Readings where the pages leave a step open (each is listed in the design
notes):

* Every virtual stage of a chunk takes that chunk's tau (the pages split the
  layers evenly and write the per-stage latency as tau_k).
* A hand-off between ranks delays the receiving stage by ``comm`` and does
  not occupy either rank (a data-flow latency); consecutive stages on one
  rank hand off for free (the fold point).
* Without packing, the first stage of a request waits for the last stage of
  the previous request; with packing it does not.
* Alg. 2's loop is read as in its worked example (4a): chunk j of the next
  request is packed when its tau fits in what is left of the window, and
  packing stops at the first chunk that does not fit.  "Scheduling C'_j into
  the idle rank slot freed by the drain" is read as: pp0 runs the entry
  stages of those chunks between the current request's last two exit stages
  (its drain slot while pp1 runs the last chunk's middle stages); t is the
  current request's first tau.  Under CPP, packing simply drops the barrier
  between requests.

Times are plain Python floats (IEEE fp64).
"""
from __future__ import annotations

CPP, VPP, VPP_ASYNC = 0, 1, 2
RANK_OF_STAGE = {CPP: (0, 0, 1, 1), VPP: (0, 1, 1, 0), VPP_ASYNC: (0, 1, 1, 0)}


def tau_linear(n_chunks: int, t: float) -> list[float]:
    """Eq. (2): tau_k = (k + 1) t for k = 0 .. n_chunks - 1."""
    return [(k + 1) * t for k in range(n_chunks)]


def rank_orders(kind: int, n: int) -> list[list[tuple[int, int]]]:
    """The (chunk, stage) sequence each rank executes (Alg. 1 for VPP)."""
    if kind == CPP:
        pp0 = [(k, s) for k in range(n) for s in (0, 1)]
        pp1 = [(k, s) for k in range(n) for s in (2, 3)]
        return [pp0, pp1]
    pp1 = [(k, s) for k in range(n) for s in (1, 2)]
    pp0 = [(0, 0)]
    for k in range(n):                       # pp1 busy with chunk k's middle stages
        tail = [(k - 1, 3)] if k >= 1 else []
        head = [(k + 1, 0)] if k + 1 < n else []
        pp0 += (head + tail) if kind == VPP_ASYNC else (tail + head)
    pp0.append((n - 1, 3))
    return [pp0, pp1]


def multi_orders(kind: int, tau, request, pack: bool) -> list[list[tuple[int, int]]]:
    """Per-rank op sequences for several requests, one after another.

    Without packing, or under CPP, each request keeps its own order.  With
    packing under the V-shaped layouts, Alg. 2 runs at every request boundary:
    the next request's first j entry stages (j from ``drain_pack`` with t the
    current request's first tau) move into pp0's drain slot, just before the
    current request's last exit stage, and are not issued again later.
    """
    groups = []                               # (first chunk, chunk count) per request
    for k, r in enumerate(request):
        if k == 0 or r != request[k - 1]:
            groups.append([k, 0])
        groups[-1][1] += 1
    orders = [[], []]
    moved = set()
    for gi, (k0, n) in enumerate(groups):
        pp0, pp1 = ([(k0 + k, st) for k, st in seq] for seq in rank_orders(kind, n))
        pp0 = [op for op in pp0 if op not in moved]
        if pack and kind != CPP and gi + 1 < len(groups):
            k1, n1 = groups[gi + 1]
            j, _ = drain_pack(n, tau[k0], tau[k1:k1 + n1])
            heads = [(k1 + i, 0) for i in range(j)]
            moved.update(heads)
            pp0 = pp0[:-1] + heads + pp0[-1:]
        orders[0] += pp0
        orders[1] += pp1
    return orders


def simulate(kind: int, tau, comm: float = 0.0, request=None, pack: bool = True) -> dict:
    """Start / end time of every (chunk, stage) and per-rank busy time.

    ``tau[k]`` is chunk k's per-virtual-stage latency; ``request[k]`` (non-
    decreasing) groups chunks into requests for the packing rule.

    With each rank's order fixed, the schedule is a precedence graph: an op
    starts once its rank has finished the op before it, once the chunk's
    previous stage has ended and been handed over, and (without packing) once
    the previous request has ended (each a constraint "start >= end of an
    earlier op + its hand-off delay").  The earliest start of every op is then
    the longest path to it from time 0, computed here in topological order
    (Kahn); a cycle means the orders cannot be run and is reported.
    """
    n = len(tau)
    request = list(request) if request is not None else [0] * n
    ranks = RANK_OF_STAGE[kind]
    last_of, first_of = {}, {}
    for k, r in enumerate(request):
        last_of[r] = k
        first_of.setdefault(r, k)
    orders = multi_orders(kind, tau, request, pack)
    preds = {op: [] for order in orders for op in order}   # op -> [(earlier op, delay after its end)]
    for order in orders:
        for u, v in zip(order, order[1:]):
            preds[v].append((u, 0.0))                       # the rank is busy with u first
    for (k, s) in preds:
        if s > 0:
            hop = comm if ranks[s - 1] != ranks[s] else 0.0
            preds[(k, s)].append(((k, s - 1), hop))
        elif not pack and k == first_of[request[k]] and request[k] != request[0]:
            prev_last = last_of[request[k - 1]]
            preds[(k, s)].append(((prev_last, 3), 0.0))
    succs = {op: [] for op in preds}
    indeg = {op: len(p) for op, p in preds.items()}
    for v, plist in preds.items():
        for u, w in plist:
            succs[u].append((v, w))
    start = {op: 0.0 for op in preds}
    end = {}
    ready = [op for op, d in indeg.items() if d == 0]
    while ready:
        u = ready.pop()
        end[u] = start[u] + tau[u[0]]
        for v, w in succs[u]:
            start[v] = max(start[v], end[u] + w)
            indeg[v] -= 1
            if indeg[v] == 0:
                ready.append(v)
    if len(end) != len(preds):
        raise RuntimeError("schedule deadlocked")
    busy = [0.0, 0.0]
    for (k, s), e in end.items():
        busy[ranks[s]] += e - start[(k, s)]
    makespan = max(end.values()) if end else 0.0
    return {"start": start, "end": end, "busy": busy, "makespan": makespan,
            "idle": [makespan - b for b in busy]}


def drain_window(n_chunks: int, t: float) -> float:
    """Alg. 2: the drain window of a request of n_chunks chunks, (N + 1) t."""
    return (n_chunks + 1) * t


def drain_pack(n_chunks: int, t: float, tau_next) -> tuple[int, float]:
    """Alg. 2 / Eq. (4a): how many leading chunks of the next request fit in the
    drain window, and what is left of it."""
    window = drain_window(n_chunks, t)
    packed = 0
    for tj in tau_next:
        if tj > window:
            break
        window -= tj
        packed += 1
    return packed, window
