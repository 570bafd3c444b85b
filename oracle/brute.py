"""TEST INFRASTRUCTURE ONLY — pure-Python brute force for tiny inputs.

An independent restatement of the attention definition (VPP technical
review, English edition, §2.2 Eq. (1) with its causal rule, and §2.3 for the
chunk offset) in plain Python floats with exactly-rounded sums
(``math.fsum``).  It exists only to pin the C oracle on tiny shapes; it is
far too slow for anything else.  Arrays are nested lists or numpy arrays of
Python-convertible numbers: ``q[i][h][e]``, ``k[j][g][e]``, ``v[j][g][e]``.
"""
import math


def attend(q, k, v, past_len, scale, group):
    """Return out[i][h][e] and lse[h][i] for every row of one chunk."""
    c = len(q)
    hq = len(q[0])
    dv = len(v[0][0])
    out = [[None] * hq for _ in range(c)]
    lse = [[None] * c for _ in range(hq)]
    for i in range(c):
        pos = past_len + i
        for h in range(hq):
            g = h // group
            logits = []
            for j in range(pos + 1):
                logits.append(scale * math.fsum(float(a) * float(b) for a, b in zip(q[i][h], k[j][g])))
            top = max(logits)
            weights = [math.exp(s - top) for s in logits]
            total = math.fsum(weights)
            out[i][h] = [math.fsum(w * float(v[j][g][e]) for j, w in enumerate(weights)) / total
                         for e in range(dv)]
            lse[h][i] = top + math.log(total)
    return out, lse
