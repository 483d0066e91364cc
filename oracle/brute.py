"""Pure-Python brute force for tiny attention problems.

TEST INFRASTRUCTURE ONLY (see oracle/sdpa.py).  Written independently of
the numpy oracle: nested Python loops, ``math.fsum`` sums, no max shift, no
matrix library.  It follows the definition directly: the output row is the
expectation of the value rows under the distribution that gives key j the
weight exp(scale*<q_i,k_j>) / sum_j' exp(scale*<q_i,k_j'>).

Only for inputs whose scores stay well inside the float64 exp range.
"""
from __future__ import annotations

import math


def attend(q, k, v, scale, is_causal=False, allowed=None):
    """q: list of nq rows, k/v: lists of nk rows (sequences of floats).
    ``allowed(i, j)``, if given, further restricts which keys row i sees; a
    row that sees no key gets a zero output row and lse = -inf.

    Returns (O as list of rows, lse as list)."""
    out, lse = [], []
    for i, qi in enumerate(q):
        keys = [j for j in range(len(k)) if ((not is_causal) or j <= i)
                and (allowed is None or allowed(i, j))]
        if not keys:
            out.append([0.0] * len(v[0]))
            lse.append(-math.inf)
            continue
        weights = []
        for j in keys:
            dot = math.fsum(float(a) * float(b) for a, b in zip(qi, k[j]))
            weights.append(math.exp(float(scale) * dot))
        z = math.fsum(weights)
        row = []
        for c in range(len(v[0])):
            row.append(math.fsum(w * float(v[j][c]) for w, j in zip(weights, keys)) / z)
        out.append(row)
        lse.append(math.log(z))
    return out, lse
