"""Pure-Python scalar-loop version of the oracle's token step, for tiny shapes.

TEST INFRASTRUCTURE ONLY (see kda_oracle.py).  It restates the same gated
delta rule element by element with explicit loops and Python floats, so that
an indexing or broadcasting mistake in the vectorized oracle shows up as a
disagreement.  Intended for dk, dv <= 8.
"""

from __future__ import annotations


def step(S, q, k, v, alpha, beta, scale):
    """One token on nested lists: S[i][j] (dk x dv), returns (new S, o)."""
    dk, dv = len(S), len(S[0])
    S1 = [[alpha[i] * S[i][j] for j in range(dv)] for i in range(dk)]
    u = [0.0] * dv
    for j in range(dv):
        acc = 0.0
        for i in range(dk):
            acc += S1[i][j] * k[i]
        u[j] = acc
    St = [[0.0] * dv for _ in range(dk)]
    for i in range(dk):
        for j in range(dv):
            erased = S1[i][j] - (beta * k[i]) * u[j]
            St[i][j] = erased + (beta * k[i]) * v[j]
    o = [0.0] * dv
    for j in range(dv):
        acc = 0.0
        for i in range(dk):
            acc += St[i][j] * q[i]
        o[j] = scale * acc
    return St, o
