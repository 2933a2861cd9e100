"""fp64 model of the chunked (WY / UT-transform) form of the gated delta rule.

Test helper only.  It checks, on the CPU, the algebra that the chunked
prefill kernel implements: within a chunk of n tokens starting from state S,

    g_r   = sum_{s<=r} log alpha_s           (per key channel)
    Kt_r  = k_r * exp(g_r)      Kh_i = k_i * exp(-g_i)      Qt_r = q_r * exp(g_r)
    A     = strictly-lower( Diag(beta) Kt Kh^T )
    Tm    = (I + A)^{-1} Diag(beta)          (forward substitution)
    W     = Tm Kt,   U = Tm V,   E = U - W S  (E's row r is beta_r (v_r - S_{r-1}^T (alpha_r k_r)))
    P     = lower-including-diagonal( Qt Kh^T )
    O     = scale (Qt S + P E)
    Kb_i  = k_i * exp(g_n - g_i)
    S'    = Diag(exp(g_n)) S + Kb^T E

which equals n single-token steps of the recurrence up to rounding.

``run_guarded`` models, in a chosen float type, the variant the prefill kernel
runs: the first token's decay is applied to the state up front (so the
cumulative products exclude it and a one-token chunk divides by nothing),
and a chunk is cut short before the first token whose product drops below a
floor in some channel, the next chunk starting there.  ``run_inclusive``
models the earlier kernel algebra (products from the chunk start, no floor)
to show where it breaks.
"""

from __future__ import annotations

import numpy as np


def chunk_step(S, q, k, v, alpha, beta, scale):
    """One chunk for one (sequence, head): S [dk][dv]; q, k, alpha [n][dk]; v [n][dv]; beta [n]."""
    n = k.shape[0]
    g = np.cumsum(np.log(alpha), axis=0)
    Kt, Kh, Qt = k * np.exp(g), k * np.exp(-g), q * np.exp(g)
    A = np.tril(beta[:, None] * (Kt @ Kh.T), -1)
    Tm = np.zeros((n, n))
    for r in range(n):                       # forward substitution: (I + A) Tm = Diag(beta)
        Tm[r] = -A[r, :r] @ Tm[:r]
        Tm[r, r] += beta[r]
    W, U = Tm @ Kt, Tm @ v
    E = U - W @ S
    P = np.tril(Qt @ Kh.T)
    O = scale * (Qt @ S + P @ E)
    Kb = k * np.exp(g[-1] - g)
    S_new = np.exp(g[-1])[:, None] * S + Kb.T @ E
    return S_new, O


def run(S0, q, k, v, alpha, beta, scale, chunk):
    """Whole sequence for one (sequence, head), chunk by chunk (last chunk may be partial)."""
    S = np.array(S0, dtype=np.float64)
    L = k.shape[0]
    O = np.empty((L, v.shape[1]))
    for c0 in range(0, L, chunk):
        c1 = min(L, c0 + chunk)
        S, O[c0:c1] = chunk_step(S, q[c0:c1], k[c0:c1], v[c0:c1], alpha[c0:c1], beta[c0:c1], scale)
    return S, O


def _chunk_guarded(S, q, k, v, alpha, beta, scale, dt):
    """One chunk with token 0's decay applied to S first; products exclude it."""
    n = k.shape[0]
    one = dt(1.0)
    S = alpha[0][:, None] * S
    a = alpha.copy()
    a[0] = one
    G = np.cumprod(a, axis=0, dtype=dt)
    Kt, Qt = k * G, q * G
    Kh = k / G
    A = np.tril(beta[:, None] * (Kt @ Kh.T), -1)
    Tm = np.zeros((n, n), dt)
    for r in range(n):
        Tm[r] = -A[r, :r] @ Tm[:r]
        Tm[r, r] += beta[r]
    E = Tm @ (v - Kt @ S)
    P = np.tril(Qt @ Kh.T)
    O = dt(scale) * (Qt @ S + P @ E)
    Kb = Kh * G[-1]
    return G[-1][:, None] * S + Kb.T @ E, O


def run_guarded(S0, q, k, v, alpha, beta, scale, chunk, dtype=np.float32, floor=2.0 ** -96):
    """Whole sequence in ``dtype`` with chunks cut where a decay product would drop below ``floor``.

    Returns (state, outputs, chunk lengths used).
    """
    dt = np.dtype(dtype).type
    S = np.asarray(S0, dt)
    q, k, v, alpha, beta = (np.asarray(x, dt) for x in (q, k, v, alpha, beta))
    L = k.shape[0]
    O = np.empty((L, v.shape[1]), dt)
    lengths = []
    t = 0
    while t < L:
        n = min(chunk, L - t)
        a = alpha[t:t + n].copy()
        a[0] = 1.0
        G = np.cumprod(a, axis=0, dtype=dt)
        bad = np.nonzero((G < floor).any(axis=1))[0]
        if bad.size:
            n = int(bad[0])          # >= 1: G_0 = 1
        sl = slice(t, t + n)
        S, O[sl] = _chunk_guarded(S, q[sl], k[sl], v[sl], alpha[sl], beta[sl], scale, dt)
        lengths.append(n)
        t += n
    return S, O, lengths


def run_inclusive(S0, q, k, v, alpha, beta, scale, chunk, dtype=np.float32):
    """The unguarded algebra: products from the chunk start including token 0, Kh = k / G."""
    dt = np.dtype(dtype).type
    S = np.asarray(S0, dt)
    q, k, v, alpha, beta = (np.asarray(x, dt) for x in (q, k, v, alpha, beta))
    L = k.shape[0]
    O = np.empty((L, v.shape[1]), dt)
    with np.errstate(all="ignore"):
        for c0 in range(0, L, chunk):
            sl = slice(c0, min(L, c0 + chunk))
            G = np.cumprod(alpha[sl], axis=0, dtype=dt)
            Kt, Qt, Kh = k[sl] * G, q[sl] * G, k[sl] / G
            n = G.shape[0]
            A = np.tril(beta[sl][:, None] * (Kt @ Kh.T), -1)
            Tm = np.zeros((n, n), dt)
            for r in range(n):
                Tm[r] = -A[r, :r] @ Tm[:r]
                Tm[r, r] += beta[sl][r]
            E = Tm @ (v[sl] - Kt @ S)
            O[sl] = dt(scale) * (Qt @ S + np.tril(Qt @ Kh.T) @ E)
            S = G[-1][:, None] * S + (Kh * G[-1]).T @ E
    return S, O
