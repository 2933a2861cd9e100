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
