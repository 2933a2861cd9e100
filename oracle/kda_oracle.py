"""fp64 CPU oracle for the KDA recurrent-state path.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this module.  The HIP library never calls it,
shares no code with it, and must not fall back to it.

What it computes
----------------
"Kimi K3: From Day-0 Availability to Optimized Inference" (nebius webinar
summary, opening paragraph) says Kimi Delta Attention keeps a fixed-size
recurrent state that it updates every token, but the pages never print the
update.  This oracle adopts the per-channel-gated delta rule as the
definition.  Per sequence b and head h the state S is a dk x dv fp32 matrix
(row i = key channel, column j = value channel); a token brings q, k (dk),
v (dv), a per-key-channel gate alpha (dk) and a scalar beta, and the step is,
in this literal order:

    S1 = Diag(alpha) S            decay each key-channel row
    u  = S1^T k                   what the memory currently returns for k
    S2 = S1 - beta k u^T          delta-rule erase
    S  = S2 + beta k v^T          delta-rule write
    o  = scale * S^T q            read after the update

Speculative verify and commit follow the webinar summary's paragraph on
rejected draft tokens: the verify pass records the recurrent inputs of every
draft token and leaves the committed state alone; the commit replays the
accepted prefix from the last committed state.  Snapshot and restore follow
its paragraph on prefix caching: the recurrent-state checkpoint sits at a
token boundary (its position is stored with it).

Everything runs in float64 on exact widenings of the stored inputs (bf16 bit
patterns and f32 values widen exactly).  Arrays use the [B][T][H][d] layout
for per-token inputs and [B][H][dk][dv] for states.

Parity status: every function here is pinned by tests that do not reuse its
formulas (closed forms, invariants, a hand-derived worked example, a
brute-force scalar implementation); see the module docstring of
tests/test_oracle_pins.py.
"""

from __future__ import annotations

import numpy as np


def widen(x) -> np.ndarray:
    """Exact float64 view of a stored input: uint16 arrays are bf16 bit patterns."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def update(S, k, v, alpha, beta):
    """The state part of one token (decay, erase, write), literal order.

    S: [..., dk, dv]; k, alpha: [..., dk]; v: [..., dv]; beta: [...].
    Returns the new state; the argument is not modified.
    """
    S1 = alpha[..., :, None] * S
    u = np.einsum("...ij,...i->...j", S1, k)
    bk = beta[..., None] * k
    S2 = S1 - bk[..., :, None] * u[..., None, :]
    return S2 + bk[..., :, None] * v[..., None, :]


def read(S, q, scale):
    """Output of a token from the already-updated state: scale * S^T q."""
    return scale * np.einsum("...ij,...i->...j", S, q)


def step(S, q, k, v, alpha, beta, scale):
    """One full token: (new state, output)."""
    St = update(S, k, v, alpha, beta)
    return St, read(St, q, scale)


def _token(inp: dict, t: int):
    return (widen(inp["q"][:, t]) if "q" in inp else None, widen(inp["k"][:, t]), widen(inp["v"][:, t]),
            widen(inp["alpha"][:, t]), widen(inp["beta"][:, t]))


def decode(S0, inp: dict, scale: float):
    """Sequential single-token decode over every token of ``inp``.

    S0: [B][H][dk][dv]; inp: q, k, v, alpha [B][n][H][d], beta [B][n][H].
    Returns (final state [B][H][dk][dv] f64, outputs [B][n][H][dv] f64).
    """
    S = widen(S0)
    n = inp["k"].shape[1]
    o = np.empty(S.shape[:2] + (n, S.shape[-1]))
    for t in range(n):
        q, k, v, a, b = _token(inp, t)
        S, o[:, :, t] = step(S, q, k, v, a, b, scale)
    return S, np.ascontiguousarray(o.transpose(0, 2, 1, 3))


def verify(S_c, inp: dict, scale: float, draft_len=None):
    """Speculative verify of draft tokens from the committed state.

    Runs the T tokens from ``S_c`` and returns (outputs [B][T][H][dv], log);
    ``S_c`` is not changed.  The log holds copies of the recurrent inputs the
    commit needs to replay the state (k, v, alpha, beta); q only shapes the
    outputs and is not logged.

    ``draft_len`` (int [B], optional) gives sequence b only its first
    ``draft_len[b]`` tokens (the rest of its T rows are padding): its outputs
    from there on are NaN (not produced), and its logged length
    (``log["len"]``) is that count.  A length outside [0, T] produces nothing,
    logs length 0 and is reported in ``log["err"]``.  Outputs of the tokens a
    sequence does verify are those of the full run, as token t's output depends
    only on tokens up to t.
    """
    _, o = decode(S_c, inp, scale)
    B, T = inp["k"].shape[:2]
    log = {name: np.array(inp[name], copy=True) for name in ("k", "v", "alpha", "beta")}
    if draft_len is None:
        log["len"] = np.full(B, T, np.int64)
        log["err"] = np.zeros(B, bool)
        return o, log
    d = np.asarray(draft_len, dtype=np.int64)
    err = (d < 0) | (d > T)
    d = np.where(err, 0, d)
    for b in range(B):
        o[b, d[b]:] = np.nan
    log["len"], log["err"] = d, err
    return o, log


def commit(S_c, pos, log: dict, accepted):
    """Replay the accepted prefix of a verified draft onto the committed state.

    For each sequence b, applies the first ``accepted[b]`` logged tokens to
    ``S_c[b]`` and advances ``pos[b]`` by that count.  A count outside
    [0, n_b], with n_b the sequence's logged draft length (T when the log has
    none), leaves that sequence's state and position unchanged and is reported
    in the returned error flags.
    Returns (state f64, pos int64, err bool [B]).
    """
    S = widen(S_c).copy()
    pos = np.array(pos, dtype=np.int64, copy=True)
    B, T = log["k"].shape[:2]
    n = np.asarray(log["len"]) if "len" in log else np.full(B, T)
    acc = np.asarray(accepted)
    err = (acc < 0) | (acc > n)
    for b in range(S.shape[0]):
        if err[b]:
            continue
        for t in range(int(acc[b])):
            S[b] = update(S[b], widen(log["k"][b, t]), widen(log["v"][b, t]),
                          widen(log["alpha"][b, t]), widen(log["beta"][b, t]))
        pos[b] += int(acc[b])
    return S, pos, err


def snapshot(state, pos, seq_ids, slot_ids, pool_states, pool_pos):
    """Copy sequence seq_ids[i]'s state (all heads) and position into slot slot_ids[i]."""
    for s, slot in zip(seq_ids, slot_ids):
        pool_states[slot] = state[s]
        pool_pos[slot] = pos[s]


def restore(state, pos, seq_ids, slot_ids, pool_states, pool_pos):
    """Copy slot slot_ids[i]'s state and position back into sequence seq_ids[i]."""
    for s, slot in zip(seq_ids, slot_ids):
        state[s] = pool_states[slot]
        pos[s] = pool_pos[slot]


def prefill(S0, pos0, inp: dict, scale: float, ckpt_every: int = 0):
    """Prompt processing as the plain token-by-token recurrence.

    The chunked form reaches the same result up to rounding, so its oracle is
    the recurrence itself.  After every ``ckpt_every`` tokens (when > 0) the
    state is checkpointed together with its token position.
    Returns (state f64, pos int64, outputs [B][L][H][dv] f64,
    checkpoints: list of (state f64 [B][H][dk][dv], pos int64 [B])).
    """
    S = widen(S0)
    pos0 = np.asarray(pos0, dtype=np.int64)
    L = inp["k"].shape[1]
    o = np.empty(S.shape[:2] + (L, S.shape[-1]))
    ckpts = []
    for t in range(L):
        q, k, v, a, b = _token(inp, t)
        S, o[:, :, t] = step(S, q, k, v, a, b, scale)
        if ckpt_every and (t + 1) % ckpt_every == 0:
            ckpts.append((S.copy(), pos0 + (t + 1)))
    return S, pos0 + L, np.ascontiguousarray(o.transpose(0, 2, 1, 3)), ckpts


# ---------------------------------------------------------------------------
# Input preparation from raw projections.
#
# The webinar summary lists removing needless copies and type conversions
# among its optimisations (paragraph on profiling the token path); fusing the
# preparation of the recurrent inputs into the decode kernel is that step for
# this path.  The pages do not print the preparation itself; it follows the
# input recipe the workloads are defined by: q and k are L2-normalised over the
# key channels, the per-channel decay is either exp(-softplus(x)) or
# sigmoid(x) of its logit x, and beta is sigmoid of its logit.  A zero q or k
# vector (no direction) is taken to normalise to zero.

GATE_EXP_NEG_SOFTPLUS = 0
GATE_SIGMOID = 1


def l2_normalize(x):
    """x / ||x||_2 over the last axis, in float64; a zero vector stays zero."""
    x = np.asarray(x, dtype=np.float64)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return np.divide(x, n, out=np.zeros_like(x), where=n > 0)


def sigmoid(x):
    """1 / (1 + e^-x); saturates to exactly 0 or 1 far out."""
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-np.asarray(x, dtype=np.float64)))


def softplus(x):
    """log(1 + e^x), evaluated without overflow."""
    return np.logaddexp(0.0, np.asarray(x, dtype=np.float64))


def decay_gate(x, kind: int):
    """Per-channel decay from its logit: exp(-softplus(x)) or sigmoid(x)."""
    if kind == GATE_EXP_NEG_SOFTPLUS:
        return np.exp(-softplus(x))
    if kind == GATE_SIGMOID:
        return sigmoid(x)
    raise ValueError(f"unknown gate kind {kind}")


def prep(raw: dict, kind: int) -> dict:
    """Prepared token inputs (float64) from raw ones.

    raw: q, k, v as stored ([..][dk] / [..][dv]), alpha_logit [..][dk] and
    beta_logit [..].  Returns q, k (unit vectors), v, alpha and beta in the
    layouts ``decode`` takes.
    """
    out = {"k": l2_normalize(widen(raw["k"])), "v": widen(raw["v"]),
           "alpha": decay_gate(widen(raw["alpha_logit"]), kind), "beta": sigmoid(widen(raw["beta_logit"]))}
    if "q" in raw:
        out["q"] = l2_normalize(widen(raw["q"]))
    return out
