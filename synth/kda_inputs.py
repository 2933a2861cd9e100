"""Seeded synthetic inputs for the five KDA workloads.

Every tensor is drawn per (sequence b, head h) from its own PCG64 stream keyed
by ``SeedSequence([seed, workload tag, phase, tensor tag, b, h])``.  Because the
streams are independent, any subset of (b, h) pairs can be regenerated on its
own (the oracle does this to check sampled heads of full-size runs), and a
large workload can be generated in parallel worker processes with results that
do not depend on the worker count.

Distributions (the workloads' recipe, stated once here):

* q, k: i.i.d. N(0, 1) per element, then divided by their L2 norm over the key
  channels in fp64 (no epsilon: a Gaussian draw has a non-zero norm), then
  rounded to the storage type.
* v: i.i.d. N(0, 1).
* alpha (per key channel, per token): either sigmoid(x) with x ~ N(3, 1)
  ("sigmoid" gate, the tiny fp32 workload) or exp(-softplus(x)) with
  x ~ N(-4, 1) ("softplus" gate: values near 1, long memory).  Stored as f32.
* beta (per token and head): sigmoid(x), x ~ N(0, 1).  Stored as f32.
* initial state: zero, or i.i.d. N(0, 0.02) (0.02 is the standard deviation).
* accepted draft counts: uniform integers in {0, ..., T}.

Rounding: fp64 -> fp32 is round-to-nearest-even (numpy's cast); fp32 -> bf16
rounds to nearest even on the fp32 bit pattern.  bf16 tensors are returned as
``uint16`` bit patterns.
"""

from __future__ import annotations

import os
from concurrent.futures import ProcessPoolExecutor
from dataclasses import dataclass, field
from multiprocessing import get_context

import numpy as np

# Stream tags: one per tensor kind.
_T_Q, _T_K, _T_V, _T_ALPHA, _T_BETA, _T_S0, _T_ACCEPT = 1, 2, 3, 4, 5, 6, 7


@dataclass(frozen=True)
class ConfigSpec:
    """One synthetic workload: sizes, storage types and distributions."""

    name: str
    tag: int                 # workload tag in every stream key
    B: tuple                 # batch sizes (a sweep when more than one)
    H: int
    dk: int
    dv: int
    in_dtype: str            # storage type of q, k, v: "f32" or "bf16"
    gate: str                # "sigmoid" (x ~ N(3,1)) or "softplus" (x ~ N(-4,1))
    state_init: str          # "zero" or "normal"
    steps: int               # decode steps, verify rounds, or prompt length
    extra: dict = field(default_factory=dict)

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.dk))


CONFIGS = {
    "tiny_decode": ConfigSpec("tiny_decode", 0, (1,), 4, 64, 64, "f32", "sigmoid", "zero", 256),
    "single_stream": ConfigSpec("single_stream", 1, (1,), 32, 128, 128, "bf16", "softplus", "normal", 1024),
    "batched_decode": ConfigSpec("batched_decode", 2, (1, 2, 4, 8, 16, 32, 64), 32, 128, 128, "bf16",
                                 "softplus", "normal", 256),
    "spec_verify": ConfigSpec("spec_verify", 3, (16,), 32, 128, 128, "bf16", "softplus", "normal", 512,
                              {"T": 4}),
    "prefill": ConfigSpec("prefill", 4, (8,), 32, 128, 128, "bf16", "softplus", "normal", 8192,
                          {"chunk": 64, "ckpt_every": 1024, "resume_pos": 4096, "resume_steps": 128}),
}


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32 exactly."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(seed: int, tag: int, phase: int, tensor: int, *idx: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tag, phase, tensor, *idx])))


def _store(x64: np.ndarray, in_dtype: str) -> np.ndarray:
    x32 = x64.astype(np.float32)
    return f32_to_bf16_bits(x32) if in_dtype == "bf16" else x32


def _gate(x: np.ndarray, gate: str) -> np.ndarray:
    if gate == "sigmoid":
        return 1.0 / (1.0 + np.exp(-x))
    if gate == "softplus":
        return np.exp(-np.logaddexp(0.0, x))
    raise ValueError(f"unknown gate {gate!r}")


def _draw_bh(args):
    seed, tag, phase, b, h, n, dk, dv, in_dtype, gate = args
    q = _rng(seed, tag, phase, _T_Q, b, h).standard_normal((n, dk))
    k = _rng(seed, tag, phase, _T_K, b, h).standard_normal((n, dk))
    v = _rng(seed, tag, phase, _T_V, b, h).standard_normal((n, dv))
    mu = 3.0 if gate == "sigmoid" else -4.0
    xa = mu + _rng(seed, tag, phase, _T_ALPHA, b, h).standard_normal((n, dk))
    xb = _rng(seed, tag, phase, _T_BETA, b, h).standard_normal((n,))
    q /= np.sqrt(np.sum(q * q, axis=1, keepdims=True))
    k /= np.sqrt(np.sum(k * k, axis=1, keepdims=True))
    return (b, h, _store(q, in_dtype), _store(k, in_dtype), _store(v, in_dtype),
            _gate(xa, gate).astype(np.float32), (1.0 / (1.0 + np.exp(-xb))).astype(np.float32))


def _draw_raw_bh(args):
    # The same streams as _draw_bh, before any transform: q, k un-normalised,
    # the gate and beta draws as logits.
    seed, tag, phase, b, h, n, dk, dv, in_dtype, gate = args
    q = _rng(seed, tag, phase, _T_Q, b, h).standard_normal((n, dk))
    k = _rng(seed, tag, phase, _T_K, b, h).standard_normal((n, dk))
    v = _rng(seed, tag, phase, _T_V, b, h).standard_normal((n, dv))
    mu = 3.0 if gate == "sigmoid" else -4.0
    xa = mu + _rng(seed, tag, phase, _T_ALPHA, b, h).standard_normal((n, dk))
    xb = _rng(seed, tag, phase, _T_BETA, b, h).standard_normal((n,))
    return (b, h, _store(q, in_dtype), _store(k, in_dtype), _store(v, in_dtype), xa.astype(np.float32),
            xb.astype(np.float32))


def default_workers() -> int:
    """Worker processes for large draws: the host cores available, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def raw_token_inputs(spec: ConfigSpec, B: int, n_tokens: int, *, seqs=None, heads=None, phase: int = 0,
                     seed: int = 0) -> dict:
    """The draws behind ``token_inputs`` before their transforms, same layout:
    q, k (un-normalised Gaussians rounded to the storage type), v, alpha_logit
    (the gate's f32 argument x) and beta_logit (f32 [B][n][H])."""
    return _collect(spec, B, n_tokens, seqs, heads, phase, seed, 1, _draw_raw_bh, ("alpha_logit", "beta_logit"))


def token_inputs(spec: ConfigSpec, B: int, n_tokens: int, *, seqs=None, heads=None, phase: int = 0,
                 seed: int = 0, workers: int | None = None) -> dict:
    """Per-token inputs in the [B][n][H][d] layout.

    ``seqs``/``heads`` select a subset of sequence and head indices (default:
    all of ``range(B)`` and ``range(spec.H)``); the result then has those
    subsets as its B and H axes, with values identical to the same slices of
    the full draw.  ``phase`` separates independent draws of the same workload
    (e.g. the decode tokens that follow a prefill).

    Returns a dict with q, k, v (uint16 bf16 bits or float32), alpha (float32)
    and beta (float32, [B][n][H]).
    """
    return _collect(spec, B, n_tokens, seqs, heads, phase, seed, workers, _draw_bh, ("alpha", "beta"))


def _collect(spec, B, n_tokens, seqs, heads, phase, seed, workers, draw, gate_names) -> dict:
    seqs = list(range(B)) if seqs is None else [int(s) for s in seqs]
    heads = list(range(spec.H)) if heads is None else [int(h) for h in heads]
    dk, dv = spec.dk, spec.dv
    sdt = np.uint16 if spec.in_dtype == "bf16" else np.float32
    nb, nh = len(seqs), len(heads)
    out = {
        "q": np.empty((nb, n_tokens, nh, dk), sdt),
        "k": np.empty((nb, n_tokens, nh, dk), sdt),
        "v": np.empty((nb, n_tokens, nh, dv), sdt),
        gate_names[0]: np.empty((nb, n_tokens, nh, dk), np.float32),
        gate_names[1]: np.empty((nb, n_tokens, nh), np.float32),
    }
    bpos = {b: i for i, b in enumerate(seqs)}
    hpos = {h: i for i, h in enumerate(heads)}
    tasks = [(seed, spec.tag, phase, b, h, n_tokens, dk, dv, spec.in_dtype, spec.gate)
             for b in seqs for h in heads]

    def scatter(res):
        b, h, q, k, v, a, be = res
        i, j = bpos[b], hpos[h]
        out["q"][i, :, j] = q
        out["k"][i, :, j] = k
        out["v"][i, :, j] = v
        out[gate_names[0]][i, :, j] = a
        out[gate_names[1]][i, :, j] = be

    if workers is None:
        big = len(tasks) * n_tokens * (3 * dk + dv) > (32 << 20)
        workers = default_workers() if big else 1
    if workers > 1 and len(tasks) > 1:
        with ProcessPoolExecutor(max_workers=workers, mp_context=get_context("spawn")) as ex:
            for res in ex.map(draw, tasks, chunksize=max(1, len(tasks) // (4 * workers))):
                scatter(res)
    else:
        for t in tasks:
            scatter(draw(t))
    return out


def initial_state(spec: ConfigSpec, B: int, *, seqs=None, heads=None, seed: int = 0) -> np.ndarray:
    """Initial recurrent state, float32 [B][H][dk][dv]: zero or N(0, 0.02) per element."""
    seqs = list(range(B)) if seqs is None else [int(s) for s in seqs]
    heads = list(range(spec.H)) if heads is None else [int(h) for h in heads]
    S = np.zeros((len(seqs), len(heads), spec.dk, spec.dv), np.float32)
    if spec.state_init == "zero":
        return S
    if spec.state_init != "normal":
        raise ValueError(spec.state_init)
    for i, b in enumerate(seqs):
        for j, h in enumerate(heads):
            S[i, j] = (0.02 * _rng(seed, spec.tag, 0, _T_S0, b, h).standard_normal((spec.dk, spec.dv))
                       ).astype(np.float32)
    return S


def accepted_counts(spec: ConfigSpec, B: int, rounds: int, T: int, *, seed: int = 0) -> np.ndarray:
    """Accepted draft-token counts, int32 [rounds][B], uniform in {0, ..., T}."""
    out = np.empty((rounds, B), np.int32)
    for b in range(B):
        out[:, b] = _rng(seed, spec.tag, 0, _T_ACCEPT, b).integers(0, T + 1, size=rounds)
    return out
