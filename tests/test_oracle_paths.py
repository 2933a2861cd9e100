"""Pins for the oracle's verify / commit / snapshot / restore / prefill functions.

These follow the webinar summary "Kimi K3: From Day-0 Availability to
Optimized Inference": rejected draft tokens are handled by logging the
recurrent inputs and replaying the accepted part from the last committed state
(paragraph on speculative decoding with a recurrent state), and the
recurrent-state checkpoint sits at a token boundary (paragraph on prefix
caching).  They also pin the chunked (WY/UT) derivation that the prefill kernel
uses against the token-by-token recurrence.
"""

from __future__ import annotations

import numpy as np
import pytest

import synth
from oracle import kda_oracle as ko
from tests import chunk_form

SPEC = synth.ConfigSpec("t", 90, (3,), 2, 8, 6, "bf16", "softplus", "normal", 0)
SPEC0 = synth.ConfigSpec("t0", 91, (2,), 3, 5, 4, "f32", "sigmoid", "normal", 0)


@pytest.mark.parametrize("spec", [SPEC, SPEC0], ids=["bf16", "f32"])
def test_verify_outputs_equal_sequential_decode(spec):
    B, T = spec.B[0], 5
    S0 = synth.initial_state(spec, B)
    inp = synth.token_inputs(spec, B, T)
    S_dec, o_dec = ko.decode(S0, inp, spec.scale)
    S_before = S0.copy()
    o_ver, log = ko.verify(S0, inp, spec.scale)
    assert np.array_equal(o_ver, o_dec)
    assert np.array_equal(S0, S_before), "verify must not touch the committed state"
    for name in ("k", "v", "alpha", "beta"):
        assert np.array_equal(log[name], inp[name])


def test_commit_replays_accepted_prefix():
    spec = SPEC
    B, T = spec.B[0], 4
    S0 = synth.initial_state(spec, B)
    inp = synth.token_inputs(spec, B, T)
    _, log = ko.verify(S0, inp, spec.scale)
    pos0 = np.array([10, 20, 30], np.int64)
    acc = np.array([0, 2, 4], np.int32)
    S, pos, err = ko.commit(S0, pos0, log, acc)
    assert not err.any()
    assert np.array_equal(pos, pos0 + acc)
    assert np.array_equal(S[0], ko.widen(S0[0])), "a = 0 leaves the state unchanged"
    for b in (1, 2):
        sub = {n: x[b:b + 1, :acc[b]] for n, x in inp.items()}
        S_ref, _ = ko.decode(S0[b:b + 1], sub, spec.scale)
        assert np.array_equal(S[b], S_ref[0]), "commit(a) == a sequential steps"


def test_commit_rejects_out_of_range_count():
    spec = SPEC
    B, T = spec.B[0], 3
    S0 = synth.initial_state(spec, B)
    inp = synth.token_inputs(spec, B, T)
    _, log = ko.verify(S0, inp, spec.scale)
    S, pos, err = ko.commit(S0, np.zeros(B, np.int64), log, np.array([-1, 4, 1], np.int32))
    assert err.tolist() == [True, True, False]
    assert np.array_equal(S[:2], ko.widen(S0[:2])) and pos.tolist() == [0, 0, 1]


def test_varlen_verify_equals_verify_of_each_shorter_draft():
    # Sequence b verifies only its first d_b tokens: its outputs there are those
    # of a verify of exactly those tokens, and nothing is produced after them.
    spec = SPEC
    B, T = spec.B[0], 5
    S0 = synth.initial_state(spec, B)
    inp = synth.token_inputs(spec, B, T)
    d = np.array([0, 5, 2], np.int32)
    o, log = ko.verify(S0, inp, spec.scale, draft_len=d)
    assert log["len"].tolist() == [0, 5, 2] and not log["err"].any()
    for b in range(B):
        if d[b]:
            sub = {n: x[b:b + 1, :d[b]] for n, x in inp.items()}
            o_b, _ = ko.verify(S0[b:b + 1], sub, spec.scale)
            assert np.array_equal(o[b, :d[b]], o_b[0])
        assert np.isnan(o[b, d[b]:]).all()


def test_varlen_commit_is_bounded_by_each_draft_length():
    spec = SPEC
    B, T = spec.B[0], 4
    S0 = synth.initial_state(spec, B)
    inp = synth.token_inputs(spec, B, T)
    _, log = ko.verify(S0, inp, spec.scale, draft_len=np.array([1, 3, 0], np.int32))
    S, pos, err = ko.commit(S0, np.zeros(B, np.int64), log, np.array([2, 3, 1], np.int32))
    assert err.tolist() == [True, False, True]
    assert pos.tolist() == [0, 3, 0]
    assert np.array_equal(S[0], ko.widen(S0[0])) and np.array_equal(S[2], ko.widen(S0[2]))
    sub = {n: x[1:2, :3] for n, x in inp.items()}
    S_ref, _ = ko.decode(S0[1:2], sub, spec.scale)
    assert np.array_equal(S[1], S_ref[0])
    _, pos, err = ko.commit(S0, np.zeros(B, np.int64), log, np.array([1, 0, 0], np.int32))
    assert not err.any() and pos.tolist() == [1, 0, 0]


def test_varlen_verify_rejects_out_of_range_length():
    spec = SPEC
    B, T = spec.B[0], 3
    S0 = synth.initial_state(spec, B)
    inp = synth.token_inputs(spec, B, T)
    o, log = ko.verify(S0, inp, spec.scale, draft_len=np.array([-1, 4, 3], np.int32))
    assert log["err"].tolist() == [True, True, False] and log["len"].tolist() == [0, 0, 3]
    assert np.isnan(o[:2]).all() and not np.isnan(o[2]).any()
    _, _, err = ko.commit(S0, np.zeros(B, np.int64), log, np.array([0, 1, 3], np.int32))
    assert err.tolist() == [False, True, False]


def test_snapshot_restore_roundtrip():
    r = np.random.default_rng(0)
    state = r.standard_normal((4, 2, 3, 5)).astype(np.float32)
    pos = np.array([5, 6, 7, 8], np.int64)
    pool, ppos = np.zeros((6, 2, 3, 5), np.float32), np.full(6, -1, np.int64)
    ko.snapshot(state, pos, [1, 3], [5, 0], pool, ppos)
    assert np.array_equal(pool[5], state[1]) and ppos[5] == 6 and ppos[0] == 8
    live, lpos = np.zeros_like(state), np.zeros(4, np.int64)
    ko.restore(live, lpos, [0, 2], [0, 5], pool, ppos)
    assert np.array_equal(live[0], state[3]) and np.array_equal(live[2], state[1])
    assert lpos.tolist() == [8, 0, 6, 0]


def test_prefill_checkpoints_sit_on_token_boundaries():
    spec = SPEC
    B, L, every = 2, 12, 4
    S0 = synth.initial_state(spec, B)
    inp = synth.token_inputs(spec, B, L)
    S, pos, o, ckpts = ko.prefill(S0, np.array([3, 0], np.int64), inp, spec.scale, every)
    assert len(ckpts) == 3 and pos.tolist() == [15, 12]
    for m, (Sm, pm) in enumerate(ckpts):
        n = (m + 1) * every
        sub = {name: x[:, :n] for name, x in inp.items()}
        S_ref, o_ref = ko.decode(S0, sub, spec.scale)
        assert np.array_equal(Sm, S_ref)
        assert pm.tolist() == [3 + n, n]
        assert np.array_equal(o[:, :n], o_ref)
    # Resume from the middle checkpoint equals continuing the prompt from there.
    rest = {name: x[:, 2 * every:] for name, x in inp.items()}
    S_res, _ = ko.decode(ckpts[1][0], rest, spec.scale)
    assert np.array_equal(S_res, S)


@pytest.mark.parametrize("chunk", [1, 2, 8, 64])
@pytest.mark.parametrize("gate", ["softplus", "sigmoid"])
def test_chunk_form_equals_recurrence(chunk, gate):
    spec = synth.ConfigSpec("c", 92, (1,), 1, 8, 6, "bf16", gate, "normal", 0)
    L = 37
    S0 = synth.initial_state(spec, 1)
    inp = synth.token_inputs(spec, 1, L)
    S_ref, o_ref = ko.decode(S0, inp, spec.scale)
    w = {n: ko.widen(x[0, :, 0]) for n, x in inp.items()}
    S, O = chunk_form.run(ko.widen(S0[0, 0]), w["q"], w["k"], w["v"], w["alpha"], w["beta"], spec.scale, chunk)
    assert np.max(np.abs(S - S_ref[0, 0])) <= 1e-12 * np.max(np.abs(S_ref))
    assert np.max(np.abs(O - o_ref[0, :, 0])) <= 1e-12 * np.max(np.abs(o_ref))


def test_chunk_form_collapses_to_recurrence_at_chunk_one():
    # With one token per chunk A = 0 and Tm = beta: E is the step's e = beta (v - S1^T k).
    r = np.random.default_rng(3)
    S = r.standard_normal((5, 4))
    k = r.standard_normal((1, 5))
    k /= np.linalg.norm(k)
    q, v, a, b = r.standard_normal((1, 5)), r.standard_normal((1, 4)), r.uniform(0.2, 1, (1, 5)), np.array([0.6])
    S_new, O = chunk_form.chunk_step(S, q, k, v, a, b, 0.5)
    S_ref, o_ref = ko.step(S, q[0], k[0], v[0], a[0], b[0], 0.5)
    assert np.allclose(S_new, S_ref, atol=1e-14) and np.allclose(O[0], o_ref, atol=1e-14)


# ---- strongly decaying gates: the guarded chunk form the prefill kernel runs ----

def _gate_case(kind, L, dk, rng):
    if kind == "sigmoid_m1":                      # sigmoid(N(-1, 1)): mean ~0.3, often below 0.1
        return 1.0 / (1.0 + np.exp(-rng.normal(-1.0, 1.0, (L, dk))))
    if kind == "const_0.05":
        return np.full((L, dk), 0.05)
    if kind == "zeros":                           # some channels shut at some tokens, the rest near 1
        a = 1.0 / (1.0 + np.exp(-rng.normal(3.0, 1.0, (L, dk))))
        a[rng.random((L, dk)) < 0.02] = 0.0
        a[:, 3] = 0.0                             # one channel forgets every token
        a[17] = 0.0                               # one token resets every channel
        return a
    if kind == "ones":
        return np.ones((L, dk))
    raise ValueError(kind)


@pytest.mark.parametrize("chunk", [32, 64])
@pytest.mark.parametrize("kind", ["sigmoid_m1", "const_0.05", "zeros", "ones"])
def test_guarded_chunk_form_fp32_matches_oracle_for_any_gate(chunk, kind):
    # The kernel's algebra in fp32 stays finite and within the parity bar for
    # gates anywhere in [0, 1], including exact zeros; the oracle is the
    # plain recurrence.
    rng = np.random.default_rng(11)
    L, dk, dv = 200, 16, 8
    k = rng.standard_normal((L, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    q = rng.standard_normal((L, dk))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    v = rng.standard_normal((L, dv))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal(L)))
    alpha = _gate_case(kind, L, dk, rng).astype(np.float32).astype(np.float64)
    S0 = rng.normal(0.0, 0.02, (dk, dv))
    inp = {"q": q[None, :, None], "k": k[None, :, None], "v": v[None, :, None], "alpha": alpha[None, :, None],
           "beta": beta[None, :, None]}
    S_ref, o_ref = ko.decode(S0[None, None], inp, dk ** -0.5)
    S, O, lengths = chunk_form.run_guarded(S0, q, k, v, alpha, beta, dk ** -0.5, chunk)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(S))
    rms = np.sqrt(np.mean(o_ref ** 2))
    assert np.max(np.abs(O - o_ref[0, :, 0])) <= 2e-3 * rms
    assert np.linalg.norm(S - S_ref[0, 0]) <= 1e-3 * np.linalg.norm(S_ref[0, 0])
    assert sum(lengths) == L and min(lengths) >= 1
    if kind == "ones":
        assert lengths == [min(chunk, L - i) for i in range(0, L, chunk)], "no cut for gates that do not decay"


def test_guarded_chunk_form_cuts_only_where_needed():
    # Gates of the decode workloads (mean ~0.97) never cut a 64-token chunk;
    # a constant 0.05 cuts before the product passes 2^-96 (0.05^22 > 2^-96 > 0.05^23).
    spec = synth.CONFIGS["prefill"]
    a = synth.token_inputs(spec, 1, 4096, heads=[0])["alpha"][0, :, 0].astype(np.float64)
    r = np.random.default_rng(1)
    z = np.zeros((4096, 128))
    _, _, lengths = chunk_form.run_guarded(np.zeros((128, 2)), z, z, np.zeros((4096, 2)), a, np.zeros(4096), 1.0, 64)
    assert set(lengths) == {64}
    c = np.full((100, 4), 0.05)
    _, _, lengths = chunk_form.run_guarded(np.zeros((4, 2)), r.random((100, 4)), r.random((100, 4)),
                                           r.random((100, 2)), c, r.random(100), 1.0, 64)
    assert lengths[:4] == [23, 23, 23, 23]


def test_unguarded_chunk_algebra_breaks_for_strong_decay():
    # The earlier algebra (k / prod alpha from the chunk start) overflows: alpha = 0.05
    # over a 64-token chunk gives 1 / 0.05^63, beyond fp32, and alpha = 0 divides by zero.
    rng = np.random.default_rng(12)
    L, dk, dv = 64, 8, 4
    k = rng.standard_normal((L, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    args = (rng.normal(0, 0.02, (dk, dv)), k, k, rng.standard_normal((L, dv)))
    _, O = chunk_form.run_inclusive(*args, np.full((L, dk), 0.05), np.full(L, 0.5), 0.5, 64)
    assert not np.all(np.isfinite(O))
    _, O, _ = chunk_form.run_guarded(*args, np.full((L, dk), 0.05), np.full(L, 0.5), 0.5, 64)
    assert np.all(np.isfinite(O))
