"""Decode from raw projections (kda_decode_step_prep): the input preparation
(L2 norms of q and k, the decay gate and beta from their logits) runs inside
the decode kernel.

Parity: against the fp64 oracle's preparation followed by its recurrence, at
the tolerance bar, for every shape and both gate forms.  Exact properties:
scaling the raw q or k by a power of two leaves every output and state bit
unchanged (the kernel's norms use IEEE square root and division), saturated
gates (a closed decay gate, beta 0) leave the state unchanged, and a zero key
writes nothing.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import recurrent_state_amd as kda
import synth
from oracle import kda_oracle as ko
from tests.kda_testutil import assert_parity, bits, dev_tensor, say, state_err
from tests.test_gpu_small import SHAPES, spec_for

pytestmark = pytest.mark.gpu

GATES = {"softplus": kda.GATE_EXP_NEG_SOFTPLUS, "sigmoid": kda.GATE_SIGMOID}


def run_prep(S, pos, raw, gate, scale=None):
    """Token-by-token decode_step_prep over raw inputs [B][n][H][d] (host arrays)."""
    B, H, _, dv = S.shape
    n = raw["k"].shape[1]
    d = {name: dev_tensor(np.ascontiguousarray(x)) for name, x in raw.items()}
    outs = []
    for t in range(n):
        o = torch.empty((B, 1, H, dv), dtype=torch.float32, device=S.device)
        kda.decode_step_prep(S, pos, d["q"][:, t:t + 1].contiguous(), d["k"][:, t:t + 1].contiguous(),
                             d["v"][:, t:t + 1].contiguous(), d["alpha_logit"][:, t:t + 1].contiguous(),
                             d["beta_logit"][:, t:t + 1].contiguous(), o, gate=gate, scale=scale)
        outs.append(o)
    if not outs:
        return torch.empty((B, 0, H, dv), dtype=torch.float32, device=S.device)
    return torch.cat(outs, dim=1)


@pytest.mark.parametrize("gate", ["softplus", "sigmoid"])
@pytest.mark.parametrize("dk,dv,dt", SHAPES)
def test_decode_prep_matches_oracle(dk, dv, dt, gate):
    spec = spec_for(dk, dv, dt, gate=gate, tag=130)
    B, n = 3, 40
    say(f"decode_prep dk={dk} dv={dv} {dt} gate={gate}")
    S0 = synth.initial_state(spec, B)
    raw = synth.raw_token_inputs(spec, B, n)
    S = dev_tensor(S0)
    pos = torch.zeros(B, dtype=torch.int64, device="cuda")
    o = run_prep(S, pos, raw, GATES[gate])
    assert kda.last_variant() == "decode_prep"
    S_ref, o_ref = ko.decode(S0, ko.prep(raw, GATES[gate]), spec.scale)
    assert_parity(o.cpu().numpy(), o_ref, S.cpu().numpy(), S_ref, f"decode_prep {dk}x{dv} {dt} {gate}")
    assert pos.cpu().tolist() == [n] * B


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_decode_prep_power_of_two_scaling_is_exact(dt):
    spec = spec_for(128, 128, dt, tag=131)
    B, n = 2, 6
    say(f"decode_prep scaling {dt}")
    S0 = synth.initial_state(spec, B)
    raw = synth.raw_token_inputs(spec, B, n)
    scaled = dict(raw)
    if dt == "bf16":
        # bf16 bit patterns: add to the exponent field (no value here is near under- or overflow).
        scaled["q"] = (raw["q"].astype(np.int32) + (5 << 7)).astype(np.uint16)    # x 2^5
        scaled["k"] = (raw["k"].astype(np.int32) - (3 << 7)).astype(np.uint16)    # x 2^-3
        nz = (raw["q"] & 0x7FFF) != 0
        assert nz.all() and ((raw["k"] & 0x7FFF) != 0).all()
    else:
        scaled["q"] = raw["q"] * np.float32(32.0)
        scaled["k"] = raw["k"] * np.float32(0.125)
    res = []
    for r in (raw, scaled):
        S = dev_tensor(S0)
        pos = torch.zeros(B, dtype=torch.int64, device="cuda")
        o = run_prep(S, pos, r, kda.GATE_EXP_NEG_SOFTPLUS)
        res.append((bits(S).clone(), bits(o).clone()))
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])


def test_decode_prep_saturated_gates_and_zero_vectors():
    spec = spec_for(128, 128, "f32", tag=132)
    B, n = 3, 3
    say("decode_prep edge cases")
    S0 = synth.initial_state(spec, B)
    raw = synth.raw_token_inputs(spec, B, n)
    raw = {k_: v_.copy() for k_, v_ in raw.items()}
    # seq 0, token 0: decay gate fully open (alpha = 1) and beta = 0: the state must not change.
    raw["alpha_logit"][0, 0] = -np.inf
    raw["beta_logit"][0, 0] = -np.inf
    # seq 1, token 1: zero key (no direction, nothing written) and zero query (output 0).
    raw["k"][1, 1] = 0.0
    raw["q"][1, 1] = 0.0
    # seq 2: saturated logits of both signs, large but finite.
    raw["alpha_logit"][2, 0, :, ::2] = 1e4
    raw["alpha_logit"][2, 0, :, 1::2] = -1e4
    raw["beta_logit"][2, 1] = 1e4
    S = dev_tensor(S0)
    pos = torch.zeros(B, dtype=torch.int64, device="cuda")
    d = {name: dev_tensor(np.ascontiguousarray(x)) for name, x in raw.items()}
    o = torch.empty((B, 1, spec.H, 128), dtype=torch.float32, device="cuda")
    tok = lambda t: [d[x][:, t:t + 1].contiguous() for x in ("q", "k", "v", "alpha_logit", "beta_logit")]  # noqa: E731
    kda.decode_step_prep(S, pos, *tok(0), o, gate=kda.GATE_EXP_NEG_SOFTPLUS)
    torch.cuda.synchronize()
    assert torch.equal(S[0], dev_tensor(S0)[0]), "alpha = 1 and beta = 0 must leave the state unchanged"
    S_after0 = S.clone()
    kda.decode_step_prep(S, pos, *tok(1), o, gate=kda.GATE_EXP_NEG_SOFTPLUS)
    # Zero key: only the decay applies (S1 = Diag(alpha) S, computed on the host from the
    # oracle's gate in fp64, rounded once: the kernel forms each product once in fp32).
    alpha1 = ko.decay_gate(raw["alpha_logit"][1, 1].astype(np.float64), ko.GATE_EXP_NEG_SOFTPLUS)
    S1 = S_after0[1].cpu().numpy().astype(np.float64) * alpha1[:, :, None]
    assert np.max(np.abs(S[1].cpu().numpy() - S1)) <= 4e-7 * np.max(np.abs(S1))
    assert torch.count_nonzero(o[1, 0]).item() == 0, "zero query: zero output"
    kda.decode_step_prep(S, pos, *tok(2), o, gate=kda.GATE_EXP_NEG_SOFTPLUS)
    S_ref, o_ref = ko.decode(S0, ko.prep(raw, ko.GATE_EXP_NEG_SOFTPLUS), spec.scale)
    assert_parity(o[:, 0].cpu().numpy(), o_ref[:, 2], S.cpu().numpy(), S_ref, "saturated gates, zero vectors")
    assert pos.cpu().tolist() == [3, 3, 3]


def _raw_dev(raw):
    return {name: dev_tensor(np.ascontiguousarray(x)) for name, x in raw.items()}


@pytest.mark.parametrize("gate", ["softplus", "sigmoid"])
@pytest.mark.parametrize("T", [1, 4, 6])
@pytest.mark.parametrize("dk,dv,dt", [(128, 128, "bf16"), (64, 64, "f32"), (128, 64, "bf16"), (64, 128, "f32")])
def test_verify_prep_matches_oracle_and_commit_equals_decode_prep(dk, dv, dt, T, gate):
    spec = spec_for(dk, dv, dt, gate=gate, tag=133)
    B = 3
    say(f"verify_prep dk={dk} dv={dv} {dt} T={T} gate={gate}")
    S0 = synth.initial_state(spec, B)
    raw = synth.raw_token_inputs(spec, B, T)
    d = _raw_dev(raw)
    S = dev_tensor(S0)
    S_keep = S.clone()
    log = kda.InputLog(S, T_max=8, in_dtype=d["q"].dtype)
    o = torch.empty((B, T, spec.H, dv), dtype=torch.float32, device="cuda")
    kda.verify_prep(S, d["q"], d["k"], d["v"], d["alpha_logit"], d["beta_logit"], o, log, gate=GATES[gate])
    assert kda.last_variant() == "verify_prep" and log.pending_T == T and log.c.pending_form == 1 + GATES[gate]
    assert torch.equal(bits(S), bits(S_keep))
    _, o_ref = ko.decode(S0, ko.prep(raw, GATES[gate]), spec.scale)
    assert_parity(o.cpu().numpy(), o_ref, what=f"verify_prep T={T}")
    # The log keeps the raw inputs.
    es = 2 if dt == "bf16" else 4
    rows = _log_rows_raw(log, B, T, spec.H, dk, dv, es)
    for name, reg in zip(("k", "v", "alpha_logit", "beta_logit"), rows):
        want = d[name].contiguous().view(torch.uint8).view(B, T, spec.H, -1)
        assert torch.equal(reg, want), name
    # Commit: bit-identical to that many decode steps from raw projections.
    acc = [T, 0, min(2, T)]
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    pos = torch.zeros(B, dtype=torch.int64, device="cuda")
    kda.commit(S, pos, log, torch.tensor(acc, dtype=torch.int32, device="cuda"), err)
    torch.cuda.synchronize()
    assert err.item() == 0 and pos.cpu().tolist() == acc
    for b, a in enumerate(acc):
        Sb = S_keep[b:b + 1].clone()
        run_prep(Sb, torch.zeros(1, dtype=torch.int64, device="cuda"),
                 {k_: v_[b:b + 1, :a] for k_, v_ in raw.items()}, GATES[gate])
        assert torch.equal(bits(S[b:b + 1]), bits(Sb)), f"commit({a}) != {a} raw decode steps (seq {b})"


def _log_rows_raw(log, B, T, H, dk, dv, es):
    Tm = log.c.T_max
    r = lambda x: (x + 255) // 256 * 256  # noqa: E731
    tok = B * Tm * H
    offs = [0]
    offs.append(r(offs[0] + tok * dk * es))
    offs.append(r(offs[1] + tok * dv * es))
    offs.append(r(offs[2] + tok * dk * 4))
    out = []
    for off, width in ((offs[0], dk * es), (offs[1], dv * es), (offs[2], dk * 4), (offs[3], 4)):
        out.append(log.buf[off:off + tok * width].view(B, Tm, H, width)[:, :T].clone())
    return out


@pytest.mark.parametrize("T1,T2", [(4, 4), (3, 6)])
def test_commit_verify_prep_equals_separate_calls(T1, T2):
    spec = spec_for(128, 128, "bf16", tag=134)
    B = 3
    say(f"commit_verify_prep T1={T1} T2={T2}")
    S0 = synth.initial_state(spec, B)
    raw = synth.raw_token_inputs(spec, B, T1 + T2)
    d = _raw_dev(raw)
    r1 = {k_: v_[:, :T1].contiguous() for k_, v_ in d.items()}
    r2 = {k_: v_[:, T1:].contiguous() for k_, v_ in d.items()}
    acc = torch.tensor([T1, 0, 1], dtype=torch.int32, device="cuda")
    outs = {}
    for path in ("separate", "fused"):
        S = dev_tensor(S0)
        pos = torch.zeros(B, dtype=torch.int64, device="cuda")
        log = kda.InputLog(S, T_max=8)
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        o1 = torch.empty((B, T1, spec.H, 128), device="cuda")
        o2 = torch.empty((B, T2, spec.H, 128), device="cuda")
        kda.verify_prep(S, r1["q"], r1["k"], r1["v"], r1["alpha_logit"], r1["beta_logit"], o1, log)
        if path == "separate":
            kda.commit(S, pos, log, acc, err)
            kda.verify_prep(S, r2["q"], r2["k"], r2["v"], r2["alpha_logit"], r2["beta_logit"], o2, log)
        else:
            kda.commit_verify_prep(S, pos, r2["q"], r2["k"], r2["v"], r2["alpha_logit"], r2["beta_logit"], o2, log,
                                   acc, err)
            assert kda.last_variant() == "commit_verify_prep"
        S_mid = S.clone()
        kda.commit(S, pos, log, torch.tensor([1, T2, 0], dtype=torch.int32, device="cuda"), err)
        torch.cuda.synchronize()
        assert err.item() == 0
        outs[path] = (bits(S_mid), bits(o2), bits(S), pos.clone())
    for x, y in zip(outs["separate"], outs["fused"]):
        assert torch.equal(x, y)


def test_fused_call_needs_the_pending_form():
    spec = spec_for(128, 128, "bf16", tag=135)
    B, T = 2, 3
    S0 = synth.initial_state(spec, B)
    raw = _raw_dev(synth.raw_token_inputs(spec, B, T))
    S = dev_tensor(S0)
    pos = torch.zeros(B, dtype=torch.int64, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    acc = torch.ones(B, dtype=torch.int32, device="cuda")
    o = torch.empty((B, T, spec.H, 128), device="cuda")
    log = kda.InputLog(S, T_max=T)
    kda.verify_prep(S, raw["q"], raw["k"], raw["v"], raw["alpha_logit"], raw["beta_logit"], o, log)
    with pytest.raises(kda.KdaError):   # a fused call of prepared inputs cannot replay a raw log
        kda.commit_verify(S, pos, raw["q"], raw["k"], raw["v"], raw["alpha_logit"], raw["beta_logit"], o, log,
                          acc, err)
    assert log.pending_T == T
    kda.commit(S, pos, log, acc, err)   # the plain commit replays either form
    torch.cuda.synchronize()
    assert err.item() == 0 and pos.cpu().tolist() == [1, 1]


@pytest.mark.parametrize("gate", ["softplus", "sigmoid"])
@pytest.mark.parametrize("dk,dv,dt", [(128, 128, "bf16"), (64, 64, "f32"), (128, 64, "bf16")])
def test_prefill_recurrent_prep_equals_decode_prep_steps(dk, dv, dt, gate):
    spec = spec_for(dk, dv, dt, gate=gate, tag=136)
    B, L = 2, 37
    say(f"prefill_recurrent_prep dk={dk} dv={dv} {dt} {gate}")
    S0 = synth.initial_state(spec, B)
    raw = synth.raw_token_inputs(spec, B, L)
    d = _raw_dev(raw)
    S = dev_tensor(S0)
    pos = torch.zeros(B, dtype=torch.int64, device="cuda")
    o = torch.empty((B, L, spec.H, dv), device="cuda")
    kda.prefill_recurrent_prep(S, pos, d["q"], d["k"], d["v"], d["alpha_logit"], d["beta_logit"], o,
                               gate=GATES[gate])
    assert kda.last_variant() == "prefill_recurrent_prep"
    S2 = dev_tensor(S0)
    pos2 = torch.zeros(B, dtype=torch.int64, device="cuda")
    o2 = run_prep(S2, pos2, raw, GATES[gate])
    assert torch.equal(bits(S), bits(S2)) and torch.equal(bits(o), bits(o2)) and torch.equal(pos, pos2)


@pytest.mark.parametrize("gate", ["softplus", "sigmoid"])
@pytest.mark.parametrize("chunk,L", [(64, 200), (32, 37), (64, 64)])
@pytest.mark.parametrize("dk,dv,dt", [(128, 128, "bf16"), (64, 64, "f32"), (64, 128, "bf16")])
def test_prefill_chunked_prep_matches_oracle(dk, dv, dt, chunk, L, gate):
    spec = spec_for(dk, dv, dt, gate=gate, tag=137)
    B = 2
    every = chunk
    say(f"prefill_chunked_prep dk={dk} dv={dv} {dt} chunk={chunk} L={L} {gate}")
    S0 = synth.initial_state(spec, B)
    raw = synth.raw_token_inputs(spec, B, L)
    d = _raw_dev(raw)
    S = dev_tensor(S0)
    pos = torch.tensor([5, 0], dtype=torch.int64, device="cuda")
    n_ck = L // every
    pool = kda.SlotPool(2 * n_ck, spec.H, dk, dv, "cuda")
    slots = torch.arange(2 * n_ck, dtype=torch.int32, device="cuda").view(2, n_ck)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    o = torch.full((B, L, spec.H, dv), float("nan"), device="cuda")
    kda.prefill_chunked_prep(S, pos, d["q"], d["k"], d["v"], d["alpha_logit"], d["beta_logit"], o, gate=GATES[gate],
                             chunk=chunk, ckpt_every=every, ckpt_slots=slots, pool=pool, dev_err=err)
    assert kda.last_variant() == "prefill_chunked_prep"
    S_ref, pos_ref, o_ref, ck = ko.prefill(S0, np.array([5, 0]), ko.prep(raw, GATES[gate]), spec.scale, every)
    assert_parity(o.cpu().numpy(), o_ref, S.cpu().numpy(), S_ref, f"prefill_chunked_prep L={L} chunk={chunk}")
    torch.cuda.synchronize()
    assert pos.cpu().tolist() == pos_ref.tolist() and err.item() == 0
    for m, (Sm, pm) in enumerate(ck):
        for b in range(B):
            slot = b * n_ck + m
            assert state_err(pool.states[slot:slot + 1].cpu().numpy(), Sm[b:b + 1]) <= 1e-3
            assert pool.pos[slot].item() == pm[b]
