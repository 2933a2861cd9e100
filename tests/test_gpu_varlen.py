"""Speculative verify with a draft length per sequence (the _varlen entry points).

Parity: the tokens a sequence verifies match the fp64 oracle at the tolerance
bar.  Bookkeeping, bit for bit: outputs and log rows past a sequence's draft
length are not written, a commit accepts at most the logged length and then
equals that many decode steps, and the fused commit + verify equals the
separate calls.  Lengths outside [0, T] and counts above the logged length
are flagged in the device error word and leave the sequence untouched.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import recurrent_state_amd as kda
import synth
from oracle import kda_oracle as ko
from tests.kda_testutil import assert_parity, bits, dev_inputs, dev_tensor, say, token_slice
from tests.test_gpu_small import SHAPES, _log_rows, decode_run, spec_for

pytestmark = pytest.mark.gpu

SENTINEL = 0x7FC0BEEF  # a NaN bit pattern no kernel produces


def sentinel_like(shape):
    return torch.full(shape, SENTINEL, dtype=torch.int32, device="cuda").view(torch.float32)


def lengths_for(T, B):
    # Full, none, one, one short of full, and a middle length.
    base = [T, 0, 1, max(T - 1, 0), min(3, T)]
    return base[:B]


@pytest.mark.parametrize("dk,dv,dt", SHAPES)
@pytest.mark.parametrize("T", [1, 4, 5, 8])
def test_verify_varlen_matches_oracle_and_bounds_commit(dk, dv, dt, T):
    spec = spec_for(dk, dv, dt, tag=120)
    B = 5
    say(f"verify_varlen dk={dk} dv={dv} {dt} T={T}")
    S0 = synth.initial_state(spec, B)
    inp = synth.token_inputs(spec, B, T)
    d = dev_inputs(inp)
    dl = lengths_for(T, B)
    draft_len = torch.tensor(dl, dtype=torch.int32, device="cuda")
    S = dev_tensor(S0)
    S_keep = S.clone()
    log = kda.InputLog(S, T_max=8, in_dtype=d["q"].dtype)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    o = sentinel_like((B, T, spec.H, dv))
    kda.verify_varlen(S, d["q"], d["k"], d["v"], d["alpha"], d["beta"], o, log, draft_len, err)
    assert kda.last_variant() == "verify_varlen" and log.pending_T == T
    torch.cuda.synchronize()
    assert err.item() == 0
    assert torch.equal(bits(S), bits(S_keep)), "verify must not write the committed state"
    o_ref, log_ref = ko.verify(S0, inp, spec.scale, draft_len=np.array(dl))
    ob = bits(o).cpu()
    for b in range(B):
        if dl[b]:
            assert_parity(o[b, :dl[b]].cpu().numpy(), o_ref[b, :dl[b]], what=f"varlen seq {b} len {dl[b]}")
        assert (ob[b, dl[b]:] == SENTINEL).all(), f"seq {b}: output rows past its draft length were written"
    # Commit: at most the logged length per sequence; seq 2 (length 1) asks for 2.
    acc = [dl[0], 0, 2, dl[3], dl[4]]
    if T == 1:
        acc[0] = 1
    accepted = torch.tensor(acc, dtype=torch.int32, device="cuda")
    pos = torch.tensor([4, 0, 1, 2, 3], dtype=torch.int64, device="cuda")
    kda.commit(S, pos, log, accepted, err)
    torch.cuda.synchronize()
    assert err.item() & kda.DEV_ERR_ACCEPTED
    S_ref, pos_ref, err_ref = ko.commit(S0, [4, 0, 1, 2, 3], log_ref, np.array(acc))
    assert err_ref.tolist() == [False, False, True, False, False]
    assert pos.cpu().tolist() == pos_ref.tolist()
    for b, a in enumerate(acc):
        Sb = S_keep[b:b + 1].clone()
        if not err_ref[b]:
            decode_run(Sb, torch.zeros(1, dtype=torch.int64, device="cuda"), {k_: v_[b:b + 1, :a] for k_, v_ in d.items()})
        assert torch.equal(bits(S[b:b + 1]), bits(Sb)), f"seq {b}: commit({a}) after a length-{dl[b]} draft"


@pytest.mark.parametrize("dk,dv,dt", [(128, 128, "bf16"), (64, 64, "f32"), (128, 64, "bf16")])
@pytest.mark.parametrize("T1,T2", [(4, 4), (7, 3), (2, 8)])
def test_commit_verify_varlen_equals_separate_calls(dk, dv, dt, T1, T2):
    spec = spec_for(dk, dv, dt, tag=121)
    B = 4
    say(f"commit_verify_varlen dk={dk} dv={dv} {dt} T1={T1} T2={T2}")
    S0 = synth.initial_state(spec, B)
    inp = synth.token_inputs(spec, B, T1 + T2)
    d = dev_inputs(inp)
    r1 = {k_: v_.contiguous() for k_, v_ in token_slice(d, 0, T1).items()}
    r2 = {k_: v_.contiguous() for k_, v_ in token_slice(d, T1, T1 + T2).items()}
    dl1 = torch.tensor([T1, 0, 1, T1 - 1], dtype=torch.int32, device="cuda")
    dl2 = torch.tensor([1, T2, 0, T2 - 1], dtype=torch.int32, device="cuda")
    acc1 = torch.tensor([T1, 0, 1, T1 // 2], dtype=torch.int32, device="cuda")
    acc2 = torch.tensor([1, T2, 0, T2 - 1], dtype=torch.int32, device="cuda")
    es = 2 if dt == "bf16" else 4
    outs = {}
    for path in ("separate", "fused"):
        S = dev_tensor(S0)
        pos = torch.tensor([5, 0, 2, 1], dtype=torch.int64, device="cuda")
        log = kda.InputLog(S, T_max=8, in_dtype=d["q"].dtype)
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        o1 = sentinel_like((B, T1, spec.H, dv))
        o2 = sentinel_like((B, T2, spec.H, dv))
        kda.verify_varlen(S, r1["q"], r1["k"], r1["v"], r1["alpha"], r1["beta"], o1, log, dl1, err)
        if path == "separate":
            kda.commit(S, pos, log, acc1, err)
            kda.verify_varlen(S, r2["q"], r2["k"], r2["v"], r2["alpha"], r2["beta"], o2, log, dl2, err)
        else:
            kda.commit_verify_varlen(S, pos, r2["q"], r2["k"], r2["v"], r2["alpha"], r2["beta"], o2, log, dl2,
                                     acc1, err)
            assert kda.last_variant() == "commit_verify_varlen" and log.pending_T == T2
        S_mid = S.clone()
        rows = _log_rows(log, B, T2, spec.H, dk, dv, es)
        kda.commit(S, pos, log, acc2, err)
        torch.cuda.synchronize()
        assert err.item() == 0
        outs[path] = (bits(S_mid), bits(o2), rows, bits(S), pos.clone())
    a, f = outs["separate"], outs["fused"]
    assert torch.equal(a[0], f[0]), "committed state differs"
    assert torch.equal(a[1], f[1]), "verify outputs differ (including the unwritten rows)"
    for b in range(B):
        n = int(dl2[b])
        for x, y in zip(a[2], f[2]):
            assert torch.equal(x[b, :n], y[b, :n]), f"log rows of seq {b} differ"
    assert torch.equal(a[3], f[3]) and torch.equal(a[4], f[4])
    ob = f[1].cpu()
    for b in range(B):
        assert (ob[b, int(dl2[b]):] == SENTINEL).all()
    # Against the oracle: round 2 outputs follow round 1's accepted prefix.
    for b in range(B):
        a1, n2 = int(acc1[b]), int(dl2[b])
        if n2 == 0:
            continue
        tok = {k_: np.concatenate([v_[b:b + 1, :a1], v_[b:b + 1, T1:T1 + n2]], axis=1) for k_, v_ in inp.items()}
        _, o_ref = ko.decode(S0[b:b + 1], tok, spec.scale)
        assert_parity(f[1].view(torch.float32)[b:b + 1, :n2].cpu().numpy(), o_ref[:, a1:], what=f"seq {b}")


def test_verify_varlen_rejects_bad_lengths():
    spec = spec_for(128, 128, "bf16", tag=122)
    B, T = 3, 4
    S0 = synth.initial_state(spec, B)
    inp = synth.token_inputs(spec, B, T)
    d = dev_inputs(inp)
    S = dev_tensor(S0)
    S_keep = S.clone()
    log = kda.InputLog(S, T_max=T)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    o = sentinel_like((B, T, spec.H, 128))
    kda.verify_varlen(S, d["q"], d["k"], d["v"], d["alpha"], d["beta"], o, log,
                      torch.tensor([-1, T + 1, 2], dtype=torch.int32, device="cuda"), err)
    torch.cuda.synchronize()
    assert err.item() == kda.DEV_ERR_DRAFT_LEN
    ob = bits(o).cpu()
    assert (ob[:2] == SENTINEL).all() and (ob[2, 2:] == SENTINEL).all() and not (ob[2, :2] == SENTINEL).any()
    # The rejected sequences logged nothing: a count of 0 passes, 1 is flagged.
    pos = torch.zeros(B, dtype=torch.int64, device="cuda")
    err.zero_()
    kda.commit(S, pos, log, torch.tensor([0, 1, 2], dtype=torch.int32, device="cuda"), err)
    torch.cuda.synchronize()
    assert err.item() == kda.DEV_ERR_ACCEPTED
    assert pos.cpu().tolist() == [0, 0, 2]
    assert torch.equal(bits(S[:2]), bits(S_keep[:2]))
