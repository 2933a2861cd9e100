"""One serving step over a mixed batch in one launch (kda_mixed_step).

A batch mixes sequences that decode one token, sequences that run a
speculative round (commit of the accepted drafts of their last round, then a
verify of new drafts) and sequences that process a prompt segment, with idle
ones in between.  Checked here:
  * oracle parity over two consecutive mixed steps: a 200-token prompt
    segment beside decoding and speculating sequences, the second step
    committing the drafts the first one logged while sequences change roles;
  * bit-identity with the standalone kernels (decode step, fused commit +
    verify, chunked prefill at chunk 64) at the headline head count, on states
    in a slot pool;
  * the device-side checks: inconsistent roles or token ranges, an accepted
    count given to a sequence that does not speculate, a bad slot id; each
    flags dev_err and leaves its sequence untouched.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import recurrent_state_amd as kda
import synth
from oracle import kda_oracle as ko
from tests.kda_testutil import assert_parity, bits, dev_tensor, say

pytestmark = pytest.mark.gpu

ROLE = {"idle": kda.ROLE_IDLE, "dec": kda.ROLE_DECODE, "spec": kda.ROLE_SPEC, "pf": kda.ROLE_PREFILL}
NAMES = ("q", "k", "v", "alpha", "beta")


def spec_for(dk, dv, dt, H, tag):
    return synth.ConfigSpec(f"mixed{dk}x{dv}{dt}", tag, (6,), H, dk, dv, dt, "softplus", "normal", 0)


class Batch:
    """Roles and token counts of one step, each sequence's seeded inputs, and
    their packed device form ([N][H][d] rows, tok_start offsets)."""

    def __init__(self, spec, roles, lens, phase):
        self.roles, self.lens = list(roles), list(lens)
        self.inp = [synth.token_inputs(spec, 1, n, seqs=[b], phase=phase) for b, n in enumerate(self.lens)]
        self.start = np.concatenate([[0], np.cumsum(self.lens)]).astype(np.int32)
        self.N = int(self.start[-1])
        self.dev = {name: dev_tensor(np.ascontiguousarray(np.concatenate([x[name][0] for x in self.inp], axis=0)))
                    for name in NAMES}
        self.o = torch.full((self.N, spec.H, spec.dv), float("nan"), device="cuda")
        self.roles_dev = torch.tensor([ROLE[r] for r in self.roles], dtype=torch.int32, device="cuda")
        self.start_dev = torch.from_numpy(self.start).cuda()

    def counts(self):
        return tuple(self.roles.count(r) for r in ("dec", "spec", "pf"))

    def rows(self, b):
        return slice(int(self.start[b]), int(self.start[b + 1]))

    def run(self, S, pos, err, log=None, accepted=None, slot_ids=None, counts=None):
        d = self.dev
        kda.mixed_step(S, pos, self.roles_dev, self.start_dev, counts or self.counts(), d["q"], d["k"], d["v"],
                       d["alpha"], d["beta"], self.o, err, log=log, accepted=accepted, slot_ids=slot_ids)
        assert kda.last_variant() == "mixed"


def oracle_step(batch, S, pos, pend_log, accepted, scale):
    """The step on the oracle: per sequence, its role's token-by-token result.

    S, pos: the oracle's states (f64 [B][H][dk][dv]) and positions before the
    step; pend_log: per sequence the oracle log of its pending drafts (or
    None).  Returns the states, positions, outputs per sequence and the new
    pending logs."""
    S, pos = S.copy(), pos.copy()
    outs, new_log = {}, [None] * len(batch.roles)
    for b, role in enumerate(batch.roles):
        inp = batch.inp[b]
        if role == "dec":
            S[b:b + 1], o = ko.decode(S[b:b + 1], inp, scale)
            pos[b] += 1
            outs[b] = o[0]
        elif role == "pf" and batch.lens[b] > 0:
            S[b:b + 1], p, o, _ = ko.prefill(S[b:b + 1], pos[b:b + 1], inp, scale)
            pos[b] = p[0]
            outs[b] = o[0]
        elif role == "spec":
            if pend_log[b] is not None:
                Sc, pc, err = ko.commit(S[b:b + 1], pos[b:b + 1], pend_log[b], [accepted[b]])
                assert not err[0]
                S[b:b + 1], pos[b] = Sc, pc[0]
            if batch.lens[b] > 0:
                o, log = ko.verify(S[b:b + 1], inp, scale)
                outs[b] = o[0]
                new_log[b] = log
    return S, pos, outs, new_log


def check_step(batch, S_dev, pos_dev, S_ref, pos_ref, outs, what):
    o = batch.o.cpu().numpy()
    got, ref = [], []
    for b, o_ref in outs.items():
        got.append(o[batch.rows(b)].reshape(-1))
        ref.append(o_ref.reshape(-1))
    assert_parity(np.concatenate(got), np.concatenate(ref), S_dev.cpu().numpy(), S_ref, what)
    assert pos_dev.cpu().tolist() == [int(p) for p in pos_ref], what


@pytest.mark.parametrize("dk,dv,dt", [(128, 128, "bf16"), (64, 64, "f32")])
def test_mixed_steps_match_oracle(dk, dv, dt):
    spec = spec_for(dk, dv, dt, 4, 160)
    B, T = 6, 4
    say(f"mixed_step oracle parity dk={dk} dv={dv} {dt}")
    S0 = synth.initial_state(spec, B)
    pos0 = np.arange(B, dtype=np.int64) * 3 + 5
    S = dev_tensor(S0)
    pos = torch.from_numpy(pos0.copy()).cuda()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    log = kda.InputLog(S, T, in_dtype=torch.bfloat16 if dt == "bf16" else torch.float32)

    # A pending verify: drafts for sequences 0 (3 tokens) and 5 (2 tokens).
    draft = np.array([3, 0, 0, 0, 0, 2], np.int32)
    pend = synth.token_inputs(spec, B, 3, phase=50)
    pd = {n: dev_tensor(x) for n, x in pend.items()}
    o_pend = torch.empty((B, 3, spec.H, dv), device="cuda")
    kda.verify_varlen(S, pd["q"], pd["k"], pd["v"], pd["alpha"], pd["beta"], o_pend, log,
                      torch.from_numpy(draft).cuda(), err)
    pend_log = [None] * B
    for b in (0, 5):
        pend_log[b] = {n: pend[n][b:b + 1] for n in ("k", "v", "alpha", "beta")}
        pend_log[b]["len"] = draft[b:b + 1].astype(np.int64)

    # Step 1: sequence 0 commits 2 drafts and verifies 4, 5 commits none and
    # verifies 3; 1 and 4 decode; 2 processes 200 prompt tokens; 3 is idle.
    b1 = Batch(spec, ["spec", "dec", "pf", "idle", "dec", "spec"], [4, 1, 200, 0, 1, 3], phase=1)
    acc1 = np.array([2, 0, 0, 0, 0, 0], np.int32)
    b1.run(S, pos, err, log=log, accepted=torch.from_numpy(acc1).cuda())
    torch.cuda.synchronize()
    assert err.item() == 0
    S_ref, pos_ref, outs, log1 = oracle_step(b1, ko.widen(S0), pos0, pend_log, acc1, spec.scale)
    check_step(b1, S, pos, S_ref, pos_ref, outs, "mixed step 1")
    assert log.pending_T == T

    # Step 2: 0 accepts all 4 drafts of step 1, 5 accepts 1 of its 3, 1 starts
    # speculating, 2 decodes after its prompt, 3 processes a 64-token segment,
    # 4 is idle.
    b2 = Batch(spec, ["spec", "spec", "dec", "pf", "idle", "spec"], [2, 4, 1, 64, 0, 1], phase=2)
    acc2 = np.array([4, 0, 0, 0, 0, 1], np.int32)
    idle_before = bits(S[4]).clone()
    b2.run(S, pos, err, log=log, accepted=torch.from_numpy(acc2).cuda())
    torch.cuda.synchronize()
    assert err.item() == 0
    S_ref, pos_ref, outs, _ = oracle_step(b2, S_ref, pos_ref, log1, acc2, spec.scale)
    check_step(b2, S, pos, S_ref, pos_ref, outs, "mixed step 2")
    assert torch.equal(bits(S[4]), idle_before), "an idle sequence's state changed"


def test_mixed_step_equals_standalone_kernels_bitwise():
    spec = spec_for(128, 128, "bf16", 32, 161)
    H, T = 32, 4
    roles = (["dec"] * 7 + ["spec"] * 2 + ["idle"]) * 3 + ["pf", "dec", "pf", "spec", "idle"]
    B = len(roles)
    lens = [{"dec": 1, "spec": T, "idle": 0}.get(r, 0) for r in roles]
    lens[roles.index("pf")] = 200
    lens[len(roles) - 1 - roles[::-1].index("pf")] = 64
    say(f"mixed_step vs standalone kernels B={B} H={H} roles={[roles.count(r) for r in ROLE]}")
    n_slots = B + 7
    pool_a = kda.SlotPool(n_slots, H, 128, 128, "cuda")
    g = torch.Generator(device="cuda").manual_seed(5)
    pool_a.states.copy_(torch.randn(pool_a.states.shape, generator=g, device="cuda") * 0.02)
    pool_a.pos.copy_(torch.arange(n_slots, device="cuda") * 10)
    pool_b = kda.SlotPool(n_slots, H, 128, 128, "cuda")
    pool_b.states.copy_(pool_a.states)
    pool_b.pos.copy_(pool_a.pos)
    ids = np.random.default_rng(6).permutation(n_slots)[:B].astype(np.int32)
    slot_ids = torch.from_numpy(ids).cuda()
    err_a = torch.zeros(1, dtype=torch.int32, device="cuda")
    err_b = torch.zeros(1, dtype=torch.int32, device="cuda")
    log_a = kda.InputLog(pool_a.states[:B], T)   # sized for a batch of B (the view only gives the shape)
    log_b = kda.InputLog(pool_a.states[:B], T)

    # The same pending verify in both pipelines: T drafts for every sequence.
    pend = {n: dev_tensor(x) for n, x in synth.token_inputs(spec, B, T, phase=70).items()}
    o_p = torch.empty((B, T, H, 128), device="cuda")
    for pool, log, err in ((pool_a, log_a, err_a), (pool_b, log_b, err_b)):
        kda.verify_slots(slot_ids, pool, pend["q"], pend["k"], pend["v"], pend["alpha"], pend["beta"], o_p, log, err)
    acc = torch.from_numpy(np.array([(b % T) + 1 if r == "spec" else 0 for b, r in enumerate(roles)],
                                    np.int32)).cuda()

    # Pipeline A: one mixed step.
    batch = Batch(spec, roles, lens, phase=3)
    batch.run(pool_a.states, pool_a.pos, err_a, log=log_a, accepted=acc, slot_ids=slot_ids)

    # Pipeline B: the standalone kernels on the same inputs.  The fused
    # commit + verify runs over the whole batch (count 0 for the sequences
    # that do not speculate, so their states are untouched).
    dense = {n: torch.zeros((B, T) + tuple(x.shape[1:]), dtype=x.dtype, device="cuda")
             for n, x in batch.dev.items()}
    for b, r in enumerate(roles):
        if r == "spec":
            for n in NAMES:
                dense[n][b] = batch.dev[n][batch.rows(b)]
    o_cv = torch.empty((B, T, H, 128), device="cuda")
    kda.commit_verify_slots(slot_ids, pool_b, dense["q"], dense["k"], dense["v"], dense["alpha"], dense["beta"], o_cv,
                            log_b, err_b, accepted=acc)
    dec = [b for b, r in enumerate(roles) if r == "dec"]
    tok = {n: torch.stack([batch.dev[n][batch.rows(b)] for b in dec]).contiguous() for n in NAMES}
    o_dec = torch.empty((len(dec), 1, H, 128), device="cuda")
    kda.decode_step_slots(slot_ids[dec].contiguous(), pool_b, tok["q"], tok["k"], tok["v"], tok["alpha"],
                          tok["beta"], o_dec, err_b)
    o_pf = {}
    for b in [b for b, r in enumerate(roles) if r == "pf"]:
        seg = {n: batch.dev[n][batch.rows(b)].unsqueeze(0).contiguous() for n in NAMES}
        o_pf[b] = torch.empty((1, lens[b], H, 128), device="cuda")
        kda.prefill_chunked_slots(slot_ids[b:b + 1].contiguous(), pool_b, seg["q"], seg["k"], seg["v"], seg["alpha"],
                                  seg["beta"], o_pf[b], err_b, chunk=64)
    torch.cuda.synchronize()
    assert err_a.item() == 0 and err_b.item() == 0
    assert torch.equal(bits(pool_a.states), bits(pool_b.states)), "states differ"
    assert torch.equal(pool_a.pos, pool_b.pos), "positions differ"
    for i, b in enumerate(dec):
        assert torch.equal(bits(batch.o[batch.rows(b)]), bits(o_dec[i])), f"decode output of sequence {b}"
    for b, o in o_pf.items():
        assert torch.equal(bits(batch.o[batch.rows(b)]), bits(o[0])), f"prompt outputs of sequence {b}"
    for b, r in enumerate(roles):
        if r == "spec":
            assert torch.equal(bits(batch.o[batch.rows(b)]), bits(o_cv[b])), f"verify outputs of sequence {b}"
    # Both logs now hold the same drafts of the speculating sequences: a
    # commit of them agrees too.
    acc2 = torch.from_numpy(np.array([T if r == "spec" else 0 for r in roles], np.int32)).cuda()
    kda.commit_slots(slot_ids, pool_a, log_a, acc2, err_a)
    kda.commit_slots(slot_ids, pool_b, log_b, acc2, err_b)
    torch.cuda.synchronize()
    assert err_a.item() == 0 and err_b.item() == 0
    assert torch.equal(bits(pool_a.states), bits(pool_b.states)), "states differ after committing the new drafts"


def test_mixed_step_flags_and_skips_bad_sequences():
    spec = spec_for(128, 128, "bf16", 4, 162)
    B, T = 6, 4
    say("mixed_step device-side checks")
    S0 = dev_tensor(synth.initial_state(spec, B))
    S = S0.clone()
    pos = torch.arange(B, dtype=torch.int64, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    log = kda.InputLog(S, T)
    pend = {n: dev_tensor(x) for n, x in synth.token_inputs(spec, B, 2, phase=9).items()}
    kda.verify(S, pend["q"], pend["k"], pend["v"], pend["alpha"], pend["beta"],
               torch.empty((B, 2, spec.H, 128), device="cuda"), log)
    # 0: decode with two tokens (bad range); 1: decode given an accepted count;
    # 2: speculation accepting more than was logged (flagged, commit skipped,
    # verify still runs); 3: prompt segment; 4: idle given an accepted count;
    # 5: decode.
    roles = ["dec", "dec", "spec", "pf", "idle", "dec"]
    batch = Batch(spec, roles, [2, 1, 2, 20, 0, 1], phase=4)
    acc = torch.tensor([0, 1, 3, 0, 1, 0], dtype=torch.int32, device="cuda")
    batch.run(S, pos, err, log=log, accepted=acc)
    torch.cuda.synchronize()
    assert err.item() == kda.DEV_ERR_MIXED | kda.DEV_ERR_ACCEPTED
    for b in (0, 1, 2, 4):
        assert torch.equal(bits(S[b]), bits(S0[b])), f"sequence {b} was changed"
    assert pos.cpu().tolist() == [0, 1, 2, 3 + 20, 4, 5 + 1]
    assert not torch.equal(bits(S[3]), bits(S0[3])) and not torch.equal(bits(S[5]), bits(S0[5]))
    o = batch.o.cpu()
    assert torch.isfinite(o[batch.rows(2)]).all(), "the verify of sequence 2 still ran"

    # Role counts that disagree with the roles array.
    err.zero_()
    batch2 = Batch(spec, ["dec", "idle", "idle", "idle", "idle", "dec"], [1, 0, 0, 0, 0, 1], phase=5)
    batch2.run(S, pos, err, counts=(1, 0, 0))
    torch.cuda.synchronize()
    assert err.item() == kda.DEV_ERR_MIXED

    # A slot id out of range skips that sequence only.
    err.zero_()
    pool = kda.SlotPool(4, spec.H, 128, 128, "cuda")
    keep = bits(pool.states).clone()
    batch3 = Batch(spec, ["dec", "dec"], [1, 1], phase=6)
    batch3.run(pool.states, pool.pos, err, slot_ids=torch.tensor([7, 2], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert err.item() == kda.DEV_ERR_SLOT_ID
    changed = [i for i in range(4) if not torch.equal(bits(pool.states[i]), keep[i])]
    assert changed == [2]
