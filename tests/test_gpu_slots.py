"""Decode on states that live in a slot pool (kda_decode_step_slots) and
slot-to-slot copies (kda_slot_copy).

Bit for bit: decoding through slot ids equals decoding the same states in a
dense batch (outputs, states, positions), slots no sequence names are not
touched, ids out of range are flagged and skipped, and a copied slot decodes
exactly like its source.  Both workgroup shapes of the decode kernel are
covered (one-wave workgroups at small batches, whole-state workgroups at
large ones).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import recurrent_state_amd as kda
import synth
from tests.kda_testutil import bits, dev_tensor, say
from tests.test_gpu_small import spec_for

pytestmark = pytest.mark.gpu

SENTINEL = 0x7FC0BEEF


def _pool(spec, n_slots, seed):
    pool = kda.SlotPool(n_slots, spec.H, spec.dk, spec.dv, "cuda")
    g = torch.Generator(device="cuda").manual_seed(seed)
    pool.states.copy_(torch.randn(pool.states.shape, generator=g, device="cuda") * 0.02)
    pool.pos.copy_(torch.arange(n_slots, device="cuda") * 10)
    return pool


@pytest.mark.parametrize("dk,dv,dt,B", [(128, 128, "bf16", 4), (64, 64, "f32", 5), (128, 128, "bf16", 128)])
def test_decode_slots_equals_dense_decode(dk, dv, dt, B):
    spec = spec_for(dk, dv, dt, tag=150)
    n_slots = 2 * B + 3
    say(f"decode_slots dk={dk} dv={dv} {dt} B={B}")
    pool = _pool(spec, n_slots, 1)
    ids = np.random.default_rng(2).permutation(n_slots)[:B].astype(np.int32)
    slot_ids = torch.from_numpy(ids).cuda()
    S = pool.states[slot_ids.long()].clone()          # the same states as a dense batch
    pos = pool.pos[slot_ids.long()].clone()
    untouched = [i for i in range(n_slots) if i not in set(ids.tolist())]
    keep = bits(pool.states[untouched]).clone()
    keep_pos = pool.pos[untouched].clone()
    inp = {name: dev_tensor(x) for name, x in synth.token_inputs(spec, B, 4).items()}
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    for t in range(4):
        tok = {name: x[:, t:t + 1].contiguous() for name, x in inp.items()}
        o_s = torch.empty((B, 1, spec.H, dv), device="cuda")
        o_d = torch.empty_like(o_s)
        kda.decode_step_slots(slot_ids, pool, tok["q"], tok["k"], tok["v"], tok["alpha"], tok["beta"], o_s, err)
        assert kda.last_variant() == "decode_slots"
        kda.decode_step(S, pos, tok["q"], tok["k"], tok["v"], tok["alpha"], tok["beta"], o_d)
        assert torch.equal(bits(o_s), bits(o_d)), f"token {t}"
    torch.cuda.synchronize()
    assert err.item() == 0
    assert torch.equal(bits(pool.states[slot_ids.long()]), bits(S))
    assert torch.equal(pool.pos[slot_ids.long()], pos)
    assert torch.equal(bits(pool.states[untouched]), keep) and torch.equal(pool.pos[untouched], keep_pos)


def test_decode_slots_out_of_range_ids_are_flagged_and_skipped():
    spec = spec_for(128, 128, "bf16", tag=151)
    B, n_slots = 4, 6
    pool = _pool(spec, n_slots, 3)
    before = bits(pool.states).clone()
    pos_before = pool.pos.clone()
    slot_ids = torch.tensor([3, n_slots, -1, 0], dtype=torch.int32, device="cuda")
    inp = {name: dev_tensor(x) for name, x in synth.token_inputs(spec, B, 1).items()}
    o = torch.full((B, 1, spec.H, 128), SENTINEL, dtype=torch.int32, device="cuda").view(torch.float32)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    kda.decode_step_slots(slot_ids, pool, inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], o, err)
    torch.cuda.synchronize()
    assert err.item() == kda.DEV_ERR_SLOT_ID
    ob = bits(o)
    assert (ob[1:3] == SENTINEL).all() and not (ob[0] == SENTINEL).any() and not (ob[3] == SENTINEL).any()
    changed = [i for i in range(n_slots) if not torch.equal(bits(pool.states[i]), before[i])]
    assert changed == [0, 3]
    assert (pool.pos - pos_before).tolist() == [1, 0, 0, 1, 0, 0]


def test_slot_copy_forks_a_prefix():
    spec = spec_for(128, 128, "bf16", tag=152)
    n_slots = 6
    say("slot_copy")
    pool = _pool(spec, n_slots, 4)
    kda.slot_copy([2, 4], [5, 1], pool)
    assert kda.last_variant() == "slot_copy"
    torch.cuda.synchronize()
    assert torch.equal(bits(pool.states[5]), bits(pool.states[2])) and torch.equal(bits(pool.states[1]),
                                                                                bits(pool.states[4]))
    assert pool.pos[5].item() == 20 and pool.pos[1].item() == 40
    # The fork and its source continue identically on the same tokens.
    inp = {name: dev_tensor(x) for name, x in synth.token_inputs(spec, 1, 3).items()}
    both = {name: torch.cat([x, x], dim=0).contiguous() for name, x in inp.items()}
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    slot_ids = torch.tensor([2, 5], dtype=torch.int32, device="cuda")
    for t in range(3):
        tok = {name: x[:, t:t + 1].contiguous() for name, x in both.items()}
        o = torch.empty((2, 1, spec.H, 128), device="cuda")
        kda.decode_step_slots(slot_ids, pool, tok["q"], tok["k"], tok["v"], tok["alpha"], tok["beta"], o, err)
        assert torch.equal(bits(o[0]), bits(o[1]))
    torch.cuda.synchronize()
    assert torch.equal(bits(pool.states[5]), bits(pool.states[2])) and pool.pos[5].item() == 23
    with pytest.raises(kda.KdaError):
        kda.slot_copy([1, 2], [2, 3], pool)    # slot 2 both read and written


@pytest.mark.parametrize("T,B,fused", [(4, 4, False), (4, 4, True), (7, 3, True), (4, 20, True)])
def test_speculative_rounds_on_slots_equal_dense(T, B, fused):
    # Two rounds (verify + commit, or fused) on pool slots against the same
    # sequences in a dense batch: states, positions and outputs bit for bit.
    spec = synth.ConfigSpec("spslots", 153, (B,), 32 if B > 8 else 5, 128, 128, "bf16", "softplus", "normal", 0)
    n_slots = 2 * B + 1
    say(f"speculative on slots T={T} B={B} fused={fused}")
    pool = _pool(spec, n_slots, 5)
    ids = np.random.default_rng(6).permutation(n_slots)[:B].astype(np.int32)
    slot_ids = torch.from_numpy(ids).cuda()
    S = pool.states[slot_ids.long()].clone()
    pos = pool.pos[slot_ids.long()].clone()
    untouched = [i for i in range(n_slots) if i not in set(ids.tolist())]
    keep = bits(pool.states[untouched]).clone()
    d = {name: dev_tensor(x) for name, x in synth.token_inputs(spec, B, 2 * T).items()}
    rounds = [{k_: v_[:, r * T:(r + 1) * T].contiguous() for k_, v_ in d.items()} for r in range(2)]
    counts = [torch.tensor(np.random.default_rng(7 + r).integers(0, T + 1, B), dtype=torch.int32, device="cuda")
              for r in range(2)]
    err_s = torch.zeros(1, dtype=torch.int32, device="cuda")
    err_d = torch.zeros(1, dtype=torch.int32, device="cuda")
    log_s = kda.InputLog(S, T_max=8)
    log_d = kda.InputLog(S, T_max=8)
    for r in range(2):
        x = rounds[r]
        o_s = torch.empty((B, T, spec.H, 128), device="cuda")
        o_d = torch.empty_like(o_s)
        if fused:
            acc = counts[r - 1] if r > 0 else None
            kda.commit_verify_slots(slot_ids, pool, x["q"], x["k"], x["v"], x["alpha"], x["beta"], o_s, log_s,
                                    err_s, accepted=acc)
            assert kda.last_variant() == "commit_verify_slots"
            kda.commit_verify(S, pos, x["q"], x["k"], x["v"], x["alpha"], x["beta"], o_d, log_d, acc,
                              err_d if acc is not None else None)
        else:
            kda.verify_slots(slot_ids, pool, x["q"], x["k"], x["v"], x["alpha"], x["beta"], o_s, log_s, err_s)
            assert kda.last_variant() == "verify_slots"
            kda.verify(S, x["q"], x["k"], x["v"], x["alpha"], x["beta"], o_d, log_d)
            kda.commit_slots(slot_ids, pool, log_s, counts[r], err_s)
            assert kda.last_variant() == "commit_slots"
            kda.commit(S, pos, log_d, counts[r], err_d)
        assert torch.equal(bits(o_s), bits(o_d)), f"round {r} outputs"
    torch.cuda.synchronize()
    assert err_s.item() == 0 and err_d.item() == 0
    assert torch.equal(bits(pool.states[slot_ids.long()]), bits(S))
    assert torch.equal(pool.pos[slot_ids.long()], pos)
    assert torch.equal(bits(pool.states[untouched]), keep)


def test_verify_slots_out_of_range_id_logs_nothing():
    spec = spec_for(128, 128, "bf16", tag=154)
    B, T, n_slots = 3, 4, 5
    pool = _pool(spec, n_slots, 8)
    before = bits(pool.states).clone()
    slot_ids = torch.tensor([1, 9, 3], dtype=torch.int32, device="cuda")
    d = {name: dev_tensor(x) for name, x in synth.token_inputs(spec, B, T).items()}
    log = kda.InputLog(torch.empty((B, spec.H, 128, 128), device="cuda"), T_max=T)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    o = torch.full((B, T, spec.H, 128), SENTINEL, dtype=torch.int32, device="cuda").view(torch.float32)
    kda.verify_slots(slot_ids, pool, d["q"], d["k"], d["v"], d["alpha"], d["beta"], o, log, err)
    torch.cuda.synchronize()
    assert err.item() == kda.DEV_ERR_SLOT_ID
    assert (bits(o)[1] == SENTINEL).all() and not (bits(o)[0] == SENTINEL).any()
    err.zero_()
    kda.commit_slots(slot_ids, pool, log, torch.tensor([2, 1, 0], dtype=torch.int32, device="cuda"), err)
    torch.cuda.synchronize()
    assert err.item() == kda.DEV_ERR_SLOT_ID          # the bad id is flagged again and skipped
    changed = [i for i in range(n_slots) if not torch.equal(bits(pool.states[i]), before[i])]
    assert changed == [1]


@pytest.mark.parametrize("L,chunk", [(200, 64), (37, 32)])
def test_prefill_chunked_on_slots_equals_dense(L, chunk):
    spec = spec_for(128, 128, "bf16", tag=155)
    B = 3
    every = chunk
    say(f"prefill on slots L={L} chunk={chunk}")
    n_ck = L // every
    n_slots = 2 * B + B * n_ck
    pool = _pool(spec, n_slots, 9)
    state_ids = torch.tensor([4, 0, 2], dtype=torch.int32, device="cuda")
    ck_ids = (2 * B + torch.arange(B * n_ck, dtype=torch.int32, device="cuda")).view(B, n_ck)
    S = pool.states[state_ids.long()].clone()
    pos = pool.pos[state_ids.long()].clone()
    dpool = kda.SlotPool(max(1, B * n_ck), spec.H, 128, 128, "cuda")
    dck = torch.arange(B * n_ck, dtype=torch.int32, device="cuda").view(B, n_ck)
    d = {name: dev_tensor(x) for name, x in synth.token_inputs(spec, B, L).items()}
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    o_s = torch.empty((B, L, spec.H, 128), device="cuda")
    o_d = torch.empty_like(o_s)
    kda.prefill_chunked_slots(state_ids, pool, d["q"], d["k"], d["v"], d["alpha"], d["beta"], o_s, err, chunk=chunk,
                              ckpt_every=every, ckpt_slots=ck_ids)
    assert kda.last_variant() == "prefill_chunked_slots"
    kda.prefill_chunked(S, pos, d["q"], d["k"], d["v"], d["alpha"], d["beta"], o_d, chunk=chunk, ckpt_every=every,
                        ckpt_slots=dck if n_ck else None, pool=dpool, dev_err=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    assert torch.equal(bits(o_s), bits(o_d))
    assert torch.equal(bits(pool.states[state_ids.long()]), bits(S)) and torch.equal(pool.pos[state_ids.long()], pos)
    for b in range(B):
        for m in range(n_ck):
            assert torch.equal(bits(pool.states[int(ck_ids[b, m])]), bits(dpool.states[int(dck[b, m])]))
            assert pool.pos[int(ck_ids[b, m])].item() == dpool.pos[int(dck[b, m])].item()
