"""GPU parity of the chunk-64 prefill at dk = dv = 128 (the shape served by the
wave-specialised kernel: separate key and value waves) for ragged prompt
lengths (a short last chunk, one-token prompts), checkpoints (whose interval
the API keeps a multiple of the chunk), fp32 and bf16 inputs, and its
checkpoint-slot error flag.  Chunks cut short by strong decay are covered in
test_gpu_decay.py.

Each case runs the prompt through the C ABI and compares outputs, the final
state, every checkpoint and every position with the fp64 oracle at the
tolerance bar.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import recurrent_state_amd as kda
import synth
from oracle import kda_oracle as ko
from tests.kda_testutil import assert_parity, dev_inputs, dev_tensor, say, state_err

pytestmark = pytest.mark.gpu


def spec_for(dt, tag):
    return synth.ConfigSpec(f"ws128{dt}", tag, (3,), 4, 128, 128, dt, "softplus", "normal", 0)


def run_prefill(spec, B, L, every, slots_fn=None):
    S0 = synth.initial_state(spec, B)
    inp = synth.token_inputs(spec, B, L)
    d = dev_inputs(inp)
    S = dev_tensor(S0)
    pos0 = np.array([5 * b for b in range(B)])
    pos = torch.from_numpy(pos0.astype(np.int64)).cuda()
    n_ck = L // every if every else 0
    pool = kda.SlotPool(max(1, B * n_ck), spec.H, 128, 128, "cuda")
    slots = None
    if n_ck:
        ids = np.arange(B * n_ck, dtype=np.int32).reshape(B, n_ck)
        if slots_fn is not None:
            ids = slots_fn(ids)
        slots = torch.from_numpy(ids).cuda()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    o = torch.full((B, L, spec.H, 128), float("nan"), dtype=torch.float32, device="cuda")
    kda.prefill_chunked(S, pos, d["q"], d["k"], d["v"], d["alpha"], d["beta"], o, chunk=64, ckpt_every=every,
                        ckpt_slots=slots, pool=pool, dev_err=err)
    torch.cuda.synchronize()
    assert kda.last_variant() == "prefill_chunked"
    S_ref, pos_ref, o_ref, ck = ko.prefill(S0, pos0, inp, spec.scale, every)
    return S, pos, o, err, pool, slots, (S_ref, pos_ref, o_ref, ck)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("L,every", [(300, 128), (129, 64), (64, 64), (65, 0), (1, 0)])
def test_chunk64_prefill_uneven_chunks_match_oracle(dt, L, every):
    spec = spec_for(dt, 211)
    B = 3
    say(f"chunk-64 prefill dk=dv=128 {dt} L={L} ckpt_every={every}")
    S, pos, o, err, pool, slots, (S_ref, pos_ref, o_ref, ck) = run_prefill(spec, B, L, every)
    assert err.item() == 0
    assert_parity(o.cpu().numpy(), o_ref, S.cpu().numpy(), S_ref, f"L={L} every={every} {dt}")
    assert pos.cpu().tolist() == pos_ref.tolist()
    n_ck = L // every if every else 0
    assert len(ck) == n_ck
    for m, (Sm, pm) in enumerate(ck):
        for b in range(B):
            slot = b * n_ck + m
            se = state_err(pool.states[slot:slot + 1].cpu().numpy(), Sm[b:b + 1])
            assert se <= 1e-3, f"checkpoint {m} of sequence {b}: {se:.3e}"
            assert pool.pos[slot].item() == pm[b]


def test_chunk64_prefill_bad_checkpoint_slot_flags_and_skips_it():
    spec = spec_for("bf16", 212)
    B, L, every = 2, 200, 64
    say("chunk-64 prefill dk=dv=128, one checkpoint slot out of range")
    bad = (1, 2)  # sequence 1, checkpoint 2

    def with_bad(ids):
        ids = ids.copy()
        ids[bad] = 10_000
        return ids

    S, pos, o, err, pool, slots, (S_ref, pos_ref, o_ref, ck) = run_prefill(spec, B, L, every, with_bad)
    assert err.item() == kda.DEV_ERR_CKPT_SLOT
    # The prompt itself still runs to the end: outputs, state and positions match.
    assert_parity(o.cpu().numpy(), o_ref, S.cpu().numpy(), S_ref, "bad checkpoint slot")
    assert pos.cpu().tolist() == pos_ref.tolist()
    n_ck = L // every
    ids = slots.cpu().numpy()
    for m, (Sm, pm) in enumerate(ck):
        for b in range(B):
            if (b, m) == bad:
                continue
            slot = int(ids[b, m])
            se = state_err(pool.states[slot:slot + 1].cpu().numpy(), Sm[b:b + 1])
            assert se <= 1e-3, f"checkpoint {m} of sequence {b}: {se:.3e}"
            assert pool.pos[slot].item() == pm[b]
    # The slot the bad id replaced is untouched: zero state, position still -1.
    untouched = int(bad[0] * n_ck + bad[1])
    assert torch.count_nonzero(pool.states[untouched]).item() == 0 and pool.pos[untouched].item() == -1


GATES = {"softplus": kda.GATE_EXP_NEG_SOFTPLUS, "sigmoid": kda.GATE_SIGMOID}


def raw_dev(raw):
    return {name: dev_tensor(np.ascontiguousarray(x)) for name, x in raw.items()}


def run_prefill_raw(spec, B, L, every, gate, scale_qk=1.0):
    """prefill_chunked_prep at chunk 64 (raw projections: the key waves form the
    norms and the gates); returns the device results and the host inputs."""
    S0 = synth.initial_state(spec, B)
    raw = synth.raw_token_inputs(spec, B, L)
    d = raw_dev(raw)
    if scale_qk != 1.0:
        d["q"] = (d["q"].view(torch.bfloat16) * scale_qk).view(d["q"].dtype)
        d["k"] = (d["k"].view(torch.bfloat16) * scale_qk).view(d["k"].dtype)
    S = dev_tensor(S0)
    pos = torch.tensor([3 * b for b in range(B)], dtype=torch.int64, device="cuda")
    n_ck = L // every if every else 0
    pool = kda.SlotPool(max(1, B * n_ck), spec.H, 128, 128, "cuda")
    slots = torch.arange(B * n_ck, dtype=torch.int32, device="cuda").view(B, n_ck) if n_ck else None
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    o = torch.full((B, L, spec.H, 128), float("nan"), dtype=torch.float32, device="cuda")
    kda.prefill_chunked_prep(S, pos, d["q"], d["k"], d["v"], d["alpha_logit"], d["beta_logit"], o, gate=GATES[gate],
                             chunk=64, ckpt_every=every, ckpt_slots=slots, pool=pool, dev_err=err)
    torch.cuda.synchronize()
    assert kda.last_variant() == "prefill_chunked_prep"
    return S0, raw, S, pos, o, err, pool, n_ck


@pytest.mark.parametrize("gate", ["softplus", "sigmoid"])
@pytest.mark.parametrize("L,every", [(300, 128), (129, 64), (65, 0), (1, 0)])
def test_chunk64_prefill_raw_projections_uneven_chunks_match_oracle(L, every, gate):
    spec = synth.ConfigSpec("ws128raw", 213, (3,), 4, 128, 128, "bf16", gate, "normal", 0)
    B = 3
    say(f"chunk-64 prefill from raw projections dk=dv=128 bf16 L={L} ckpt_every={every} {gate}")
    S0, raw, S, pos, o, err, pool, n_ck = run_prefill_raw(spec, B, L, every, gate)
    assert err.item() == 0
    S_ref, pos_ref, o_ref, ck = ko.prefill(S0, np.array([3 * b for b in range(B)]), ko.prep(raw, GATES[gate]),
                                           spec.scale, every)
    assert_parity(o.cpu().numpy(), o_ref, S.cpu().numpy(), S_ref, f"raw L={L} every={every} {gate}")
    assert pos.cpu().tolist() == pos_ref.tolist()
    assert len(ck) == n_ck
    for m, (Sm, pm) in enumerate(ck):
        for b in range(B):
            se = state_err(pool.states[b * n_ck + m:b * n_ck + m + 1].cpu().numpy(), Sm[b:b + 1])
            assert se <= 1e-3, f"checkpoint {m} of sequence {b}: {se:.3e}"
            assert pool.pos[b * n_ck + m].item() == pm[b]


def test_chunk64_prefill_raw_projections_power_of_two_scaling_is_exact():
    # The norms are sums of squares, an IEEE square root and a division:
    # scaling every q and k by 2 scales each by exactly 2, and the unit
    # vectors, so every output and state bit, stay the same.
    spec = synth.ConfigSpec("ws128raw", 214, (2,), 4, 128, 128, "bf16", "softplus", "normal", 0)
    say("chunk-64 prefill from raw projections: q, k scaled by 2")
    _, _, S1, _, o1, _, _, _ = run_prefill_raw(spec, 2, 150, 0, "softplus")
    _, _, S2, _, o2, _, _, _ = run_prefill_raw(spec, 2, 150, 0, "softplus", scale_qk=2.0)
    assert torch.equal(o1.view(torch.int32), o2.view(torch.int32))
    assert torch.equal(S1.view(torch.int32), S2.view(torch.int32))


@pytest.mark.parametrize("raw", [False, True])
@pytest.mark.parametrize("L,every", [(200, 64), (1, 0)])
@pytest.mark.parametrize("dk", [128, 64])
def test_chunk64_prefill_dv64_matches_oracle(dk, L, every, raw):
    # dv = 64: four value waves beside the dk / 16 key waves.
    spec = synth.ConfigSpec("ws64", 215, (2,), 4, dk, 64, "bf16", "softplus", "normal", 0)
    B = 2
    say(f"chunk-64 prefill dk={dk} dv=64 bf16 L={L} ckpt_every={every} raw={raw}")
    S0 = synth.initial_state(spec, B)
    pos0 = np.array([4, 0])
    pos = torch.from_numpy(pos0.astype(np.int64)).cuda()
    S = dev_tensor(S0)
    n_ck = L // every if every else 0
    pool = kda.SlotPool(max(1, B * n_ck), spec.H, dk, 64, "cuda")
    slots = torch.arange(B * n_ck, dtype=torch.int32, device="cuda").view(B, n_ck) if n_ck else None
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    o = torch.full((B, L, spec.H, 64), float("nan"), dtype=torch.float32, device="cuda")
    if raw:
        host = synth.raw_token_inputs(spec, B, L)
        d = raw_dev(host)
        kda.prefill_chunked_prep(S, pos, d["q"], d["k"], d["v"], d["alpha_logit"], d["beta_logit"], o,
                                 gate=GATES["softplus"], chunk=64, ckpt_every=every, ckpt_slots=slots, pool=pool,
                                 dev_err=err)
        ref_inp = ko.prep(host, GATES["softplus"])
    else:
        host = synth.token_inputs(spec, B, L)
        d = dev_inputs(host)
        kda.prefill_chunked(S, pos, d["q"], d["k"], d["v"], d["alpha"], d["beta"], o, chunk=64, ckpt_every=every,
                            ckpt_slots=slots, pool=pool, dev_err=err)
        ref_inp = host
    torch.cuda.synchronize()
    assert err.item() == 0
    S_ref, pos_ref, o_ref, ck = ko.prefill(S0, pos0, ref_inp, spec.scale, every)
    assert_parity(o.cpu().numpy(), o_ref, S.cpu().numpy(), S_ref, f"dv=64 L={L} raw={raw}")
    assert pos.cpu().tolist() == pos_ref.tolist()
    for m, (Sm, pm) in enumerate(ck):
        for b in range(B):
            se = state_err(pool.states[b * n_ck + m:b * n_ck + m + 1].cpu().numpy(), Sm[b:b + 1])
            assert se <= 1e-3, f"checkpoint {m} of sequence {b}: {se:.3e}"
            assert pool.pos[b * n_ck + m].item() == pm[b]


@pytest.mark.parametrize("L,every", [(129, 64), (1, 0)])
def test_chunk64_prefill_raw_projections_f32_match_oracle(L, every):
    # fp32 raw projections: keys and queries a period ahead as for bf16.
    spec = synth.ConfigSpec("ws128rawf", 216, (2,), 4, 128, 128, "f32", "sigmoid", "normal", 0)
    B = 2
    say(f"chunk-64 prefill from fp32 raw projections dk=dv=128 L={L} ckpt_every={every}")
    S0, raw, S, pos, o, err, pool, n_ck = run_prefill_raw(spec, B, L, every, "sigmoid")
    assert err.item() == 0
    S_ref, pos_ref, o_ref, ck = ko.prefill(S0, np.array([3 * b for b in range(B)]), ko.prep(raw, GATES["sigmoid"]),
                                           spec.scale, every)
    assert_parity(o.cpu().numpy(), o_ref, S.cpu().numpy(), S_ref, f"f32 raw L={L} every={every}")
    assert pos.cpu().tolist() == pos_ref.tolist()
    for m, (Sm, pm) in enumerate(ck):
        for b in range(B):
            se = state_err(pool.states[b * n_ck + m:b * n_ck + m + 1].cpu().numpy(), Sm[b:b + 1])
            assert se <= 1e-3, f"checkpoint {m} of sequence {b}: {se:.3e}"
