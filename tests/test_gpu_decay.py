"""GPU parity of the chunked prefill for gates that decay strongly, and empty prompts.

The chunked form divides by in-chunk decay products; the kernel keeps them
finite by applying each chunk's first decay to the state up front and by
cutting a chunk where some channel's product would drop below 2^-96 (the fp32
model of that algebra is checked against the oracle on the CPU in
tests/test_oracle_paths.py).  These cases drive the kernel through those cuts:
gates of mean ~0.3 (sigmoid of N(-1, 1)), a constant 0.05, and exact zeros (a
channel that forgets every token, a token that resets every channel, scattered
zeros), at both chunk sizes, with checkpoints whose boundaries the cut chunks
must still land on, and from raw logits whose gates saturate to exactly 0.
Every case is compared with the fp64 oracle (the token-by-token recurrence).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import recurrent_state_amd as kda
import synth
from oracle import kda_oracle as ko
from tests.kda_testutil import assert_parity, bits, dev_inputs, dev_tensor, say, state_err

pytestmark = pytest.mark.gpu

GATES = {"softplus": kda.GATE_EXP_NEG_SOFTPLUS, "sigmoid": kda.GATE_SIGMOID}


def strong_gates(kind, B, L, H, dk, seed):
    r = np.random.default_rng(seed)
    if kind == "sigmoid_m1":
        a = 1.0 / (1.0 + np.exp(-r.normal(-1.0, 1.0, (B, L, H, dk))))
    elif kind == "const_0.05":
        a = np.full((B, L, H, dk), 0.05)
    elif kind == "zeros":
        a = 1.0 / (1.0 + np.exp(-r.normal(3.0, 1.0, (B, L, H, dk))))
        a[r.random((B, L, H, dk)) < 0.01] = 0.0
        a[:, :, :, 5] = 0.0          # a channel that forgets every token
        a[:, 41] = 0.0               # a token that resets every channel
        a[0, 100:103, 1] = 0.0       # three resets in a row in one head
    else:
        raise ValueError(kind)
    return a.astype(np.float32)


def run_chunked(spec, B, L, chunk, inp, every, S0, pos0=(7, 0)):
    d = dev_inputs(inp)
    S = dev_tensor(S0)
    pos = torch.tensor(list(pos0)[:B], dtype=torch.int64, device="cuda")
    n_ck = L // every if every else 0
    pool = kda.SlotPool(max(1, B * n_ck), spec.H, spec.dk, spec.dv, "cuda")
    slots = torch.arange(B * n_ck, dtype=torch.int32, device="cuda").view(B, n_ck) if n_ck else None
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    o = torch.full((B, L, spec.H, spec.dv), float("nan"), device="cuda")
    kda.prefill_chunked(S, pos, d["q"], d["k"], d["v"], d["alpha"], d["beta"], o, chunk=chunk, ckpt_every=every,
                        ckpt_slots=slots, pool=pool, dev_err=err)
    assert kda.last_variant() == "prefill_chunked"
    torch.cuda.synchronize()
    return S, pos, o, pool, n_ck, err


@pytest.mark.parametrize("kind", ["sigmoid_m1", "const_0.05", "zeros"])
@pytest.mark.parametrize("chunk", [32, 64])
@pytest.mark.parametrize("dk,dv,dt", [(128, 128, "bf16"), (64, 64, "f32")])
def test_prefill_chunked_strong_decay_matches_oracle(dk, dv, dt, chunk, kind):
    spec = synth.ConfigSpec(f"decay{dk}{dt}", 140, (2,), 4, dk, dv, dt, "softplus", "normal", 0)
    B, L = 2, 200
    every = 2 * chunk
    say(f"prefill_chunked strong decay {kind} dk={dk} dv={dv} {dt} chunk={chunk} L={L}")
    inp = synth.token_inputs(spec, B, L)
    inp["alpha"] = strong_gates(kind, B, L, spec.H, dk, seed=dk + chunk)
    S0 = synth.initial_state(spec, B)
    S, pos, o, pool, n_ck, err = run_chunked(spec, B, L, chunk, inp, every, S0)
    S_ref, pos_ref, o_ref, ck = ko.prefill(S0, np.array([7, 0]), inp, spec.scale, every)
    o_np = o.cpu().numpy()
    assert np.all(np.isfinite(o_np)), "every output written and finite"
    assert_parity(o_np, o_ref, S.cpu().numpy(), S_ref, f"strong decay {kind} chunk={chunk}")
    assert pos.cpu().tolist() == pos_ref.tolist() and err.item() == 0
    for m, (Sm, pm) in enumerate(ck):
        for b in range(B):
            slot = b * n_ck + m
            assert state_err(pool.states[slot:slot + 1].cpu().numpy(), Sm[b:b + 1]) <= 1e-3, (m, b)
            assert pool.pos[slot].item() == pm[b]


def test_prefill_chunked_strong_decay_equals_recurrent_prefill_to_tolerance():
    # The token-by-token kernel on the same inputs (a second HIP path, no cuts at all).
    spec = synth.ConfigSpec("decay_rec", 141, (2,), 4, 128, 128, "bf16", "softplus", "normal", 0)
    B, L = 2, 160
    inp = synth.token_inputs(spec, B, L)
    inp["alpha"] = strong_gates("zeros", B, L, spec.H, 128, seed=3)
    S0 = synth.initial_state(spec, B)
    S, _, o, _, _, _ = run_chunked(spec, B, L, 64, inp, 0, S0)
    d = dev_inputs(inp)
    S2 = dev_tensor(S0)
    o2 = torch.empty_like(o)
    kda.prefill_recurrent(S2, torch.zeros(B, dtype=torch.int64, device="cuda"), d["q"], d["k"], d["v"], d["alpha"],
                          d["beta"], o2)
    assert_parity(o.cpu().numpy(), o2.cpu().numpy().astype(np.float64), S.cpu().numpy(),
                  S2.cpu().numpy().astype(np.float64), "chunked vs recurrent, strong decay")


@pytest.mark.parametrize("gate", ["softplus", "sigmoid"])
@pytest.mark.parametrize("chunk", [32, 64])
def test_prefill_chunked_prep_saturated_gates_match_oracle(gate, chunk):
    # Logits far out saturate the fp32 gate to exactly 0 (and 1 the other way).
    spec = synth.ConfigSpec("decay_prep", 142, (2,), 4, 128, 128, "bf16", gate, "normal", 0)
    B, L = 2, 200
    say(f"prefill_chunked_prep saturated gates {gate} chunk={chunk}")
    raw = synth.raw_token_inputs(spec, B, L)
    r = np.random.default_rng(chunk)
    x = r.normal(0.0, 40.0, raw["alpha_logit"].shape)           # ~2% beyond +-100
    x[:, 77] = 300.0 if gate == "softplus" else -300.0          # closes every gate: alpha = 0
    raw["alpha_logit"] = x.astype(np.float32)
    S0 = synth.initial_state(spec, B)
    d = dev_inputs(raw)
    S = dev_tensor(S0)
    pos = torch.zeros(B, dtype=torch.int64, device="cuda")
    o = torch.full((B, L, spec.H, 128), float("nan"), device="cuda")
    kda.prefill_chunked_prep(S, pos, d["q"], d["k"], d["v"], d["alpha_logit"], d["beta_logit"], o,
                             gate=GATES[gate], chunk=chunk)
    assert kda.last_variant() == "prefill_chunked_prep"
    S_ref, _, o_ref, _ = ko.prefill(S0, np.zeros(B, np.int64), ko.prep(raw, GATES[gate]), spec.scale, 0)
    o_np = o.cpu().numpy()
    assert np.all(np.isfinite(o_np))
    assert_parity(o_np, o_ref, S.cpu().numpy(), S_ref, f"prep saturated {gate} chunk={chunk}")


@pytest.mark.parametrize("which", ["chunked", "recurrent", "chunked_prep", "recurrent_prep", "chunked_slots"])
def test_empty_prompt_is_a_noop(which):
    spec = synth.ConfigSpec("empty", 143, (2,), 4, 128, 128, "bf16", "softplus", "normal", 0)
    B = 2
    S0 = dev_tensor(synth.initial_state(spec, B))
    S = S0.clone()
    pos = torch.tensor([5, 9], dtype=torch.int64, device="cuda")
    z = lambda *s, dt=torch.bfloat16: torch.zeros(s, dtype=dt, device="cuda")  # noqa: E731
    q, k, v = z(B, 0, 4, 128), z(B, 0, 4, 128), z(B, 0, 4, 128)
    a, b = z(B, 0, 4, 128, dt=torch.float32), z(B, 0, 4, dt=torch.float32)
    o = z(B, 0, 4, 128, dt=torch.float32)
    before = kda.last_variant()
    if which == "chunked":
        kda.prefill_chunked(S, pos, q, k, v, a, b, o, chunk=64)
    elif which == "recurrent":
        kda.prefill_recurrent(S, pos, q, k, v, a, b, o)
    elif which == "chunked_prep":
        kda.prefill_chunked_prep(S, pos, q, k, v, a, b, o, chunk=32)
    elif which == "recurrent_prep":
        kda.prefill_recurrent_prep(S, pos, q, k, v, a, b, o)
    else:
        pool = kda.SlotPool(3, 4, 128, 128, "cuda")
        pool.states.copy_(torch.randn_like(pool.states))
        keep = pool.states.clone()
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        kda.prefill_chunked_slots(torch.tensor([2, 0], dtype=torch.int32, device="cuda"), pool, q, k, v, a, b, o,
                                  err, chunk=64)
        torch.cuda.synchronize()
        assert torch.equal(bits(pool.states), bits(keep)) and err.item() == 0
    torch.cuda.synchronize()
    assert kda.last_variant() == before, "nothing is launched for an empty prompt"
    assert torch.equal(bits(S), bits(S0)) and pos.cpu().tolist() == [5, 9]
