"""GPU parity and bookkeeping on small shapes (every dk/dv/dtype combination).

Parity: the HIP path against the fp64 oracle at the tolerance bar.  Bit-exact
bookkeeping: commit(a) equals a decode steps, a = 0 leaves the state
untouched, snapshot/restore round-trips, and positions add up; these compare
GPU results with each other.  Verify computes its outputs in the chunk form of
the rule (a different rounding order from the token loop), so its outputs are
held to the tolerance bar, against the oracle and against decode steps.  Every test also
checks that the kernel variant it meant to exercise is the one that ran.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import recurrent_state_amd as kda
import synth
from oracle import kda_oracle as ko
from tests.kda_testutil import assert_parity, bits, dev_inputs, dev_tensor, say, state_err, token_slice

pytestmark = pytest.mark.gpu

SHAPES = [(64, 64, "f32"), (64, 128, "bf16"), (128, 64, "f32"), (128, 128, "bf16"), (128, 128, "f32"),
          (64, 64, "bf16")]


def spec_for(dk, dv, dt, gate="softplus", tag=100):
    return synth.ConfigSpec(f"s{dk}x{dv}{dt}", tag, (3,), 5, dk, dv, dt, gate, "normal", 0)


def decode_run(S, pos, inp_dev, scale=None):
    B, H, _, dv = S.shape
    n = inp_dev["k"].shape[1]
    outs = []
    for t in range(n):
        o = torch.empty((B, 1, H, dv), dtype=torch.float32, device=S.device)
        tok = token_slice(inp_dev, t, t + 1)
        kda.decode_step(S, pos, tok["q"].contiguous(), tok["k"].contiguous(), tok["v"].contiguous(),
                        tok["alpha"].contiguous(), tok["beta"].contiguous(), o, scale=scale)
        outs.append(o)
    if not outs:
        return torch.empty((B, 0, H, dv), dtype=torch.float32, device=S.device)
    return torch.cat(outs, dim=1)


@pytest.mark.parametrize("dk,dv,dt", SHAPES)
def test_decode_matches_oracle(dk, dv, dt):
    spec = spec_for(dk, dv, dt)
    B, n = 3, 40
    say(f"decode dk={dk} dv={dv} {dt} B={B} steps={n}")
    S0 = synth.initial_state(spec, B)
    inp = synth.token_inputs(spec, B, n)
    S = dev_tensor(S0)
    pos = torch.zeros(B, dtype=torch.int64, device="cuda")
    o = decode_run(S, pos, dev_inputs(inp))
    assert kda.last_variant() == "decode"
    S_ref, o_ref = ko.decode(S0, inp, spec.scale)
    assert_parity(o.cpu().numpy(), o_ref, S.cpu().numpy(), S_ref, f"decode {dk}x{dv} {dt}")
    assert pos.cpu().tolist() == [n] * B


@pytest.mark.parametrize("dk,dv,dt", SHAPES)
@pytest.mark.parametrize("T", [1, 3, 4, 5, 8, 16])
def test_verify_commit_matches_oracle_and_decode(dk, dv, dt, T):
    spec = spec_for(dk, dv, dt, tag=101)
    B = 3
    say(f"verify/commit dk={dk} dv={dv} {dt} T={T}")
    S0 = synth.initial_state(spec, B)
    inp = synth.token_inputs(spec, B, T)
    d = dev_inputs(inp)
    S = dev_tensor(S0)
    S_keep = S.clone()
    pos = torch.tensor([7, 0, 3], dtype=torch.int64, device="cuda")
    log = kda.InputLog(S, T_max=16, in_dtype=d["q"].dtype)
    o = torch.empty((B, T, spec.H, dv), dtype=torch.float32, device="cuda")
    kda.verify(S, d["q"], d["k"], d["v"], d["alpha"], d["beta"], o, log)
    assert kda.last_variant() == "verify" and log.pending_T == T
    assert torch.equal(bits(S), bits(S_keep)), "verify must not write the committed state"
    _, o_ref = ko.decode(S0, inp, spec.scale)
    assert_parity(o.cpu().numpy(), o_ref, what=f"verify T={T}")
    # Verify outputs agree with decode steps from the same state to the bar.
    S_dec = S.clone()
    pos_dec = pos.clone()
    o_dec = decode_run(S_dec, pos_dec, d)
    assert_parity(o.cpu().numpy(), o_dec.cpu().numpy().astype(np.float64), what=f"verify vs decode T={T}")
    # Commit a different count per sequence; compare with that many decode steps.
    acc = [T, 0, min(1, T)] if T > 1 else [1, 0, 1]
    accepted = torch.tensor(acc, dtype=torch.int32, device="cuda")
    dev_err = torch.zeros(1, dtype=torch.int32, device="cuda")
    kda.commit(S, pos, log, accepted, dev_err)
    assert kda.last_variant() == "commit" and log.pending_T == 0
    assert dev_err.item() == 0
    for b, a in enumerate(acc):
        Sb = S_keep[b:b + 1].clone()
        pb = torch.zeros(1, dtype=torch.int64, device="cuda")
        decode_run(Sb, pb, {k_: v_[b:b + 1, :a] for k_, v_ in d.items()})
        assert torch.equal(bits(S[b:b + 1]), bits(Sb)), f"commit({a}) != {a} decode steps (seq {b})"
    assert pos.cpu().tolist() == [7 + acc[0], 0 + acc[1], 3 + acc[2]]


@pytest.mark.parametrize("T", [4, 7])
def test_verify_extreme_gates(T):
    # Gates of exactly 0 (a full reset of a key channel), exactly 1, and beta
    # of 0 and 1: the verify's decay products never divide by a cumulative
    # decay, so these stay finite and match the oracle; commit still equals
    # the decode steps bit for bit.
    spec = spec_for(128, 128, "bf16", tag=113)
    B = 2
    inp = synth.token_inputs(spec, B, T)
    rng = np.random.default_rng(5)
    a = inp["alpha"]
    a[rng.random(a.shape) < 0.2] = 0.0
    a[rng.random(a.shape) < 0.2] = 1.0
    bt = inp["beta"]
    bt[:, 0] = 1.0
    bt[:, -1] = 0.0
    S0 = synth.initial_state(spec, B)
    d = dev_inputs(inp)
    S = dev_tensor(S0)
    S_keep = S.clone()
    pos = torch.zeros(B, dtype=torch.int64, device="cuda")
    log = kda.InputLog(S, T_max=T)
    o = torch.empty((B, T, spec.H, 128), dtype=torch.float32, device="cuda")
    kda.verify(S, d["q"], d["k"], d["v"], d["alpha"], d["beta"], o, log)
    assert torch.isfinite(o).all()
    _, o_ref = ko.decode(S0, inp, spec.scale)
    assert_parity(o.cpu().numpy(), o_ref, what=f"verify extreme gates T={T}")
    accepted = torch.tensor([T, T - 1], dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    kda.commit(S, pos, log, accepted, err)
    for b, n in enumerate([T, T - 1]):
        Sb = S_keep[b:b + 1].clone()
        decode_run(Sb, torch.zeros(1, dtype=torch.int64, device="cuda"), {k_: v_[b:b + 1, :n] for k_, v_ in d.items()})
        assert torch.equal(bits(S[b:b + 1]), bits(Sb))


def test_commit_rejects_out_of_range_counts():
    spec = spec_for(128, 128, "bf16", tag=102)
    B, T = 3, 4
    S0 = synth.initial_state(spec, B)
    d = dev_inputs(synth.token_inputs(spec, B, T))
    S = dev_tensor(S0)
    S_keep = S.clone()
    pos = torch.zeros(B, dtype=torch.int64, device="cuda")
    log = kda.InputLog(S, T_max=4)
    o = torch.empty((B, T, spec.H, 128), dtype=torch.float32, device="cuda")
    kda.verify(S, d["q"], d["k"], d["v"], d["alpha"], d["beta"], o, log)
    dev_err = torch.zeros(1, dtype=torch.int32, device="cuda")
    kda.commit(S, pos, log, torch.tensor([-1, 5, 2], dtype=torch.int32, device="cuda"), dev_err)
    assert dev_err.item() == kda.DEV_ERR_ACCEPTED
    assert torch.equal(bits(S[:2]), bits(S_keep[:2])) and not torch.equal(bits(S[2]), bits(S_keep[2]))
    assert pos.cpu().tolist() == [0, 0, 2]


def test_order_errors():
    spec = spec_for(64, 64, "f32", tag=103)
    S = dev_tensor(synth.initial_state(spec, 3))
    pos = torch.zeros(3, dtype=torch.int64, device="cuda")
    d = dev_inputs(synth.token_inputs(spec, 3, 2))
    log = kda.InputLog(S, T_max=2, in_dtype=torch.float32)
    acc = torch.zeros(3, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(kda.KdaError) as ei:
        kda.commit(S, pos, log, acc, err)
    assert ei.value.status == 5
    o = torch.empty((3, 2, spec.H, 64), dtype=torch.float32, device="cuda")
    kda.verify(S, d["q"], d["k"], d["v"], d["alpha"], d["beta"], o, log)
    with pytest.raises(kda.KdaError) as ei:
        kda.verify(S, d["q"], d["k"], d["v"], d["alpha"], d["beta"], o, log)
    assert ei.value.status == 5
    kda.commit(S, pos, log, acc, err)
    torch.cuda.synchronize()


def test_snapshot_restore_bitwise():
    spec = spec_for(128, 128, "bf16", tag=104)
    B = 4
    S = dev_tensor(synth.initial_state(spec, B))
    pos = torch.tensor([11, 22, 33, 44], dtype=torch.int64, device="cuda")
    pool = kda.SlotPool(6, spec.H, 128, 128, "cuda")
    kda.snapshot(S, pos, [2, 0, 3], [5, 1, 1], pool)   # slot 1 written twice: the later pair wins
    assert kda.last_variant() == "snapshot"
    assert torch.equal(bits(pool.states[5]), bits(S[2])) and torch.equal(bits(pool.states[1]), bits(S[3]))
    assert pool.pos.cpu().tolist() == [-1, 44, -1, -1, -1, 33]
    live = torch.zeros_like(S)
    lpos = torch.zeros(B, dtype=torch.int64, device="cuda")
    kda.restore(live, lpos, [0, 3], [5, 1], pool)
    assert kda.last_variant() == "restore"
    assert torch.equal(bits(live[0]), bits(S[2])) and torch.equal(bits(live[3]), bits(S[3]))
    assert not live[1].any() and lpos.cpu().tolist() == [33, 0, 0, 44]
    with pytest.raises(kda.KdaError):
        kda.snapshot(S, pos, [4], [0], pool)
    with pytest.raises(kda.KdaError):
        kda.restore(live, lpos, [0], [6], pool)


def test_snapshot_many_pairs_batches():
    # More pairs than one launch carries: exercises the host-side batching.
    spec = spec_for(64, 64, "f32", tag=105)
    B = 70
    S = torch.randn((B, 2, 64, 64), device="cuda")
    pos = torch.arange(B, dtype=torch.int64, device="cuda")
    pool = kda.SlotPool(B, 2, 64, 64, "cuda")
    kda.snapshot(S, pos, list(range(B)), list(reversed(range(B))), pool)
    assert torch.equal(bits(pool.states), bits(S.flip(0)))
    assert torch.equal(pool.pos, pos.flip(0))


@pytest.mark.parametrize("dk,dv,dt", [(128, 128, "bf16"), (64, 64, "f32"), (64, 128, "bf16")])
@pytest.mark.parametrize("L", [1, 37, 96])
def test_prefill_recurrent_matches_oracle_and_decode(dk, dv, dt, L):
    spec = spec_for(dk, dv, dt, tag=106)
    B = 2
    every = 32
    say(f"prefill_recurrent dk={dk} dv={dv} {dt} L={L}")
    S0 = synth.initial_state(spec, B)
    inp = synth.token_inputs(spec, B, L)
    d = dev_inputs(inp)
    S = dev_tensor(S0)
    pos = torch.tensor([5, 0], dtype=torch.int64, device="cuda")
    n_ck = L // every
    pool = kda.SlotPool(max(1, 2 * n_ck), spec.H, dk, dv, "cuda")
    slots = torch.arange(2 * n_ck, dtype=torch.int32, device="cuda").view(2, n_ck) if n_ck else None
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    o = torch.empty((B, L, spec.H, dv), dtype=torch.float32, device="cuda")
    kda.prefill_recurrent(S, pos, d["q"], d["k"], d["v"], d["alpha"], d["beta"], o, ckpt_every=every,
                          ckpt_slots=slots, pool=pool, dev_err=err)
    assert kda.last_variant() == "prefill_recurrent"
    S_ref, pos_ref, o_ref, ck = ko.prefill(S0, np.array([5, 0]), inp, spec.scale, every)
    assert_parity(o.cpu().numpy(), o_ref, S.cpu().numpy(), S_ref, f"prefill_recurrent L={L}")
    assert pos.cpu().tolist() == pos_ref.tolist() and err.item() == 0
    for m, (Sm, pm) in enumerate(ck):
        for b in range(B):
            slot = b * n_ck + m
            assert_parity(o.cpu().numpy(), o_ref, pool.states[slot:slot + 1].cpu().numpy(), Sm[b:b + 1],
                          f"checkpoint {m} seq {b}")
            assert pool.pos[slot].item() == pm[b]
    # Bit-exact with L decode steps from the same state.
    S2 = dev_tensor(S0)
    decode_run(S2, torch.zeros(B, dtype=torch.int64, device="cuda"), d)
    assert torch.equal(bits(S), bits(S2))


def test_prefill_bad_checkpoint_slot_flags_error():
    spec = spec_for(64, 64, "f32", tag=107)
    B, L = 2, 8
    d = dev_inputs(synth.token_inputs(spec, B, L))
    S = dev_tensor(synth.initial_state(spec, B))
    pos = torch.zeros(B, dtype=torch.int64, device="cuda")
    pool = kda.SlotPool(2, spec.H, 64, 64, "cuda")
    slots = torch.tensor([[0], [9]], dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    o = torch.empty((B, L, spec.H, 64), dtype=torch.float32, device="cuda")
    kda.prefill_recurrent(S, pos, d["q"], d["k"], d["v"], d["alpha"], d["beta"], o, ckpt_every=8,
                          ckpt_slots=slots, pool=pool, dev_err=err)
    assert err.item() == kda.DEV_ERR_CKPT_SLOT
    assert pool.pos.cpu().tolist() == [8, -1]


def test_empty_batch_is_noop():
    S = torch.zeros((0, 2, 64, 64), device="cuda")
    pos = torch.zeros(0, dtype=torch.int64, device="cuda")
    z = lambda *s, dt=torch.float32: torch.zeros(s, dtype=dt, device="cuda")  # noqa: E731
    kda.decode_step(S, pos, z(0, 1, 2, 64), z(0, 1, 2, 64), z(0, 1, 2, 64), z(0, 1, 2, 64), z(0, 1, 2),
                    z(0, 1, 2, 64))


def test_decode_is_deterministic():
    spec = spec_for(128, 128, "bf16", tag=108)
    B = 4
    S0 = dev_tensor(synth.initial_state(spec, B))
    d = dev_inputs(synth.token_inputs(spec, B, 3))
    outs = []
    for _ in range(2):
        S = S0.clone()
        o = decode_run(S, torch.zeros(B, dtype=torch.int64, device="cuda"), d)
        outs.append((bits(S).clone(), bits(o).clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("dk,dv,dt", [(128, 128, "bf16"), (64, 64, "f32"), (64, 128, "bf16"), (128, 64, "f32")])
@pytest.mark.parametrize("chunk", [32, 64])
@pytest.mark.parametrize("L", [1, 37, 64, 200])
def test_prefill_chunked_matches_oracle(dk, dv, dt, chunk, L):
    spec = spec_for(dk, dv, dt, tag=109)
    B = 2
    every = 2 * chunk
    say(f"prefill_chunked dk={dk} dv={dv} {dt} chunk={chunk} L={L}")
    S0 = synth.initial_state(spec, B)
    inp = synth.token_inputs(spec, B, L)
    d = dev_inputs(inp)
    S = dev_tensor(S0)
    pos = torch.tensor([3, 0], dtype=torch.int64, device="cuda")
    n_ck = L // every
    pool = kda.SlotPool(max(1, 2 * n_ck), spec.H, dk, dv, "cuda")
    slots = torch.arange(2 * n_ck, dtype=torch.int32, device="cuda").view(2, n_ck) if n_ck else None
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    o = torch.full((B, L, spec.H, dv), float("nan"), dtype=torch.float32, device="cuda")
    kda.prefill_chunked(S, pos, d["q"], d["k"], d["v"], d["alpha"], d["beta"], o, chunk=chunk, ckpt_every=every,
                        ckpt_slots=slots, pool=pool, dev_err=err)
    assert kda.last_variant() == "prefill_chunked"
    S_ref, pos_ref, o_ref, ck = ko.prefill(S0, np.array([3, 0]), inp, spec.scale, every)
    assert_parity(o.cpu().numpy(), o_ref, S.cpu().numpy(), S_ref, f"prefill_chunked L={L} chunk={chunk}")
    assert pos.cpu().tolist() == pos_ref.tolist() and err.item() == 0
    for m, (Sm, pm) in enumerate(ck):
        for b in range(B):
            slot = b * n_ck + m
            se = state_err(pool.states[slot:slot + 1].cpu().numpy(), Sm[b:b + 1])
            assert se <= 1e-3, f"checkpoint {m} seq {b}: {se:.3e}"
            assert pool.pos[slot].item() == pm[b]


@pytest.mark.parametrize("gate", ["sigmoid", "softplus"])
def test_prefill_chunked_gate_ranges_and_zero_state(gate):
    # Stronger decay (the tiny workload's gates) and a zero initial state.
    spec = synth.ConfigSpec("gates", 111, (2,), 4, 128, 128, "bf16", gate, "zero", 0)
    B, L = 2, 300
    S0 = synth.initial_state(spec, B)
    inp = synth.token_inputs(spec, B, L)
    d = dev_inputs(inp)
    S = dev_tensor(S0)
    pos = torch.zeros(B, dtype=torch.int64, device="cuda")
    o = torch.empty((B, L, spec.H, 128), dtype=torch.float32, device="cuda")
    kda.prefill_chunked(S, pos, d["q"], d["k"], d["v"], d["alpha"], d["beta"], o, chunk=64)
    S_ref, _, o_ref, _ = ko.prefill(S0, np.zeros(B, np.int64), inp, spec.scale, 0)
    assert_parity(o.cpu().numpy(), o_ref, S.cpu().numpy(), S_ref, f"prefill_chunked gate={gate}")


def test_prefill_chunked_then_decode_continues():
    # A prompt processed in two chunked calls equals one call (positions and
    # state carry over), and decode continues from it.
    spec = spec_for(128, 128, "bf16", tag=112)
    B, L1, L2 = 2, 96, 70
    S0 = synth.initial_state(spec, B)
    inp = synth.token_inputs(spec, B, L1 + L2 + 3)
    d = dev_inputs(inp)
    S = dev_tensor(S0)
    pos = torch.zeros(B, dtype=torch.int64, device="cuda")
    part = lambda t0, t1: {k_: v_[:, t0:t1].contiguous() for k_, v_ in d.items()}  # noqa: E731
    o1 = torch.empty((B, L1, spec.H, 128), device="cuda")
    o2 = torch.empty((B, L2, spec.H, 128), device="cuda")
    p1, p2 = part(0, L1), part(L1, L1 + L2)
    kda.prefill_chunked(S, pos, p1["q"], p1["k"], p1["v"], p1["alpha"], p1["beta"], o1, chunk=32)
    kda.prefill_chunked(S, pos, p2["q"], p2["k"], p2["v"], p2["alpha"], p2["beta"], o2, chunk=64)
    o3 = decode_run(S, pos, part(L1 + L2, L1 + L2 + 3))
    assert pos.cpu().tolist() == [L1 + L2 + 3] * B
    S_ref, o_ref = ko.decode(S0, inp, spec.scale)
    assert_parity(torch.cat([o1, o2, o3], dim=1).cpu().numpy(), o_ref, S.cpu().numpy(), S_ref,
                  "two chunked prefills + decode")


def _log_rows(log, B, T, H, dk, dv, es):
    """The filled rows (t < T) of the four log regions as int tensors, for bitwise comparison."""
    n = log.buf.numel()
    Tm = log.c.T_max
    r = lambda x: (x + 255) // 256 * 256  # noqa: E731
    tok = B * Tm * H
    offs = [0]
    offs.append(r(offs[0] + tok * dk * es))
    offs.append(r(offs[1] + tok * dv * es))
    offs.append(r(offs[2] + tok * dk * 4))
    assert r(offs[3] + tok * 4) <= n
    out = []
    for off, width, e in ((offs[0], dk, es), (offs[1], dv, es), (offs[2], dk, 4), (offs[3], 1, 4)):
        reg = log.buf[off:off + tok * width * e].view(B, Tm, H, width * e)[:, :T]
        out.append(reg.clone())
    return out


@pytest.mark.parametrize("dk,dv,dt", SHAPES)
@pytest.mark.parametrize("T1,T2", [(3, 3), (4, 2), (2, 5), (8, 4)])
def test_commit_verify_equals_commit_then_verify(dk, dv, dt, T1, T2):
    spec = spec_for(dk, dv, dt, tag=114)
    B = 3
    say(f"commit_verify dk={dk} dv={dv} {dt} T1={T1} T2={T2}")
    S0 = synth.initial_state(spec, B)
    inp = synth.token_inputs(spec, B, T1 + T2)
    d = dev_inputs(inp)
    r1 = token_slice(d, 0, T1)
    r2 = {k_: v_.contiguous() for k_, v_ in token_slice(d, T1, T1 + T2).items()}
    r1 = {k_: v_.contiguous() for k_, v_ in r1.items()}
    acc = torch.tensor([T1, 0, min(2, T1)], dtype=torch.int32, device="cuda")
    outs = {}
    for path in ("separate", "fused"):
        S = dev_tensor(S0)
        pos = torch.tensor([5, 0, 2], dtype=torch.int64, device="cuda")
        log = kda.InputLog(S, T_max=8, in_dtype=d["q"].dtype)
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        o1 = torch.empty((B, T1, spec.H, dv), dtype=torch.float32, device="cuda")
        o2 = torch.empty((B, T2, spec.H, dv), dtype=torch.float32, device="cuda")
        kda.verify(S, r1["q"], r1["k"], r1["v"], r1["alpha"], r1["beta"], o1, log)
        if path == "separate":
            kda.commit(S, pos, log, acc, err)
            kda.verify(S, r2["q"], r2["k"], r2["v"], r2["alpha"], r2["beta"], o2, log)
        else:
            kda.commit_verify(S, pos, r2["q"], r2["k"], r2["v"], r2["alpha"], r2["beta"], o2, log, acc, err)
            assert kda.last_variant() == "commit_verify" and log.pending_T == T2
        S_mid = S.clone()
        rows = _log_rows(log, B, T2, spec.H, dk, dv, 2 if dt == "bf16" else 4)
        # Commit the second round too (a different count per sequence).
        acc2 = torch.tensor([1, T2, 0], dtype=torch.int32, device="cuda")
        kda.commit(S, pos, log, acc2, err)
        torch.cuda.synchronize()
        assert err.item() == 0
        outs[path] = (bits(S_mid), bits(o2), rows, bits(S), pos.clone())
    a, b_ = outs["separate"], outs["fused"]
    assert torch.equal(a[0], b_[0]), "committed state differs"
    assert torch.equal(a[1], b_[1]), "verify outputs differ"
    for x, y in zip(a[2], b_[2]):
        assert torch.equal(x, y), "log rows differ"
    assert torch.equal(a[3], b_[3]) and torch.equal(a[4], b_[4])
    # And against the oracle: the second verify's outputs follow the accepted prefix of round 1.
    for bi in range(B):
        a1 = int(acc[bi])
        tok = {k_: np.concatenate([v_[bi:bi + 1, :a1], v_[bi:bi + 1, T1:T1 + T2]], axis=1) for k_, v_ in inp.items()}
        _, o_ref = ko.decode(S0[bi:bi + 1], tok, spec.scale)
        o_gpu = b_[1].view(torch.float32)[bi:bi + 1].cpu().numpy()
        assert_parity(o_gpu, o_ref[:, a1:], what=f"commit_verify seq {bi}")


def test_commit_verify_bad_count_and_nothing_pending():
    spec = spec_for(128, 128, "bf16", tag=115)
    B, T = 2, 4
    S0 = synth.initial_state(spec, B)
    inp = synth.token_inputs(spec, B, 2 * T)
    d = dev_inputs(inp)
    r1 = {k_: v_.contiguous() for k_, v_ in token_slice(d, 0, T).items()}
    r2 = {k_: v_.contiguous() for k_, v_ in token_slice(d, T, 2 * T).items()}
    S = dev_tensor(S0)
    S_keep = S.clone()
    pos = torch.zeros(B, dtype=torch.int64, device="cuda")
    log = kda.InputLog(S, T_max=T)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    o1 = torch.empty((B, T, spec.H, 128), dtype=torch.float32, device="cuda")
    o_ref = torch.empty_like(o1)
    # Nothing pending: a plain verify (no accepted / dev_err needed).
    kda.commit_verify(S, pos, r1["q"], r1["k"], r1["v"], r1["alpha"], r1["beta"], o1, log)
    log2 = kda.InputLog(S, T_max=T)
    kda.verify(S, r1["q"], r1["k"], r1["v"], r1["alpha"], r1["beta"], o_ref, log2)
    assert torch.equal(bits(o1), bits(o_ref)) and torch.equal(bits(S), bits(S_keep))
    assert pos.cpu().tolist() == [0, 0]
    # Count out of range for sequence 1: flagged, sequence 1 untouched, verify still runs from it.
    acc = torch.tensor([2, T + 1], dtype=torch.int32, device="cuda")
    o2 = torch.empty_like(o1)
    kda.commit_verify(S, pos, r2["q"], r2["k"], r2["v"], r2["alpha"], r2["beta"], o2, log, acc, err)
    torch.cuda.synchronize()
    assert err.item() & kda.DEV_ERR_ACCEPTED
    assert torch.equal(bits(S[1]), bits(S_keep[1])) and not torch.equal(bits(S[0]), bits(S_keep[0]))
    assert pos.cpu().tolist() == [2, 0]
    o3 = torch.empty_like(o1)
    log3 = kda.InputLog(S, T_max=T)
    kda.verify(S, r2["q"], r2["k"], r2["v"], r2["alpha"], r2["beta"], o3, log3)
    assert torch.equal(bits(o2), bits(o3))


def test_workgroup_shapes_bit_identical():
    # Large batches run decode and commit with whole-state workgroups, small
    # ones with one-wave workgroups, and the smallest decode (B = 2 here) with
    # one-wave workgroups of 16 value columns; the arithmetic of every column
    # is the same, so a sequence's results do not depend on the batch it ran
    # in, and commit(a) equals a decode steps in every shape.
    spec = synth.ConfigSpec("wg", 117, (16,), 32, 128, 128, "bf16", "softplus", "normal", 0)
    Bbig, T = 16, 3                      # 16 x 32 x 4 = 2,048 slices (>= 1,024): whole-state workgroups
    S0 = synth.initial_state(spec, Bbig)
    inp = synth.token_inputs(spec, Bbig, T)
    d = dev_inputs(inp)
    res = {}
    for B in (Bbig, 2):
        dd = {k_: v_[:B].contiguous() for k_, v_ in d.items()}
        S = dev_tensor(S0[:B])
        pos = torch.zeros(B, dtype=torch.int64, device="cuda")
        o_dec = decode_run(S, pos, dd)
        Sc = dev_tensor(S0[:B])
        posc = torch.zeros(B, dtype=torch.int64, device="cuda")
        log = kda.InputLog(Sc, T_max=T)
        o_v = torch.empty((B, T, spec.H, 128), dtype=torch.float32, device="cuda")
        kda.verify(Sc, dd["q"], dd["k"], dd["v"], dd["alpha"], dd["beta"], o_v, log)
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        kda.commit(Sc, posc, log, torch.full((B,), T, dtype=torch.int32, device="cuda"), err)
        assert err.item() == 0
        assert torch.equal(bits(Sc), bits(S)), f"commit({T}) != {T} decode steps at B={B}"
        res[B] = (bits(S[:2]).clone(), bits(o_dec[:2]).clone())
    assert torch.equal(res[2][0], res[Bbig][0]) and torch.equal(res[2][1], res[Bbig][1])


@pytest.mark.parametrize("T1,T2", [(4, 4), (7, 7)])
def test_commit_verify_large_batch_equals_separate_calls(T1, T2):
    # Batches of 512 (sequence, head) pairs and more take the fused kernel
    # without the replay prefetch that small batches use; both must equal
    # commit followed by verify bit for bit.
    spec = synth.ConfigSpec("cvlarge", 116, (17,), 32, 128, 128, "bf16", "softplus", "normal", 0)
    B = 17
    say(f"commit_verify large batch T1={T1} T2={T2}")
    S0 = synth.initial_state(spec, B)
    d = dev_inputs(synth.token_inputs(spec, B, T1 + T2))
    r1 = {k_: v_[:, :T1].contiguous() for k_, v_ in d.items()}
    r2 = {k_: v_[:, T1:].contiguous() for k_, v_ in d.items()}
    acc = torch.tensor(np.random.default_rng(5).integers(0, T1 + 1, B), dtype=torch.int32, device="cuda")
    outs = {}
    for path in ("separate", "fused"):
        S = dev_tensor(S0)
        pos = torch.zeros(B, dtype=torch.int64, device="cuda")
        log = kda.InputLog(S, T_max=8)
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        o1 = torch.empty((B, T1, spec.H, 128), device="cuda")
        o2 = torch.empty((B, T2, spec.H, 128), device="cuda")
        kda.verify(S, r1["q"], r1["k"], r1["v"], r1["alpha"], r1["beta"], o1, log)
        if path == "separate":
            kda.commit(S, pos, log, acc, err)
            kda.verify(S, r2["q"], r2["k"], r2["v"], r2["alpha"], r2["beta"], o2, log)
        else:
            kda.commit_verify(S, pos, r2["q"], r2["k"], r2["v"], r2["alpha"], r2["beta"], o2, log, acc, err)
        torch.cuda.synchronize()
        assert err.item() == 0
        outs[path] = (bits(S), bits(o2), pos.clone())
    for x, y in zip(outs["separate"], outs["fused"]):
        assert torch.equal(x, y)
