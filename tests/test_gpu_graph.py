"""The library's launches captured in HIP graphs (as a serving loop replays its
per-step work) give the same bits as eager launches.

Each graph is replayed several times with unrelated eager work and host
synchronisation between replays, and every replay is compared with the eager
result of the same step.
"""

from __future__ import annotations

import pytest
import torch

import recurrent_state_amd as kda
import synth
from tests.kda_testutil import bits, dev_tensor, say

pytestmark = pytest.mark.gpu

SPEC = synth.ConfigSpec("graph", 110, (4,), 8, 128, 128, "bf16", "softplus", "normal", 0)


def steps_major(inp):
    return {k: dev_tensor(v).transpose(0, 1).contiguous() for k, v in inp.items()}


def test_decode_graph_replays_match_eager():
    B, layers, n = 4, 3, 6
    say("graph: decode")
    S0 = dev_tensor(synth.initial_state(SPEC, B))
    d = steps_major(synth.token_inputs(SPEC, B, n))
    o_e = torch.empty((B, SPEC.H, 128), device="cuda")
    SA = [S0.clone() for _ in range(layers)]
    posA = torch.zeros(B, dtype=torch.int64, device="cuda")
    ref = []
    for t in range(n):
        for S in SA:
            kda.decode_step(S, posA, d["q"][t], d["k"][t], d["v"][t], d["alpha"][t], d["beta"][t], o_e)
        ref.append(([bits(S).clone() for S in SA], bits(o_e).clone(), posA.clone()))
    SB = [S0.clone() for _ in range(layers)]
    posB = torch.zeros(B, dtype=torch.int64, device="cuda")
    o_g = torch.empty_like(o_e)
    graphs = []
    for t in range(n):
        plans = [kda.DecodePlan(S, posB, d["q"][t], d["k"][t], d["v"][t], d["alpha"][t], d["beta"][t], o_g)
                 for S in SB]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for p in plans:
                p()
        graphs.append(g)
    torch.cuda.synchronize()
    assert posB.sum().item() == 0, "capture must not run the kernels"
    for t in range(n):
        graphs[t].replay()
        junk = torch.randn(1000, device="cuda").cumsum(0)  # unrelated eager work between replays
        torch.cuda.synchronize()
        assert junk.numel() == 1000
        states, o_ref, pos_ref = ref[t]
        for l in range(layers):
            assert torch.equal(bits(SB[l]), states[l]), f"replay {t} layer {l}"
        assert torch.equal(bits(o_g), o_ref) and torch.equal(posB, pos_ref)


def test_verify_commit_graph_replays_match_eager():
    B, T, rounds = 4, 3, 4
    say("graph: verify + commit")
    S0 = dev_tensor(synth.initial_state(SPEC, B))
    d = {k: dev_tensor(v) for k, v in synth.token_inputs(SPEC, B, T).items()}
    counts = [[3, 0, 1, 2], [0, 0, 0, 0], [2, 3, 3, 1], [1, 2, 0, 3]]
    # Eager reference.
    SA = S0.clone()
    posA = torch.zeros(B, dtype=torch.int64, device="cuda")
    logA = kda.InputLog(SA, T_max=T)
    errA = torch.zeros(1, dtype=torch.int32, device="cuda")
    oA = torch.empty((B, T, SPEC.H, 128), device="cuda")
    ref = []
    for r in range(rounds):
        kda.verify(SA, d["q"], d["k"], d["v"], d["alpha"], d["beta"], oA, logA)
        kda.commit(SA, posA, logA, torch.tensor(counts[r], dtype=torch.int32, device="cuda"), errA)
        ref.append((bits(SA).clone(), bits(oA).clone(), posA.clone()))
    # One captured round, replayed with new accepted counts written in between.
    SB = S0.clone()
    posB = torch.zeros(B, dtype=torch.int64, device="cuda")
    logB = kda.InputLog(SB, T_max=T)
    errB = torch.zeros(1, dtype=torch.int32, device="cuda")
    oB = torch.empty_like(oA)
    acc = torch.zeros(B, dtype=torch.int32, device="cuda")
    vp = kda.VerifyPlan(SB, d["q"], d["k"], d["v"], d["alpha"], d["beta"], oB, logB)
    cp = kda.CommitPlan(SB, posB, logB, acc, errB)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        vp()
        cp()
    assert logB.pending_T == 0
    for r in range(rounds):
        acc.copy_(torch.tensor(counts[r], dtype=torch.int32))
        g.replay()
        torch.cuda.synchronize()
        S_ref, o_ref, pos_ref = ref[r]
        assert torch.equal(bits(SB), S_ref) and torch.equal(bits(oB), o_ref) and torch.equal(posB, pos_ref), r
    assert errA.item() == 0 and errB.item() == 0


def test_commit_verify_graph_replays_match_eager():
    # Round r commits counts[r - 1] of the previous round and verifies new drafts;
    # one captured fused round is replayed with new counts written in between.
    B, T, rounds = 4, 3, 4
    say("graph: fused commit + verify")
    S0 = dev_tensor(synth.initial_state(SPEC, B))
    d = {k: dev_tensor(v) for k, v in synth.token_inputs(SPEC, B, T).items()}
    counts = [[3, 0, 1, 2], [0, 0, 0, 0], [2, 3, 3, 1], [1, 2, 0, 3]]
    SA = S0.clone()
    posA = torch.zeros(B, dtype=torch.int64, device="cuda")
    logA = kda.InputLog(SA, T_max=T)
    errA = torch.zeros(1, dtype=torch.int32, device="cuda")
    oA = torch.empty((B, T, SPEC.H, 128), device="cuda")
    kda.commit_verify(SA, posA, d["q"], d["k"], d["v"], d["alpha"], d["beta"], oA, logA)
    ref = []
    for r in range(rounds):
        kda.commit_verify(SA, posA, d["q"], d["k"], d["v"], d["alpha"], d["beta"], oA, logA,
                          torch.tensor(counts[r], dtype=torch.int32, device="cuda"), errA)
        ref.append((bits(SA).clone(), bits(oA).clone(), posA.clone()))
    SB = S0.clone()
    posB = torch.zeros(B, dtype=torch.int64, device="cuda")
    logB = kda.InputLog(SB, T_max=T)
    errB = torch.zeros(1, dtype=torch.int32, device="cuda")
    oB = torch.empty_like(oA)
    acc = torch.zeros(B, dtype=torch.int32, device="cuda")
    kda.commit_verify(SB, posB, d["q"], d["k"], d["v"], d["alpha"], d["beta"], oB, logB)   # round 0, eager
    plan = kda.CommitVerifyPlan(SB, posB, d["q"], d["k"], d["v"], d["alpha"], d["beta"], oB, logB, acc, errB)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan()
    assert logB.pending_T == T
    for r in range(rounds):
        acc.copy_(torch.tensor(counts[r], dtype=torch.int32))
        g.replay()
        junk = torch.randn(1000, device="cuda").cumsum(0)
        torch.cuda.synchronize()
        assert junk.numel() == 1000
        S_ref, o_ref, pos_ref = ref[r]
        assert torch.equal(bits(SB), S_ref) and torch.equal(bits(oB), o_ref) and torch.equal(posB, pos_ref), r
    assert errA.item() == 0 and errB.item() == 0


def test_commit_verify_varlen_graph_replays_match_eager():
    # As above with a draft length per sequence that changes every round.
    B, T, rounds = 4, 4, 4
    say("graph: fused commit + verify, per-sequence draft lengths")
    S0 = dev_tensor(synth.initial_state(SPEC, B))
    d = {k: dev_tensor(v) for k, v in synth.token_inputs(SPEC, B, T).items()}
    lens = [[4, 0, 2, 3], [1, 4, 4, 0], [0, 0, 0, 0], [3, 2, 1, 4]]
    counts = [[4, 0, 1, 3], [1, 2, 4, 0], [0, 0, 0, 0], [2, 2, 0, 4]]   # round r commits within lens[r - 1]
    SA = S0.clone()
    posA = torch.zeros(B, dtype=torch.int64, device="cuda")
    logA = kda.InputLog(SA, T_max=T)
    errA = torch.zeros(1, dtype=torch.int32, device="cuda")
    oA = torch.zeros((B, T, SPEC.H, 128), device="cuda")
    kda.commit_verify_varlen(SA, posA, d["q"], d["k"], d["v"], d["alpha"], d["beta"], oA, logA,
                             torch.tensor(lens[0], dtype=torch.int32, device="cuda"), None, errA)
    ref = []
    for r in range(1, rounds):
        kda.commit_verify_varlen(SA, posA, d["q"], d["k"], d["v"], d["alpha"], d["beta"], oA, logA,
                                 torch.tensor(lens[r], dtype=torch.int32, device="cuda"),
                                 torch.tensor(counts[r - 1], dtype=torch.int32, device="cuda"), errA)
        ref.append((bits(SA).clone(), bits(oA).clone(), posA.clone()))
    SB = S0.clone()
    posB = torch.zeros(B, dtype=torch.int64, device="cuda")
    logB = kda.InputLog(SB, T_max=T)
    errB = torch.zeros(1, dtype=torch.int32, device="cuda")
    oB = torch.zeros_like(oA)
    dl = torch.tensor(lens[0], dtype=torch.int32, device="cuda")
    acc = torch.zeros(B, dtype=torch.int32, device="cuda")
    kda.commit_verify_varlen(SB, posB, d["q"], d["k"], d["v"], d["alpha"], d["beta"], oB, logB, dl, None, errB)
    plan = kda.CommitVerifyPlan(SB, posB, d["q"], d["k"], d["v"], d["alpha"], d["beta"], oB, logB, acc, errB,
                                draft_len=dl)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan()
    for r in range(1, rounds):
        dl.copy_(torch.tensor(lens[r], dtype=torch.int32))
        acc.copy_(torch.tensor(counts[r - 1], dtype=torch.int32))
        g.replay()
        junk = torch.randn(1000, device="cuda").cumsum(0)
        torch.cuda.synchronize()
        assert junk.numel() == 1000
        S_ref, o_ref, pos_ref = ref[r - 1]
        assert torch.equal(bits(SB), S_ref) and torch.equal(bits(oB), o_ref) and torch.equal(posB, pos_ref), r
    assert errA.item() == 0 and errB.item() == 0


def test_prefill_graph_replays_match_eager():
    # The chunk-64 prompt at dk = dv = 128 (the wave-specialised kernel: 1,024
    # threads and 157 KiB of LDS per workgroup) and the chunk-32 one (the
    # single-role kernel) in one graph, with checkpoints; each replay starts
    # from the same state, restored eagerly before it.
    B, L, every = 2, 130, 64
    say("graph: chunked prefill, chunk 64 and 32")
    S0 = dev_tensor(synth.initial_state(SPEC, B))
    d = {k: dev_tensor(v) for k, v in synth.token_inputs(SPEC, B, L).items()}
    n_ck = L // every
    ck = torch.arange(B * n_ck, dtype=torch.int32, device="cuda").view(B, n_ck)
    pos0 = torch.tensor([7, 0], dtype=torch.int64, device="cuda")

    def fresh():
        return ([S0.clone(), S0.clone()], [pos0.clone(), pos0.clone()],
                [kda.SlotPool(B * n_ck, SPEC.H, 128, 128, "cuda") for _ in range(2)],
                [torch.empty((B, L, SPEC.H, 128), device="cuda") for _ in range(2)],
                torch.zeros(1, dtype=torch.int32, device="cuda"))

    def run(S, pos, pools, outs, err):
        for i, chunk in enumerate((64, 32)):
            kda.prefill_chunked(S[i], pos[i], d["q"], d["k"], d["v"], d["alpha"], d["beta"], outs[i], chunk=chunk,
                                ckpt_every=every, ckpt_slots=ck, pool=pools[i], dev_err=err)

    Se, pe, poolse, oe, erre = fresh()
    run(Se, pe, poolse, oe, erre)
    torch.cuda.synchronize()
    assert erre.item() == 0
    Sg, pg, poolsg, og, errg = fresh()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(Sg, pg, poolsg, og, errg)
    torch.cuda.synchronize()
    assert torch.equal(pg[0], pos0), "capture must not run the kernels"
    for rep in range(3):
        for i in range(2):
            Sg[i].copy_(S0)
            pg[i].copy_(pos0)
            og[i].fill_(float("nan"))
            poolsg[i].states.zero_()
        torch.cuda.synchronize()
        g.replay()
        junk = torch.randn(1000, device="cuda").cumsum(0)  # unrelated eager work between replays
        torch.cuda.synchronize()
        assert junk.numel() == 1000 and errg.item() == 0
        for i in range(2):
            assert torch.equal(bits(Sg[i]), bits(Se[i])), f"replay {rep} state (chunk {(64, 32)[i]})"
            assert torch.equal(bits(og[i]), bits(oe[i])), f"replay {rep} outputs (chunk {(64, 32)[i]})"
            assert torch.equal(pg[i], pe[i])
            assert torch.equal(bits(poolsg[i].states), bits(poolse[i].states)), f"replay {rep} checkpoints"
            assert torch.equal(poolsg[i].pos, poolse[i].pos)


def test_prefill_raw_projections_graph_replays_match_eager():
    # The chunk-64 prompt from raw projections (the key waves form the norms
    # and gates, exchanging norm parts through LDS), with checkpoints.
    B, L, every = 2, 130, 64
    say("graph: chunked prefill from raw projections, chunk 64")
    S0 = dev_tensor(synth.initial_state(SPEC, B))
    d = {k: dev_tensor(v) for k, v in synth.raw_token_inputs(SPEC, B, L).items()}
    n_ck = L // every
    ck = torch.arange(B * n_ck, dtype=torch.int32, device="cuda").view(B, n_ck)
    pos0 = torch.tensor([2, 9], dtype=torch.int64, device="cuda")

    def fresh():
        return (S0.clone(), pos0.clone(), kda.SlotPool(B * n_ck, SPEC.H, 128, 128, "cuda"),
                torch.empty((B, L, SPEC.H, 128), device="cuda"), torch.zeros(1, dtype=torch.int32, device="cuda"))

    def run(S, pos, pool, o, err):
        kda.prefill_chunked_prep(S, pos, d["q"], d["k"], d["v"], d["alpha_logit"], d["beta_logit"], o,
                                 gate=kda.GATE_SIGMOID, chunk=64, ckpt_every=every, ckpt_slots=ck, pool=pool,
                                 dev_err=err)

    Se, pe, poole, oe, erre = fresh()
    run(Se, pe, poole, oe, erre)
    torch.cuda.synchronize()
    assert erre.item() == 0
    Sg, pg, poolg, og, errg = fresh()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(Sg, pg, poolg, og, errg)
    torch.cuda.synchronize()
    assert torch.equal(pg, pos0), "capture must not run the kernels"
    for rep in range(3):
        Sg.copy_(S0)
        pg.copy_(pos0)
        og.fill_(float("nan"))
        poolg.states.zero_()
        torch.cuda.synchronize()
        g.replay()
        junk = torch.randn(1000, device="cuda").cumsum(0)  # unrelated eager work between replays
        torch.cuda.synchronize()
        assert junk.numel() == 1000 and errg.item() == 0
        assert torch.equal(bits(Sg), bits(Se)), f"replay {rep} state"
        assert torch.equal(bits(og), bits(oe)), f"replay {rep} outputs"
        assert torch.equal(pg, pe)
        assert torch.equal(bits(poolg.states), bits(poole.states)), f"replay {rep} checkpoints"
        assert torch.equal(poolg.pos, poole.pos)
