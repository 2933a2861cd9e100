"""GPU parity on the five full-size workloads, in the launch configuration the
benchmark times.

Where the whole run is too large for the fp64 oracle, it is checked on sampled
(sequence, head) pairs: pairs are independent in the recurrence, so the
oracle's result for a pair is exact for that pair at any batch size.

Workloads (seeded, synthetic):
  tiny_decode     B=1, H=4, d=64, fp32 inputs, 256 steps from a zero state
  single_stream   B=1, H=32, d=128, bf16 inputs, 1024 steps
  batched_decode  B in {1..64}, H=32, d=128, bf16, 256 steps each
  spec_verify     B=16, H=32, d=128, bf16, T=4 drafts, 512 verify+commit rounds
  prefill         B=8, H=32, d=128, bf16, 8192-token prompt, checkpoint every
                  1024 tokens into a 64-slot pool, then 128 decode steps resumed
                  from the checkpoint at token 4096
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import recurrent_state_amd as kda
import synth
from oracle import kda_oracle as ko
from tests.kda_testutil import assert_parity, dev_tensor, say, state_err, S_TOL

pytestmark = pytest.mark.gpu

CFG = synth.CONFIGS


def steps_major(inp: dict) -> dict:
    """Device copies in [n][B][H][d] layout, so step t is a contiguous x[t]."""
    out = {}
    for k, v in inp.items():
        t = dev_tensor(v)
        out[k] = t.transpose(0, 1).contiguous()
    return out


def run_decode(S, pos, steps: dict, n: int, keep=None):
    """n decode steps; returns outputs [n][B][H][dv] (or only the `keep` (b, h) pairs)."""
    B, H, _, dv = S.shape
    o = torch.empty((B, H, dv), dtype=torch.float32, device="cuda")
    outs = []
    for t in range(n):
        kda.decode_step(S, pos, steps["q"][t], steps["k"][t], steps["v"][t], steps["alpha"][t], steps["beta"][t], o)
        outs.append(o[keep[0], keep[1]].clone() if keep is not None else o.clone())
    return torch.stack(outs)


def pairs_inputs(inp: dict, bs, hs) -> dict:
    """Oracle inputs for (b, h) pairs: pair p becomes sequence p with one head."""
    return {k: v[bs, :, hs][:, :, None] for k, v in inp.items()}


def test_tiny_decode():
    spec = CFG["tiny_decode"]
    B, n = 1, spec.steps
    say("tiny_decode: generating")
    S0 = synth.initial_state(spec, B)
    inp = synth.token_inputs(spec, B, n)
    S = dev_tensor(S0)
    pos = torch.zeros(B, dtype=torch.int64, device="cuda")
    o = run_decode(S, pos, steps_major(inp), n)
    assert kda.last_variant() == "decode"
    S_ref, o_ref = ko.decode(S0, inp, spec.scale)
    assert_parity(o.permute(1, 0, 2, 3).cpu().numpy(), o_ref, S.cpu().numpy(), S_ref, "tiny_decode")
    assert pos.item() == n


def test_single_stream_decode():
    spec = CFG["single_stream"]
    B, n = 1, spec.steps
    say("single_stream: generating")
    S0 = synth.initial_state(spec, B)
    inp = synth.token_inputs(spec, B, n)
    S = dev_tensor(S0)
    pos = torch.zeros(B, dtype=torch.int64, device="cuda")
    o = run_decode(S, pos, steps_major(inp), n)
    say("single_stream: oracle")
    S_ref, o_ref = ko.decode(S0, inp, spec.scale)
    assert_parity(o.permute(1, 0, 2, 3).cpu().numpy(), o_ref, S.cpu().numpy(), S_ref, "single_stream 1024 steps")


@pytest.fixture(scope="module")
def batched_inputs():
    spec = CFG["batched_decode"]
    Bmax = max(spec.B)
    say("batched_decode: generating B=64 inputs")
    return synth.initial_state(spec, Bmax), synth.token_inputs(spec, Bmax, spec.steps)


@pytest.mark.parametrize("B", CFG["batched_decode"].B)
def test_batched_decode(batched_inputs, B):
    spec = CFG["batched_decode"]
    n = spec.steps
    S0_all, inp_all = batched_inputs
    S0 = S0_all[:B]
    inp = {k: v[:B] for k, v in inp_all.items()}
    rng = np.random.default_rng(1000 + B)
    P = min(8, B * spec.H)
    flat = rng.choice(B * spec.H, size=P, replace=False)
    bs, hs = flat // spec.H, flat % spec.H
    say(f"batched_decode B={B}: pairs {list(zip(bs.tolist(), hs.tolist()))}")
    S = dev_tensor(S0)
    pos = torch.zeros(B, dtype=torch.int64, device="cuda")
    o = run_decode(S, pos, steps_major(inp), n, keep=(torch.as_tensor(bs), torch.as_tensor(hs)))
    S_ref, o_ref = ko.decode(S0[bs, hs][:, None], pairs_inputs(inp, bs, hs), spec.scale)
    o_gpu = o.permute(1, 0, 2).cpu().numpy()[:, :, None]          # [P][n][1][dv]
    assert_parity(o_gpu, o_ref, S[bs, hs].cpu().numpy()[:, None], S_ref, f"batched_decode B={B}")
    assert (pos.cpu().numpy() == n).all()


def test_spec_verify_rounds():
    spec = CFG["spec_verify"]
    B, T, R = spec.B[0], spec.extra["T"], spec.steps
    heads = [0, 17]
    say("spec_verify: generating")
    S0 = synth.initial_state(spec, B)
    inp = synth.token_inputs(spec, B, R * T)
    acc = synth.accepted_counts(spec, B, R, T)
    # Device inputs per round: [R][B][T][H][d], contiguous per round.
    dev = {}
    for k, v in inp.items():
        t = dev_tensor(v)
        t = t.view(B, R, T, *t.shape[2:])
        dev[k] = t.transpose(0, 1).contiguous()
    acc_dev = torch.from_numpy(acc).to("cuda")
    S = dev_tensor(S0)
    pos = torch.zeros(B, dtype=torch.int64, device="cuda")
    log = kda.InputLog(S, T_max=T)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    o = torch.empty((B, T, spec.H, spec.dv), dtype=torch.float32, device="cuda")
    o_keep = []
    for r in range(R):
        kda.verify(S, dev["q"][r], dev["k"][r], dev["v"][r], dev["alpha"][r], dev["beta"][r], o, log)
        o_keep.append(o[:, :, heads].clone())
        kda.commit(S, pos, log, acc_dev[r], err)
    assert err.item() == 0
    assert np.array_equal(pos.cpu().numpy(), acc.sum(axis=0))
    say("spec_verify: oracle on heads", heads)
    Sr = ko.widen(S0[:, heads])
    o_ref = []
    for r in range(R):
        tok = {k: v[:, r * T:(r + 1) * T][:, :, heads] for k, v in inp.items()}
        o_r, log_r = ko.verify(Sr, tok, spec.scale)
        o_ref.append(o_r)
        Sr, _, _ = ko.commit(Sr, np.zeros(B, np.int64), log_r, acc[r])
    o_gpu = torch.stack(o_keep).cpu().numpy()
    assert_parity(o_gpu, np.stack(o_ref), S[:, heads].cpu().numpy(), Sr, "spec_verify 512 rounds")


@pytest.mark.parametrize("variant", ["chunked", "recurrent"])
def test_prefill_checkpoints_and_resume(variant):
    spec = CFG["prefill"]
    B, L, H = spec.B[0], spec.steps, spec.H
    every, rpos, rsteps = spec.extra["ckpt_every"], spec.extra["resume_pos"], spec.extra["resume_steps"]
    n_ck = L // every
    say("prefill: generating 8 x 8192 x 32 inputs")
    S0 = synth.initial_state(spec, B)
    inp = synth.token_inputs(spec, B, L)
    res = synth.token_inputs(spec, B, rsteps, phase=1)
    d = {k: dev_tensor(v) for k, v in inp.items()}
    S = dev_tensor(S0)
    pos = torch.zeros(B, dtype=torch.int64, device="cuda")
    pool = kda.SlotPool(B * n_ck, H, spec.dk, spec.dv, "cuda")
    slots = torch.arange(B * n_ck, dtype=torch.int32, device="cuda").view(B, n_ck)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    o = torch.empty((B, L, H, spec.dv), dtype=torch.float32, device="cuda")
    say(f"prefill ({variant}): GPU")
    if variant == "chunked":
        kda.prefill_chunked(S, pos, d["q"], d["k"], d["v"], d["alpha"], d["beta"], o, chunk=spec.extra["chunk"],
                            ckpt_every=every, ckpt_slots=slots, pool=pool, dev_err=err)
    else:
        kda.prefill_recurrent(S, pos, d["q"], d["k"], d["v"], d["alpha"], d["beta"], o, ckpt_every=every,
                              ckpt_slots=slots, pool=pool, dev_err=err)
    torch.cuda.synchronize()
    assert kda.last_variant() == f"prefill_{variant}"
    assert err.item() == 0 and pos.cpu().tolist() == [L] * B
    m_res = rpos // every - 1
    kda.restore(S, pos, list(range(B)), [b * n_ck + m_res for b in range(B)], pool)
    assert pos.cpu().tolist() == [rpos] * B
    rng = np.random.default_rng(7)
    flat = rng.choice(B * H, size=6, replace=False)
    bs, hs = flat // H, flat % H
    o_res = run_decode(S, pos, steps_major(res), rsteps, keep=(torch.as_tensor(bs), torch.as_tensor(hs)))
    say(f"prefill: oracle on pairs {list(zip(bs.tolist(), hs.tolist()))}")
    S_ref, _, o_ref, ck = ko.prefill(S0[bs, hs][:, None], np.zeros(len(bs), np.int64), pairs_inputs(inp, bs, hs),
                                     spec.scale, every)
    o_gpu = o[torch.as_tensor(bs), :, torch.as_tensor(hs)].cpu().numpy()[:, :, None]
    assert_parity(o_gpu, o_ref, what="prefill outputs (8192 tokens)")
    for m, (Sm, pm) in enumerate(ck):
        slot_ids = torch.as_tensor(bs * n_ck + m)
        se = state_err(pool.states[slot_ids, torch.as_tensor(hs)].cpu().numpy()[:, None], Sm)
        assert se <= S_TOL, f"checkpoint {m}: state rel err {se:.3e}"
        assert pool.pos[slot_ids].cpu().tolist() == [every * (m + 1)] * len(bs)
    say("prefill: oracle resume")
    S_res, o_res_ref = ko.decode(ck[m_res][0], pairs_inputs(res, bs, hs), spec.scale)
    assert_parity(o_res.permute(1, 0, 2).cpu().numpy()[:, :, None], o_res_ref,
                  S[torch.as_tensor(bs), torch.as_tensor(hs)].cpu().numpy()[:, None], S_res,
                  "resume 128 decode steps from token 4096")
