#!/usr/bin/env python3
"""Benchmark of the KDA recurrent-state hot path on one MI355X.

Headline (`value`): decode state-updates per second (tokens x heads / s) for
B = 64 sequences, H = 32 heads, dk = dv = 128, bf16 q/k/v, fp32 state.  One
step is one decode token through L_LAYERS independent layer states (1 GiB in
total, four times the Infinity Cache), i.e. L_LAYERS kda_decode_step launches,
so every launch streams its state from HBM as a multi-layer model would.

`rows` reports the other parts of the path, each against its own roofline:
the decode batch sweep B = 1..64, speculative verify (T = 4) and commit,
snapshot/restore, the prompt prefill with checkpoints (B = 8, L = 8192), mixed
batches (decode, speculative rounds and prompt segments in one launch, against
the standalone kernels one after another), and a measured device-to-device
copy for reference.  `roofline` is the decode
kernel's: algorithmic bytes per launch / measured average launch time.
`cpu_baseline` times the fp64 oracle on a bounded sample of the headline
workload on the host.

Timing: every figure is the median of 5 samples of at least 200 ms each
(HIP events on the launch stream); the headline's samples are whole blocks of
the K steps asked for, and its first K-step block is reported beside them.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick] [--no-cpu]
                       [--rows decode,spec,slots,prefill,mixed] [--samples N] [--min-sample-ms M]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
B_HEAD, H, DK, DV = 64, 32, 128, 128
L_LAYERS = 8                   # 8 x 128 MiB of state per step
N_TOKENS_IN = 16               # distinct seeded input tokens cycled through the timed steps
STEPS_PER_GRAPH = 8            # decode steps captured in one HIP graph (N_TOKENS_IN is a multiple)
SCALE = DK ** -0.5

# Algorithmic bytes per unit (bf16 q/k/v, fp32 alpha/beta/o/state; dk = dv = 128).
STATE_BYTES = DK * DV * 4
DECODE_BYTES = 2 * STATE_BYTES + 3 * 128 * 2 + 128 * 4 + 4 + 128 * 4        # 132,868 per state-update
TOKEN_IN_BYTES = 3 * 128 * 2 + 128 * 4 + 4                                    # 1,284: q, k, v, alpha, beta
LOG_BYTES = 128 * 2 * 2 + 128 * 4 + 4                                         # 1,028: k, v, alpha, beta copy
PREFILL_BYTES_PER_TOKEN_HEAD = TOKEN_IN_BYTES + 128 * 4                       # + o; state and ckpts added per run


MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_sha() -> str:
    h = hashlib.sha256()
    for f in ("kda_common.h", "kda_state.hip"):
        with open(os.path.join(ROOT, "recurrent_state_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def counted_traffic():
    """HBM bytes per decode launch from the committed rocprofv3 counter summary,
    or None when the decode kernel's source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "decode_b64_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_src_sha") != kernel_sha():
        return None
    return t.get("hbm_bytes_per_launch")


class Timer:
    """HIP events on the current stream (the stream the library launches on)."""

    def __init__(self, torch):
        self.torch = torch
        self.a = torch.cuda.Event(enable_timing=True)
        self.b = torch.cuda.Event(enable_timing=True)

    def __enter__(self):
        self.torch.cuda.synchronize()
        self.a.record()
        return self

    def __exit__(self, *exc):
        self.b.record()
        self.torch.cuda.synchronize()
        self.ms = self.a.elapsed_time(self.b)


MIN_SAMPLE_MS = 200.0   # each timed sample lasts at least this long
N_SAMPLES = 5           # samples per figure; the median is reported


def sampled(torch, run, unit, min_units=1):
    """Median time per unit over N_SAMPLES samples of at least MIN_SAMPLE_MS.

    run(n) enqueues n units of work back to back (no synchronisation); the
    first call calibrates how many units one sample needs.  Returns
    (median ms per unit, {"count", "units_per_sample", "unit", "ms_per_unit"}).
    """
    with Timer(torch) as tm:
        run(min_units)
    per = max(tm.ms / min_units, 1e-6)
    n = max(min_units, int(np.ceil(MIN_SAMPLE_MS / per)))
    ms = []
    for _ in range(N_SAMPLES):
        with Timer(torch) as tm:
            run(n)
        ms.append(tm.ms / n)
    return float(np.median(ms)), {"count": N_SAMPLES, "units_per_sample": n, "unit": unit, "ms_per_unit": ms}


def dev_tensor(torch, x, device):
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def decode_inputs(torch, kda_synth, B, n, device, raw=False):
    """n seeded tokens in [n][B][H][d] layout (token t is a contiguous slice);
    with raw, the un-prepared projections and logits of the same draws, under
    the names of the prepared inputs."""
    spec = kda_synth.CONFIGS["batched_decode"]
    if raw:
        r = kda_synth.raw_token_inputs(spec, B, n)
        inp = {"q": r["q"], "k": r["k"], "v": r["v"], "alpha": r["alpha_logit"], "beta": r["beta_logit"]}
    else:
        inp = kda_synth.token_inputs(spec, B, n)
    return {k: dev_tensor(torch, v, device).transpose(0, 1).contiguous() for k, v in inp.items()}


def capture(torch, fns):
    """A HIP graph of the given launches (no kernel runs during capture)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in fns:
            f()
    return g


def bench_decode(torch, kda, synth, B, layers, steps, warmup, device, use_graph=True, prep=False):
    """Decode through `layers` independent states per step; returns timing dict.

    Step s uses seeded input token s mod 16 for every layer.  With use_graph,
    the launches are replayed from captured HIP graphs (how a serving loop
    drives per-step work), eight steps per graph where the step count allows:
    a model step's graph holds every kernel of the step, so the gap between
    two graph launches is spread over far more work than these layer states'
    launches alone, and timing one graph per step would count that gap against
    the kernel.  Otherwise the launches are issued eagerly from plans.
    With prep, the launches take raw projections and logits and prepare them
    in the kernel (decode_step_prep); the bytes moved are the same.
    """
    spec = synth.CONFIGS["batched_decode"]
    inp = decode_inputs(torch, synth, B, N_TOKENS_IN, device, raw=prep)
    gate = kda.GATE_EXP_NEG_SOFTPLUS if prep else None
    S0 = dev_tensor(torch, synth.initial_state(spec, B), device)
    states = [S0.clone() for _ in range(layers)]
    pos = torch.zeros(B, dtype=torch.int64, device=device)
    o = torch.empty((B, H, DV), dtype=torch.float32, device=device)
    plans = [[kda.DecodePlan(S, pos, inp["q"][t], inp["k"][t], inp["v"][t], inp["alpha"][t], inp["beta"][t], o,
                             prep_gate=gate)
              for S in states] for t in range(N_TOKENS_IN)]
    if use_graph:
        single = [capture(torch, ps) for ps in plans]
        multi = [capture(torch, [f for t in range(t0, t0 + STEPS_PER_GRAPH) for f in plans[t]])
                 for t0 in range(0, N_TOKENS_IN, STEPS_PER_GRAPH)]

        def run(n):  # steps 0 .. n - 1
            s = 0
            while s < n:
                if s % STEPS_PER_GRAPH == 0 and s + STEPS_PER_GRAPH <= n:
                    multi[(s % N_TOKENS_IN) // STEPS_PER_GRAPH].replay()
                    s += STEPS_PER_GRAPH
                else:
                    single[s % N_TOKENS_IN].replay()
                    s += 1
    else:
        def run(n):
            for s in range(n):
                for p in plans[s % N_TOKENS_IN]:
                    p()
    run(warmup)
    # The first timed block is exactly `steps` steps; the reported figure is
    # the median of the samples, each a whole number of `steps`-step blocks.
    with Timer(torch) as tm:
        run(steps)
    first_ms = tm.ms / steps
    step_ms, samples = sampled(torch, lambda n: [run(steps) for _ in range(n)], f"{steps} steps")
    step_ms /= steps
    samples["ms_per_step"] = [x / steps for x in samples.pop("ms_per_unit")]
    launch_us = step_ms * 1e3 / layers
    bytes_per_launch = DECODE_BYTES * B * H
    return {
        "B": B, "layers": layers, "steps": steps, "graph": use_graph,
        "steps_per_graph": STEPS_PER_GRAPH if use_graph else None, "ms_per_step": step_ms,
        "first_block_ms_per_step": first_ms,
        "launch_us": launch_us, "updates_per_s": B * H * layers / (step_ms / 1e3),
        "achieved_GBs": bytes_per_launch / (launch_us * 1e-6) / 1e9,
        "hbm_frac": bytes_per_launch / (launch_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
        "state_bytes_total": layers * B * H * STATE_BYTES, "samples": samples,
    }


def bench_decode_slots(torch, kda, synth, B, layers, steps, warmup, device):
    """Decode on states kept in one slot pool (B * layers slots): layer l of
    step s updates the slots of its own id set, a seeded permutation of the
    pool, so consecutive sequences read scattered 2 MiB slots."""
    spec = synth.CONFIGS["batched_decode"]
    inp = decode_inputs(torch, synth, B, N_TOKENS_IN, device)
    pool = kda.SlotPool(B * layers, H, DK, DV, device)
    S0 = dev_tensor(torch, synth.initial_state(spec, B), device)
    perm = np.random.default_rng(7).permutation(B * layers).astype(np.int32)
    ids = [torch.from_numpy(perm[l * B:(l + 1) * B].copy()).to(device) for l in range(layers)]
    for l in range(layers):
        pool.states[ids[l].long()] = S0
    err = torch.zeros(1, dtype=torch.int32, device=device)
    o = torch.empty((B, H, DV), dtype=torch.float32, device=device)
    graphs = [capture(torch, [kda.DecodeSlotsPlan(ids[l], pool, inp["q"][t], inp["k"][t], inp["v"][t],
                                                  inp["alpha"][t], inp["beta"][t], o, err) for l in range(layers)])
              for t in range(N_TOKENS_IN)]
    for s in range(warmup):
        graphs[s % N_TOKENS_IN].replay()

    def run(n):
        for s in range(n):
            graphs[s % N_TOKENS_IN].replay()

    step_ms, samples = sampled(torch, run, "step", steps)
    launch_us = step_ms * 1e3 / layers
    bytes_per_launch = DECODE_BYTES * B * H
    assert err.item() == 0
    return {"B": B, "layers": layers, "launch_us": launch_us,
            "updates_per_s": B * H * layers / (step_ms / 1e3),
            "hbm_frac": bytes_per_launch / (launch_us * 1e-6) / 1e9 / HBM_PEAK_GBS, "samples": samples}


def bench_verify_commit(torch, kda, synth, B, T, rounds, layers, device):
    """Speculative rounds (verify T drafts, commit the accepted prefix) over
    `layers` independent states; verify and commit are captured as separate
    graphs per round and timed with events recorded between replays."""
    spec = synth.CONFIGS["spec_verify"]
    inp = synth.token_inputs(spec, B, 4 * T)
    d = {}
    for k, v in inp.items():
        t = dev_tensor(torch, v, device)
        d[k] = t.view(B, 4, T, *t.shape[2:]).transpose(0, 1).contiguous()   # [4][B][T][H][d]
    acc_np = synth.accepted_counts(spec, B, rounds, T)
    acc = torch.from_numpy(acc_np).to(device)
    S0 = dev_tensor(torch, synth.initial_state(spec, B), device)
    states = [S0.clone() for _ in range(layers)]
    logs = [kda.InputLog(S0, T_max=T) for _ in range(layers)]
    pos = torch.zeros(B, dtype=torch.int64, device=device)
    err = torch.zeros(1, dtype=torch.int32, device=device)
    o = torch.empty((B, T, H, DV), dtype=torch.float32, device=device)
    vg, cg = [], []
    for r in range(rounds):
        j = r % 4
        vg.append(capture(torch, [kda.VerifyPlan(S, d["q"][j], d["k"][j], d["v"][j], d["alpha"][j], d["beta"][j],
                                                 o, lg) for S, lg in zip(states, logs)]))
        cg.append(capture(torch, [kda.CommitPlan(S, pos, lg, acc[r], err) for S, lg in zip(states, logs)]))
    for r in range(rounds):          # warm-up pass
        vg[r].replay()
        cg[r].replay()

    def one_pass():
        """All rounds once, with events between the verify and commit replays."""
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * rounds + 1)]
        ev[0].record()
        for r in range(rounds):
            vg[r].replay()
            ev[2 * r + 1].record()
            cg[r].replay()
            ev[2 * r + 2].record()
        return ev

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    one_pass()
    torch.cuda.synchronize()
    passes = max(1, int(np.ceil(MIN_SAMPLE_MS / 1e3 / (time.perf_counter() - t0))))
    per_sample = []
    for _ in range(N_SAMPLES):
        evs = [one_pass() for _ in range(passes)]
        torch.cuda.synchronize()
        v = sum(ev[2 * r].elapsed_time(ev[2 * r + 1]) for ev in evs for r in range(rounds))
        c = sum(ev[2 * r + 1].elapsed_time(ev[2 * r + 2]) for ev in evs for r in range(rounds))
        t = sum(ev[0].elapsed_time(ev[-1]) for ev in evs)
        per_sample.append((v / passes, c / passes, t / passes))
    med = lambda i: float(np.median([x[i] for x in per_sample]))  # noqa: E731
    ver_ms, com_ms, tot_ms = med(0), med(1), med(2)
    samples = {"count": N_SAMPLES, "units_per_sample": passes, "unit": f"{rounds} rounds",
               "ms_per_unit": [x[2] for x in per_sample]}
    n_launch = rounds * layers
    ver_bytes = B * H * (STATE_BYTES + T * (TOKEN_IN_BYTES + 128 * 4 + LOG_BYTES))
    com_bytes = float((int((acc_np > 0).sum()) * 2 * STATE_BYTES + int(acc_np.sum()) * LOG_BYTES) * H) * layers
    return {
        "B": B, "T": T, "rounds": rounds, "layers": layers, "mean_accepted": float(acc_np.mean()),
        "verify_us": ver_ms * 1e3 / n_launch, "commit_us": com_ms * 1e3 / n_launch,
        "round_us": tot_ms * 1e3 / n_launch,
        "verify_hbm_frac": ver_bytes * n_launch / (ver_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "commit_hbm_frac": com_bytes / (com_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "round_hbm_frac": (ver_bytes * n_launch + com_bytes) / (tot_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "verified_token_heads_per_s": B * H * n_launch * T / (tot_ms / 1e3),
        "committed_token_heads_per_s": float(acc_np.sum()) * H * layers / (tot_ms / 1e3),
        "samples": samples,
    }


def bench_spec_fused(torch, kda, synth, B, T, rounds, layers, device, fixed_accept=None):
    """Speculative rounds through the fused entry point: each round is one
    launch per layer that commits the previous round's accepted prefix and
    verifies T new drafts (the first round is a plain verify).  Accepted
    counts are the seeded uniform draws, or `fixed_accept` every round."""
    spec = synth.CONFIGS["spec_verify"]
    inp = synth.token_inputs(spec, B, 4 * T)
    d = {}
    for k, v in inp.items():
        t = dev_tensor(torch, v, device)
        d[k] = t.view(B, 4, T, *t.shape[2:]).transpose(0, 1).contiguous()   # [4][B][T][H][d]
    if fixed_accept is None:
        acc_np = synth.accepted_counts(spec, B, rounds + 1, T)
    else:
        acc_np = np.full((rounds + 1, B), fixed_accept, dtype=np.int32)
    acc = torch.from_numpy(acc_np).to(device)
    S0 = dev_tensor(torch, synth.initial_state(spec, B), device)
    states = [S0.clone() for _ in range(layers)]
    logs = [kda.InputLog(S0, T_max=T) for _ in range(layers)]
    pos = torch.zeros(B, dtype=torch.int64, device=device)
    err = torch.zeros(1, dtype=torch.int32, device=device)
    o = torch.empty((B, T, H, DV), dtype=torch.float32, device=device)
    for S, lg in zip(states, logs):     # round 0: nothing pending yet
        kda.commit_verify(S, pos, d["q"][0], d["k"][0], d["v"][0], d["alpha"][0], d["beta"][0], o, lg)
    graphs = []
    for r in range(rounds):
        j = (r + 1) % 4
        graphs.append(capture(torch, [kda.CommitVerifyPlan(S, pos, d["q"][j], d["k"][j], d["v"][j], d["alpha"][j],
                                                           d["beta"][j], o, lg, acc[r], err)
                                      for S, lg in zip(states, logs)]))
    for g in graphs:
        g.replay()

    def run(n):
        for _ in range(n):
            for g in graphs:
                g.replay()

    pass_ms, samples = sampled(torch, run, f"{rounds} rounds")
    n_launch = rounds * layers
    us = pass_ms * 1e3 / n_launch
    a = acc_np[:rounds]
    per_bh = (STATE_BYTES + T * (TOKEN_IN_BYTES + 128 * 4 + LOG_BYTES)) * a.size
    per_bh += int((a > 0).sum()) * STATE_BYTES + int(a.sum()) * LOG_BYTES
    bytes_total = float(per_bh) * H * layers
    return {"B": B, "T": T, "rounds": rounds, "layers": layers, "mean_accepted": float(a.mean()),
            "round_us": us, "hbm_frac": bytes_total / (pass_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "verified_token_heads_per_s": B * H * T / (us * 1e-6),
            "committed_token_heads_per_s": float(a.sum()) * H * layers / (pass_ms * 1e-3), "samples": samples}


def bench_verify_only(torch, kda, synth, B, T, layers, reps, device):
    """Verify alone: T drafts through `layers` independent states per round,
    replayed back to back from one captured graph (each layer has its own log;
    nothing is committed, so the states are only read)."""
    spec = synth.CONFIGS["spec_verify"]
    inp = synth.token_inputs(spec, B, T)
    d = {k: dev_tensor(torch, v, device) for k, v in inp.items()}
    S0 = dev_tensor(torch, synth.initial_state(spec, B), device)
    states = [S0.clone() for _ in range(layers)]
    logs = [kda.InputLog(S0, T_max=T) for _ in range(layers)]
    o = torch.empty((B, T, H, DV), dtype=torch.float32, device=device)
    g = capture(torch, [kda.VerifyPlan(S, d["q"], d["k"], d["v"], d["alpha"], d["beta"], o, lg)
                        for S, lg in zip(states, logs)])
    for _ in range(3):
        g.replay()

    def run(n):
        for _ in range(n):
            g.replay()

    rep_ms, samples = sampled(torch, run, f"{layers} launches", reps)
    us = rep_ms * 1e3 / layers
    ver_bytes = B * H * (STATE_BYTES + T * (TOKEN_IN_BYTES + 128 * 4 + LOG_BYTES))
    return {"B": B, "T": T, "layers": layers, "launch_us": us,
            "verified_token_heads_per_s": B * H * T / (us * 1e-6),
            "hbm_frac": ver_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, "samples": samples}


def bench_prefill(torch, kda, synth, device, variant):
    spec = synth.CONFIGS["prefill"]
    B, L = spec.B[0], spec.steps
    every = spec.extra["ckpt_every"]
    # Timing only: the first 1024 seeded tokens tiled 8x along the prompt (the
    # parity tests use the full 8192-token draw).
    if variant == "chunked_prep":   # raw projections and logits, prepared in the kernel
        r = synth.raw_token_inputs(spec, B, 1024)
        base = {"q": r["q"], "k": r["k"], "v": r["v"], "alpha": r["alpha_logit"], "beta": r["beta_logit"]}
    else:
        base = synth.token_inputs(spec, B, 1024)
    d = {k: dev_tensor(torch, np.concatenate([v] * (L // 1024), axis=1), device) for k, v in base.items()}
    S0 = dev_tensor(torch, synth.initial_state(spec, B), device)
    S = S0.clone()
    pos = torch.zeros(B, dtype=torch.int64, device=device)
    n_ck = L // every
    pool = kda.SlotPool(B * n_ck, H, DK, DV, device)
    slots = torch.arange(B * n_ck, dtype=torch.int32, device=device).view(B, n_ck)
    err = torch.zeros(1, dtype=torch.int32, device=device)
    o = torch.empty((B, L, H, DV), dtype=torch.float32, device=device)
    fn = {"chunked": kda.prefill_chunked, "chunked_prep": kda.prefill_chunked_prep,
          "recurrent": kda.prefill_recurrent}[variant]
    kw = dict(ckpt_every=every, ckpt_slots=slots, pool=pool, dev_err=err)
    if variant != "recurrent":
        kw["chunk"] = spec.extra["chunk"]

    def run(n):  # back-to-back prompts continue from the state the last one left
        for _ in range(n):
            fn(S, pos, d["q"], d["k"], d["v"], d["alpha"], d["beta"], o, **kw)

    run(1)
    best, samples = sampled(torch, run, "prompt")
    th = B * L * H
    total_bytes = th * PREFILL_BYTES_PER_TOKEN_HEAD + B * H * STATE_BYTES * (2 + n_ck)
    row = {"variant": variant, "B": B, "L": L, "ms": best, "token_heads_per_s": th / (best / 1e3),
           "hbm_frac": total_bytes / (best * 1e-3) / 1e9 / HBM_PEAK_GBS, "algorithmic_bytes": total_bytes,
           "samples": samples}
    if variant == "chunked":
        C = spec.extra["chunk"]
        chunks = B * H * (L // C)
        alg, exe = prefill_flops_per_chunk(C, DK, DV)
        row.update({"algorithmic_tflops": alg * chunks / (best * 1e-3) / 1e12,
                    "mfma_executed_tflops": exe * chunks / (best * 1e-3) / 1e12,
                    "mfma_executed_frac": exe * chunks / (best * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                    "mfma_algorithmic_frac": alg * chunks / (best * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS})
    return row


def prefill_flops_per_chunk(C, K, V):
    """(algorithmic, executed) flops of one chunk of one (sequence, head).

    Algorithmic: the chunk form's products counted once, triangular parts
    halved -- A = Diag(beta) Kt Kh^T and P = Qt Kh^T (C^2/2 K each), the two
    triangular applications of (I + A)^-1 (C^2/2 K and C^2/2 V), the inverse
    (C^3/6), Kt S, Qt S and Kb^T E (C K V each) and P E (C^2/2 V); 2 flops per
    multiply-add.  Executed: the v_mfma_f32_16x16x32_bf16 instructions the
    chunked kernel issues (three per fp32-accurate product), 16,384 flops each.
    """
    alg = 2 * (3 * (C * C / 2) * K + (C * C / 2) * V + C ** 3 / 6 + 3 * C * K * V + (C * C / 2) * V)
    NB, KB, MT = C // 16, K // 32, K // 16
    NA = NB * (NB + 1) // 2
    per_wave = 3 * (2 * NB * KB                                                     # X = [Kt; Qt] S
                    + sum(1 + (i > 0) * ((i - 1) // 2 + 1) for i in range(NB))     # block solve
                    + sum(mt // 2 + 1 for mt in range(NB))                         # P E
                    + MT * (NB // 2))                                              # Kb^T E
    mfmas = 3 * 2 * NA * KB + (V // 16) * per_wave                                 # + A and P tiles
    return alg, mfmas * 16384


def bench_mixed(torch, kda, synth, device, n_dec, n_spec, pf_lens, T=4, accept=2, layers=8):
    """A serving step over a mixed batch, one step = every layer's state
    (slot pools of B = n_dec + n_spec + len(pf_lens) sequences, one per layer):
    n_dec sequences decode a token, n_spec run a speculative round (commit of
    `accept` drafts, verify of T new ones) and each prompt segment of pf_lens
    is processed.  Timed two ways on the same inputs, each captured in one
    graph per step: the one-launch mixed step per layer, and the standalone
    kernels (fused commit + verify, decode, one chunked prefill per segment
    length) launched one after another per layer."""
    spec = synth.CONFIGS["spec_verify"]
    roles = ["pf"] * len(pf_lens) + ["spec"] * n_spec + ["dec"] * n_dec
    lens = list(pf_lens) + [T] * n_spec + [1] * n_dec
    B = len(roles)
    code = {"dec": kda.ROLE_DECODE, "spec": kda.ROLE_SPEC, "pf": kda.ROLE_PREFILL}
    start = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    N = int(start[-1])
    inp = synth.token_inputs(spec, 1, N, phase=11)
    packed = {k: dev_tensor(torch, v[0], device) for k, v in inp.items()}          # [N][H][d]
    o = torch.empty((N, H, DV), dtype=torch.float32, device=device)
    roles_dev = torch.tensor([code[r] for r in roles], dtype=torch.int32, device=device)
    start_dev = torch.from_numpy(start).to(device)
    slot_ids = torch.arange(B, dtype=torch.int32, device=device)
    S0 = dev_tensor(torch, synth.initial_state(spec, 1), device)
    err = torch.zeros(1, dtype=torch.int32, device=device)
    acc = torch.tensor([accept if r == "spec" else 0 for r in roles], dtype=torch.int32, device=device)

    def pools():
        out = []
        for _ in range(layers):
            p = kda.SlotPool(B, H, DK, DV, device)
            p.states.copy_(S0.expand(B, -1, -1, -1))
            p.pos.zero_()
            out.append(p)
        return out

    # One launch per layer.
    pool_m = pools()
    logs_m = [kda.InputLog(p.states, T) for p in pool_m]
    counts = (n_dec, n_spec, len(pf_lens))

    def mixed_layer(p, lg):
        return lambda: kda.mixed_step(p.states, p.pos, roles_dev, start_dev, counts, packed["q"], packed["k"],
                                      packed["v"], packed["alpha"], packed["beta"], o, err, log=lg, accepted=acc,
                                      slot_ids=slot_ids)

    for p, lg in zip(pool_m, logs_m):   # a first step leaves drafts pending
        mixed_layer(p, lg)()
    g_mixed = capture(torch, [mixed_layer(p, lg) for p, lg in zip(pool_m, logs_m)])

    # The standalone kernels per layer: sub-batches by role, inputs copied into
    # their dense layouts once.
    pool_s = pools()
    spec_ids = slot_ids[len(pf_lens):len(pf_lens) + n_spec].contiguous()
    dec_ids = slot_ids[len(pf_lens) + n_spec:].contiguous()
    rows = lambda b: slice(int(start[b]), int(start[b + 1]))  # noqa: E731
    sp = {k: torch.stack([v[rows(len(pf_lens) + i)] for i in range(n_spec)]).contiguous() for k, v in packed.items()}
    dc = {k: torch.stack([v[rows(len(pf_lens) + n_spec + i)] for i in range(n_dec)]).contiguous()
          for k, v in packed.items()}
    by_len = {}
    for i, n in enumerate(pf_lens):
        by_len.setdefault(n, []).append(i)
    pf = {n: ({k: torch.stack([v[rows(i)] for i in ix]).contiguous() for k, v in packed.items()},
              slot_ids[ix].contiguous(), torch.empty((len(ix), n, H, DV), dtype=torch.float32, device=device))
          for n, ix in by_len.items()}
    o_sp = torch.empty((n_spec, T, H, DV), dtype=torch.float32, device=device)
    o_dc = torch.empty((n_dec, 1, H, DV), dtype=torch.float32, device=device)
    logs_s = [kda.InputLog(p.states[:n_spec], T) for p in pool_s]
    acc_s = torch.full((n_spec,), accept, dtype=torch.int32, device=device)

    def separate_layer(p, lg):
        def f():
            kda.commit_verify_slots(spec_ids, p, sp["q"], sp["k"], sp["v"], sp["alpha"], sp["beta"], o_sp, lg, err,
                                    accepted=acc_s)
            kda.decode_step_slots(dec_ids, p, dc["q"], dc["k"], dc["v"], dc["alpha"], dc["beta"], o_dc, err)
            for n, (d, ids, o_pf) in pf.items():
                kda.prefill_chunked_slots(ids, p, d["q"], d["k"], d["v"], d["alpha"], d["beta"], o_pf, err, chunk=64)
        return f

    for p, lg in zip(pool_s, logs_s):
        kda.verify_slots(spec_ids, p, sp["q"], sp["k"], sp["v"], sp["alpha"], sp["beta"], o_sp, lg, err)
    g_sep = capture(torch, [separate_layer(p, lg) for p, lg in zip(pool_s, logs_s)])

    def runner(g):
        def run(n):
            for _ in range(n):
                g.replay()
        return run

    for g in (g_mixed, g_sep):
        g.replay()
    ms_m, samp_m = sampled(torch, runner(g_mixed), f"step of {layers} layers")
    ms_s, samp_s = sampled(torch, runner(g_sep), f"step of {layers} layers")
    torch.cuda.synchronize()
    if err.item() != 0:
        raise RuntimeError(f"mixed bench: device error flags {err.item()}")
    per_layer = (n_dec * DECODE_BYTES
                 + n_spec * (2 * STATE_BYTES + T * (TOKEN_IN_BYTES + 128 * 4 + LOG_BYTES) + accept * LOG_BYTES)
                 + sum(2 * STATE_BYTES + n * PREFILL_BYTES_PER_TOKEN_HEAD for n in pf_lens)) * H
    return {"B": B, "decode": n_dec, "spec": n_spec, "T": T, "accepted": accept, "prompt_segments": list(pf_lens),
            "layers": layers, "mixed_us_per_layer": ms_m * 1e3 / layers, "separate_us_per_layer": ms_s * 1e3 / layers,
            "speedup": ms_s / ms_m, "mixed_hbm_frac": per_layer * layers / (ms_m * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "algorithmic_bytes_per_layer": per_layer, "samples_mixed": samp_m, "samples_separate": samp_s}


def bench_snapshot_restore(torch, kda, synth, device, reps=20):
    B, n_slots = 64, 64
    S = torch.randn((B, H, DK, DV), device=device)
    pos = torch.arange(B, dtype=torch.int64, device=device)
    pool = kda.SlotPool(n_slots, H, DK, DV, device)
    ids = list(range(B))
    kda.snapshot(S, pos, ids, ids, pool)
    snap_ms, s_samples = sampled(torch, lambda n: [kda.snapshot(S, pos, ids, ids, pool) for _ in range(n)],
                                 "snapshot", reps)
    rest_ms, r_samples = sampled(torch, lambda n: [kda.restore(S, pos, ids, ids, pool) for _ in range(n)],
                                 "restore", reps)
    nbytes = 2 * B * H * STATE_BYTES
    return {"pairs": B, "snapshot_us": snap_ms * 1e3, "restore_us": rest_ms * 1e3,
            "snapshot_hbm_frac": nbytes / (snap_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "restore_hbm_frac": nbytes / (rest_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "samples": {"snapshot": s_samples, "restore": r_samples}}


def bench_resume(torch, kda, synth, device, steps=128):
    """The prefill workload's resume: restore the 8 sequences' mid-prompt
    checkpoints from a 64-slot pool into the live states, then 128 decode
    steps on fresh tokens (one layer, graph-replayed steps)."""
    spec = synth.CONFIGS["prefill"]
    B = spec.B[0]
    pool = kda.SlotPool(8 * B, H, DK, DV, device)
    pool.states.normal_(0.0, 0.02)
    pool.pos.copy_(torch.arange(8 * B, device=device) * 1024)
    S = torch.zeros((B, H, DK, DV), device=device)
    pos = torch.zeros(B, dtype=torch.int64, device=device)
    inp = decode_inputs(torch, synth, B, N_TOKENS_IN, device)
    o = torch.empty((B, H, DV), dtype=torch.float32, device=device)
    graphs = [capture(torch, [kda.DecodePlan(S, pos, inp["q"][t], inp["k"][t], inp["v"][t], inp["alpha"][t],
                                             inp["beta"][t], o)]) for t in range(N_TOKENS_IN)]
    seqs, slots = list(range(B)), [8 * b + 3 for b in range(B)]   # the checkpoint at token 4096
    kda.restore(S, pos, seqs, slots, pool)
    for s in range(8):
        graphs[s % N_TOKENS_IN].replay()
    rest_ms, r_samples = sampled(torch, lambda n: [kda.restore(S, pos, seqs, slots, pool) for _ in range(n)],
                                 "restore of the 8 checkpoints")

    def resume(n):  # n whole resumes: restore, then the decode steps
        for _ in range(n):
            kda.restore(S, pos, seqs, slots, pool)
            for s in range(steps):
                graphs[s % N_TOKENS_IN].replay()

    tot_ms, samples = sampled(torch, resume, f"restore + {steps} decode steps")
    dec_ms = (tot_ms - rest_ms) / steps
    return {"B": B, "restore_us": rest_ms * 1e3, "decode_steps": steps, "decode_us_per_step": dec_ms * 1e3,
            "total_us": tot_ms * 1e3,
            "decode_hbm_frac": DECODE_BYTES * B * H / (dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "samples": {"restore": r_samples, "resume": samples}}


def bench_copy(torch, device, reps=20):
    n = 1 << 28  # 1 GiB of fp32
    a = torch.empty(n, dtype=torch.float32, device=device).fill_(1.0)
    b = torch.empty_like(a)
    b.copy_(a)
    ms, samples = sampled(torch, lambda k: [b.copy_(a) for _ in range(k)], "1 GiB copy", reps)
    return {"bytes_per_copy": 2 * 4 * n, "GBs": 2 * 4 * n / (ms * 1e-3) / 1e9, "samples": samples}


_CPU = {}  # inputs shared with the forked oracle workers


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_worker(args):
    """Decode steps of the fp64 oracle on sequences [b0, b1), one thread, until `budget_s` passes."""
    b0, b1, budget_s = args
    from threadpoolctl import threadpool_limits

    from oracle import kda_oracle as ko
    inp, S = _CPU["inp"], ko.widen(_CPU["S0"][b0:b1])
    done = 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while True:
            t = done % N_TOKENS_IN
            tok = [ko.widen(inp[n][b0:b1, t]) for n in ("q", "k", "v", "alpha", "beta")]
            S, _ = ko.step(S, *tok, SCALE)
            done += 1
            el = time.perf_counter() - t0
            if el >= budget_s:
                break
    return done * (b1 - b0) * H, el


def cpu_baseline(synth, budget_s=8.0):
    """The fp64 oracle (as it stands) on bounded samples of the headline
    workload, B = 64, H = 32 decode steps: split over the host's cores by
    sequence (one single-threaded worker process per core, each stepping its
    own sequences for `budget_s`), and on one core over all 64 sequences.
    Runs before the GPU is initialised, so the workers fork from a process
    that has not touched it."""
    import multiprocessing as mp

    spec = synth.CONFIGS["batched_decode"]
    _CPU["S0"] = synth.initial_state(spec, B_HEAD)
    _CPU["inp"] = synth.token_inputs(spec, B_HEAD, N_TOKENS_IN)
    cores = max(1, min(len(os.sched_getaffinity(0)), 16, B_HEAD))
    one, el1 = _oracle_worker((0, B_HEAD, budget_s))
    per = B_HEAD // cores
    parts = [(i * per, B_HEAD if i == cores - 1 else (i + 1) * per, budget_s) for i in range(cores)]
    env = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    for k in env:
        os.environ[k] = "1"
    try:
        with mp.get_context("fork").Pool(cores) as pool:
            res = pool.map(_oracle_worker, parts)
    finally:
        for k, v in env.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    updates = sum(u for u, _ in res)
    wall = max(e for _, e in res)
    return {"value": updates / wall, "unit": "state-updates/s", "cores": cores, "kind": "oracle",
            "cpu_model": _cpu_model(), "one_core": {"value": one / el1, "unit": "state-updates/s", "seconds": el1},
            "sample": f"fp64 oracle decode steps of the B=64 x H=32 (dk=dv=128) headline workload: {cores} "
                      f"single-threaded worker processes, one per core, each stepping {per} or more of the 64 "
                      f"sequences for {budget_s:.0f} s ({updates} state-updates); plus one core over all 64 "
                      f"sequences for {el1:.1f} s"}


def main():
    global N_SAMPLES, MIN_SAMPLE_MS
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--quick", action="store_true", help="headline only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--with-copy-ref", action="store_true",
                    help="also run one 256 MiB device copy (known bytes) to scale profiler byte counters")
    ap.add_argument("--samples", type=int, default=5,
                    help="timed samples per figure, median reported (profiling runs: 1)")
    ap.add_argument("--min-sample-ms", type=float, default=200.0,
                    help="minimum length of one sample (profiling runs: 0)")
    ap.add_argument("--rows", default="all",
                    help="comma-separated row groups after the headline: decode, spec, slots, prefill, mixed "
                         "(default all)")
    args = ap.parse_args()
    N_SAMPLES, MIN_SAMPLE_MS = max(1, args.samples), max(0.0, args.min_sample_ms)
    groups = {"decode", "spec", "slots", "prefill", "mixed"}
    picked = groups if args.rows == "all" else set(args.rows.split(","))
    if not picked <= groups:
        ap.error(f"--rows: unknown group(s) {sorted(picked - groups)}")
    if args.gpus != 1:
        print("bench.py measures one GPU: this library's path has no multi-GPU part "
              "(sequences and heads shard with no exchange); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import synth

    # The oracle's CPU baseline runs first: its worker processes fork from
    # this process, which must not have initialised the GPU yet.
    cpu = None if args.no_cpu else cpu_baseline(synth)
    if cpu is not None:
        log(f"cpu baseline: {cpu['value']:.0f} state-updates/s on {cpu['cores']} cores")

    import torch

    import recurrent_state_amd as kda

    kda.lib()  # fails loudly if libkda.so is missing
    device = torch.device("cuda:0")
    torch.cuda.set_device(device)
    props = torch.cuda.get_device_properties(device)
    log(f"device: {props.name}, {props.multi_processor_count} CUs")

    if args.with_copy_ref:
        ref_a = torch.ones(1 << 26, dtype=torch.float32, device=device)   # 256 MiB
        ref_b = torch.empty_like(ref_a)
        ref_b.copy_(ref_a)
        torch.cuda.synchronize()
        log("copy reference: 268435456 bytes read, 268435456 bytes written")
        del ref_a, ref_b

    log("headline: decode B=64 x 8 layers")
    head = bench_decode(torch, kda, synth, B_HEAD, L_LAYERS, args.steps, args.warmup, device)
    rows = {}
    if not args.quick and "decode" in picked:
        log("headline workload launched eagerly (no graph)")
        rows["decode_b64_eager"] = bench_decode(torch, kda, synth, B_HEAD, L_LAYERS, 100, 10, device,
                                                use_graph=False)
        log("headline workload from raw projections (input preparation in the kernel)")
        rows["decode_prep_b64"] = bench_decode(torch, kda, synth, B_HEAD, L_LAYERS, 100, 10, device, prep=True)
        log("headline workload on states in a slot pool (scattered slot ids)")
        rows["decode_slots_b64"] = bench_decode_slots(torch, kda, synth, B_HEAD, L_LAYERS, 100, 10, device)
        log("copy reference")
        rows["d2d_copy_1GiB"] = bench_copy(torch, device)
        log("decode B=64, one layer state (128 MiB)")
        rows["decode_b64_one_layer"] = bench_decode(torch, kda, synth, 64, 1, 400, 40, device)
        sweep = []
        for B in (1, 2, 4, 8, 16, 32, 64):
            layers = max(L_LAYERS, (1 << 30) // (B * H * STATE_BYTES))
            steps = max(10, min(200, int(2e4 // layers)))
            log(f"sweep B={B} layers={layers} steps={steps}")
            sweep.append(bench_decode(torch, kda, synth, B, layers, steps, 3, device))
        rows["decode_sweep"] = sweep
    if not args.quick and "spec" in picked:
        log("verify/commit")
        rows["verify_commit_b16"] = bench_verify_commit(torch, kda, synth, 16, 4, 32, 32, device)
        rows["verify_commit_b64"] = bench_verify_commit(torch, kda, synth, 64, 4, 32, 8, device)
        log("fused commit + verify rounds")
        rows["spec_fused_b16"] = bench_spec_fused(torch, kda, synth, 16, 4, 32, 32, device)
        rows["spec_fused_b64"] = bench_spec_fused(torch, kda, synth, 64, 4, 32, 8, device)
        log("fused rounds, seven drafts with six accepted")
        rows["spec_fused_dl7_al6_b1"] = bench_spec_fused(torch, kda, synth, 1, 7, 8, 512, device, fixed_accept=6)
        rows["spec_fused_dl7_al6_b64"] = bench_spec_fused(torch, kda, synth, 64, 7, 16, 8, device, fixed_accept=6)
        log("verify alone")
        rows["verify_only_b16"] = bench_verify_only(torch, kda, synth, 16, 4, 32, 20, device)
        rows["verify_only_b64"] = bench_verify_only(torch, kda, synth, 64, 4, 8, 50, device)
    if not args.quick and "slots" in picked:
        log("snapshot/restore")
        rows["snapshot_restore"] = bench_snapshot_restore(torch, kda, synth, device)
        log("resume from a mid-prompt checkpoint")
        rows["resume_b8"] = bench_resume(torch, kda, synth, device)
    if not args.quick and "prefill" in picked:
        log("prefill")
        for variant in ("chunked", "chunked_prep", "recurrent"):
            rows[f"prefill_{variant}"] = bench_prefill(torch, kda, synth, device, variant)
    if not args.quick and "mixed" in picked:
        log("mixed batches: one launch against the standalone kernels")
        rows["mixed_b64_pf200"] = bench_mixed(torch, kda, synth, device, 55, 8, [200])
        rows["mixed_b64_pf4x512"] = bench_mixed(torch, kda, synth, device, 52, 8, [512] * 4)
        rows["mixed_b16_pf200"] = bench_mixed(torch, kda, synth, device, 11, 4, [200], layers=16)

    bytes_per_launch = DECODE_BYTES * B_HEAD * H
    line = {
        "metric": "KDA state-updates/s (tokens*heads/s) and % HBM roofline, B=1..64, 1 GPU",
        "value": head["updates_per_s"],
        "unit": "state-updates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "samples": head["samples"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded generator: unit-norm Gaussian q/k, N(0,1) v, exp(-softplus(N(-4,1))) gates, "
                "sigmoid(N(0,1)) beta, N(0,0.02) initial state)",
        "config": {"workload": "batched decode, B=64, H=32, dk=dv=128, bf16 q/k/v, fp32 state; one step = one "
                               "token through 8 independent layer states (1 GiB)",
                   "B": B_HEAD, "H": H, "dk": DK, "dv": DV, "layers": L_LAYERS, "in_dtype": "bf16",
                   "steps_per_graph": STEPS_PER_GRAPH},
        "device": {"name": props.name, "compute_units": props.multi_processor_count,
                   "memory_bytes": props.total_memory},
        "roofline": {"bound": "hbm", "kernel": "decode_kernel<128,128,bf16,4,false,false,4>",
                     "achieved": head["achieved_GBs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": head["achieved_GBs"] / HBM_PEAK_GBS, "traffic": counted_traffic(),
                     "algorithmic_bytes_per_launch": bytes_per_launch, "launch_us": head["launch_us"]},
        "cpu_baseline": cpu,
        "rows": rows,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
