"""The seeded input generator: determinism, subset slicing, rounding, distributions."""

from __future__ import annotations

import numpy as np
import torch

import synth

SPEC = synth.ConfigSpec("t", 93, (4,), 3, 16, 8, "bf16", "softplus", "normal", 0)


def test_bf16_rounding_matches_torch():
    r = np.random.default_rng(0)
    x = np.concatenate([r.standard_normal(100000).astype(np.float32) * 10.0 ** r.integers(-30, 30, 100000),
                        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, 1e-40], np.float32)]).astype(np.float32)
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = synth.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_deterministic_and_subset_equals_slice():
    a = synth.token_inputs(SPEC, 4, 7)
    b = synth.token_inputs(SPEC, 4, 7)
    sub = synth.token_inputs(SPEC, 4, 7, seqs=[3, 1], heads=[2])
    for n in a:
        assert np.array_equal(a[n], b[n])
        assert np.array_equal(sub[n], a[n][[3, 1]][:, :, [2]])
    s_full = synth.initial_state(SPEC, 4)
    assert np.array_equal(synth.initial_state(SPEC, 4, seqs=[2], heads=[0, 2]), s_full[[2]][:, [0, 2]])


def test_worker_count_does_not_change_values():
    spec = synth.ConfigSpec("w", 94, (2,), 4, 128, 128, "bf16", "softplus", "normal", 0)
    a = synth.token_inputs(spec, 2, 4200, workers=1)
    b = synth.token_inputs(spec, 2, 4200, workers=3)
    for n in a:
        assert np.array_equal(a[n], b[n])


def test_distributions():
    spec = synth.ConfigSpec("d", 95, (2,), 4, 128, 128, "bf16", "softplus", "normal", 0)
    x = synth.token_inputs(spec, 2, 512)
    k = synth.bf16_bits_to_f32(x["k"]).astype(np.float64)
    nk = np.linalg.norm(k, axis=-1)
    assert np.all(np.abs(nk - 1.0) < 4e-3)            # unit norm up to bf16 rounding
    a = x["alpha"]
    assert np.all((a > 0) & (a < 1)) and 0.96 < a.mean() < 0.99
    be = x["beta"]
    assert np.all((be > 0) & (be < 1)) and abs(be.mean() - 0.5) < 0.02
    s = synth.initial_state(spec, 2)
    assert abs(s.std() - 0.02) < 5e-4
    t0 = synth.CONFIGS["tiny_decode"]
    y = synth.token_inputs(t0, 1, 64)
    assert y["q"].dtype == np.float32 and np.allclose(np.linalg.norm(y["q"], axis=-1), 1.0, atol=1e-6)
    assert 0.85 < y["alpha"].mean() < 0.95              # sigmoid(N(3, 1))
    assert not synth.initial_state(t0, 1).any()
    acc = synth.accepted_counts(synth.CONFIGS["spec_verify"], 16, 512, 4)
    assert acc.min() == 0 and acc.max() == 4 and abs(acc.mean() - 2.0) < 0.1
