"""Pins for the oracle's input preparation (raw projections -> recurrent inputs).

Each function is checked against facts that do not reuse its formula:
hand-derived values (a 3-4-5 vector, gate logits of 0 and ln 3), limits,
exact invariances (scaling by powers of two), and scipy's logistic function
as an independent library implementation of the sigmoid.  A final check
plants plausible mistakes in copies of the preparation and sees each caught.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
from scipy.special import expit

import synth
from oracle import kda_oracle as ko


def test_l2_normalize_hand_values_and_zero():
    x = np.array([[0.0, 3.0, 0.0, -4.0], [0.0, 0.0, 0.0, 0.0], [0.0, 0.0, 2.5, 0.0]])
    y = ko.l2_normalize(x)
    assert np.array_equal(y[0], [0.0, 0.6, 0.0, -0.8])
    assert np.array_equal(y[1], np.zeros(4)), "a zero vector normalises to zero"
    assert np.array_equal(y[2], [0.0, 0.0, 1.0, 0.0])


def test_l2_normalize_unit_norm_direction_and_scale_invariance():
    r = np.random.default_rng(5)
    x = r.standard_normal((200, 128))
    y = ko.l2_normalize(x)
    assert np.max(np.abs(np.linalg.norm(y, axis=1) - 1.0)) < 1e-15
    # Same direction: y . x = ||x||, and the component ratios are kept.
    assert np.allclose(np.sum(y * x, axis=1), np.linalg.norm(x, axis=1), rtol=1e-14, atol=0)
    assert np.allclose(y[:, 1:] * x[:, :1], x[:, 1:] * y[:, :1], rtol=1e-12, atol=1e-15)
    for p in (-40, -3, 7, 60):
        assert np.array_equal(ko.l2_normalize(x * 2.0 ** p), y), f"scaling by 2^{p} must not change the result"


def test_gates_hand_values():
    ln3 = math.log(3.0)
    g = ko.decay_gate(np.array([0.0, ln3, -ln3]), ko.GATE_EXP_NEG_SOFTPLUS)
    assert g[0] == 0.5 and abs(g[1] - 0.25) < 1e-16 and abs(g[2] - 0.75) < 1e-16
    s = ko.decay_gate(np.array([0.0, ln3, -ln3]), ko.GATE_SIGMOID)
    assert s[0] == 0.5 and abs(s[1] - 0.75) < 1e-16 and abs(s[2] - 0.25) < 1e-16
    b = ko.sigmoid(np.array([0.0, ln3]))
    assert b[0] == 0.5 and abs(b[1] - 0.75) < 1e-16


def test_gates_limits_are_exact_and_finite():
    big = np.array([-1e4, -800.0, 800.0, 1e4, -np.inf, np.inf])
    soft = ko.decay_gate(big, ko.GATE_EXP_NEG_SOFTPLUS)     # a large logit closes the gate
    assert soft.tolist() == [1.0, 1.0, 0.0, 0.0, 1.0, 0.0]
    sig = ko.decay_gate(big, ko.GATE_SIGMOID)
    assert sig.tolist() == [0.0, 0.0, 1.0, 1.0, 0.0, 1.0]


def test_gates_match_library_logistic():
    r = np.random.default_rng(6)
    x = np.concatenate([r.normal(-4, 1, 5000), r.normal(3, 1, 5000), r.normal(0, 6, 5000)])
    soft = ko.decay_gate(x, ko.GATE_EXP_NEG_SOFTPLUS)
    assert np.max(np.abs(soft - expit(-x)) / expit(-x)) < 1e-13, "exp(-softplus(x)) = 1 / (1 + e^x)"
    assert np.max(np.abs(ko.decay_gate(x, ko.GATE_SIGMOID) - expit(x)) / expit(x)) < 1e-13
    assert np.max(np.abs(ko.sigmoid(x) - expit(x)) / expit(x)) < 1e-13


def _check_prep(prep_fn):
    spec = synth.CONFIGS["batched_decode"]
    raw = synth.raw_token_inputs(spec, 2, 3)
    for kind, lib in ((ko.GATE_EXP_NEG_SOFTPLUS, lambda x: expit(-x)), (ko.GATE_SIGMOID, expit)):
        p = prep_fn(raw, kind)
        for name in ("q", "k"):
            x = ko.widen(raw[name])
            assert np.max(np.abs(np.linalg.norm(p[name], axis=-1) - 1.0)) < 1e-14, name
            assert np.allclose(np.sum(p[name] * x, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13), name
        assert np.array_equal(p["v"], ko.widen(raw["v"]))
        a = raw["alpha_logit"].astype(np.float64)
        assert np.allclose(p["alpha"], lib(a), rtol=1e-13, atol=0)
        assert np.allclose(p["beta"], expit(raw["beta_logit"].astype(np.float64)), rtol=1e-13, atol=0)


def test_prep_pins():
    _check_prep(ko.prep)


def _mutants():
    def swap_qk(raw, kind):
        p = ko.prep(raw, kind)
        p["q"] = ko.widen(raw["q"]) / np.linalg.norm(ko.widen(raw["k"]), axis=-1, keepdims=True)
        return p

    def gate_sign(raw, kind):
        p = ko.prep(raw, kind)
        p["alpha"] = ko.decay_gate(-ko.widen(raw["alpha_logit"]), kind)
        return p

    def beta_sign(raw, kind):
        p = ko.prep(raw, kind)
        p["beta"] = ko.sigmoid(-ko.widen(raw["beta_logit"]))
        return p

    def norm_squared(raw, kind):
        p = ko.prep(raw, kind)
        k = ko.widen(raw["k"])
        p["k"] = k / np.sum(k * k, axis=-1, keepdims=True)
        return p

    def kinds_swapped(raw, kind):
        return ko.prep(raw, 1 - kind)

    return [swap_qk, gate_sign, beta_sign, norm_squared, kinds_swapped]


@pytest.mark.parametrize("mutant", _mutants(), ids=lambda f: f.__name__)
def test_planted_prep_mistake_fails_a_pin(mutant):
    with pytest.raises(AssertionError):
        _check_prep(mutant)
