"""Pins for two oracle pieces the step pins do not reach: how stored inputs are
widened, and where each output lands in the [B][n][H][dv] layout.

* ``widen`` treats uint16 arrays as bfloat16 bit patterns.  It is checked
  against hand-built bit patterns (their values follow from the bfloat16
  format: sign, 8 exponent bits with bias 127, 7 fraction bits) and against
  torch's own bfloat16 -> float32 conversion, an implementation that shares
  nothing with the oracle.
* ``decode`` and ``prefill`` return outputs as [B][n][H][dv].  They are checked
  against a hand-indexed run: the scalar-loop step (oracle/kda_scalar.py, nested
  Python lists) applied per (b, h) in token order, each output written to
  o[b, t, h] by explicit indices.

Planted mistakes at the end (a widening that reads the bit patterns as
integers, and outputs left in the oracle's internal [B][H][n][dv] order) must
each fail one of these pins.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from oracle import kda_oracle as ko
from oracle import kda_scalar

# (bit pattern, value) pairs written out from the bfloat16 format.
BF16_HAND = [
    (0x0000, 0.0),
    (0x3F80, 1.0),                     # exponent 127, fraction 0
    (0xBF80, -1.0),
    (0x4000, 2.0),                     # exponent 128
    (0xC040, -3.0),                    # -(1 + 1/2) * 2
    (0x3F00, 0.5),
    (0x3FC0, 1.5),
    (0x4120, 10.0),                    # (1 + 1/4) * 8
    (0x3DCD, 0.10009765625),           # (1 + 77/128) * 2^-4
    (0x7F7F, (2.0 - 2.0 ** -7) * 2.0 ** 127),   # largest finite
    (0x0080, 2.0 ** -126),             # smallest normal
    (0x0001, 2.0 ** -133),             # smallest subnormal: 2^-7 * 2^-126
]


def check_widen(widen):
    bits = np.array([b for b, _ in BF16_HAND], np.uint16)
    got = widen(bits)
    assert got.dtype == np.float64
    assert got.tolist() == [v for _, v in BF16_HAND]
    special = widen(np.array([0x8000, 0x7F80, 0xFF80, 0x7FC0], np.uint16))
    assert np.signbit(special[0]) and special[0] == 0.0, "0x8000 is -0.0"
    assert special[1] == np.inf and special[2] == -np.inf and np.isnan(special[3])
    # Every finite bit pattern against torch's conversion.
    every = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(every.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    with np.errstate(invalid="ignore"):  # the NaN patterns
        w = widen(every)
    fin = np.isfinite(ref)
    assert np.array_equal(w[fin], ref[fin])
    assert np.array_equal(np.isnan(w), np.isnan(ref)) and np.array_equal(np.isinf(w), np.isinf(ref))
    # float32 inputs widen exactly (no reinterpretation).
    x = np.array([0.1, -3.5e-39, 7.0e37], np.float32)
    assert widen(x).tolist() == [float(v) for v in x]


def _hand_indexed_run(S0, inp, scale):
    """Scalar-loop steps per (b, h) in token order; output of token t of (b, h) at o[b, t, h]."""
    B, n, H = inp["k"].shape[:3]
    dv = inp["v"].shape[-1]
    o = np.full((B, n, H, dv), np.nan)
    S_out = np.empty(np.asarray(S0).shape)
    for b in range(B):
        for h in range(H):
            S = np.asarray(S0[b, h], np.float64).tolist()
            for t in range(n):
                tok = [np.asarray(inp[name][b, t, h], np.float64) for name in ("q", "k", "v", "alpha")]
                S, ov = kda_scalar.step(S, *(x.tolist() for x in tok), float(inp["beta"][b, t, h]), scale)
                for j in range(dv):
                    o[b, t, h, j] = ov[j]
            S_out[b, h] = S
    return S_out, o


def _layout_inputs():
    spec = synth.ConfigSpec("layout", 96, (2,), 3, 5, 4, "f32", "sigmoid", "normal", 0)
    B, n = 2, 4
    return spec, synth.initial_state(spec, B), synth.token_inputs(spec, B, n)


def check_decode_layout(decode):
    spec, S0, inp = _layout_inputs()
    S_ref, o_ref = _hand_indexed_run(S0, inp, spec.scale)
    S, o = decode(S0, inp, spec.scale)
    assert o.shape == o_ref.shape == (2, 4, 3, 4)
    assert np.allclose(o, o_ref, rtol=1e-13, atol=1e-14)
    assert np.allclose(S, S_ref, rtol=1e-13, atol=1e-14)


def check_prefill_layout(prefill):
    spec, S0, inp = _layout_inputs()
    S_ref, o_ref = _hand_indexed_run(S0, inp, spec.scale)
    S, pos, o, ckpts = prefill(S0, np.array([7, 0], np.int64), inp, spec.scale, 2)
    assert o.shape == o_ref.shape
    assert np.allclose(o, o_ref, rtol=1e-13, atol=1e-14)
    assert np.allclose(S, S_ref, rtol=1e-13, atol=1e-14)
    assert pos.tolist() == [11, 4] and [c[1].tolist() for c in ckpts] == [[9, 2], [11, 4]]


def test_widen_pins():
    check_widen(ko.widen)


def test_decode_output_layout():
    check_decode_layout(ko.decode)


def test_prefill_output_layout():
    check_prefill_layout(ko.prefill)


# ------------------------------------------------- planted mistakes ----

def m_widen_integer_values(x):
    return np.asarray(x).astype(np.float64)


def m_widen_low_half(x):
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return x.astype(np.uint32).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def m_decode_untransposed(S0, inp, scale):
    S = ko.widen(S0)
    n = inp["k"].shape[1]
    o = np.empty(S.shape[:2] + (n, S.shape[-1]))
    for t in range(n):
        q, k, v, a, b = (ko.widen(inp[name][:, t]) for name in ("q", "k", "v", "alpha", "beta"))
        S, o[:, :, t] = ko.step(S, q, k, v, a, b, scale)
    return S, o.reshape(o.shape[0], n, o.shape[1], o.shape[-1])


def m_prefill_untransposed(S0, pos0, inp, scale, ckpt_every=0):
    S, pos, o, ckpts = ko.prefill(S0, pos0, inp, scale, ckpt_every)
    B, L, H, dv = o.shape
    return S, pos, np.ascontiguousarray(o.transpose(0, 2, 1, 3)).reshape(B, L, H, dv), ckpts


@pytest.mark.parametrize("mutant", [m_widen_integer_values, m_widen_low_half], ids=lambda f: f.__name__)
def test_planted_widen_mistake_fails(mutant):
    with pytest.raises(AssertionError):
        check_widen(mutant)


def test_planted_decode_layout_mistake_fails():
    with pytest.raises(AssertionError):
        check_decode_layout(m_decode_untransposed)


def test_planted_prefill_layout_mistake_fails():
    with pytest.raises(AssertionError):
        check_prefill_layout(m_prefill_untransposed)
