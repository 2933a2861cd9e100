"""Pins for the fp64 oracle that do not reuse its formulas.

Each pin checks the token step against something fixed independently of the
oracle's code: a closed form, an invariant, a textbook special case, a
hand-derived worked example, or a brute-force scalar implementation.  The
planted-mistake tests at the end run every pin against deliberately wrong
variants of the step (planted in copies of the oracle, on the CPU) and require
each variant to fail at least one pin.

Pins (the step is the gated delta rule adopted for KDA's recurrent state):
  identity        alpha = 1, beta = 0 leaves S unchanged; o = scale S^T q
  exact_write     alpha = 1, beta = 1, basis key e_i: row i becomes v exactly,
                  and reading with q = e_i returns scale v (read after update)
  unit_key_write  alpha = 1, beta = 1, random unit k: S^T k = v to 1e-13
  decay           beta = 0 for n steps: S_n = Diag(prod alpha) S_0 (dk != dv)
  assoc_memory    alpha = 1, beta = 1, orthonormal keys from S_0 = 0:
                  S_n = sum k_t v_t^T and S_n^T k_t = v_t
  scalar          dk = dv = 1: first-order linear recurrence in closed form
  lms             alpha = 1: one gradient step of 1/2 |S^T k - v|^2 with rate
                  beta (Widrow-Hoff), gradient by central differences
  linearity       (S_0, v) -> S_T is linear; value columns are independent
  norm_bound      |S_t|_F <= |S_{t-1}|_F + beta |k| |v| when |k| <= 1
  worked_example  tests/golden/kda_worked_example.json, bit for bit
  scalar_loops    oracle/kda_scalar.py agrees to 1e-14
"""

from __future__ import annotations

import json
import os

import numpy as np
import pytest

from oracle import kda_oracle as ko
from oracle import kda_scalar

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kda_worked_example.json")


def _rng(seed):
    return np.random.default_rng(seed)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


# ---------------------------------------------------------------- pins ----

def pin_identity(step):
    r = _rng(1)
    S = r.standard_normal((2, 3, 5, 4))
    q, k = r.standard_normal((2, 3, 5)), _unit(r.standard_normal((2, 3, 5)))
    v = r.standard_normal((2, 3, 4))
    St, o = step(S, q, k, v, np.ones((2, 3, 5)), np.zeros((2, 3)), 0.3)
    assert np.array_equal(St, S)
    ref = 0.3 * np.matmul(np.swapaxes(S, -1, -2), q[..., None])[..., 0]
    assert np.allclose(o, ref, rtol=1e-14, atol=1e-14)


def pin_exact_write(step):
    r = _rng(2)
    dk, dv = 6, 4
    S = r.standard_normal((dk, dv))
    v = r.standard_normal(dv)
    for i in range(dk):
        e = np.zeros(dk)
        e[i] = 1.0
        St, o = step(S, e, e, v, np.ones(dk), np.float64(1.0), 0.5)
        assert np.array_equal(St[i], v), "S^T k must equal v exactly for a basis key"
        assert np.array_equal(np.delete(St, i, axis=0), np.delete(S, i, axis=0))
        assert np.array_equal(o, 0.5 * v), "the read must see the updated state"


def pin_unit_key_write(step):
    r = _rng(3)
    for _ in range(20):
        S = r.standard_normal((8, 5))
        k, v = _unit(r.standard_normal(8)), r.standard_normal(5)
        St, _ = step(S, k, k, v, np.ones(8), np.float64(1.0), 1.0)
        assert np.max(np.abs(St.T @ k - v)) <= 1e-13


def pin_decay(step):
    r = _rng(4)
    dk, dv, n = 5, 3, 6
    S0 = r.standard_normal((dk, dv))
    alphas = r.uniform(0.5, 1.0, (n, dk))
    S = S0
    for t in range(n):
        S, _ = step(S, r.standard_normal(dk), _unit(r.standard_normal(dk)), r.standard_normal(dv),
                    alphas[t], np.float64(0.0), 1.0)
    ref = np.prod(alphas, axis=0)[:, None] * S0
    assert np.allclose(S, ref, rtol=1e-14, atol=0)


def pin_assoc_memory(step):
    r = _rng(5)
    dk, dv, n = 6, 4, 5
    Kq, _ = np.linalg.qr(r.standard_normal((dk, dk)))
    K = Kq.T[:n]                                   # n orthonormal keys, one per row
    V = r.standard_normal((n, dv))
    S = np.zeros((dk, dv))
    for t in range(n):
        S, _ = step(S, K[t], K[t], V[t], np.ones(dk), np.float64(1.0), 1.0)
    assert np.allclose(S, K.T @ V, atol=1e-13)
    for t in range(n):
        assert np.allclose(S.T @ K[t], V[t], atol=1e-13)


def pin_scalar(step):
    r = _rng(6)
    n = 40
    al, be = r.uniform(0.2, 1.0, n), r.uniform(0.0, 1.0, n)
    kk, vv = r.uniform(-1.5, 1.5, n), r.standard_normal(n)
    s0 = 0.7
    S = np.array([[s0]])
    for t in range(n):
        S, _ = step(S, np.array([1.0]), np.array([kk[t]]), np.array([vv[t]]), np.array([al[t]]),
                    np.float64(be[t]), 1.0)
    a = al * (1.0 - be * kk * kk)
    b = be * kk * vv
    ref = np.prod(a) * s0 + sum(np.prod(a[t + 1:]) * b[t] for t in range(n))
    assert abs(S[0, 0] - ref) <= 1e-12 * max(1.0, abs(ref))


def pin_lms(step):
    r = _rng(7)
    dk, dv = 5, 4
    S = r.standard_normal((dk, dv))
    k, v = r.standard_normal(dk), r.standard_normal(dv)
    beta = 0.37

    def loss(M):
        d = M.T @ k - v
        return 0.5 * float(d @ d)

    h = 1e-3
    grad = np.zeros_like(S)
    for i in range(dk):
        for j in range(dv):
            Ep = S.copy()
            Ep[i, j] += h
            Em = S.copy()
            Em[i, j] -= h
            grad[i, j] = (loss(Ep) - loss(Em)) / (2 * h)
    St, _ = step(S, k, k, v, np.ones(dk), np.float64(beta), 1.0)
    assert np.allclose(St, S - beta * grad, atol=1e-9)


def pin_linearity(step):
    r = _rng(8)
    dk, dv, n = 6, 5, 7
    ks = _unit(r.standard_normal((n, dk)))
    qs = r.standard_normal((n, dk))
    al = r.uniform(0.3, 1.0, (n, dk))
    be = r.uniform(0.0, 1.0, n)

    def run(S, V):
        os_ = []
        for t in range(n):
            S, o = step(S, qs[t], ks[t], V[t], al[t], np.float64(be[t]), 0.5)
            os_.append(o)
        return S, np.array(os_)

    X, Y = r.standard_normal((dk, dv)), r.standard_normal((dk, dv))
    VX, VY = r.standard_normal((n, dv)), r.standard_normal((n, dv))
    lam, mu = 0.3, -1.7
    SZ, OZ = run(lam * X + mu * Y, lam * VX + mu * VY)
    SX, OX = run(X, VX)
    SY, OY = run(Y, VY)
    assert np.allclose(SZ, lam * SX + mu * SY, atol=1e-12)
    assert np.allclose(OZ, lam * OX + mu * OY, atol=1e-12)
    perm = r.permutation(dv)
    SP, OP = run(X[:, perm], VX[:, perm])
    assert np.array_equal(SP, SX[:, perm]) or np.allclose(SP, SX[:, perm], rtol=0, atol=1e-15)
    assert np.allclose(OP, OX[:, perm], rtol=0, atol=1e-15)


def pin_norm_bound(step):
    r = _rng(9)
    dk, dv = 8, 6
    S = r.standard_normal((dk, dv))
    for _ in range(300):
        k = _unit(r.standard_normal(dk)) * r.uniform(0.0, 1.0)
        v = r.standard_normal(dv)
        beta = r.uniform(0.0, 1.0)
        St, _ = step(S, r.standard_normal(dk), k, v, r.uniform(0.0, 1.0, dk), np.float64(beta), 1.0)
        assert np.linalg.norm(St) <= np.linalg.norm(S) + beta * np.linalg.norm(k) * np.linalg.norm(v) + 1e-12
        S = St


def pin_worked_example(step):
    with open(GOLDEN) as f:
        g = json.load(f)
    S = np.array(g["S0"])
    for tok in g["tokens"]:
        S, o = step(S, np.array(tok["q"]), np.array(tok["k"]), np.array(tok["v"]), np.array(tok["alpha"]),
                    np.float64(tok["beta"]), tok["scale"])
        assert np.array_equal(S, np.array(tok["S"]))
        assert np.array_equal(o, np.array(tok["o"]))


def pin_scalar_loops(step):
    r = _rng(10)
    for dk, dv in ((1, 1), (3, 2), (4, 7), (8, 8)):
        S = r.standard_normal((dk, dv))
        for _ in range(5):
            q, k, v = r.standard_normal(dk), _unit(r.standard_normal(dk)), r.standard_normal(dv)
            a, b = r.uniform(0.1, 1.0, dk), np.float64(r.uniform())
            Sv, ov = step(S, q, k, v, a, b, 0.25)
            Ss, os_ = kda_scalar.step(S.tolist(), q.tolist(), k.tolist(), v.tolist(), a.tolist(), float(b), 0.25)
            assert np.allclose(Sv, np.array(Ss), rtol=1e-14, atol=1e-14)
            assert np.allclose(ov, np.array(os_), rtol=1e-14, atol=1e-14)
            S = Sv


PINS = [pin_identity, pin_exact_write, pin_unit_key_write, pin_decay, pin_assoc_memory, pin_scalar,
        pin_lms, pin_linearity, pin_norm_bound, pin_worked_example, pin_scalar_loops]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_step_satisfies_pin(pin):
    pin(ko.step)


# ------------------------------------------------- planted mistakes ----
# Each mutant is a plausible error in writing the step; every one must fail
# at least one pin.  (Pins compare against ko.step only through kda_scalar,
# which is a separate implementation, so a mutant cannot pass by agreeing
# with itself.)

def _bk(beta, k):
    return beta[..., None] * k


def m_decay_on_columns(S, q, k, v, alpha, beta, scale):
    S1 = S * alpha[..., None, :]
    u = np.einsum("...ij,...i->...j", S1, k)
    St = S1 - _bk(beta, k)[..., :, None] * u[..., None, :] + _bk(beta, k)[..., :, None] * v[..., None, :]
    return St, ko.read(St, q, scale)


def m_read_before_update(S, q, k, v, alpha, beta, scale):
    return ko.update(S, k, v, alpha, beta), ko.read(S, q, scale)


def m_erase_without_beta(S, q, k, v, alpha, beta, scale):
    S1 = alpha[..., :, None] * S
    u = np.einsum("...ij,...i->...j", S1, k)
    St = S1 - k[..., :, None] * u[..., None, :] + _bk(beta, k)[..., :, None] * v[..., None, :]
    return St, ko.read(St, q, scale)


def m_erase_sign(S, q, k, v, alpha, beta, scale):
    S1 = alpha[..., :, None] * S
    u = np.einsum("...ij,...i->...j", S1, k)
    St = S1 + _bk(beta, k)[..., :, None] * u[..., None, :] + _bk(beta, k)[..., :, None] * v[..., None, :]
    return St, ko.read(St, q, scale)


def m_decay_after_write(S, q, k, v, alpha, beta, scale):
    u = np.einsum("...ij,...i->...j", S, k)
    St = alpha[..., :, None] * (S - _bk(beta, k)[..., :, None] * u[..., None, :]
                                + _bk(beta, k)[..., :, None] * v[..., None, :])
    return St, ko.read(St, q, scale)


def m_erase_uses_undecayed_state(S, q, k, v, alpha, beta, scale):
    S1 = alpha[..., :, None] * S
    u = np.einsum("...ij,...i->...j", S, k)
    St = S1 - _bk(beta, k)[..., :, None] * u[..., None, :] + _bk(beta, k)[..., :, None] * v[..., None, :]
    return St, ko.read(St, q, scale)


def m_transposed_read(S, q, k, v, alpha, beta, scale):
    St = ko.update(S, k, v, alpha, beta)
    if St.shape[-1] != St.shape[-2]:
        raise ValueError("shape")
    return St, scale * np.einsum("...ij,...j->...i", St, q)


def m_unscaled_read(S, q, k, v, alpha, beta, scale):
    St = ko.update(S, k, v, alpha, beta)
    return St, ko.read(St, q, 1.0)


def m_beta_squared_erase(S, q, k, v, alpha, beta, scale):
    S1 = alpha[..., :, None] * S
    u = np.einsum("...ij,...i->...j", S1, k)
    bb = (beta * beta)[..., None] * k
    St = S1 - bb[..., :, None] * u[..., None, :] + _bk(beta, k)[..., :, None] * v[..., None, :]
    return St, ko.read(St, q, scale)


def m_gate_inverted(S, q, k, v, alpha, beta, scale):
    return ko.step(S, q, k, v, 1.0 - alpha + 0.0 * alpha, beta, scale)


MUTANTS = [m_decay_on_columns, m_read_before_update, m_erase_without_beta, m_erase_sign, m_decay_after_write,
           m_erase_uses_undecayed_state, m_transposed_read, m_unscaled_read, m_beta_squared_erase,
           m_gate_inverted]


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda m: m.__name__)
def test_planted_mistake_fails_a_pin(mutant):
    failed = []
    for pin in PINS:
        try:
            pin(mutant)
        except Exception:  # assertion or shape error: the pin rejects the mutant
            failed.append(pin.__name__)
    assert failed, f"{mutant.__name__} passed every pin"
