"""Helpers shared by the GPU tests: moving seeded inputs to the device and the
parity bar (max |o - o_ref| <= 2e-3 RMS(o_ref); per-(b, h) relative Frobenius
state error <= 1e-3)."""

from __future__ import annotations

import sys

import numpy as np
import torch

O_TOL = 2e-3       # max |o - o_ref| / RMS(o_ref), over all outputs of a run
S_TOL = 1e-3       # ||S - S_ref||_F / ||S_ref||_F, per (sequence, head)


def say(*a):
    """Progress line, flushed, so a log names the case that was running."""
    print(*a, flush=True)
    sys.stdout.flush()


def dev_tensor(x: np.ndarray, device="cuda"):
    """Device tensor from a seeded input: uint16 arrays are bf16 bit patterns."""
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def dev_inputs(inp: dict, device="cuda") -> dict:
    return {k: dev_tensor(v, device) for k, v in inp.items()}


def token_slice(inp: dict, t0: int, t1: int) -> dict:
    return {k: v[:, t0:t1] for k, v in inp.items()}


def sub_heads(inp: dict, seqs, heads) -> dict:
    return {k: v[seqs][:, :, heads] for k, v in inp.items()}


def out_err(o, o_ref) -> tuple[float, float]:
    o = np.asarray(o, dtype=np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(o_ref * o_ref)))
    return float(np.max(np.abs(o - o_ref))) / rms, rms


def state_err(S, S_ref) -> float:
    S = np.asarray(S, dtype=np.float64)
    S_ref = np.asarray(S_ref, dtype=np.float64)
    num = np.sqrt(np.sum((S - S_ref) ** 2, axis=(-1, -2)))
    den = np.sqrt(np.sum(S_ref ** 2, axis=(-1, -2)))
    return float(np.max(num / np.maximum(den, 1e-300)))


def assert_parity(o, o_ref, S=None, S_ref=None, what=""):
    e, rms = out_err(o, o_ref)
    msg = f"{what}: max|o-o_ref|/RMS = {e:.3e} (RMS {rms:.3e})"
    if S is not None:
        se = state_err(S, S_ref)
        msg += f", state rel err {se:.3e}"
        assert se <= S_TOL, msg
    say(msg)
    assert e <= O_TOL, msg


def bits(t: torch.Tensor) -> torch.Tensor:
    """The tensor's bytes as int32 (for bit-exact comparisons of fp32 tensors)."""
    return t.contiguous().view(torch.int32)
