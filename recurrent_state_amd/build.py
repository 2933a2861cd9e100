"""Build libkda.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Usage: python -m recurrent_state_amd.build   (or call build()).
The library lands next to this file; the Python binding loads it from there.
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkda.so")

SOURCES = ["kda_api.cpp", "kda_state.hip", "kda_verify.hip", "kda_slots.hip", "kda_prefill.hip"]

# -ffp-contract=off: every fused multiply-add in the kernels is written out,
#   so decode and commit round identically.
# -packed-fp32-ops off: no packed fp32 VALU instructions are generated.
HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-result",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def build(verbose: bool = False, extra_flags=(), out: str = LIB) -> str:
    """Compile every HIP/C++ source into libkda.so (or `out`); returns its path."""
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr[-8000:]}")
    if verbose and res.stderr.strip():
        print(res.stderr[-4000:], file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
