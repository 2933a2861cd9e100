"""Build libkda.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Usage: python -m recurrent_state_amd.build   (or call build()).
The library lands next to this file; the Python binding loads it from there.
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkda.so")

SOURCES = ["kda_api.cpp", "kda_state.hip", "kda_verify.hip", "kda_slots.hip", "kda_prefill.hip", "kda_mixed.hip"]

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


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr[-8000:]}")
    if verbose and res.stderr.strip():
        print(res.stderr[-4000:], file=sys.stderr)


def build(verbose: bool = False, extra_flags=(), out: str = LIB, jobs: int = 0) -> str:
    """Compile every HIP/C++ source into libkda.so (or `out`); returns its path.

    Each source is compiled to its own object (in parallel), then the objects
    are linked; every object carries its own gfx950 code, so no device-side
    linking is involved.
    """
    objdir = os.path.join(os.path.dirname(out), "_build")
    os.makedirs(objdir, exist_ok=True)
    flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    objs = [os.path.join(objdir, s + ".o") for s in SOURCES]
    cmds = [[hipcc(), *flags, *extra_flags, "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c",
             os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    n = jobs or min(len(cmds), os.cpu_count() or 1, 16)
    with ThreadPoolExecutor(max_workers=n) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = out + ".tmp"
    _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
