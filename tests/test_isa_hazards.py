"""Machine-code check on the kernels built here (gfx950 assembly from hipcc -S).

A VALU write to the data registers of a buffer store wider than 32 bits, too
soon after the store issues, can change the stored value.  The compiler's
hazard tracking assumes no such hazard when the store takes an SGPR offset,
and on gfx950 that assumption was seen to fail (a decode step's state row
picked up the next value of its register).  Every wide buffer store in the
library therefore folds its uniform offset into the lane offset and passes a
zero SGPR offset; this test keeps it that way.
"""

from __future__ import annotations

import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from recurrent_state_amd import build as b

WIDE_STORE_SGPR_OFFSET = re.compile(r"buffer_store_dwordx[234]\s+v\[[0-9:]+\],\s*v[0-9]+,\s*s\[[0-9:]+\],\s*s[0-9]+")
WIDE_STORE = re.compile(r"buffer_store_dwordx[234]\b")


def _asm(src, out):
    flags = [f for f in b.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [b.hipcc(), *flags, "-I", os.path.join(b.ROOT, "include"), "-I", b.CSRC, "-S", "--offload-device-only",
           os.path.join(b.CSRC, src), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    with open(out) as f:
        return f.read()


@pytest.mark.skipif(not (os.path.exists(b.hipcc()) or shutil.which(b.hipcc())), reason="hipcc not available")
def test_no_wide_buffer_store_takes_an_sgpr_offset(tmp_path):
    srcs = [s for s in b.SOURCES if s.endswith(".hip")]
    with ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        asm = dict(zip(srcs, ex.map(lambda s: _asm(s, str(tmp_path / (s + ".s"))), srcs)))
    total = 0
    for src, text in asm.items():
        bad = WIDE_STORE_SGPR_OFFSET.findall(text)
        assert not bad, f"{src}: {len(bad)} wide buffer stores with an SGPR offset, e.g. {bad[0]}"
        total += len(WIDE_STORE.findall(text))
    assert total > 0, "the pattern must see the library's wide stores"
