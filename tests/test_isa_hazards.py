"""Machine-code check on the kernels built here (gfx950 assembly from hipcc -S).

A VALU write to the data registers of a buffer store wider than 32 bits, too
soon after the store issues, can change the stored value.  The compiler's
hazard tracking assumes no such hazard when the store takes an SGPR offset,
and on gfx950 that assumption was seen to fail (a decode step's state row
picked up the next value of its register).  Every wide buffer store in the
library therefore folds its uniform offset into the lane offset and passes a
zero SGPR offset; this test keeps it that way.

A buffer resource built from a value the compiler cannot prove wave-uniform
(one read from LDS, or merged after a branch it takes to be divergent) is held
in vector registers, and every access through it becomes a loop over the
distinct resources in the wave: readfirstlane, compare, exec mask, access.
Such loops once sat around every input load and output store of the chunked
prefill's chunk loop (1.83 against 1.58 ms without them); the second test
finds none in any kernel.

A private array whose address escapes (say, into a lambda that captures it
by reference) can be moved by the compiler into LDS; the verify kernels once
waited for such an array's loads before issuing their state tile (verify at
B = 64 30.5 against 39.5 us).  The third test holds every verify kernel to
exactly the LDS it declares.

A register spill goes to scratch memory, and a spill of a value that is
still being loaded waits for the load first: the wave-specialised prefill,
in a form whose key waves needed more registers than their share, spilled
its fresh key and query loads that way (2.09 against 1.32 ms).  The last
tests find no scratch use in any kernel and keep that prefill within the
128 registers of four waves per SIMD.
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
# readfirstlane into a resource, then an access under a per-resource exec mask.
RESOURCE_LOOP = re.compile(r"v_readfirstlane_b32[^\n]*\n(?:[^\n]*\n){0,10}?\s*s_and_saveexec_b64[^\n]*\n\s*buffer_(?:load|store)")
HAVE_HIPCC = os.path.exists(b.hipcc()) or shutil.which(b.hipcc())


def _asm(src, out):
    flags = [f for f in b.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [b.hipcc(), *flags, "-I", os.path.join(b.ROOT, "include"), "-I", b.CSRC, "-S", "--offload-device-only",
           os.path.join(b.CSRC, src), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    with open(out) as f:
        return f.read()


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if not HAVE_HIPCC:
        pytest.skip("hipcc not available")
    d = tmp_path_factory.mktemp("asm")
    srcs = [s for s in b.SOURCES if s.endswith(".hip")]
    with ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        return dict(zip(srcs, ex.map(lambda s: _asm(s, str(d / (s + ".s"))), srcs)))


def test_no_wide_buffer_store_takes_an_sgpr_offset(asm):
    total = 0
    for src, text in asm.items():
        bad = WIDE_STORE_SGPR_OFFSET.findall(text)
        assert not bad, f"{src}: {len(bad)} wide buffer stores with an SGPR offset, e.g. {bad[0]}"
        total += len(WIDE_STORE.findall(text))
    assert total > 0, "the pattern must see the library's wide stores"


def test_no_buffer_access_loops_over_resources(asm):
    for src, text in asm.items():
        bad = RESOURCE_LOOP.findall(text)
        assert not bad, f"{src}: {len(bad)} buffer accesses through a resource held in vector registers"


def test_resource_loop_pattern_matches_its_shape():
    # The shape the compiler emits for a divergent resource (taken from an
    # earlier build of the chunked prefill), so the pattern above is live.
    sample = """	v_readfirstlane_b32 s8, v50
	v_readfirstlane_b32 s9, v51
	v_readfirstlane_b32 s10, v52
	v_readfirstlane_b32 s11, v53
	v_cmp_eq_u64_e64 s[2:3], s[8:9], v[50:51]
	s_nop 0
	v_cmp_eq_u64_e64 s[4:5], s[10:11], v[52:53]
	s_and_b64 s[2:3], s[2:3], s[4:5]
	s_and_saveexec_b64 s[2:3], s[2:3]
	buffer_load_dwordx2 v[64:65], v41, s[8:11], 0 offen
	s_xor_b64 exec, exec, s[2:3]
	s_cbranch_execnz .LBB0_117
"""
    assert len(RESOURCE_LOOP.findall(sample)) == 1


# Declared LDS of a verify workgroup (VerifyLds<DK>): three token vectors and
# the group-end decay of 8 row groups x (R + 4) floats each, plus two 4 x 4
# float blocks.
def _verify_lds(dk):
    r = dk // 8
    vec = 8 * (r + 4)
    return 4 * (3 * 4 * vec + vec + 2 * 16)


def test_verify_kernels_use_only_their_declared_lds(asm):
    text = asm["kda_verify.hip"]
    found = re.findall(r"\.amdhsa_kernel (_ZN3kda12_GLOBAL__N_119verify_chunk_kernelILi(\d+)\S*)\n(.*?)\.end_amdhsa_kernel",
                       text, flags=re.S)
    assert len(found) >= 32
    for name, dk, body in found:
        lds = int(re.search(r"\.amdhsa_group_segment_fixed_size (\d+)", body).group(1))
        assert lds == _verify_lds(int(dk)), f"{name}: {lds} bytes of LDS, {_verify_lds(int(dk))} declared"


def _kernels(text):
    return re.findall(r"\.amdhsa_kernel (\S+)\n(.*?)\.end_amdhsa_kernel", text, flags=re.S)


def test_no_kernel_spills_to_scratch(asm):
    n = 0
    for src, text in asm.items():
        for name, body in _kernels(text):
            size = int(re.search(r"\.amdhsa_private_segment_fixed_size (\d+)", body).group(1))
            assert size == 0, f"{src}: {name} uses {size} bytes of scratch per lane"
            n += 1
    assert n > 100, "the pattern must see the library's kernels"


def test_wave_specialised_prefill_fits_its_workgroup_on_one_cu(asm):
    # dv / 16 value waves and dk / 16 key waves spread over the CU's four
    # SIMDs: 16 waves (dk = dv = 128) need at most 128 VGPRs, 12 waves 168,
    # 8 waves 256.
    found = [(name, body) for name, body in _kernels(asm["kda_prefill.hip"]) if "prefill_ws_kernel" in name]
    assert found, "the wave-specialised prefill kernel must be built"
    shapes = set()
    for name, body in found:
        dk, dv = map(int, re.search(r"prefill_ws_kernelILi(\d+)ELi(\d+)ELi64E", name).groups())
        shapes.add((dk, dv))
        waves_per_simd = -(-(dv // 16 + dk // 16) // 4)
        budget = min(512 // waves_per_simd // 8 * 8, 256)
        vgprs = int(re.search(r"\.amdhsa_next_free_vgpr (\d+)", body).group(1))
        assert vgprs <= budget, f"{name}: {vgprs} VGPRs, more than {waves_per_simd} waves per SIMD allow ({budget})"
    assert shapes == {(128, 128), (128, 64), (64, 128), (64, 64)}, shapes
