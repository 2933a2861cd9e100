"""The C ABI on the host: the library loads, exports every function that
include/kda.h declares, and rejects invalid arguments before enqueuing
anything.

Every call here is built to fail host-side validation (or to be a pure size
query), so no kernel is ever launched: the pointers passed are fake but never
reach a device.  Safe with or without a GPU.  The one exception, an empty
prompt (which must return before any launch), runs only where no GPU is
visible; tests/test_gpu_decay.py covers it on the GPU with real buffers.
"""

from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

OK, NULL, SHAPE, DTYPE, ALIGN, ORDER, SLOT, HIP = range(8)


@pytest.fixture(scope="module")
def k():
    import recurrent_state_amd as kda
    if not os.path.exists(kda.LIB_PATH):
        from recurrent_state_amd import build
        build.build()
    return kda


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_\w+)\s*\(", text)))


def test_exports_every_declared_function(k):
    names = declared_functions()
    assert len(names) >= 13
    lib = ctypes.CDLL(k.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in kda.h but not exported"
    assert set(names) == set(k.exported_symbols()), "binding and header disagree"
    assert k.lib().kda_abi_version() == 1


def shape(k, B=2, H=3, dk=128, dv=128, dt=0, scale=0.1):
    return k.Shape(B, H, dk, dv, dt, scale)


P = ctypes.c_void_p
GOOD = P(0x10000)      # 16-byte aligned fake pointer: only ever paired with an invalid argument
MIS = P(0x10004)       # misaligned


def test_sizes(k):
    s = shape(k, B=16, H=32)
    assert k.slot_bytes(s) == 32 * 128 * 128 * 4
    nb = k.log_bytes(s, 4)
    tok = 16 * 4 * 32
    assert nb >= tok * (128 * 2 * 2 + 128 * 4 + 4) + 16 * 32 * 4 and nb % 256 == 0   # + per-(b, h) counts
    assert k.log_bytes(s, 0) == 0 and k.log_bytes(s, 17) == 0
    assert k.log_bytes(shape(k, dk=96), 4) == 0 and k.slot_bytes(shape(k, dt=5)) == 0
    f32 = shape(k, B=16, H=32, dt=1)
    assert k.log_bytes(f32, 4) > nb


def test_decode_validation(k):
    L = k.lib()
    dec = lambda s, state=GOOD, pos=GOOD, q=GOOD, o=GOOD: L.kda_decode_step(  # noqa: E731
        ctypes.byref(s) if s is not None else None, state, pos, q, GOOD, GOOD, GOOD, GOOD, o, None)
    assert dec(None) == NULL
    assert dec(shape(k, dk=96)) == SHAPE
    assert dec(shape(k, dv=256)) == SHAPE
    assert dec(shape(k, H=0)) == SHAPE
    assert dec(shape(k, B=-1)) == SHAPE
    assert dec(shape(k, dt=2)) == DTYPE
    assert dec(shape(k), state=None) == NULL
    assert dec(shape(k), q=None) == NULL
    assert dec(shape(k), pos=None) == NULL
    assert dec(shape(k), o=MIS) == ALIGN
    assert dec(shape(k), state=MIS) == ALIGN
    # An empty batch is a no-op that needs no buffers.
    assert dec(shape(k, B=0), state=None, pos=None, q=None, o=None) == OK


def test_decode_prep_validation(k):
    L = k.lib()
    dec = lambda s, gate=0, state=GOOD, pos=GOOD, q=GOOD, a=GOOD, o=GOOD: L.kda_decode_step_prep(  # noqa: E731
        ctypes.byref(s) if s is not None else None, gate, state, pos, q, GOOD, GOOD, a, GOOD, o, None)
    assert dec(None) == NULL
    assert dec(shape(k, dk=96)) == SHAPE
    assert dec(shape(k), gate=2) == SHAPE and dec(shape(k), gate=-1) == SHAPE
    assert dec(shape(k, B=0), gate=7) == SHAPE, "the gate is checked before the empty-batch shortcut"
    assert dec(shape(k), state=None) == NULL
    assert dec(shape(k), q=None) == NULL
    assert dec(shape(k), a=None) == NULL
    assert dec(shape(k), pos=None) == NULL
    assert dec(shape(k), o=MIS) == ALIGN
    assert dec(shape(k, B=0), gate=1, state=None, pos=None, q=None, a=None, o=None) == OK


def test_prep_verify_validation(k):
    L = k.lib()
    s = shape(k)
    need = k.log_bytes(s, 4)
    log = k._lib._Log(0x100000, need, 4, 0, 0)
    ver = lambda gate, T=2, lg=log: L.kda_verify_prep(  # noqa: E731
        ctypes.byref(s), gate, T, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, None, ctypes.byref(lg), None)
    assert ver(3) == SHAPE and ver(-1) == SHAPE
    assert ver(0) == NULL                                  # o is NULL: rejected before any launch
    assert ver(0, lg=k._lib._Log(0x100000, need, 4, 0, 7)) == SHAPE   # unknown pending form
    # The fused calls need the pending verify's form: raw after verify_prep, prepared otherwise.
    raw_pend = k._lib._Log(0x100000, need, 4, 2, 1)
    prep_pend = k._lib._Log(0x100000, need, 4, 2, 0)
    assert L.kda_commit_verify(ctypes.byref(s), 2, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD,
                               ctypes.byref(raw_pend), GOOD, GOOD, None) == ORDER
    assert L.kda_commit_verify_prep(ctypes.byref(s), 0, 2, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD,
                                    ctypes.byref(prep_pend), GOOD, GOOD, None) == ORDER
    assert L.kda_commit_verify_prep(ctypes.byref(s), 9, 2, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD,
                                    ctypes.byref(raw_pend), GOOD, GOOD, None) == SHAPE
    assert raw_pend.pending_T == 2 and raw_pend.pending_form == 1 and prep_pend.pending_form == 0
    slots = k._lib._Slots(0x200000, 0x300000, 8)
    assert L.kda_prefill_chunked_prep(ctypes.byref(s), 2, 64, 64, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 0,
                                      None, ctypes.byref(slots), None, None) == SHAPE
    assert L.kda_prefill_recurrent_prep(ctypes.byref(s), -1, 64, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 0,
                                        None, ctypes.byref(slots), None, None) == SHAPE
    assert L.kda_prefill_chunked_prep(ctypes.byref(s), 1, 64, 48, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 0,
                                      None, ctypes.byref(slots), None, None) == SHAPE   # chunk 48


def test_verify_commit_validation(k):
    L = k.lib()
    s = shape(k)
    need = k.log_bytes(s, 4)
    log = k._lib._Log(0x100000, need, 4, 0)
    ver = lambda T, lg, st=GOOD: L.kda_verify(ctypes.byref(s), T, st, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD,  # noqa
                                              ctypes.byref(lg) if lg is not None else None, None)
    assert ver(1, None) == NULL
    assert ver(0, log) == SHAPE
    assert ver(5, log) == SHAPE                                   # T > T_max
    assert ver(1, k._lib._Log(0x100000, need - 256, 4, 0)) == SHAPE  # buffer too small
    assert ver(1, k._lib._Log(0x100080, need, 4, 0)) == ALIGN        # log not 256-byte aligned
    assert ver(1, k._lib._Log(0x100000, need, 4, 2)) == ORDER        # a verify is already pending
    assert ver(2, log, st=None) == NULL
    com = lambda lg, acc=GOOD, err=GOOD: L.kda_commit(ctypes.byref(s), GOOD, GOOD, ctypes.byref(lg), acc,  # noqa
                                                      err, None)
    assert com(log) == ORDER                                      # nothing pending
    pend = k._lib._Log(0x100000, need, 4, 3)
    assert com(pend, acc=None) == NULL
    assert com(pend, err=None) == NULL
    assert com(pend, acc=P(0x10002)) == ALIGN
    assert pend.pending_T == 3, "a rejected commit must not consume the pending verify"


def test_commit_verify_validation(k):
    L = k.lib()
    s = shape(k)
    need = k.log_bytes(s, 4)

    def cv(T, lg, pos=GOOD, acc=GOOD, err=GOOD, st=GOOD):
        return L.kda_commit_verify(ctypes.byref(s), T, st, pos, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD,
                                   ctypes.byref(lg) if lg is not None else None, acc, err, None)

    log = k._lib._Log(0x100000, need, 4, 2)
    assert cv(1, None) == NULL
    assert cv(0, log) == SHAPE
    assert cv(5, log) == SHAPE                                    # T > T_max
    assert cv(2, log, pos=None) == NULL
    assert cv(2, log, pos=P(0x10004)) == ALIGN
    assert cv(2, log, acc=None) == NULL                           # a verify is pending: counts needed
    assert cv(2, log, err=None) == NULL
    assert cv(2, log, acc=P(0x10002)) == ALIGN
    assert cv(2, log, st=None) == NULL
    assert log.pending_T == 2, "a rejected call must not touch the pending count"
    assert cv(2, k._lib._Log(0x100000, need - 256, 4, 0)) == SHAPE
    # An empty batch needs no buffers and moves the log to the new pending count.
    empty = shape(k, B=0)
    lg0 = k._lib._Log(0x100000, k.log_bytes(empty, 4) or 256, 4, 3)
    assert L.kda_commit_verify(ctypes.byref(empty), 4, None, None, None, None, None, None, None, None,
                               ctypes.byref(lg0), None, None, None) == OK
    assert lg0.pending_T == 4


def test_varlen_validation(k):
    L = k.lib()
    s = shape(k)
    need = k.log_bytes(s, 4)
    MIS4 = P(0x10002)

    def ver(T, lg, dl=GOOD, err=GOOD):
        return L.kda_verify_varlen(ctypes.byref(s), T, dl, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD,
                                   ctypes.byref(lg), err, None)

    log = k._lib._Log(0x100000, need, 4, 0)
    assert ver(2, log, dl=None) == NULL
    assert ver(2, log, err=None) == NULL
    assert ver(2, log, dl=MIS4) == ALIGN
    assert ver(2, log, err=MIS4) == ALIGN
    assert ver(0, log) == SHAPE and ver(5, log) == SHAPE
    assert ver(2, k._lib._Log(0x100000, need, 4, 3)) == ORDER
    assert log.pending_T == 0

    def cv(lg, dl=GOOD, acc=GOOD, err=GOOD):
        return L.kda_commit_verify_varlen(ctypes.byref(s), 3, dl, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD,
                                          ctypes.byref(lg), acc, err, None)

    idle = k._lib._Log(0x100000, need, 4, 0)
    assert cv(idle, dl=None) == NULL
    assert cv(idle, err=None) == NULL          # nothing pending, but draft lengths can be rejected
    assert cv(idle, dl=MIS4) == ALIGN
    pend = k._lib._Log(0x100000, need, 4, 2)
    assert cv(pend, acc=None) == NULL
    assert cv(pend, acc=MIS4) == ALIGN
    assert idle.pending_T == 0 and pend.pending_T == 2
    # An empty batch needs no buffers.
    empty = shape(k, B=0)
    lg0 = k._lib._Log(0x100000, k.log_bytes(empty, 4) or 256, 4, 0)
    assert L.kda_verify_varlen(ctypes.byref(empty), 3, None, None, None, None, None, None, None, None,
                               ctypes.byref(lg0), None, None) == OK
    assert lg0.pending_T == 3


def test_slot_decode_and_copy_validation(k):
    L = k.lib()
    s = shape(k, B=4)
    slots = k._lib._Slots(0x200000, 0x300000, 8)
    dec = lambda sl=slots, ids=GOOD, err=GOOD, q=GOOD, shp=s: L.kda_decode_step_slots(  # noqa: E731
        ctypes.byref(shp), ids, ctypes.byref(sl) if sl is not None else None, q, GOOD, GOOD, GOOD, GOOD, GOOD, err,
        None)
    assert dec(sl=None) == NULL
    assert dec(ids=None) == NULL and dec(err=None) == NULL and dec(q=None) == NULL
    assert dec(ids=P(0x10002)) == ALIGN
    assert dec(sl=k._lib._Slots(0x200000, 0x300000, -1)) == SHAPE
    assert dec(shp=shape(k, B=0), ids=None, err=None, q=None) == OK
    ids = lambda *v: (ctypes.c_int32 * len(v))(*v)  # noqa: E731
    cp = lambda a, b, n=None: L.kda_slot_copy(ctypes.byref(s), a, b, len(a) if n is None else n,  # noqa: E731
                                              ctypes.byref(slots), None)
    assert cp(ids(0), ids(8)) == SLOT and cp(ids(-1), ids(0)) == SLOT
    assert cp(ids(1, 2), ids(2, 3)) == SLOT, "a slot that is both a source and a destination"
    assert cp(ids(1), ids(1)) == SLOT
    assert cp(ids(), ids(), 0) == OK
    assert cp(ids(0), ids(1), -1) == SHAPE
    assert L.kda_slot_copy(ctypes.byref(s), None, None, 1, ctypes.byref(slots), None) == NULL
    log = k._lib._Log(0x100000, k.log_bytes(s, 4), 4, 0, 0)
    assert L.kda_verify_slots(ctypes.byref(s), 2, None, ctypes.byref(slots), GOOD, GOOD, GOOD, GOOD, GOOD, GOOD,
                              ctypes.byref(log), GOOD, None) == NULL
    assert L.kda_verify_slots(ctypes.byref(s), 2, GOOD, ctypes.byref(slots), GOOD, GOOD, GOOD, GOOD, GOOD, GOOD,
                              ctypes.byref(log), None, None) == NULL
    assert L.kda_verify_slots(ctypes.byref(s), 2, GOOD, ctypes.byref(k._lib._Slots(0x200000, 0x300000, 0)), GOOD,
                              GOOD, GOOD, GOOD, GOOD, GOOD, ctypes.byref(log), GOOD, None) == SLOT
    assert log.pending_T == 0
    assert L.kda_commit_slots(ctypes.byref(s), GOOD, ctypes.byref(slots), ctypes.byref(log), GOOD, GOOD,
                              None) == ORDER                      # nothing pending
    pend = k._lib._Log(0x100000, k.log_bytes(s, 4), 4, 2, 0)
    assert L.kda_commit_slots(ctypes.byref(s), P(0x10002), ctypes.byref(slots), ctypes.byref(pend), GOOD, GOOD,
                              None) == ALIGN
    assert L.kda_commit_verify_slots(ctypes.byref(s), 2, GOOD, ctypes.byref(slots), GOOD, GOOD, GOOD, GOOD, GOOD,
                                     GOOD, ctypes.byref(pend), GOOD, None, None) == NULL
    assert pend.pending_T == 2
    assert L.kda_prefill_chunked_slots(ctypes.byref(s), 64, 64, GOOD, ctypes.byref(slots), GOOD, GOOD, GOOD, GOOD,
                                       GOOD, GOOD, 0, None, None, None) == NULL          # dev_err
    assert L.kda_prefill_chunked_slots(ctypes.byref(s), 64, 64, P(0x10002), ctypes.byref(slots), GOOD, GOOD, GOOD,
                                       GOOD, GOOD, GOOD, 0, None, GOOD, None) == ALIGN
    assert L.kda_prefill_chunked_slots(ctypes.byref(s), 64, 64, GOOD,
                                       ctypes.byref(k._lib._Slots(0x200000, 0x300000, 0)), GOOD, GOOD, GOOD, GOOD,
                                       GOOD, GOOD, 0, None, GOOD, None) == SLOT


def test_snapshot_restore_validation(k):
    L = k.lib()
    s = shape(k, B=4)
    slots = k._lib._Slots(0x200000, 0x300000, 8)
    ids = lambda *v: (ctypes.c_int32 * len(v))(*v)  # noqa: E731
    for fn in (L.kda_snapshot, L.kda_restore):
        assert fn(ctypes.byref(s), GOOD, GOOD, ids(0), ids(8), 1, ctypes.byref(slots), None) == SLOT
        assert fn(ctypes.byref(s), GOOD, GOOD, ids(4), ids(0), 1, ctypes.byref(slots), None) == SLOT
        assert fn(ctypes.byref(s), GOOD, GOOD, ids(-1), ids(0), 1, ctypes.byref(slots), None) == SLOT
        assert fn(ctypes.byref(s), GOOD, GOOD, ids(0, 1), ids(0, -3), 2, ctypes.byref(slots), None) == SLOT
        assert fn(ctypes.byref(s), GOOD, GOOD, None, ids(0), 1, ctypes.byref(slots), None) == NULL
        assert fn(ctypes.byref(s), GOOD, GOOD, ids(0), ids(0), -1, ctypes.byref(slots), None) == SHAPE
        assert fn(ctypes.byref(s), GOOD, GOOD, ids(0), ids(0), 1, None, None) == NULL
        assert fn(ctypes.byref(s), MIS, GOOD, ids(0), ids(0), 1, ctypes.byref(slots), None) == ALIGN
        assert fn(ctypes.byref(s), GOOD, GOOD, ids(), ids(), 0, ctypes.byref(slots), None) == OK


def test_prefill_validation(k):
    L = k.lib()
    s = shape(k)
    slots = k._lib._Slots(0x200000, 0x300000, 8)

    def pre(Lt=64, chunk=64, every=0, ck=GOOD, sl=slots, err=GOOD, q=GOOD):
        return L.kda_prefill_chunked(ctypes.byref(s), Lt, chunk, GOOD, GOOD, q, GOOD, GOOD, GOOD, GOOD, GOOD,
                                     every, ck, ctypes.byref(sl) if sl is not None else None, err, None)

    assert pre(chunk=48) == SHAPE
    assert pre(chunk=16) == SHAPE
    assert pre(Lt=-1) == SHAPE
    assert pre(every=100) == SHAPE             # not a multiple of the chunk
    assert pre(every=-64) == SHAPE
    assert pre(every=64, ck=None) == NULL
    assert pre(every=64, sl=None) == NULL
    assert pre(every=64, err=None) == NULL
    assert pre(q=None) == NULL
    assert pre(q=MIS) == ALIGN
    rec = L.kda_prefill_recurrent
    assert rec(ctypes.byref(s), -2, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 0, None, None, None,
               None) == SHAPE
    assert rec(ctypes.byref(s), 8, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 4, None, None, None,
               None) == NULL


def test_empty_prompt_returns_before_any_launch(k):
    import torch
    if torch.cuda.is_available():
        pytest.skip("fake pointers: host-only check (the GPU suite tests empty prompts with real buffers)")
    L = k.lib()
    s = shape(k)
    before = L.kda_last_variant()
    # NULL token pointers are allowed when L = 0, and nothing is enqueued.
    assert L.kda_prefill_chunked(ctypes.byref(s), 0, 64, GOOD, GOOD, None, None, None, None, None, None, 0, None,
                                 None, None, None) == OK
    assert L.kda_prefill_chunked_prep(ctypes.byref(s), 0, 0, 32, GOOD, GOOD, None, None, None, None, None, None, 0,
                                      None, None, None, None) == OK
    assert L.kda_prefill_recurrent(ctypes.byref(s), 0, GOOD, GOOD, None, None, None, None, None, None, 0, None, None,
                                   None, None) == OK
    assert L.kda_prefill_recurrent_prep(ctypes.byref(s), 1, 0, GOOD, GOOD, None, None, None, None, None, None, 0,
                                        None, None, None, None) == OK
    slots = k._lib._Slots(0x200000, 0x300000, 8)
    assert L.kda_prefill_chunked_slots(ctypes.byref(s), 0, 64, GOOD, ctypes.byref(slots), None, None, None, None,
                                       None, None, 0, None, GOOD, None) == OK
    assert L.kda_last_variant() == before
    # The state and position are still required.
    assert L.kda_prefill_chunked(ctypes.byref(s), 0, 64, None, GOOD, None, None, None, None, None, None, 0, None,
                                 None, None, None) == NULL


def test_mixed_step_validation(k):
    L = k.lib()
    s = shape(k, B=4)
    need = k.log_bytes(s, 4)

    def mx(counts=(1, 1, 1), n_tok=8, lg=None, roles=GOOD, ts=GOOD, err=GOOD, pos=GOOD, st=GOOD, acc=GOOD,
           slot_ids=None, n_slots=0, q=GOOD, sh=s):
        return L.kda_mixed_step(ctypes.byref(sh), roles, ts, n_tok, *counts, st, pos, slot_ids, n_slots, q, GOOD,
                                GOOD, GOOD, GOOD, GOOD, ctypes.byref(lg) if lg is not None else None, acc, err, None)

    log = k._lib._Log(0x100000, need, 4, 0)
    assert mx(lg=None) == NULL                                   # a speculating sequence needs a log
    assert mx(counts=(-1, 0, 0)) == SHAPE
    assert mx(counts=(2, 2, 1), lg=log) == SHAPE                 # 5 roles for 4 sequences
    assert mx(n_tok=-1, lg=log) == SHAPE
    assert mx(lg=log, roles=None) == NULL
    assert mx(lg=log, ts=None) == NULL
    assert mx(lg=log, err=None) == NULL
    assert mx(lg=log, pos=P(0x10004)) == ALIGN
    assert mx(lg=log, roles=P(0x10002)) == ALIGN
    assert mx(lg=log, q=None) == NULL                            # tokens present: token pointers required
    assert mx(lg=log, slot_ids=GOOD, n_slots=0) == SHAPE
    assert mx(lg=k._lib._Log(0x100000, need - 256, 4, 0)) == SHAPE
    raw = k._lib._Log(0x100000, need, 4, 3, 1)                   # a pending verify of raw projections
    assert mx(lg=raw) == ORDER and raw.pending_T == 3
    pend = k._lib._Log(0x100000, need, 4, 3, 0)
    assert mx(lg=pend, acc=None) == NULL                         # pending rows: counts needed
    assert pend.pending_T == 3, "a rejected call must not touch the pending count"
    # An empty batch enqueues nothing and leaves nothing pending.
    empty = shape(k, B=0)
    lg0 = k._lib._Log(0x100000, k.log_bytes(empty, 4) or 256, 4, 3, 0)
    before = L.kda_last_variant()
    assert mx(counts=(0, 0, 0), n_tok=0, lg=lg0, roles=None, ts=None, err=None, pos=None, st=None, acc=None,
              q=None, sh=empty) == OK
    assert lg0.pending_T == 0 and L.kda_last_variant() == before


def test_status_strings(k):
    L = k.lib()
    names = [L.kda_status_str(i).decode() for i in range(8)]
    assert names[0] == "ok" and len(set(names)) == 8
    assert L.kda_status_str(99).decode() == "unknown status"


def test_binding_refuses_missing_library(tmp_path, monkeypatch):
    import recurrent_state_amd._lib as binding
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "absent.so"))
    monkeypatch.setattr(binding, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        binding.lib()
