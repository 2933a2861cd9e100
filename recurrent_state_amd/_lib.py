"""ctypes binding of libkda (the C ABI declared in include/kda.h).

Argument marshalling only: every function checks that the torch tensors it is
given have the sizes, types, device and contiguity the C ABI expects (the C
side only sees pointers), then passes their device pointers and the current
HIP stream.  All arithmetic happens in the library's HIP kernels.  There is no
fallback: if libkda.so is missing or a call fails, an exception is raised.
"""

from __future__ import annotations

import ctypes
import os

import torch  # loads the HIP runtime that libkda then shares (same soname)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")

KDA_BF16, KDA_F32 = 0, 1
VARIANTS = {0: "none", 1: "decode", 2: "verify", 3: "commit", 4: "snapshot", 5: "restore",
            6: "prefill_recurrent", 7: "prefill_chunked", 8: "commit_verify", 9: "verify_varlen",
            10: "commit_verify_varlen", 11: "decode_prep", 12: "verify_prep", 13: "commit_verify_prep",
            14: "decode_slots", 15: "slot_copy", 16: "prefill_chunked_prep", 17: "prefill_recurrent_prep",
            18: "verify_slots", 19: "commit_slots", 20: "commit_verify_slots", 21: "prefill_chunked_slots",
            22: "mixed"}
GATE_EXP_NEG_SOFTPLUS, GATE_SIGMOID = 0, 1
DEV_ERR_ACCEPTED, DEV_ERR_CKPT_SLOT, DEV_ERR_DRAFT_LEN, DEV_ERR_SLOT_ID, DEV_ERR_MIXED = 1, 2, 4, 8, 16
ROLE_IDLE, ROLE_DECODE, ROLE_SPEC, ROLE_PREFILL = 0, 1, 2, 3


class KdaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libkda status {status}: {msg}")
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("dk", ctypes.c_int32), ("dv", ctypes.c_int32),
                ("in_dtype", ctypes.c_int32), ("scale", ctypes.c_float)]


class _Log(ctypes.Structure):
    _fields_ = [("dev", ctypes.c_void_p), ("bytes", ctypes.c_size_t), ("T_max", ctypes.c_int32),
                ("pending_T", ctypes.c_int32), ("pending_form", ctypes.c_int32)]


class _Slots(ctypes.Structure):
    _fields_ = [("states", ctypes.c_void_p), ("pos", ctypes.c_void_p), ("n_slots", ctypes.c_int32)]


_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int32
_SIGS = {
    "kda_log_bytes": (ctypes.c_size_t, [ctypes.POINTER(Shape), _I]),
    "kda_slot_bytes": (ctypes.c_size_t, [ctypes.POINTER(Shape)]),
    "kda_decode_step": (_I, [ctypes.POINTER(Shape), _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "kda_decode_step_prep": (_I, [ctypes.POINTER(Shape), _I, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "kda_verify_prep": (_I, [ctypes.POINTER(Shape), _I, _I, _P, _P, _P, _P, _P, _P, _P, ctypes.POINTER(_Log), _P]),
    "kda_commit_verify_prep": (_I, [ctypes.POINTER(Shape), _I, _I, _P, _P, _P, _P, _P, _P, _P, _P,
                                    ctypes.POINTER(_Log), _P, _P, _P]),
    "kda_verify": (_I, [ctypes.POINTER(Shape), _I, _P, _P, _P, _P, _P, _P, _P, ctypes.POINTER(_Log), _P]),
    "kda_commit": (_I, [ctypes.POINTER(Shape), _P, _P, ctypes.POINTER(_Log), _P, _P, _P]),
    "kda_commit_verify": (_I, [ctypes.POINTER(Shape), _I, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.POINTER(_Log), _P,
                               _P, _P]),
    "kda_verify_varlen": (_I, [ctypes.POINTER(Shape), _I, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.POINTER(_Log), _P,
                               _P]),
    "kda_commit_verify_varlen": (_I, [ctypes.POINTER(Shape), _I, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                      ctypes.POINTER(_Log), _P, _P, _P]),
    "kda_decode_step_slots": (_I, [ctypes.POINTER(Shape), _P, ctypes.POINTER(_Slots), _P, _P, _P, _P, _P, _P, _P,
                                   _P]),
    "kda_slot_copy": (_I, [ctypes.POINTER(Shape), _P, _P, _I, ctypes.POINTER(_Slots), _P]),
    "kda_prefill_chunked_slots": (_I, [ctypes.POINTER(Shape), _I, _I, _P, ctypes.POINTER(_Slots), _P, _P, _P, _P, _P,
                                       _P, _I, _P, _P, _P]),
    "kda_verify_slots": (_I, [ctypes.POINTER(Shape), _I, _P, ctypes.POINTER(_Slots), _P, _P, _P, _P, _P, _P,
                              ctypes.POINTER(_Log), _P, _P]),
    "kda_commit_slots": (_I, [ctypes.POINTER(Shape), _P, ctypes.POINTER(_Slots), ctypes.POINTER(_Log), _P, _P, _P]),
    "kda_commit_verify_slots": (_I, [ctypes.POINTER(Shape), _I, _P, ctypes.POINTER(_Slots), _P, _P, _P, _P, _P, _P,
                                     ctypes.POINTER(_Log), _P, _P, _P]),
    "kda_snapshot": (_I, [ctypes.POINTER(Shape), _P, _P, _P, _P, _I, ctypes.POINTER(_Slots), _P]),
    "kda_restore": (_I, [ctypes.POINTER(Shape), _P, _P, _P, _P, _I, ctypes.POINTER(_Slots), _P]),
    "kda_prefill_chunked": (_I, [ctypes.POINTER(Shape), _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _I, _P,
                                 ctypes.POINTER(_Slots), _P, _P]),
    "kda_prefill_recurrent": (_I, [ctypes.POINTER(Shape), _I, _P, _P, _P, _P, _P, _P, _P, _P, _I, _P,
                                   ctypes.POINTER(_Slots), _P, _P]),
    "kda_prefill_chunked_prep": (_I, [ctypes.POINTER(Shape), _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _I, _P,
                                      ctypes.POINTER(_Slots), _P, _P]),
    "kda_prefill_recurrent_prep": (_I, [ctypes.POINTER(Shape), _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _I, _P,
                                        ctypes.POINTER(_Slots), _P, _P]),
    "kda_mixed_step": (_I, [ctypes.POINTER(Shape), _P, _P, _I, _I, _I, _I, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P,
                            ctypes.POINTER(_Log), _P, _P, _P]),
    "kda_status_str": (ctypes.c_char_p, [_I]),
    "kda_last_variant": (_I, []),
    "kda_abi_version": (_I, []),
}


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m recurrent_state_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def exported_symbols():
    return list(_SIGS)


def _check(status: int):
    if status != 0:
        raise KdaError(status, lib().kda_status_str(status).decode())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, shape, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _shape(state, in_dtype, scale):
    B, H, dk, dv = state.shape
    code = KDA_BF16 if in_dtype == torch.bfloat16 else KDA_F32 if in_dtype == torch.float32 else None
    if code is None:
        raise TypeError(f"q/k/v dtype must be bfloat16 or float32, not {in_dtype}")
    sc = float(dk) ** -0.5 if scale is None else float(scale)
    return Shape(B, H, dk, dv, code, sc)


def _check_tokens(state, T, q, k, v, alpha, beta, o):
    B, H, dk, dv = state.shape
    dev = state.device
    dt = q.dtype
    _need(q, "q", (B, T, H, dk), dt, dev)
    _need(k, "k", (B, T, H, dk), dt, dev)
    _need(v, "v", (B, T, H, dv), dt, dev)
    _need(alpha, "alpha", (B, T, H, dk), torch.float32, dev)
    _need(beta, "beta", (B, T, H), torch.float32, dev)
    _need(o, "o", (B, T, H, dv), torch.float32, dev)


def log_bytes(shape: Shape, T_max: int) -> int:
    return int(lib().kda_log_bytes(ctypes.byref(shape), T_max))


def slot_bytes(shape: Shape) -> int:
    return int(lib().kda_slot_bytes(ctypes.byref(shape)))


def last_variant() -> str:
    return VARIANTS.get(int(lib().kda_last_variant()), "unknown")


class InputLog:
    """Device buffer for the verify input log plus its host-side bookkeeping."""

    def __init__(self, state: torch.Tensor, T_max: int, in_dtype=torch.bfloat16):
        self.shape = _shape(state, in_dtype, None)
        n = log_bytes(self.shape, T_max)
        if n == 0:
            raise ValueError("unsupported log shape")
        self.buf = torch.empty(n, dtype=torch.uint8, device=state.device)
        self.c = _Log(self.buf.data_ptr(), n, T_max, 0)

    @property
    def pending_T(self) -> int:
        return int(self.c.pending_T)


class SlotPool:
    """Caller-owned slot pool: states f32 [n_slots][H][dk][dv], pos i64 [n_slots]."""

    def __init__(self, n_slots: int, H: int, dk: int, dv: int, device):
        self.states = torch.zeros((n_slots, H, dk, dv), dtype=torch.float32, device=device)
        self.pos = torch.full((n_slots,), -1, dtype=torch.int64, device=device)
        self.c = _Slots(self.states.data_ptr(), self.pos.data_ptr(), n_slots)

    @property
    def n_slots(self) -> int:
        return int(self.c.n_slots)


def decode_step(state, pos, q, k, v, alpha, beta, o, scale=None):
    """One decode token for every (sequence, head); inputs [B][1][H][d] (or [B][H][d])."""
    B, H, dk, dv = state.shape
    if beta.dim() == 2:  # [B][H] form: add the token axis
        q, k, v, alpha, beta, o = (x.unsqueeze(1) for x in (q, k, v, alpha, beta, o))
    _need(state, "state", (B, H, dk, dv), torch.float32, state.device)
    _need(pos, "pos", (B,), torch.int64, state.device)
    _check_tokens(state, 1, q, k, v, alpha, beta, o)
    sh = _shape(state, q.dtype, scale)
    _check(lib().kda_decode_step(ctypes.byref(sh), _ptr(state), _ptr(pos), _ptr(q), _ptr(k), _ptr(v),
                                 _ptr(alpha), _ptr(beta), _ptr(o), _stream()))


def decode_step_prep(state, pos, q, k, v, alpha_logit, beta_logit, o, gate=GATE_EXP_NEG_SOFTPLUS, scale=None):
    """decode_step from raw projections: q, k un-normalised, the decay and beta as logits
    (decay = exp(-softplus(x)) for GATE_EXP_NEG_SOFTPLUS, sigmoid(x) for GATE_SIGMOID)."""
    B, H, dk, dv = state.shape
    if beta_logit.dim() == 2:
        q, k, v, alpha_logit, beta_logit, o = (x.unsqueeze(1) for x in (q, k, v, alpha_logit, beta_logit, o))
    _need(state, "state", (B, H, dk, dv), torch.float32, state.device)
    _need(pos, "pos", (B,), torch.int64, state.device)
    _check_tokens(state, 1, q, k, v, alpha_logit, beta_logit, o)
    sh = _shape(state, q.dtype, scale)
    _check(lib().kda_decode_step_prep(ctypes.byref(sh), int(gate), _ptr(state), _ptr(pos), _ptr(q), _ptr(k),
                                      _ptr(v), _ptr(alpha_logit), _ptr(beta_logit), _ptr(o), _stream()))


def _verify_args(state, q, k, v, alpha, beta, o, log: InputLog, scale):
    B, H, dk, dv = state.shape
    T = q.shape[1]
    _need(state, "state", (B, H, dk, dv), torch.float32, state.device)
    _check_tokens(state, T, q, k, v, alpha, beta, o)
    sh = _shape(state, q.dtype, scale)
    if sh.in_dtype != log.shape.in_dtype or (B, H, dk, dv) != (log.shape.B, log.shape.H, log.shape.dk,
                                                               log.shape.dv):
        raise ValueError("log was sized for a different shape")
    return sh, T, tuple(_ptr(t) for t in (state, q, k, v, alpha, beta, o))


def verify(state, q, k, v, alpha, beta, o, log: InputLog, scale=None):
    """Verify T draft tokens (inputs [B][T][H][d]) from the committed state; fills the log."""
    sh, T, ptrs = _verify_args(state, q, k, v, alpha, beta, o, log, scale)
    _check(lib().kda_verify(ctypes.byref(sh), T, *ptrs, ctypes.byref(log.c), _stream()))


def verify_prep(state, q, k, v, alpha_logit, beta_logit, o, log: InputLog, gate=GATE_EXP_NEG_SOFTPLUS, scale=None):
    """verify from raw projections and logits (prepared in the kernel, logged raw)."""
    sh, T, ptrs = _verify_args(state, q, k, v, alpha_logit, beta_logit, o, log, scale)
    _check(lib().kda_verify_prep(ctypes.byref(sh), int(gate), T, *ptrs, ctypes.byref(log.c), _stream()))


def verify_varlen(state, q, k, v, alpha, beta, o, log: InputLog, draft_len, dev_err, scale=None):
    """verify where sequence b has only its first draft_len[b] tokens (device int32 [B], each in [0, T])."""
    sh, T, ptrs = _verify_args(state, q, k, v, alpha, beta, o, log, scale)
    _need(draft_len, "draft_len", (state.shape[0],), torch.int32, state.device)
    _need(dev_err, "dev_err", (1,), torch.int32, state.device)
    _check(lib().kda_verify_varlen(ctypes.byref(sh), T, _ptr(draft_len), *ptrs, ctypes.byref(log.c), _ptr(dev_err),
                                   _stream()))


def commit(state, pos, log: InputLog, accepted, dev_err):
    """Replay accepted[b] logged tokens onto the committed state (accepted: device int32 [B])."""
    B, H, dk, dv = state.shape
    _need(state, "state", (B, H, dk, dv), torch.float32, state.device)
    _need(pos, "pos", (B,), torch.int64, state.device)
    _need(accepted, "accepted", (B,), torch.int32, state.device)
    _need(dev_err, "dev_err", (1,), torch.int32, state.device)
    if (B, H, dk, dv) != (log.shape.B, log.shape.H, log.shape.dk, log.shape.dv):
        raise ValueError("log was sized for a different shape")
    _check(lib().kda_commit(ctypes.byref(log.shape), _ptr(state), _ptr(pos), ctypes.byref(log.c),
                            _ptr(accepted), _ptr(dev_err), _stream()))


def _commit_verify_args(state, pos, q, k, v, alpha, beta, o, log: InputLog, accepted, dev_err, scale):
    B, H, dk, dv = state.shape
    T = q.shape[1]
    _need(state, "state", (B, H, dk, dv), torch.float32, state.device)
    _need(pos, "pos", (B,), torch.int64, state.device)
    _check_tokens(state, T, q, k, v, alpha, beta, o)
    if accepted is not None:
        _need(accepted, "accepted", (B,), torch.int32, state.device)
    if dev_err is not None:
        _need(dev_err, "dev_err", (1,), torch.int32, state.device)
    sh = _shape(state, q.dtype, scale)
    if (B, H, dk, dv, sh.in_dtype) != (log.shape.B, log.shape.H, log.shape.dk, log.shape.dv, log.shape.in_dtype):
        raise ValueError("log was sized for a different shape")
    ptrs = tuple(_ptr(t) for t in (state, pos, q, k, v, alpha, beta, o))
    extra = (_ptr(accepted) if accepted is not None else None, _ptr(dev_err) if dev_err is not None else None)
    return sh, T, ptrs, extra


def commit_verify(state, pos, q, k, v, alpha, beta, o, log: InputLog, accepted=None, dev_err=None, scale=None):
    """Commit the pending verify's accepted prefix, then verify T new drafts, in one launch."""
    sh, T, ptrs, extra = _commit_verify_args(state, pos, q, k, v, alpha, beta, o, log, accepted, dev_err, scale)
    _check(lib().kda_commit_verify(ctypes.byref(sh), T, *ptrs, ctypes.byref(log.c), *extra, _stream()))


def commit_verify_prep(state, pos, q, k, v, alpha_logit, beta_logit, o, log: InputLog, accepted=None, dev_err=None,
                       gate=GATE_EXP_NEG_SOFTPLUS, scale=None):
    """commit_verify whose new drafts are raw projections and logits (as verify_prep)."""
    sh, T, ptrs, extra = _commit_verify_args(state, pos, q, k, v, alpha_logit, beta_logit, o, log, accepted, dev_err,
                                             scale)
    _check(lib().kda_commit_verify_prep(ctypes.byref(sh), int(gate), T, *ptrs, ctypes.byref(log.c), *extra,
                                        _stream()))


def commit_verify_varlen(state, pos, q, k, v, alpha, beta, o, log: InputLog, draft_len, accepted=None, dev_err=None,
                         scale=None):
    """commit_verify whose new drafts have a length per sequence (draft_len: device int32 [B])."""
    sh, T, ptrs, extra = _commit_verify_args(state, pos, q, k, v, alpha, beta, o, log, accepted, dev_err, scale)
    _need(draft_len, "draft_len", (state.shape[0],), torch.int32, state.device)
    _check(lib().kda_commit_verify_varlen(ctypes.byref(sh), T, _ptr(draft_len), *ptrs, ctypes.byref(log.c), *extra,
                                          _stream()))


def _pairs(seq_ids, slot_ids):
    s = (ctypes.c_int32 * len(seq_ids))(*[int(x) for x in seq_ids])
    t = (ctypes.c_int32 * len(slot_ids))(*[int(x) for x in slot_ids])
    if len(seq_ids) != len(slot_ids):
        raise ValueError("seq_ids and slot_ids differ in length")
    return s, t


class _Batch:
    """Stands in for a [B][H][dk][dv] state tensor where only its shape and device matter."""

    def __init__(self, B, pool: SlotPool):
        _, H, dk, dv = pool.states.shape
        self.shape = (B, H, dk, dv)
        self.device = pool.states.device


def _decode_slots_args(slot_ids, pool: SlotPool, q, k, v, alpha, beta, o, dev_err, scale):
    B = slot_ids.shape[0]
    _need(slot_ids, "slot_ids", (B,), torch.int32, pool.states.device)
    _need(dev_err, "dev_err", (1,), torch.int32, pool.states.device)
    if beta.dim() == 2:
        q, k, v, alpha, beta, o = (x.unsqueeze(1) for x in (q, k, v, alpha, beta, o))
    batch = _Batch(B, pool)
    _check_tokens(batch, 1, q, k, v, alpha, beta, o)
    sh = _shape(batch, q.dtype, scale)
    return sh, (slot_ids, q, k, v, alpha, beta, o, dev_err)


def decode_step_slots(slot_ids, pool: SlotPool, q, k, v, alpha, beta, o, dev_err, scale=None):
    """decode_step on states in a slot pool: sequence b updates pool slot slot_ids[b] (device int32 [B])."""
    sh, t = _decode_slots_args(slot_ids, pool, q, k, v, alpha, beta, o, dev_err, scale)
    slot_ids, q, k, v, alpha, beta, o, dev_err = t
    _check(lib().kda_decode_step_slots(ctypes.byref(sh), _ptr(slot_ids), ctypes.byref(pool.c), _ptr(q), _ptr(k),
                                       _ptr(v), _ptr(alpha), _ptr(beta), _ptr(o), _ptr(dev_err), _stream()))


class DecodeSlotsPlan:
    """A decode_step_slots call validated once (see DecodePlan)."""

    def __init__(self, slot_ids, pool: SlotPool, q, k, v, alpha, beta, o, dev_err, scale=None):
        self._shape, t = _decode_slots_args(slot_ids, pool, q, k, v, alpha, beta, o, dev_err, scale)
        self._keep = (pool,) + t
        slot_ids, q, k, v, alpha, beta, o, dev_err = t
        self._args = (ctypes.byref(self._shape), _ptr(slot_ids), ctypes.byref(pool.c)) + tuple(
            _ptr(x) for x in (q, k, v, alpha, beta, o, dev_err))
        self._fn = lib().kda_decode_step_slots

    def __call__(self):
        _check(self._fn(*self._args, _stream()))


def _slots_batch(slot_ids, pool: SlotPool, log: InputLog, dev_err):
    B = slot_ids.shape[0]
    _need(slot_ids, "slot_ids", (B,), torch.int32, pool.states.device)
    _need(dev_err, "dev_err", (1,), torch.int32, pool.states.device)
    batch = _Batch(B, pool)
    if batch.shape != (log.shape.B, log.shape.H, log.shape.dk, log.shape.dv):
        raise ValueError("log was sized for a different shape")
    return batch


def verify_slots(slot_ids, pool: SlotPool, q, k, v, alpha, beta, o, log: InputLog, dev_err, scale=None):
    """verify on states in a slot pool (sequence b reads slot slot_ids[b]); log, inputs and o are the batch's."""
    batch = _slots_batch(slot_ids, pool, log, dev_err)
    T = q.shape[1]
    _check_tokens(batch, T, q, k, v, alpha, beta, o)
    sh = _shape(batch, q.dtype, scale)
    _check(lib().kda_verify_slots(ctypes.byref(sh), T, _ptr(slot_ids), ctypes.byref(pool.c),
                                  *(_ptr(x) for x in (q, k, v, alpha, beta, o)), ctypes.byref(log.c), _ptr(dev_err),
                                  _stream()))


def commit_slots(slot_ids, pool: SlotPool, log: InputLog, accepted, dev_err):
    """commit onto states and positions in a slot pool (sequence b updates slot slot_ids[b])."""
    batch = _slots_batch(slot_ids, pool, log, dev_err)
    _need(accepted, "accepted", (batch.shape[0],), torch.int32, pool.states.device)
    _check(lib().kda_commit_slots(ctypes.byref(log.shape), _ptr(slot_ids), ctypes.byref(pool.c), ctypes.byref(log.c),
                                  _ptr(accepted), _ptr(dev_err), _stream()))


def commit_verify_slots(slot_ids, pool: SlotPool, q, k, v, alpha, beta, o, log: InputLog, dev_err, accepted=None,
                        scale=None):
    """commit_verify on states and positions in a slot pool."""
    batch = _slots_batch(slot_ids, pool, log, dev_err)
    T = q.shape[1]
    _check_tokens(batch, T, q, k, v, alpha, beta, o)
    if accepted is not None:
        _need(accepted, "accepted", (batch.shape[0],), torch.int32, pool.states.device)
    sh = _shape(batch, q.dtype, scale)
    _check(lib().kda_commit_verify_slots(ctypes.byref(sh), T, _ptr(slot_ids), ctypes.byref(pool.c),
                                         *(_ptr(x) for x in (q, k, v, alpha, beta, o)), ctypes.byref(log.c),
                                         _ptr(accepted) if accepted is not None else None, _ptr(dev_err), _stream()))


def prefill_chunked_slots(state_slots, pool: SlotPool, q, k, v, alpha, beta, o, dev_err, *, chunk=64, ckpt_every=0,
                          ckpt_slots=None, scale=None):
    """prefill_chunked on states in a slot pool: sequence b starts from and ends in slot state_slots[b]."""
    B = state_slots.shape[0]
    _need(state_slots, "state_slots", (B,), torch.int32, pool.states.device)
    _need(dev_err, "dev_err", (1,), torch.int32, pool.states.device)
    batch = _Batch(B, pool)
    L = q.shape[1]
    _check_tokens(batch, L, q, k, v, alpha, beta, o)
    n_ckpt = L // ckpt_every if ckpt_every > 0 else 0
    if n_ckpt > 0:
        _need(ckpt_slots, "ckpt_slots", (B, n_ckpt), torch.int32, pool.states.device)
    sh = _shape(batch, q.dtype, scale)
    _check(lib().kda_prefill_chunked_slots(ctypes.byref(sh), L, chunk, _ptr(state_slots), ctypes.byref(pool.c),
                                           *(_ptr(x) for x in (q, k, v, alpha, beta, o)), ckpt_every,
                                           _ptr(ckpt_slots) if n_ckpt else None, _ptr(dev_err), _stream()))


def mixed_step(state, pos, roles, tok_start, counts, q, k, v, alpha, beta, o, dev_err, *, log: InputLog = None,
               accepted=None, slot_ids=None, scale=None):
    """One serving step over a mixed batch in one launch (kda_mixed_step).

    roles (device int32 [B], ROLE_*) and tok_start (device int32 [B + 1])
    describe the batch; counts = (n_decode, n_spec, n_prefill) are the host's
    role counts.  Tokens are packed: q, k [N][H][dk], v [N][H][dv], alpha
    [N][H][dk], beta [N][H], o [N][H][dv].  state / pos are the dense [B]
    states, or a slot pool's arrays when slot_ids (device int32 [B]) is given.
    """
    B = roles.shape[0]
    dev = state.device
    _need(roles, "roles", (B,), torch.int32, dev)
    _need(tok_start, "tok_start", (B + 1,), torch.int32, dev)
    _need(dev_err, "dev_err", (1,), torch.int32, dev)
    n_slots, H, dk, dv = state.shape
    _need(state, "state", (n_slots, H, dk, dv), torch.float32, dev)
    _need(pos, "pos", (n_slots,), torch.int64, dev)
    if slot_ids is None:
        if n_slots != B:
            raise ValueError("without slot_ids, state holds one entry per sequence")
    else:
        _need(slot_ids, "slot_ids", (B,), torch.int32, dev)
    N = q.shape[0]
    _need(q, "q", (N, H, dk), q.dtype, dev)
    _need(k, "k", (N, H, dk), q.dtype, dev)
    _need(v, "v", (N, H, dv), q.dtype, dev)
    _need(alpha, "alpha", (N, H, dk), torch.float32, dev)
    _need(beta, "beta", (N, H), torch.float32, dev)
    _need(o, "o", (N, H, dv), torch.float32, dev)
    if accepted is not None:
        _need(accepted, "accepted", (B,), torch.int32, dev)
    sh = _shape(torch.empty((B, H, dk, dv), device="meta"), q.dtype, scale)
    if log is not None and (B, H, dk, dv, sh.in_dtype) != (log.shape.B, log.shape.H, log.shape.dk, log.shape.dv,
                                                           log.shape.in_dtype):
        raise ValueError("log was sized for a different shape")
    n_dec, n_spec, n_pf = (int(c) for c in counts)
    _check(lib().kda_mixed_step(ctypes.byref(sh), _ptr(roles), _ptr(tok_start), N, n_dec, n_spec, n_pf, _ptr(state),
                                _ptr(pos), _ptr(slot_ids), n_slots if slot_ids is not None else 0,
                                *(_ptr(x) for x in (q, k, v, alpha, beta, o)),
                                ctypes.byref(log.c) if log is not None else None, _ptr(accepted), _ptr(dev_err),
                                _stream()))


def slot_copy(src_slots, dst_slots, pool: SlotPool):
    """Copy whole states and positions between pool slots: dst_slots[i] <- src_slots[i] (host ids)."""
    s, t = _pairs(src_slots, dst_slots)
    _, H, dk, dv = pool.states.shape
    sh = Shape(0, H, dk, dv, KDA_BF16, 1.0)
    _check(lib().kda_slot_copy(ctypes.byref(sh), s, t, len(src_slots), ctypes.byref(pool.c), _stream()))


def snapshot(state, pos, seq_ids, slot_ids, pool: SlotPool):
    B, H, dk, dv = state.shape
    _need(state, "state", (B, H, dk, dv), torch.float32, state.device)
    _need(pos, "pos", (B,), torch.int64, state.device)
    _need(pool.states, "pool.states", (pool.n_slots, H, dk, dv), torch.float32, state.device)
    s, t = _pairs(seq_ids, slot_ids)
    sh = Shape(B, H, dk, dv, KDA_BF16, 1.0)
    _check(lib().kda_snapshot(ctypes.byref(sh), _ptr(state), _ptr(pos), s, t, len(seq_ids),
                              ctypes.byref(pool.c), _stream()))


def restore(state, pos, seq_ids, slot_ids, pool: SlotPool):
    B, H, dk, dv = state.shape
    _need(state, "state", (B, H, dk, dv), torch.float32, state.device)
    _need(pos, "pos", (B,), torch.int64, state.device)
    _need(pool.states, "pool.states", (pool.n_slots, H, dk, dv), torch.float32, state.device)
    s, t = _pairs(seq_ids, slot_ids)
    sh = Shape(B, H, dk, dv, KDA_BF16, 1.0)
    _check(lib().kda_restore(ctypes.byref(sh), _ptr(state), _ptr(pos), s, t, len(seq_ids),
                             ctypes.byref(pool.c), _stream()))


def _prefill_args(state, pos, q, k, v, alpha, beta, o, ckpt_every, ckpt_slots, pool, dev_err):
    B, H, dk, dv = state.shape
    L = q.shape[1]
    _need(state, "state", (B, H, dk, dv), torch.float32, state.device)
    _need(pos, "pos", (B,), torch.int64, state.device)
    _check_tokens(state, L, q, k, v, alpha, beta, o)
    n_ckpt = L // ckpt_every if ckpt_every > 0 else 0
    if n_ckpt > 0:
        if pool is None or ckpt_slots is None or dev_err is None:
            raise ValueError("checkpoints need ckpt_slots, a slot pool and dev_err")
        _need(ckpt_slots, "ckpt_slots", (B, n_ckpt), torch.int32, state.device)
        _need(dev_err, "dev_err", (1,), torch.int32, state.device)
        _need(pool.states, "pool.states", (pool.n_slots, H, dk, dv), torch.float32, state.device)
    return L, n_ckpt


def prefill_chunked(state, pos, q, k, v, alpha, beta, o, *, chunk=64, ckpt_every=0, ckpt_slots=None,
                    pool: SlotPool | None = None, dev_err=None, scale=None):
    """Chunked (WY/UT form) prompt processing of L tokens ([B][L][H][d]) into the state."""
    L, n_ckpt = _prefill_args(state, pos, q, k, v, alpha, beta, o, ckpt_every, ckpt_slots, pool, dev_err)
    sh = _shape(state, q.dtype, scale)
    _check(lib().kda_prefill_chunked(ctypes.byref(sh), L, chunk, _ptr(state), _ptr(pos), _ptr(q), _ptr(k),
                                     _ptr(v), _ptr(alpha), _ptr(beta), _ptr(o), ckpt_every,
                                     _ptr(ckpt_slots) if n_ckpt else None,
                                     ctypes.byref(pool.c) if pool is not None else None,
                                     _ptr(dev_err), _stream()))


def prefill_recurrent(state, pos, q, k, v, alpha, beta, o, *, ckpt_every=0, ckpt_slots=None,
                      pool: SlotPool | None = None, dev_err=None, scale=None):
    """Token-by-token prompt processing (state in registers for the whole prompt)."""
    L, n_ckpt = _prefill_args(state, pos, q, k, v, alpha, beta, o, ckpt_every, ckpt_slots, pool, dev_err)
    sh = _shape(state, q.dtype, scale)
    _check(lib().kda_prefill_recurrent(ctypes.byref(sh), L, _ptr(state), _ptr(pos), _ptr(q), _ptr(k), _ptr(v),
                                       _ptr(alpha), _ptr(beta), _ptr(o), ckpt_every,
                                       _ptr(ckpt_slots) if n_ckpt else None,
                                       ctypes.byref(pool.c) if pool is not None else None,
                                       _ptr(dev_err), _stream()))


def prefill_chunked_prep(state, pos, q, k, v, alpha_logit, beta_logit, o, *, gate=GATE_EXP_NEG_SOFTPLUS, chunk=64,
                         ckpt_every=0, ckpt_slots=None, pool: SlotPool | None = None, dev_err=None, scale=None):
    """prefill_chunked from raw projections and logits (prepared in the kernel)."""
    L, n_ckpt = _prefill_args(state, pos, q, k, v, alpha_logit, beta_logit, o, ckpt_every, ckpt_slots, pool, dev_err)
    sh = _shape(state, q.dtype, scale)
    _check(lib().kda_prefill_chunked_prep(ctypes.byref(sh), int(gate), L, chunk, _ptr(state), _ptr(pos), _ptr(q),
                                          _ptr(k), _ptr(v), _ptr(alpha_logit), _ptr(beta_logit), _ptr(o), ckpt_every,
                                          _ptr(ckpt_slots) if n_ckpt else None,
                                          ctypes.byref(pool.c) if pool is not None else None,
                                          _ptr(dev_err), _stream()))


def prefill_recurrent_prep(state, pos, q, k, v, alpha_logit, beta_logit, o, *, gate=GATE_EXP_NEG_SOFTPLUS,
                           ckpt_every=0, ckpt_slots=None, pool: SlotPool | None = None, dev_err=None, scale=None):
    """prefill_recurrent from raw projections and logits (bit-identical to decode_step_prep token by token)."""
    L, n_ckpt = _prefill_args(state, pos, q, k, v, alpha_logit, beta_logit, o, ckpt_every, ckpt_slots, pool, dev_err)
    sh = _shape(state, q.dtype, scale)
    _check(lib().kda_prefill_recurrent_prep(ctypes.byref(sh), int(gate), L, _ptr(state), _ptr(pos), _ptr(q),
                                            _ptr(k), _ptr(v), _ptr(alpha_logit), _ptr(beta_logit), _ptr(o),
                                            ckpt_every, _ptr(ckpt_slots) if n_ckpt else None,
                                            ctypes.byref(pool.c) if pool is not None else None,
                                            _ptr(dev_err), _stream()))


class DecodePlan:
    """A decode_step call validated once, for launch-bound loops and HIP-graph
    capture: calling the plan only passes the stored pointers and the current
    stream to the library."""

    def __init__(self, state, pos, q, k, v, alpha, beta, o, scale=None, prep_gate=None):
        B, H, dk, dv = state.shape
        if beta.dim() == 2:
            q, k, v, alpha, beta, o = (x.unsqueeze(1) for x in (q, k, v, alpha, beta, o))
        _need(state, "state", (B, H, dk, dv), torch.float32, state.device)
        _need(pos, "pos", (B,), torch.int64, state.device)
        _check_tokens(state, 1, q, k, v, alpha, beta, o)
        self._keep = (state, pos, q, k, v, alpha, beta, o)
        self._shape = _shape(state, q.dtype, scale)
        if prep_gate is None:      # prepared inputs
            self._args = (ctypes.byref(self._shape),) + tuple(_ptr(t) for t in self._keep)
            self._fn = lib().kda_decode_step
        else:                      # raw projections and logits (decode_step_prep)
            self._args = (ctypes.byref(self._shape), int(prep_gate)) + tuple(_ptr(t) for t in self._keep)
            self._fn = lib().kda_decode_step_prep

    def __call__(self):
        _check(self._fn(*self._args, _stream()))


class VerifyPlan:
    """A verify call validated once (see DecodePlan); with draft_len (and
    dev_err) it is a verify_varlen call."""

    def __init__(self, state, q, k, v, alpha, beta, o, log: InputLog, scale=None, draft_len=None, dev_err=None,
                 prep_gate=None):
        self._shape, T, ptrs = _verify_args(state, q, k, v, alpha, beta, o, log, scale)
        self._keep = (state, q, k, v, alpha, beta, o, log, draft_len, dev_err)
        if prep_gate is not None:
            if draft_len is not None:
                raise ValueError("draft lengths and raw projections do not combine")
            self._args = (ctypes.byref(self._shape), int(prep_gate), T) + ptrs + (ctypes.byref(log.c),)
            self._fn = lib().kda_verify_prep
        elif draft_len is None:
            self._args = (ctypes.byref(self._shape), T) + ptrs + (ctypes.byref(log.c),)
            self._fn = lib().kda_verify
        else:
            _need(draft_len, "draft_len", (state.shape[0],), torch.int32, state.device)
            _need(dev_err, "dev_err", (1,), torch.int32, state.device)
            self._args = (ctypes.byref(self._shape), T, _ptr(draft_len)) + ptrs + (ctypes.byref(log.c),
                                                                                   _ptr(dev_err))
            self._fn = lib().kda_verify_varlen

    def __call__(self):
        _check(self._fn(*self._args, _stream()))


class CommitPlan:
    """A commit call validated once (see DecodePlan)."""

    def __init__(self, state, pos, log: InputLog, accepted, dev_err):
        B, H, dk, dv = state.shape
        _need(state, "state", (B, H, dk, dv), torch.float32, state.device)
        _need(pos, "pos", (B,), torch.int64, state.device)
        _need(accepted, "accepted", (B,), torch.int32, state.device)
        _need(dev_err, "dev_err", (1,), torch.int32, state.device)
        if (B, H, dk, dv) != (log.shape.B, log.shape.H, log.shape.dk, log.shape.dv):
            raise ValueError("log was sized for a different shape")
        self._keep = (state, pos, log, accepted, dev_err)
        self._args = (ctypes.byref(log.shape), _ptr(state), _ptr(pos), ctypes.byref(log.c), _ptr(accepted),
                      _ptr(dev_err))
        self._fn = lib().kda_commit

    def __call__(self):
        _check(self._fn(*self._args, _stream()))


class CommitVerifyPlan:
    """A commit_verify call validated once (see DecodePlan).  The pending
    count of the log when the plan is called is the one committed."""

    def __init__(self, state, pos, q, k, v, alpha, beta, o, log: InputLog, accepted=None, dev_err=None, scale=None,
                 draft_len=None, prep_gate=None):
        self._shape, T, ptrs, extra = _commit_verify_args(state, pos, q, k, v, alpha, beta, o, log, accepted,
                                                          dev_err, scale)
        self._keep = (state, pos, q, k, v, alpha, beta, o, log, accepted, dev_err, draft_len)
        if prep_gate is not None:
            if draft_len is not None:
                raise ValueError("draft lengths and raw projections do not combine")
            self._args = (ctypes.byref(self._shape), int(prep_gate), T) + ptrs + (ctypes.byref(log.c),) + extra
            self._fn = lib().kda_commit_verify_prep
        elif draft_len is None:
            self._args = (ctypes.byref(self._shape), T) + ptrs + (ctypes.byref(log.c),) + extra
            self._fn = lib().kda_commit_verify
        else:
            _need(draft_len, "draft_len", (state.shape[0],), torch.int32, state.device)
            self._args = (ctypes.byref(self._shape), T, _ptr(draft_len)) + ptrs + (ctypes.byref(log.c),) + extra
            self._fn = lib().kda_commit_verify_varlen

    def __call__(self):
        _check(self._fn(*self._args, _stream()))
