"""MI355X (gfx950) KDA recurrent-state library: Python binding of libkda.

The hot path (decode step, speculative verify and commit, snapshot/restore,
chunked prefill) runs in hand-written HIP kernels inside libkda.so; this
package only marshals torch tensors (device memory and streams) into the C ABI
of include/kda.h.
"""

from ._lib import (  # noqa: F401
    DEV_ERR_ACCEPTED,
    DEV_ERR_CKPT_SLOT,
    DEV_ERR_DRAFT_LEN,
    DEV_ERR_SLOT_ID,
    GATE_EXP_NEG_SOFTPLUS,
    GATE_SIGMOID,
    CommitPlan,
    CommitVerifyPlan,
    DecodePlan,
    DecodeSlotsPlan,
    LIB_PATH,
    InputLog,
    KdaError,
    VerifyPlan,
    Shape,
    SlotPool,
    commit,
    commit_verify,
    commit_verify_prep,
    commit_verify_varlen,
    decode_step,
    decode_step_prep,
    decode_step_slots,
    exported_symbols,
    last_variant,
    lib,
    log_bytes,
    prefill_chunked,
    prefill_chunked_prep,
    prefill_recurrent,
    prefill_recurrent_prep,
    restore,
    slot_bytes,
    slot_copy,
    snapshot,
    verify,
    verify_prep,
    verify_varlen,
)
