// Internal launch interface between the C ABI layer (kda_api.cpp) and the
// kernel translation units.  Host-only types; no torch, no allocation.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "kda.h"

namespace kda {

// Byte offsets of the four log regions for a log sized for T_max tokens.
struct LogLayout {
  size_t k, v, alpha, beta, len, total;
};

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Regions hold [B][T_max][H] token rows, so every (sequence, head) owns the
// same rows whatever T a call uses.
inline LogLayout log_layout(const kda_shape& s, int32_t T_max) {
  const size_t es = s.in_dtype == KDA_BF16 ? 2 : 4;
  const size_t tok = (size_t)s.B * (size_t)T_max * (size_t)s.H;
  LogLayout L;
  L.k = 0;
  L.v = round_up(L.k + tok * s.dk * es, 256);
  L.alpha = round_up(L.v + tok * s.dv * es, 256);
  L.beta = round_up(L.alpha + tok * s.dk * 4, 256);
  L.len = round_up(L.beta + tok * 4, 256);
  L.total = round_up(L.len + (size_t)s.B * s.H * 4, 256);
  return L;
}

struct TokenInputs {
  const void* q;
  const void* k;
  const void* v;
  const float* alpha;
  const float* beta;
};

// The log regions; token t of (b, h) is row (b * T_max + t) * H + h, and
// len[b * H + h] is the number of rows the last verify of (b, h) wrote.
struct LogPtrs {
  void* k;
  void* v;
  float* alpha;
  float* beta;
  int32_t* len;
  int32_t T_max;
};

hipError_t launch_decode(const kda_shape& s, float* state, int64_t* pos, TokenInputs in, float* o,
                         hipStream_t st);
// draft_len (device [B], may be null: every sequence has T tokens) limits
// sequence b to its first draft_len[b] tokens; a length outside [0, T] sets
// KDA_DEV_ERR_DRAFT_LEN in *dev_err and counts as 0.
// gate < 0: prepared inputs; otherwise raw projections and logits with that
// KDA_GATE_* (prepared in the kernel, logged raw).
// slot_ids (device [B], may be null) puts the states (and, for the commits,
// the positions) in a slot pool of n_slots: sequence b uses slot slot_ids[b];
// an id out of range sets KDA_DEV_ERR_SLOT_ID and the sequence is skipped.
hipError_t launch_verify(const kda_shape& s, int32_t T, const int32_t* draft_len, const float* state, TokenInputs in,
                         float* o, LogPtrs log, int32_t* dev_err, int32_t gate, hipStream_t st,
                         const int32_t* slot_ids = nullptr, int32_t n_slots = 0);
// Decode from raw projections: q, k un-normalised, `alpha` / `beta` hold the
// decay and beta logits; decay = sigmoid(gate_sign * logit).
hipError_t launch_decode_prep(const kda_shape& s, float* state, int64_t* pos, TokenInputs raw, float* o,
                              float gate_sign, hipStream_t st);
// form: the logged inputs' form (0 prepared, 1 + KDA_GATE_* raw projections).
// Decode on states in a slot pool: sequence b updates pool_states[slot_ids[b]]
// and pool_pos[slot_ids[b]]; an id outside [0, n_slots) sets
// KDA_DEV_ERR_SLOT_ID and that sequence is skipped.
hipError_t launch_decode_slots(const kda_shape& s, const int32_t* slot_ids, float* pool_states, int64_t* pool_pos,
                               int32_t n_slots, TokenInputs in, float* o, int32_t* dev_err, hipStream_t st);
hipError_t launch_commit(const kda_shape& s, int32_t T, float* state, int64_t* pos, LogPtrs log,
                         const int32_t* accepted, int32_t* dev_err, int32_t form, hipStream_t st,
                         const int32_t* slot_ids = nullptr, int32_t n_slots = 0);
// Commit of the pending T_pend logged tokens (T_pend = 0: none) followed by
// the verify of T new tokens from the committed state, in one launch.
// The pending log must be prepared when gate < 0 and raw when gate >= 0;
// pend_gate is the gate of a raw pending log.
hipError_t launch_commit_verify(const kda_shape& s, int32_t T_pend, int32_t T, const int32_t* draft_len, float* state,
                                int64_t* pos, const int32_t* accepted, int32_t* dev_err, TokenInputs in, float* o,
                                LogPtrs log, int32_t gate, int32_t pend_gate, hipStream_t st,
                                const int32_t* slot_ids = nullptr, int32_t n_slots = 0);
// Prefills: gate < 0 prepared inputs, otherwise raw projections and logits.
// state_slots (device [B], may be null): the states and positions are the
// slot pool's (slot_states, slot_pos, n_slots), sequence b using slot
// state_slots[b]; state and pos must then be the pool's arrays too.
hipError_t launch_prefill_recurrent(const kda_shape& s, int32_t L, float* state, int64_t* pos,
                                    TokenInputs in, float* o, int32_t ckpt_every, const int32_t* ckpt_slots,
                                    float* slot_states, int64_t* slot_pos, int32_t n_slots,
                                    int32_t* dev_err, int32_t gate, hipStream_t st,
                                    const int32_t* state_slots = nullptr);
hipError_t launch_prefill_chunked(const kda_shape& s, int32_t L, int32_t chunk, float* state, int64_t* pos,
                                  TokenInputs in, float* o, int32_t ckpt_every, const int32_t* ckpt_slots,
                                  float* slot_states, int64_t* slot_pos, int32_t n_slots, int32_t* dev_err,
                                  int32_t gate, hipStream_t st, const int32_t* state_slots = nullptr);

// A mixed batch (kda_mixed_step): device roles [B] and token offsets
// [B + 1] into the packed token rows, with the host's role counts.
struct MixedBatch {
  const int32_t* roles;
  const int32_t* tok_start;
  int32_t n_tokens, n_decode, n_spec, n_prefill;
};
// log may be null (no speculating sequence, nothing pending); T_pend is the
// pending verify's row count (0: none, accepted unused).
hipError_t launch_mixed(const kda_shape& s, const MixedBatch& m, float* state, int64_t* pos, const int32_t* slot_ids,
                        int32_t n_slots, TokenInputs in, float* o, const LogPtrs* log, int32_t T_pend,
                        const int32_t* accepted, int32_t* dev_err, hipStream_t st);

// Copies whole per-sequence states (n_floats each) and positions for up to
// kMaxPairs (src, dst) index pairs per launch.
constexpr int kMaxPairs = 64;
struct CopyPairs {
  int32_t n;
  int32_t src[kMaxPairs];
  int32_t dst[kMaxPairs];
};
hipError_t launch_copy_states(const float* src, const int64_t* src_pos, float* dst, int64_t* dst_pos,
                              size_t n_floats, const CopyPairs& pairs, hipStream_t st);

}  // namespace kda
