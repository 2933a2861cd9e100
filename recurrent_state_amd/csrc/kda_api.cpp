// C ABI of libkda: host-side argument validation and kernel launches.
// Every entry point validates everything it can see on the host first and
// returns a status without enqueuing anything when a check fails; after that
// it only enqueues kernels on the caller's stream.  Nothing here allocates
// device memory or synchronizes.

#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>

#include <vector>

#include "kda.h"
#include "kda_internal.h"

namespace {

thread_local int32_t g_last_variant = KDA_VARIANT_NONE;

constexpr int32_t kMaxT = 16;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

kda_status check_shape(const kda_shape* s) {
  if (!s) return KDA_ERR_NULL;
  if (s->in_dtype != KDA_BF16 && s->in_dtype != KDA_F32) return KDA_ERR_DTYPE;
  if (s->B < 0 || s->H < 1) return KDA_ERR_SHAPE;
  if (!(s->dk == 64 || s->dk == 128) || !(s->dv == 64 || s->dv == 128)) return KDA_ERR_SHAPE;
  // Grid of one wave per 32-column slice must fit a launch dimension.
  if ((int64_t)s->B * s->H * (s->dv / 32) > (int64_t)INT32_MAX) return KDA_ERR_SHAPE;
  return KDA_OK;
}

// All pointers non-null and 16-byte aligned.
kda_status check_ptrs(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (!p) return KDA_ERR_NULL;
  for (const void* p : ps)
    if (!aligned(p, 16)) return KDA_ERR_ALIGN;
  return KDA_OK;
}

// Per-token inputs and outputs: q, k, v, alpha, o are read/written with
// 16-byte vector accesses; beta is read one float at a time.
kda_status check_tokens(const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                        const float* o) {
  kda_status r = check_ptrs({q, k, v, alpha, o});
  if (r != KDA_OK) return r;
  if (!beta) return KDA_ERR_NULL;
  if (!aligned(beta, 4)) return KDA_ERR_ALIGN;
  return KDA_OK;
}

kda_status launched(hipError_t e, int32_t variant) {
  if (e != hipSuccess) return KDA_ERR_HIP;
  g_last_variant = variant;
  return KDA_OK;
}

kda_status check_log(const kda_shape& s, const kda_log* log) {
  if (!log || !log->dev) return KDA_ERR_NULL;
  if (!aligned(log->dev, 256)) return KDA_ERR_ALIGN;
  if (log->T_max < 1 || log->T_max > kMaxT) return KDA_ERR_SHAPE;
  if (log->pending_form < 0 || log->pending_form > 2) return KDA_ERR_SHAPE;
  if (log->bytes < kda::log_layout(s, log->T_max).total) return KDA_ERR_SHAPE;
  return KDA_OK;
}

kda::LogPtrs log_ptrs(const kda_shape& s, const kda_log* log) {
  const kda::LogLayout L = kda::log_layout(s, log->T_max);
  char* base = static_cast<char*>(log->dev);
  return kda::LogPtrs{base + L.k, base + L.v, reinterpret_cast<float*>(base + L.alpha),
                      reinterpret_cast<float*>(base + L.beta), reinterpret_cast<int32_t*>(base + L.len),
                      log->T_max};
}

kda_status check_slots(const kda_slots* slots) {
  if (!slots || !slots->states || !slots->pos) return KDA_ERR_NULL;
  if (!aligned(slots->states, 16) || !aligned(slots->pos, 8)) return KDA_ERR_ALIGN;
  if (slots->n_slots < 0) return KDA_ERR_SHAPE;
  return KDA_OK;
}

// Launches bitwise copies for the (src, dst) pairs, at most kMaxPairs per
// launch.  When a destination repeats, only its last pair is kept, so the
// later pair wins deterministically.
kda_status copy_pairs(const std::vector<int32_t>& src, const std::vector<int32_t>& dst, const float* src_states,
                      const int64_t* src_pos, float* dst_states, int64_t* dst_pos, size_t n_floats,
                      hipStream_t st) {
  std::vector<char> later(src.size(), 0);
  for (size_t i = 0; i < dst.size(); ++i)
    for (size_t j = i + 1; j < dst.size(); ++j)
      if (dst[j] == dst[i]) later[i] = 1;
  kda::CopyPairs batch;
  batch.n = 0;
  for (size_t i = 0; i < src.size(); ++i) {
    if (later[i]) continue;
    batch.src[batch.n] = src[i];
    batch.dst[batch.n] = dst[i];
    if (++batch.n == kda::kMaxPairs) {
      if (kda::launch_copy_states(src_states, src_pos, dst_states, dst_pos, n_floats, batch, st) != hipSuccess)
        return KDA_ERR_HIP;
      batch.n = 0;
    }
  }
  if (batch.n > 0 &&
      kda::launch_copy_states(src_states, src_pos, dst_states, dst_pos, n_floats, batch, st) != hipSuccess)
    return KDA_ERR_HIP;
  return KDA_OK;
}

kda_status check_pairs(const kda_shape& s, const int32_t* seq_ids, const int32_t* slot_ids, int32_t n,
                       const kda_slots* slots) {
  if (n < 0) return KDA_ERR_SHAPE;
  if (n > 0 && (!seq_ids || !slot_ids)) return KDA_ERR_NULL;
  for (int32_t i = 0; i < n; ++i) {
    if (seq_ids[i] < 0 || seq_ids[i] >= s.B) return KDA_ERR_SLOT;
    if (slot_ids[i] < 0 || slot_ids[i] >= slots->n_slots) return KDA_ERR_SLOT;
  }
  return KDA_OK;
}

kda_status check_prefill(const kda_shape* shape, int32_t L, int32_t chunk, float* state, int64_t* pos,
                         const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                         float* o, int32_t ckpt_every, const int32_t* ckpt_slots, const kda_slots* slots,
                         int32_t* dev_err) {
  kda_status r = check_shape(shape);
  if (r != KDA_OK) return r;
  if (L < 0 || !(chunk == 32 || chunk == 64)) return KDA_ERR_SHAPE;
  if (ckpt_every < 0 || (ckpt_every > 0 && ckpt_every % chunk != 0)) return KDA_ERR_SHAPE;
  if ((int64_t)shape->B * L * shape->H > (int64_t)1 << 40) return KDA_ERR_SHAPE;
  if (shape->B == 0) return KDA_OK;
  if (!state || !pos) return KDA_ERR_NULL;
  if (L > 0 && (r = check_tokens(q, k, v, alpha, beta, o)) != KDA_OK) return r;
  if ((r = check_ptrs({state})) != KDA_OK) return r;
  if (!aligned(pos, 8)) return KDA_ERR_ALIGN;
  if (ckpt_every > 0 && L >= ckpt_every) {
    if (!ckpt_slots || !dev_err) return KDA_ERR_NULL;
    if ((r = check_slots(slots)) != KDA_OK) return r;
    if (!aligned(ckpt_slots, 4) || !aligned(dev_err, 4)) return KDA_ERR_ALIGN;
  }
  return KDA_OK;
}

}  // namespace

extern "C" {

size_t kda_log_bytes(const kda_shape* shape, int32_t T_max) {
  if (check_shape(shape) != KDA_OK || T_max < 1 || T_max > kMaxT) return 0;
  return kda::log_layout(*shape, T_max).total;
}

size_t kda_slot_bytes(const kda_shape* shape) {
  if (check_shape(shape) != KDA_OK) return 0;
  return (size_t)shape->H * shape->dk * shape->dv * sizeof(float);
}

kda_status kda_decode_step(const kda_shape* shape, float* state, int64_t* pos, const void* q, const void* k,
                           const void* v, const float* alpha, const float* beta, float* o, void* stream) {
  kda_status r = check_shape(shape);
  if (r != KDA_OK) return r;
  if (shape->B == 0) return KDA_OK;
  if ((r = check_ptrs({state})) != KDA_OK) return r;
  if ((r = check_tokens(q, k, v, alpha, beta, o)) != KDA_OK) return r;
  if (!pos) return KDA_ERR_NULL;
  if (!aligned(pos, 8)) return KDA_ERR_ALIGN;
  return launched(kda::launch_decode(*shape, state, pos, kda::TokenInputs{q, k, v, alpha, beta}, o,
                                     static_cast<hipStream_t>(stream)),
                  KDA_VARIANT_DECODE);
}

kda_status kda_decode_step_prep(const kda_shape* shape, int32_t gate, float* state, int64_t* pos, const void* q,
                                const void* k, const void* v, const float* alpha_logit, const float* beta_logit,
                                float* o, void* stream) {
  kda_status r = check_shape(shape);
  if (r != KDA_OK) return r;
  if (gate != KDA_GATE_EXP_NEG_SOFTPLUS && gate != KDA_GATE_SIGMOID) return KDA_ERR_SHAPE;
  if (shape->B == 0) return KDA_OK;
  if ((r = check_ptrs({state})) != KDA_OK) return r;
  if ((r = check_tokens(q, k, v, alpha_logit, beta_logit, o)) != KDA_OK) return r;
  if (!pos) return KDA_ERR_NULL;
  if (!aligned(pos, 8)) return KDA_ERR_ALIGN;
  const float gate_sign = gate == KDA_GATE_SIGMOID ? 1.f : -1.f;
  return launched(kda::launch_decode_prep(*shape, state, pos, kda::TokenInputs{q, k, v, alpha_logit, beta_logit}, o,
                                          gate_sign, static_cast<hipStream_t>(stream)),
                  KDA_VARIANT_DECODE_PREP);
}

namespace {

bool valid_gate(int32_t gate) { return gate == KDA_GATE_EXP_NEG_SOFTPLUS || gate == KDA_GATE_SIGMOID; }

// gate < 0: prepared inputs; otherwise raw projections and logits.
kda_status check_slot_ids(const int32_t* slot_ids, int32_t* dev_err) {
  if (!slot_ids || !dev_err) return KDA_ERR_NULL;
  if (!aligned(slot_ids, 4) || !aligned(dev_err, 4)) return KDA_ERR_ALIGN;
  return KDA_OK;
}

// slot_ids non-null: state (and pos) are a slot pool's arrays of n_slots.
kda_status verify_impl(const kda_shape* shape, int32_t T, const int32_t* draft_len, const float* state, const void* q,
                       const void* k, const void* v, const float* alpha, const float* beta, float* o, kda_log* log,
                       int32_t* dev_err, bool varlen, int32_t gate, void* stream, const int32_t* slot_ids = nullptr,
                       int32_t n_slots = 0) {
  kda_status r = check_shape(shape);
  if (r != KDA_OK) return r;
  if ((r = check_log(*shape, log)) != KDA_OK) return r;
  if (T < 1 || T > log->T_max) return KDA_ERR_SHAPE;
  if (log->pending_T != 0) return KDA_ERR_ORDER;
  if (shape->B > 0) {
    if ((r = check_ptrs({state})) != KDA_OK) return r;
    if ((r = check_tokens(q, k, v, alpha, beta, o)) != KDA_OK) return r;
    if (varlen) {
      if (!draft_len || !dev_err) return KDA_ERR_NULL;
      if (!aligned(draft_len, 4) || !aligned(dev_err, 4)) return KDA_ERR_ALIGN;
    }
    if (n_slots > 0 && (r = check_slot_ids(slot_ids, dev_err)) != KDA_OK) return r;
    r = launched(kda::launch_verify(*shape, T, draft_len, state, kda::TokenInputs{q, k, v, alpha, beta}, o,
                                    log_ptrs(*shape, log), dev_err, gate, static_cast<hipStream_t>(stream), slot_ids,
                                    n_slots),
                 n_slots > 0 ? KDA_VARIANT_VERIFY_SLOTS
                 : gate >= 0 ? KDA_VARIANT_VERIFY_PREP
                 : varlen    ? KDA_VARIANT_VERIFY_VARLEN
                             : KDA_VARIANT_VERIFY);
    if (r != KDA_OK) return r;
  }
  log->pending_T = T;
  log->pending_form = gate < 0 ? 0 : 1 + gate;
  return KDA_OK;
}

kda_status commit_verify_impl(const kda_shape* shape, int32_t T, const int32_t* draft_len, float* state,
                              int64_t* pos, const void* q, const void* k, const void* v, const float* alpha,
                              const float* beta, float* o, kda_log* log, const int32_t* accepted, int32_t* dev_err,
                              bool varlen, int32_t gate, void* stream, const int32_t* slot_ids = nullptr,
                              int32_t n_slots = 0) {
  kda_status r = check_shape(shape);
  if (r != KDA_OK) return r;
  if ((r = check_log(*shape, log)) != KDA_OK) return r;
  if (T < 1 || T > log->T_max) return KDA_ERR_SHAPE;
  const int32_t pend = log->pending_T;
  if (pend < 0 || pend > log->T_max) return KDA_ERR_ORDER;
  // One fused launch replays one logged form: raw after the _prep verify only.
  if (pend > 0 && (log->pending_form != 0) != (gate >= 0)) return KDA_ERR_ORDER;
  if (shape->B > 0) {
    if ((r = check_ptrs({state})) != KDA_OK) return r;
    if ((r = check_tokens(q, k, v, alpha, beta, o)) != KDA_OK) return r;
    if (!pos) return KDA_ERR_NULL;
    if (!aligned(pos, 8)) return KDA_ERR_ALIGN;
    if (pend > 0) {
      if (!accepted) return KDA_ERR_NULL;
      if (!aligned(accepted, 4)) return KDA_ERR_ALIGN;
    }
    if (varlen) {
      if (!draft_len) return KDA_ERR_NULL;
      if (!aligned(draft_len, 4)) return KDA_ERR_ALIGN;
    }
    if (pend > 0 || varlen) {
      if (!dev_err) return KDA_ERR_NULL;
      if (!aligned(dev_err, 4)) return KDA_ERR_ALIGN;
    }
    if (n_slots > 0 && (r = check_slot_ids(slot_ids, dev_err)) != KDA_OK) return r;
    r = launched(kda::launch_commit_verify(*shape, pend, T, draft_len, state, pos, accepted, dev_err,
                                           kda::TokenInputs{q, k, v, alpha, beta}, o, log_ptrs(*shape, log), gate,
                                           log->pending_form - 1, static_cast<hipStream_t>(stream), slot_ids,
                                           n_slots),
                 n_slots > 0 ? KDA_VARIANT_COMMIT_VERIFY_SLOTS
                 : gate >= 0 ? KDA_VARIANT_COMMIT_VERIFY_PREP
                 : varlen    ? KDA_VARIANT_COMMIT_VERIFY_VARLEN
                             : KDA_VARIANT_COMMIT_VERIFY);
    if (r != KDA_OK) return r;
  }
  log->pending_T = T;
  log->pending_form = gate < 0 ? 0 : 1 + gate;
  return KDA_OK;
}

}  // namespace

kda_status kda_verify(const kda_shape* shape, int32_t T, const float* state, const void* q, const void* k,
                      const void* v, const float* alpha, const float* beta, float* o, kda_log* log, void* stream) {
  return verify_impl(shape, T, nullptr, state, q, k, v, alpha, beta, o, log, nullptr, false, -1, stream);
}

kda_status kda_verify_prep(const kda_shape* shape, int32_t gate, int32_t T, const float* state, const void* q,
                           const void* k, const void* v, const float* alpha_logit, const float* beta_logit, float* o,
                           kda_log* log, void* stream) {
  if (!valid_gate(gate)) return KDA_ERR_SHAPE;
  return verify_impl(shape, T, nullptr, state, q, k, v, alpha_logit, beta_logit, o, log, nullptr, false, gate, stream);
}

kda_status kda_verify_varlen(const kda_shape* shape, int32_t T, const int32_t* draft_len, const float* state,
                             const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                             float* o, kda_log* log, int32_t* dev_err, void* stream) {
  return verify_impl(shape, T, draft_len, state, q, k, v, alpha, beta, o, log, dev_err, true, -1, stream);
}

namespace {

kda_status commit_impl(const kda_shape* shape, float* state, int64_t* pos, kda_log* log, const int32_t* accepted,
                       int32_t* dev_err, void* stream, const int32_t* slot_ids, int32_t n_slots) {
  kda_status r = check_shape(shape);
  if (r != KDA_OK) return r;
  if ((r = check_log(*shape, log)) != KDA_OK) return r;
  if (log->pending_T < 1 || log->pending_T > log->T_max) return KDA_ERR_ORDER;
  if (shape->B > 0) {
    if ((r = check_ptrs({state})) != KDA_OK) return r;
    if (!pos || !accepted || !dev_err) return KDA_ERR_NULL;
    if (!aligned(pos, 8) || !aligned(accepted, 4) || !aligned(dev_err, 4)) return KDA_ERR_ALIGN;
    if (n_slots > 0 && (r = check_slot_ids(slot_ids, dev_err)) != KDA_OK) return r;
    r = launched(kda::launch_commit(*shape, log->pending_T, state, pos, log_ptrs(*shape, log), accepted, dev_err,
                                    log->pending_form, static_cast<hipStream_t>(stream), slot_ids, n_slots),
                 n_slots > 0 ? KDA_VARIANT_COMMIT_SLOTS : KDA_VARIANT_COMMIT);
    if (r != KDA_OK) return r;
  }
  log->pending_T = 0;
  return KDA_OK;
}

}  // namespace

kda_status kda_commit(const kda_shape* shape, float* state, int64_t* pos, kda_log* log, const int32_t* accepted,
                      int32_t* dev_err, void* stream) {
  return commit_impl(shape, state, pos, log, accepted, dev_err, stream, nullptr, 0);
}

kda_status kda_verify_slots(const kda_shape* shape, int32_t T, const int32_t* slot_ids, const kda_slots* slots,
                            const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                            float* o, kda_log* log, int32_t* dev_err, void* stream) {
  kda_status r = check_slots(slots);
  if (r != KDA_OK) return r;
  if (slots->n_slots == 0 && shape && shape->B > 0) return KDA_ERR_SLOT;
  return verify_impl(shape, T, nullptr, slots->states, q, k, v, alpha, beta, o, log, dev_err, false, -1, stream,
                     slot_ids, slots->n_slots);
}

kda_status kda_commit_slots(const kda_shape* shape, const int32_t* slot_ids, const kda_slots* slots, kda_log* log,
                            const int32_t* accepted, int32_t* dev_err, void* stream) {
  kda_status r = check_slots(slots);
  if (r != KDA_OK) return r;
  if (slots->n_slots == 0 && shape && shape->B > 0) return KDA_ERR_SLOT;
  return commit_impl(shape, slots->states, slots->pos, log, accepted, dev_err, stream, slot_ids, slots->n_slots);
}

kda_status kda_commit_verify_slots(const kda_shape* shape, int32_t T, const int32_t* slot_ids, const kda_slots* slots,
                                   const void* q, const void* k, const void* v, const float* alpha,
                                   const float* beta, float* o, kda_log* log, const int32_t* accepted,
                                   int32_t* dev_err, void* stream) {
  kda_status r = check_slots(slots);
  if (r != KDA_OK) return r;
  if (slots->n_slots == 0 && shape && shape->B > 0) return KDA_ERR_SLOT;
  if (!dev_err) return KDA_ERR_NULL;
  return commit_verify_impl(shape, T, nullptr, slots->states, slots->pos, q, k, v, alpha, beta, o, log, accepted,
                            dev_err, false, -1, stream, slot_ids, slots->n_slots);
}

kda_status kda_commit_verify(const kda_shape* shape, int32_t T, float* state, int64_t* pos, const void* q,
                             const void* k, const void* v, const float* alpha, const float* beta, float* o,
                             kda_log* log, const int32_t* accepted, int32_t* dev_err, void* stream) {
  return commit_verify_impl(shape, T, nullptr, state, pos, q, k, v, alpha, beta, o, log, accepted, dev_err, false,
                            -1, stream);
}

kda_status kda_commit_verify_prep(const kda_shape* shape, int32_t gate, int32_t T, float* state, int64_t* pos,
                                  const void* q, const void* k, const void* v, const float* alpha_logit,
                                  const float* beta_logit, float* o, kda_log* log, const int32_t* accepted,
                                  int32_t* dev_err, void* stream) {
  if (!valid_gate(gate)) return KDA_ERR_SHAPE;
  return commit_verify_impl(shape, T, nullptr, state, pos, q, k, v, alpha_logit, beta_logit, o, log, accepted,
                            dev_err, false, gate, stream);
}

kda_status kda_commit_verify_varlen(const kda_shape* shape, int32_t T, const int32_t* draft_len, float* state,
                                    int64_t* pos, const void* q, const void* k, const void* v, const float* alpha,
                                    const float* beta, float* o, kda_log* log, const int32_t* accepted,
                                    int32_t* dev_err, void* stream) {
  return commit_verify_impl(shape, T, draft_len, state, pos, q, k, v, alpha, beta, o, log, accepted, dev_err, true,
                            -1, stream);
}

kda_status kda_decode_step_slots(const kda_shape* shape, const int32_t* slot_ids, const kda_slots* slots,
                                 const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                                 float* o, int32_t* dev_err, void* stream) {
  kda_status r = check_shape(shape);
  if (r != KDA_OK) return r;
  if ((r = check_slots(slots)) != KDA_OK) return r;
  if (shape->B == 0) return KDA_OK;
  if ((r = check_tokens(q, k, v, alpha, beta, o)) != KDA_OK) return r;
  if (!slot_ids || !dev_err) return KDA_ERR_NULL;
  if (!aligned(slot_ids, 4) || !aligned(dev_err, 4)) return KDA_ERR_ALIGN;
  return launched(kda::launch_decode_slots(*shape, slot_ids, slots->states, slots->pos, slots->n_slots,
                                           kda::TokenInputs{q, k, v, alpha, beta}, o, dev_err,
                                           static_cast<hipStream_t>(stream)),
                  KDA_VARIANT_DECODE_SLOTS);
}

kda_status kda_slot_copy(const kda_shape* shape, const int32_t* src_slots, const int32_t* dst_slots, int32_t n,
                         const kda_slots* slots, void* stream) {
  kda_status r = check_shape(shape);
  if (r != KDA_OK) return r;
  if ((r = check_slots(slots)) != KDA_OK) return r;
  if (n < 0) return KDA_ERR_SHAPE;
  if (n == 0) return KDA_OK;
  if (!src_slots || !dst_slots) return KDA_ERR_NULL;
  for (int32_t i = 0; i < n; ++i) {
    if (src_slots[i] < 0 || src_slots[i] >= slots->n_slots) return KDA_ERR_SLOT;
    if (dst_slots[i] < 0 || dst_slots[i] >= slots->n_slots) return KDA_ERR_SLOT;
  }
  for (int32_t i = 0; i < n; ++i)
    for (int32_t j = 0; j < n; ++j)
      if (src_slots[i] == dst_slots[j]) return KDA_ERR_SLOT;  // copies of one call run concurrently
  const size_t n_floats = (size_t)shape->H * shape->dk * shape->dv;
  r = copy_pairs(std::vector<int32_t>(src_slots, src_slots + n), std::vector<int32_t>(dst_slots, dst_slots + n),
                 slots->states, slots->pos, slots->states, slots->pos, n_floats, static_cast<hipStream_t>(stream));
  if (r == KDA_OK) g_last_variant = KDA_VARIANT_SLOT_COPY;
  return r;
}

kda_status kda_snapshot(const kda_shape* shape, const float* state, const int64_t* pos, const int32_t* seq_ids,
                        const int32_t* slot_ids, int32_t n, const kda_slots* slots, void* stream) {
  kda_status r = check_shape(shape);
  if (r != KDA_OK) return r;
  if ((r = check_slots(slots)) != KDA_OK) return r;
  if ((r = check_pairs(*shape, seq_ids, slot_ids, n, slots)) != KDA_OK) return r;
  if (n == 0) return KDA_OK;
  if ((r = check_ptrs({state})) != KDA_OK) return r;
  if (!pos) return KDA_ERR_NULL;
  if (!aligned(pos, 8)) return KDA_ERR_ALIGN;
  const size_t n_floats = (size_t)shape->H * shape->dk * shape->dv;
  r = copy_pairs(std::vector<int32_t>(seq_ids, seq_ids + n), std::vector<int32_t>(slot_ids, slot_ids + n), state,
                 pos, slots->states, slots->pos, n_floats, static_cast<hipStream_t>(stream));
  if (r == KDA_OK) g_last_variant = KDA_VARIANT_SNAPSHOT;
  return r;
}

kda_status kda_restore(const kda_shape* shape, float* state, int64_t* pos, const int32_t* seq_ids,
                       const int32_t* slot_ids, int32_t n, const kda_slots* slots, void* stream) {
  kda_status r = check_shape(shape);
  if (r != KDA_OK) return r;
  if ((r = check_slots(slots)) != KDA_OK) return r;
  if ((r = check_pairs(*shape, seq_ids, slot_ids, n, slots)) != KDA_OK) return r;
  if (n == 0) return KDA_OK;
  if ((r = check_ptrs({state})) != KDA_OK) return r;
  if (!pos) return KDA_ERR_NULL;
  if (!aligned(pos, 8)) return KDA_ERR_ALIGN;
  const size_t n_floats = (size_t)shape->H * shape->dk * shape->dv;
  r = copy_pairs(std::vector<int32_t>(slot_ids, slot_ids + n), std::vector<int32_t>(seq_ids, seq_ids + n),
                 slots->states, slots->pos, state, pos, n_floats, static_cast<hipStream_t>(stream));
  if (r == KDA_OK) g_last_variant = KDA_VARIANT_RESTORE;
  return r;
}

namespace {

kda_status prefill_chunked_impl(const kda_shape* shape, int32_t L, int32_t chunk, float* state, int64_t* pos,
                                const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                                float* o, int32_t ckpt_every, const int32_t* ckpt_slots, const kda_slots* slots,
                                int32_t* dev_err, int32_t gate, void* stream, const int32_t* state_slots = nullptr) {
  kda_status r = check_prefill(shape, L, chunk, state, pos, q, k, v, alpha, beta, o, ckpt_every, ckpt_slots, slots,
                               dev_err);
  // An empty prompt leaves every state and position as it is: nothing to launch.
  if (r != KDA_OK || shape->B == 0 || L == 0) return r;
  const bool ck = ckpt_every > 0 && L >= ckpt_every;
  if (state_slots) {  // the caller passed the pool's arrays as state and pos
    if ((r = check_slot_ids(state_slots, dev_err)) != KDA_OK) return r;
    return launched(kda::launch_prefill_chunked(*shape, L, chunk, state, pos, kda::TokenInputs{q, k, v, alpha, beta},
                                                o, ck ? ckpt_every : 0, ck ? ckpt_slots : nullptr, slots->states,
                                                slots->pos, slots->n_slots, dev_err, gate,
                                                static_cast<hipStream_t>(stream), state_slots),
                    KDA_VARIANT_PREFILL_CHUNKED_SLOTS);
  }
  return launched(kda::launch_prefill_chunked(*shape, L, chunk, state, pos, kda::TokenInputs{q, k, v, alpha, beta},
                                              o, ck ? ckpt_every : 0, ck ? ckpt_slots : nullptr,
                                              ck ? slots->states : nullptr, ck ? slots->pos : nullptr,
                                              ck ? slots->n_slots : 0, dev_err, gate,
                                              static_cast<hipStream_t>(stream)),
                  gate < 0 ? KDA_VARIANT_PREFILL_CHUNKED : KDA_VARIANT_PREFILL_CHUNKED_PREP);
}

kda_status prefill_recurrent_impl(const kda_shape* shape, int32_t L, float* state, int64_t* pos, const void* q,
                                  const void* k, const void* v, const float* alpha, const float* beta, float* o,
                                  int32_t ckpt_every, const int32_t* ckpt_slots, const kda_slots* slots,
                                  int32_t* dev_err, int32_t gate, void* stream) {
  // Same checks as the chunked form except the chunk size, which does not
  // apply here, so any positive checkpoint interval is allowed.
  kda_status r = check_prefill(shape, L, 32, state, pos, q, k, v, alpha, beta, o, 0, nullptr, nullptr, dev_err);
  if (r != KDA_OK || shape->B == 0) return r;
  if (ckpt_every < 0) return KDA_ERR_SHAPE;
  if (L == 0) return KDA_OK;  // an empty prompt: nothing to launch
  const bool ck = ckpt_every > 0 && L >= ckpt_every;
  if (ck) {
    if (!ckpt_slots || !dev_err) return KDA_ERR_NULL;
    if ((r = check_slots(slots)) != KDA_OK) return r;
    if (!aligned(ckpt_slots, 4) || !aligned(dev_err, 4)) return KDA_ERR_ALIGN;
  }
  return launched(kda::launch_prefill_recurrent(*shape, L, state, pos, kda::TokenInputs{q, k, v, alpha, beta}, o,
                                                ck ? ckpt_every : 0, ck ? ckpt_slots : nullptr,
                                                ck ? slots->states : nullptr, ck ? slots->pos : nullptr,
                                                ck ? slots->n_slots : 0, dev_err, gate,
                                                static_cast<hipStream_t>(stream)),
                  gate < 0 ? KDA_VARIANT_PREFILL_RECURRENT : KDA_VARIANT_PREFILL_RECURRENT_PREP);
}

}  // namespace

kda_status kda_prefill_chunked(const kda_shape* shape, int32_t L, int32_t chunk, float* state, int64_t* pos,
                               const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                               float* o, int32_t ckpt_every, const int32_t* ckpt_slots, const kda_slots* slots,
                               int32_t* dev_err, void* stream) {
  return prefill_chunked_impl(shape, L, chunk, state, pos, q, k, v, alpha, beta, o, ckpt_every, ckpt_slots, slots,
                              dev_err, -1, stream);
}

kda_status kda_prefill_chunked_slots(const kda_shape* shape, int32_t L, int32_t chunk, const int32_t* state_slots,
                                     const kda_slots* slots, const void* q, const void* k, const void* v,
                                     const float* alpha, const float* beta, float* o, int32_t ckpt_every,
                                     const int32_t* ckpt_slots, int32_t* dev_err, void* stream) {
  kda_status r = check_slots(slots);
  if (r != KDA_OK) return r;
  if (slots->n_slots == 0 && shape && shape->B > 0) return KDA_ERR_SLOT;
  if (!dev_err && shape && shape->B > 0) return KDA_ERR_NULL;
  return prefill_chunked_impl(shape, L, chunk, slots->states, slots->pos, q, k, v, alpha, beta, o, ckpt_every,
                              ckpt_slots, slots, dev_err, -1, stream, state_slots);
}

kda_status kda_prefill_chunked_prep(const kda_shape* shape, int32_t gate, int32_t L, int32_t chunk, float* state,
                                    int64_t* pos, const void* q, const void* k, const void* v,
                                    const float* alpha_logit, const float* beta_logit, float* o, int32_t ckpt_every,
                                    const int32_t* ckpt_slots, const kda_slots* slots, int32_t* dev_err,
                                    void* stream) {
  if (!valid_gate(gate)) return KDA_ERR_SHAPE;
  return prefill_chunked_impl(shape, L, chunk, state, pos, q, k, v, alpha_logit, beta_logit, o, ckpt_every,
                              ckpt_slots, slots, dev_err, gate, stream);
}

kda_status kda_prefill_recurrent(const kda_shape* shape, int32_t L, float* state, int64_t* pos, const void* q,
                                 const void* k, const void* v, const float* alpha, const float* beta, float* o,
                                 int32_t ckpt_every, const int32_t* ckpt_slots, const kda_slots* slots,
                                 int32_t* dev_err, void* stream) {
  return prefill_recurrent_impl(shape, L, state, pos, q, k, v, alpha, beta, o, ckpt_every, ckpt_slots, slots, dev_err,
                                -1, stream);
}

kda_status kda_prefill_recurrent_prep(const kda_shape* shape, int32_t gate, int32_t L, float* state, int64_t* pos,
                                      const void* q, const void* k, const void* v, const float* alpha_logit,
                                      const float* beta_logit, float* o, int32_t ckpt_every,
                                      const int32_t* ckpt_slots, const kda_slots* slots, int32_t* dev_err,
                                      void* stream) {
  if (!valid_gate(gate)) return KDA_ERR_SHAPE;
  return prefill_recurrent_impl(shape, L, state, pos, q, k, v, alpha_logit, beta_logit, o, ckpt_every, ckpt_slots,
                                slots, dev_err, gate, stream);
}

kda_status kda_mixed_step(const kda_shape* shape, const int32_t* roles, const int32_t* tok_start, int32_t n_tokens,
                          int32_t n_decode, int32_t n_spec, int32_t n_prefill, float* state, int64_t* pos,
                          const int32_t* slot_ids, int32_t n_slots, const void* q, const void* k, const void* v,
                          const float* alpha, const float* beta, float* o, kda_log* log, const int32_t* accepted,
                          int32_t* dev_err, void* stream) {
  kda_status r = check_shape(shape);
  if (r != KDA_OK) return r;
  if (n_tokens < 0 || n_decode < 0 || n_spec < 0 || n_prefill < 0) return KDA_ERR_SHAPE;
  if ((int64_t)n_decode + n_spec + n_prefill > shape->B) return KDA_ERR_SHAPE;
  if (slot_ids && n_slots < 1) return KDA_ERR_SHAPE;
  int32_t pend = 0;
  if (log) {
    if ((r = check_log(*shape, log)) != KDA_OK) return r;
    pend = log->pending_T;
    if (pend < 0 || pend > log->T_max) return KDA_ERR_ORDER;
    if (pend > 0 && log->pending_form != 0) return KDA_ERR_ORDER;  // one replay form: prepared
  } else if (n_spec > 0) {
    return KDA_ERR_NULL;
  }
  if (shape->B > 0) {
    if (!roles || !tok_start || !dev_err || !pos) return KDA_ERR_NULL;
    if (!aligned(roles, 4) || !aligned(tok_start, 4) || !aligned(dev_err, 4) || !aligned(pos, 8))
      return KDA_ERR_ALIGN;
    if ((r = check_ptrs({state})) != KDA_OK) return r;
    if (n_tokens > 0 && (r = check_tokens(q, k, v, alpha, beta, o)) != KDA_OK) return r;
    if (pend > 0) {
      if (!accepted) return KDA_ERR_NULL;
      if (!aligned(accepted, 4)) return KDA_ERR_ALIGN;
    }
    if (slot_ids && !aligned(slot_ids, 4)) return KDA_ERR_ALIGN;
    const kda::LogPtrs lp = log ? log_ptrs(*shape, log) : kda::LogPtrs{};
    const kda::MixedBatch m{roles, tok_start, n_tokens, n_decode, n_spec, n_prefill};
    r = launched(kda::launch_mixed(*shape, m, state, pos, slot_ids, slot_ids ? n_slots : shape->B,
                                   kda::TokenInputs{q, k, v, alpha, beta}, o, log ? &lp : nullptr, pend, accepted,
                                   dev_err, static_cast<hipStream_t>(stream)),
                 KDA_VARIANT_MIXED);
    if (r != KDA_OK) return r;
  }
  if (log) {
    log->pending_T = n_spec > 0 ? log->T_max : 0;
    log->pending_form = 0;
  }
  return KDA_OK;
}

const char* kda_status_str(kda_status status) {
  switch (status) {
    case KDA_OK: return "ok";
    case KDA_ERR_NULL: return "null pointer";
    case KDA_ERR_SHAPE: return "unsupported or inconsistent size";
    case KDA_ERR_DTYPE: return "unknown input dtype";
    case KDA_ERR_ALIGN: return "misaligned pointer";
    case KDA_ERR_ORDER: return "verify/commit out of order";
    case KDA_ERR_SLOT: return "sequence or slot index out of range";
    case KDA_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

int32_t kda_last_variant(void) { return g_last_variant; }

int32_t kda_abi_version(void) { return KDA_ABI_VERSION; }

}  // extern "C"
