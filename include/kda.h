/*
 * kda.h - C ABI of libkda, the MI355X (gfx950) KDA recurrent-state library.
 *
 * Kimi Delta Attention keeps, per sequence and head, a fixed-size recurrent
 * state that every token updates ("Kimi K3: From Day-0 Availability to
 * Optimized Inference", nebius webinar summary, opening paragraph).  The
 * pages do not print the update; this library implements the
 * per-channel-gated delta rule.  Per sequence b and head h the state S is a
 * dk x dv fp32 matrix (row i = key channel, column j = value channel), and a
 * token with q, k (dk), v (dv), per-key-channel gate alpha (dk) and scalar
 * beta does
 *
 *     S <- Diag(alpha) S
 *     S <- S - beta k (k^T S) + beta k v^T
 *     o  = scale * S^T q              (read after the update)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layouts (all dense, row-major, device memory unless stated otherwise):
 *   state   f32 [B][H][dk][dv]        updated in place
 *   q, k    in_dtype [B][T][H][dk]    (T = 1 for a decode step)
 *   v       in_dtype [B][T][H][dv]
 *   alpha   f32 [B][T][H][dk]         gates in [0, 1] (0 forgets the channel)
 *   beta    f32 [B][T][H]
 *   o       f32 [B][T][H][dv]         must not alias any input
 *   pos     i64 [B]                   token position of each sequence
 * in_dtype is KDA_BF16 (bfloat16 bit patterns) or KDA_F32.
 *
 * Ownership: the caller allocates every buffer (state, inputs, outputs, log,
 * slot pool, positions, counters).  The library never allocates or frees
 * device memory and never synchronizes; each call validates its arguments on
 * the host and then only enqueues kernels on `stream` (a hipStream_t; NULL
 * is the null stream).  Results are available when the stream reaches them.
 *
 * Alignment: state, q, k, v, alpha, o and the slot states must be 16-byte
 * aligned; beta, accepted, dev_err and checkpoint slot ids 4-byte; pos and
 * slot positions 8-byte; the log buffer 256-byte.  (Any row-aligned slice of
 * a dense tensor along B, T or H satisfies these.)
 *
 * Errors: argument errors are detected on the host before anything is
 * enqueued and return a status without side effects.  Values the host
 * cannot see (accepted counts, checkpoint slot ids in device memory) are
 * checked on the device: a bad value sets bits in the caller's sticky
 * `dev_err` word and leaves the affected sequence untouched.  Launch
 * failures return KDA_ERR_HIP.  No call prints, throws or aborts.  Values
 * are not checked: NaN and Inf propagate.
 *
 * Threading: calls are reentrant; calls on different streams with disjoint
 * buffers may run concurrently.  Calls that share a buffer must be ordered
 * by the caller (same stream or events).
 *
 * Supported sizes: dk, dv in {64, 128}; B >= 0 (B = 0 is a no-op); H >= 1;
 * verify 1 <= T <= T_max <= 16; prefill chunk in {32, 64}.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 1

typedef enum kda_status {
  KDA_OK = 0,
  KDA_ERR_NULL = 1,   /* a required pointer is NULL */
  KDA_ERR_SHAPE = 2,  /* unsupported or inconsistent size */
  KDA_ERR_DTYPE = 3,  /* unknown in_dtype code */
  KDA_ERR_ALIGN = 4,  /* a pointer is not aligned as required */
  KDA_ERR_ORDER = 5,  /* commit without a pending verify, or verify while one is pending */
  KDA_ERR_SLOT = 6,   /* a sequence or slot index is out of range */
  KDA_ERR_HIP = 7     /* the HIP runtime rejected a launch */
} kda_status;

typedef enum kda_dtype { KDA_BF16 = 0, KDA_F32 = 1 } kda_dtype;

/* Bits set in the device error word. */
#define KDA_DEV_ERR_ACCEPTED 1 /* an accepted count was outside [0, T] */
#define KDA_DEV_ERR_CKPT_SLOT 2 /* a checkpoint slot id was outside [0, n_slots) */
#define KDA_DEV_ERR_DRAFT_LEN 4 /* a per-sequence draft length was outside [0, T] */
#define KDA_DEV_ERR_SLOT_ID 8   /* a device-side state slot id was outside [0, n_slots) */
#define KDA_DEV_ERR_MIXED 16    /* kda_mixed_step: roles or token ranges inconsistent with the launch */

/* Kernel variants reported by kda_last_variant(). */
#define KDA_VARIANT_NONE 0
#define KDA_VARIANT_DECODE 1
#define KDA_VARIANT_VERIFY 2
#define KDA_VARIANT_COMMIT 3
#define KDA_VARIANT_SNAPSHOT 4
#define KDA_VARIANT_RESTORE 5
#define KDA_VARIANT_PREFILL_RECURRENT 6
#define KDA_VARIANT_PREFILL_CHUNKED 7
#define KDA_VARIANT_COMMIT_VERIFY 8
#define KDA_VARIANT_VERIFY_VARLEN 9
#define KDA_VARIANT_COMMIT_VERIFY_VARLEN 10
#define KDA_VARIANT_DECODE_PREP 11
#define KDA_VARIANT_VERIFY_PREP 12
#define KDA_VARIANT_COMMIT_VERIFY_PREP 13
#define KDA_VARIANT_DECODE_SLOTS 14
#define KDA_VARIANT_SLOT_COPY 15
#define KDA_VARIANT_PREFILL_CHUNKED_PREP 16
#define KDA_VARIANT_PREFILL_RECURRENT_PREP 17
#define KDA_VARIANT_VERIFY_SLOTS 18
#define KDA_VARIANT_COMMIT_SLOTS 19
#define KDA_VARIANT_COMMIT_VERIFY_SLOTS 20
#define KDA_VARIANT_PREFILL_CHUNKED_SLOTS 21
#define KDA_VARIANT_MIXED 22

/* What a sequence does in a kda_mixed_step. */
#define KDA_ROLE_IDLE 0    /* nothing this step */
#define KDA_ROLE_DECODE 1  /* one token, as kda_decode_step */
#define KDA_ROLE_SPEC 2    /* commit of its accepted drafts, then a verify of new ones */
#define KDA_ROLE_PREFILL 3 /* a segment of its prompt, as kda_prefill_chunked */

/* Decay gate of kda_decode_step_prep: alpha = f(x) of the logit x. */
#define KDA_GATE_EXP_NEG_SOFTPLUS 0 /* alpha = exp(-softplus(x)) = 1 / (1 + e^x) */
#define KDA_GATE_SIGMOID 1          /* alpha = sigmoid(x) = 1 / (1 + e^-x) */

typedef struct kda_shape {
  int32_t B;        /* sequences in the batch */
  int32_t H;        /* heads */
  int32_t dk;       /* key/query width: 64 or 128 */
  int32_t dv;       /* value width: 64 or 128 */
  int32_t in_dtype; /* kda_dtype of q, k, v */
  float scale;      /* output scale, normally 1/sqrt(dk) */
} kda_shape;

/*
 * Speculative-decoding input log ("Kimi K3: From Day-0 Availability to
 * Optimized Inference", paragraph on rejected draft tokens: the recurrent
 * inputs are stored and the accepted part is replayed from the last
 * committed state).  `dev` is a caller-owned device buffer of
 * kda_log_bytes(shape, T_max) bytes.  It holds five regions, each starting
 * at a 256-byte boundary, in this order, with T_max token rows per sequence
 * of which the first n_bh (of the pending verify) are filled:
 *   k      in_dtype [B][T_max][H][dk]
 *   v      in_dtype [B][T_max][H][dv]
 *   alpha  f32 [B][T_max][H][dk]
 *   beta   f32 [B][T_max][H]
 *   n      i32 [B][H]   per (b, h): bits 0-15 the rows the pending verify
 *                       filled (T, or the sequence's draft length under the
 *                       _varlen calls); bits 16 and up the form of the logged
 *                       inputs: 0 prepared, 1 + gate for raw projections
 *                       (the _prep calls, which log their inputs raw)
 * The device writes n; a commit accepts at most n_bh tokens of (b, h) and
 * replays them with the update of their form.
 * `pending_T` and `pending_form` are host-side bookkeeping: the verify calls
 * set pending_T to T and pending_form to the form they logged (0 prepared
 * inputs, 1 + gate for the _prep calls), kda_commit consumes them and resets
 * pending_T to 0.  Initialise both to 0.
 */
typedef struct kda_log {
  void* dev;
  size_t bytes;
  int32_t T_max;
  int32_t pending_T;
  int32_t pending_form;
} kda_log;

/*
 * Slot pool for recurrent-state checkpoints (same webinar summary, paragraph
 * on prefix caching: the checkpoint sits at a token boundary shared with the
 * attention cache).  Caller-owned device memory:
 *   states  f32 [n_slots][H][dk][dv]
 *   pos     i64 [n_slots]   token position at which the slot's state was taken
 */
typedef struct kda_slots {
  float* states;
  int64_t* pos;
  int32_t n_slots;
} kda_slots;

/* Bytes needed for a log of up to T_max draft tokens; 0 for an invalid shape. */
size_t kda_log_bytes(const kda_shape* shape, int32_t T_max);

/* Bytes of one slot's state (H * dk * dv * 4); 0 for an invalid shape. */
size_t kda_slot_bytes(const kda_shape* shape);

/*
 * One decode token for every (sequence, head): the update above applied in
 * place to `state`, o = scale * S^T q written to `o` (f32 [B][H][dv]), and
 * pos[b] += 1.  Inputs use the layouts above with T = 1.
 * ("Hyper-optimizing Kimi K3 in vLLM", Part 1, section 1: a dedicated KDA
 * decode kernel scheduled for the batch size and heads per GPU.)
 */
kda_status kda_decode_step(const kda_shape* shape, float* state, int64_t* pos, const void* q,
                           const void* k, const void* v, const float* alpha, const float* beta,
                           float* o, void* stream);

/*
 * kda_decode_step from raw projections, with the input preparation done in
 * the kernel ("Kimi K3: From Day-0 Availability to Optimized Inference",
 * paragraph on profiling the token path: needless copies and type
 * conversions removed).  q and k (in_dtype [B][H][dk]) are taken
 * un-normalised and divided by their L2 norm over dk in fp32 (a zero vector
 * stays zero); alpha_logit (f32 [B][H][dk]) gives the decay through `gate`
 * (KDA_GATE_*); beta_logit (f32 [B][H]) gives beta = sigmoid(beta_logit).
 * v, state, o and pos as kda_decode_step.  Fails with KDA_ERR_SHAPE for an
 * unknown gate.
 */
kda_status kda_decode_step_prep(const kda_shape* shape, int32_t gate, float* state, int64_t* pos,
                                const void* q, const void* k, const void* v, const float* alpha_logit,
                                const float* beta_logit, float* o, void* stream);

/*
 * Speculative verify of T draft tokens per sequence from the committed
 * state: runs the T tokens on a private copy of each (b, h) state, writes
 * every output o_t (f32 [B][T][H][dv]) and copies k, v, alpha, beta of all T
 * tokens into the log.  `state` is read, never written.  Fails with
 * KDA_ERR_ORDER if `log` already has a pending verify.  The outputs are
 * computed in the chunk form of the rule (groups of up to four tokens from
 * the group's start state), so o_t agrees with what t decode steps would
 * produce to rounding, not bit for bit.
 * (Webinar summary, paragraph on rejected draft tokens.)
 */
kda_status kda_verify(const kda_shape* shape, int32_t T, const float* state, const void* q,
                      const void* k, const void* v, const float* alpha, const float* beta,
                      float* o, kda_log* log, void* stream);

/*
 * Commit: for each sequence b, replays the first accepted[b] logged tokens
 * onto the committed state in place and adds accepted[b] to pos[b].
 * `accepted` is a device int32 [B].  A count of 0 leaves the state bytes
 * untouched; a count outside [0, n_bh] (the rows the pending verify logged
 * for the sequence: pending_T, or its draft length) sets KDA_DEV_ERR_ACCEPTED in
 * *dev_err (device int32, sticky, never cleared by the library) and leaves
 * that sequence untouched.  The resulting state is bit-identical to
 * accepted[b] kda_decode_step calls on the same tokens.  Fails with
 * KDA_ERR_ORDER when no verify is pending; on success the log is released.
 * (Webinar summary, paragraph on rejected draft tokens.)
 */
kda_status kda_commit(const kda_shape* shape, float* state, int64_t* pos, kda_log* log,
                      const int32_t* accepted, int32_t* dev_err, void* stream);

/*
 * Commit of the pending verify fused with the next verify, in one launch:
 * for each sequence b, replays the first accepted[b] tokens of the pending
 * verify onto the state (exactly as kda_commit: bit-identical to that many
 * decode steps, pos[b] += accepted[b], KDA_DEV_ERR_ACCEPTED and no change
 * for a count outside [0, pending_T]), then verifies T new draft tokens from
 * the committed state (exactly as kda_verify: outputs o and the log of the
 * new tokens).  With no verify pending (pending_T == 0) it is a verify.
 * The committed state is written once and not read back: one state read per
 * speculative round instead of two.  accepted and dev_err may be NULL only
 * when nothing is pending.  On success pending_T = T.
 * (Webinar summary, paragraph on rejected draft tokens: the accepted part is
 * replayed from the last committed state; here the replay happens at the
 * start of the next round's verify.)
 */
kda_status kda_commit_verify(const kda_shape* shape, int32_t T, float* state, int64_t* pos, const void* q,
                             const void* k, const void* v, const float* alpha, const float* beta, float* o,
                             kda_log* log, const int32_t* accepted, int32_t* dev_err, void* stream);

/*
 * kda_verify with a draft length per sequence ("Hyper-optimizing Kimi K3 in
 * vLLM", section 2 on bounding the scope: speculative decoding is validated
 * over various draft lengths).  Inputs keep the [B][T][H][d] layout with T
 * the longest draft; sequence b verifies only its first draft_len[b] tokens
 * (device int32 [B], each in [0, T]; 0 = the sequence sits this round out).
 * For t >= draft_len[b] nothing is read, o is not written and no log row is
 * filled; the log records draft_len[b] so that a later commit accepts at most
 * that many tokens of b (KDA_DEV_ERR_ACCEPTED above it).  A length outside
 * [0, T] sets KDA_DEV_ERR_DRAFT_LEN in *dev_err and counts as 0.  draft_len
 * and dev_err must not be NULL when B > 0.  Otherwise as kda_verify.
 */
kda_status kda_verify_varlen(const kda_shape* shape, int32_t T, const int32_t* draft_len, const float* state,
                             const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                             float* o, kda_log* log, int32_t* dev_err, void* stream);

/*
 * kda_commit_verify whose new drafts have a length per sequence, as in
 * kda_verify_varlen.  The commit half accepts at most the length logged by
 * the pending verify; dev_err must not be NULL when B > 0.
 */
kda_status kda_commit_verify_varlen(const kda_shape* shape, int32_t T, const int32_t* draft_len, float* state,
                                    int64_t* pos, const void* q, const void* k, const void* v, const float* alpha,
                                    const float* beta, float* o, kda_log* log, const int32_t* accepted,
                                    int32_t* dev_err, void* stream);

/*
 * kda_verify from raw projections: q, k, alpha_logit, beta_logit as in
 * kda_decode_step_prep, with the [B][T][H][d] token layout.  The kernel
 * prepares them (unit q and k, decay and beta from their logits) and logs
 * them raw (k, v, alpha_logit, beta_logit), marking the log's records as raw
 * with this gate; kda_commit then replays them through the same preparation,
 * so the committed state is bit-identical to that many
 * kda_decode_step_prep calls.  Fails with KDA_ERR_SHAPE for an unknown gate.
 * (Webinar summary: rejected draft tokens, and needless conversions removed.)
 */
kda_status kda_verify_prep(const kda_shape* shape, int32_t gate, int32_t T, const float* state, const void* q,
                           const void* k, const void* v, const float* alpha_logit, const float* beta_logit,
                           float* o, kda_log* log, void* stream);

/*
 * kda_commit_verify whose new drafts are raw projections (as kda_verify_prep).
 * The pending verify, if any, must have logged raw projections too (any gate:
 * it is replayed with its own); after a verify of prepared inputs commit with
 * kda_commit first (KDA_ERR_ORDER otherwise).  Likewise kda_commit_verify and
 * kda_commit_verify_varlen need a pending verify of prepared inputs.
 */
kda_status kda_commit_verify_prep(const kda_shape* shape, int32_t gate, int32_t T, float* state, int64_t* pos,
                                  const void* q, const void* k, const void* v, const float* alpha_logit,
                                  const float* beta_logit, float* o, kda_log* log, const int32_t* accepted,
                                  int32_t* dev_err, void* stream);

/*
 * kda_decode_step on states that live in a slot pool, for serving loops that
 * keep every request's recurrent state in one pool and reuse cached prefixes
 * without copying states in and out (webinar summary, paragraph on the two
 * state systems and their allocation and reuse).  Sequence b of the batch
 * (inputs and o as kda_decode_step, batch B = shape->B) updates
 * slots->states[slot_ids[b]] in place and adds 1 to slots->pos[slot_ids[b]].
 * slot_ids is a DEVICE int32 [B]; the ids must be distinct (two sequences
 * naming one slot race).  An id outside [0, n_slots) sets KDA_DEV_ERR_SLOT_ID
 * in *dev_err and that sequence is skipped (its o rows are not written).
 * The arithmetic is kda_decode_step's, so the states are bit-identical.
 */
kda_status kda_decode_step_slots(const kda_shape* shape, const int32_t* slot_ids, const kda_slots* slots,
                                 const void* q, const void* k, const void* v, const float* alpha,
                                 const float* beta, float* o, int32_t* dev_err, void* stream);

/*
 * The speculative calls on states in a slot pool (as kda_decode_step_slots):
 * sequence b's state is slots->states[slot_ids[b]] (read by the verify,
 * updated by the commits) and its position slots->pos[slot_ids[b]] (advanced
 * by the commits).  slot_ids is a DEVICE int32 [B] of distinct ids; an id out
 * of range sets KDA_DEV_ERR_SLOT_ID and the sequence is skipped (its verify
 * logs no row, so a later count above 0 for it is flagged too).  The log,
 * inputs, outputs and counts are the batch's, as in kda_verify, kda_commit
 * and kda_commit_verify; the arithmetic is theirs, so states and outputs are
 * bit-identical.  dev_err must not be NULL.
 */
kda_status kda_verify_slots(const kda_shape* shape, int32_t T, const int32_t* slot_ids, const kda_slots* slots,
                            const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                            float* o, kda_log* log, int32_t* dev_err, void* stream);
kda_status kda_commit_slots(const kda_shape* shape, const int32_t* slot_ids, const kda_slots* slots, kda_log* log,
                            const int32_t* accepted, int32_t* dev_err, void* stream);
kda_status kda_commit_verify_slots(const kda_shape* shape, int32_t T, const int32_t* slot_ids, const kda_slots* slots,
                                   const void* q, const void* k, const void* v, const float* alpha,
                                   const float* beta, float* o, kda_log* log, const int32_t* accepted,
                                   int32_t* dev_err, void* stream);

/*
 * Slot-to-slot copy of whole states (all H heads) and positions:
 * slot dst_slots[i] <- slot src_slots[i], i < n (HOST int32 arrays,
 * range-checked before anything is enqueued: KDA_ERR_SLOT).  Forks a cached
 * prefix into the slot of a new request.  A destination named twice gets the
 * later pair; a slot that is both a source and a destination of one call is
 * rejected (KDA_ERR_SLOT), as the copies run concurrently.  Bitwise.
 */
kda_status kda_slot_copy(const kda_shape* shape, const int32_t* src_slots, const int32_t* dst_slots, int32_t n,
                         const kda_slots* slots, void* stream);

/*
 * Snapshot: copies the whole state of sequence seq_ids[i] (all H heads) and
 * its position into slot slot_ids[i], for i < n.  seq_ids and slot_ids are
 * HOST int32 arrays; every id is range-checked before anything is enqueued
 * (KDA_ERR_SLOT).  Slots written twice in one call get the later pair.
 * The copy is bitwise.  (Webinar summary, paragraph on prefix caching.)
 */
kda_status kda_snapshot(const kda_shape* shape, const float* state, const int64_t* pos,
                        const int32_t* seq_ids, const int32_t* slot_ids, int32_t n,
                        const kda_slots* slots, void* stream);

/*
 * Restore: copies slot slot_ids[i]'s state and position into sequence
 * seq_ids[i], for i < n (host arrays, range-checked as above).  Bitwise.
 * A sequence named twice gets the later pair.
 */
kda_status kda_restore(const kda_shape* shape, float* state, int64_t* pos, const int32_t* seq_ids,
                       const int32_t* slot_ids, int32_t n, const kda_slots* slots, void* stream);

/*
 * Prompt processing of L tokens per sequence into the state (in place), in
 * the chunked (WY / UT-transform) form with `chunk` tokens per chunk; the last
 * chunk may be partial.  Writes o for every token (f32 [B][L][H][dv]) and
 * adds L to pos.  Inputs use the layouts above with T = L.
 * When ckpt_every > 0 (a multiple of chunk) the state after every
 * ckpt_every tokens is also written to slot ckpt_slots[b * n_ckpt + m]
 * (m = 0 .. n_ckpt - 1, n_ckpt = L / ckpt_every), with slot position
 * pos[b] + (m + 1) * ckpt_every.  ckpt_slots is a DEVICE int32 array; an id
 * outside [0, slots->n_slots) sets KDA_DEV_ERR_CKPT_SLOT and that checkpoint
 * is skipped.  `dev_err` may be NULL only when ckpt_every == 0.
 * Gates: every alpha in [0, 1] is handled exactly (up to rounding).  The
 * chunk form divides by in-chunk decay products, so a chunk ends early, and
 * the next one starts, where some key channel's product of alphas since the
 * chunk's first token would fall below 2^-96; gates that decay that fast
 * make the call slower (shorter chunks), never less accurate.
 * L = 0 is a no-op: nothing is enqueued, the token pointers may be NULL, and
 * state and pos are left as they are.
 * (Webinar summary: prompt processing that prefix caching avoids, and the
 * recurrent-state checkpoint at a token boundary.)
 */
kda_status kda_prefill_chunked(const kda_shape* shape, int32_t L, int32_t chunk, float* state,
                               int64_t* pos, const void* q, const void* k, const void* v,
                               const float* alpha, const float* beta, float* o, int32_t ckpt_every,
                               const int32_t* ckpt_slots, const kda_slots* slots, int32_t* dev_err,
                               void* stream);

/*
 * The same prompt processing as kda_prefill_chunked, computed token by token
 * with the decode update while each (sequence, head) state stays in
 * registers for the whole prompt.  Arguments as for kda_prefill_chunked
 * without `chunk`; any ckpt_every > 0 is allowed (L = 0 is a no-op).  It is the cross-check for
 * the chunked form and the cheaper choice for very short prompts.
 */
kda_status kda_prefill_recurrent(const kda_shape* shape, int32_t L, float* state, int64_t* pos,
                                 const void* q, const void* k, const void* v, const float* alpha,
                                 const float* beta, float* o, int32_t ckpt_every,
                                 const int32_t* ckpt_slots, const kda_slots* slots, int32_t* dev_err,
                                 void* stream);

/*
 * kda_prefill_chunked on states in the slot pool: sequence b starts from
 * slot state_slots[b] (device int32 [B], distinct ids) and leaves its final
 * state and position there, so a prompt can continue from a cached prefix
 * without copies.  Checkpoints go to the same pool (ckpt_slots as above, none
 * of them one of the state slots).  An id outside [0, n_slots) sets
 * KDA_DEV_ERR_SLOT_ID and the sequence is skipped.  dev_err must not be NULL.
 */
kda_status kda_prefill_chunked_slots(const kda_shape* shape, int32_t L, int32_t chunk, const int32_t* state_slots,
                                     const kda_slots* slots, const void* q, const void* k, const void* v,
                                     const float* alpha, const float* beta, float* o, int32_t ckpt_every,
                                     const int32_t* ckpt_slots, int32_t* dev_err, void* stream);

/*
 * The two prefills from raw projections (q, k, alpha_logit, beta_logit as in
 * kda_decode_step_prep, with the [B][L][H][d] token layout), the inputs
 * prepared inside the kernels (webinar summary: needless conversions removed).
 * The token-by-token form is bit-identical to L kda_decode_step_prep calls.
 * Fails with KDA_ERR_SHAPE for an unknown gate; otherwise as above.
 */
kda_status kda_prefill_chunked_prep(const kda_shape* shape, int32_t gate, int32_t L, int32_t chunk, float* state,
                                    int64_t* pos, const void* q, const void* k, const void* v,
                                    const float* alpha_logit, const float* beta_logit, float* o, int32_t ckpt_every,
                                    const int32_t* ckpt_slots, const kda_slots* slots, int32_t* dev_err,
                                    void* stream);
kda_status kda_prefill_recurrent_prep(const kda_shape* shape, int32_t gate, int32_t L, float* state, int64_t* pos,
                                      const void* q, const void* k, const void* v, const float* alpha_logit,
                                      const float* beta_logit, float* o, int32_t ckpt_every,
                                      const int32_t* ckpt_slots, const kda_slots* slots, int32_t* dev_err,
                                      void* stream);

/*
 * One serving step over a mixed batch, in one launch: each sequence b of
 * the batch (shape->B of them) decodes, speculates or processes a prompt
 * segment, as roles[b] says ("Hyper-optimizing Kimi K3 in vLLM", Part 2,
 * section 4: pure decode and mixed workloads are measured apart; "What's
 * Next": prefill and mixed batches).
 *   roles      device int32 [B], KDA_ROLE_*; exactly n_decode, n_spec and
 *              n_prefill of them DECODE, SPEC and PREFILL (host counts: the
 *              grid is sized from them).
 *   tok_start  device int32 [B + 1]: sequence b's tokens are rows
 *              tok_start[b] .. tok_start[b + 1] - 1 of the packed inputs
 *              q, k, v, alpha (in_dtype / f32 [n_tokens][H][d]) and beta
 *              (f32 [n_tokens][H]); its outputs go to the same rows of o
 *              (f32 [n_tokens][H][dv]).  DECODE takes exactly 1 token, SPEC
 *              0 .. log->T_max drafts, PREFILL any number (0: nothing).
 *   state/pos  the states and positions: dense [B] when slot_ids is NULL,
 *              otherwise a slot pool of n_slots entries that sequence b
 *              reaches through slot_ids[b] (device int32 [B], distinct ids).
 *   log        the speculative log, sized for this B (NULL allowed when
 *              n_spec == 0 and nothing is pending).  Rows are indexed by
 *              batch position, so a speculating sequence keeps its position
 *              from one step to the next.  SPEC sequences first commit
 *              accepted[b] rows of the pending verify (device int32 [B],
 *              read when log->pending_T > 0; the pending verify must have
 *              logged prepared inputs), then verify and log their drafts.
 *              Every other role must have accepted[b] == 0; after the step
 *              the log holds this step's drafts only (pending_T = T_max when
 *              n_spec > 0, else 0).
 * Prepared inputs only (unit q, k; gates and beta as for kda_decode_step).
 * The arithmetic of each role is that of kda_decode_step, kda_commit_verify
 * and kda_prefill_chunked with chunk 64, so states and outputs are bit-
 * identical to those calls (no checkpoints are taken).  Device-side checks
 * set bits in *dev_err (device int32, required) and skip the sequence:
 * KDA_DEV_ERR_MIXED for role counts that differ from roles[], an unknown
 * role or a token range outside [0, n_tokens] or wrong for its role;
 * KDA_DEV_ERR_SLOT_ID; KDA_DEV_ERR_ACCEPTED for a count out of range or one
 * given to a sequence that does not speculate.  Host-side failures:
 * KDA_ERR_SHAPE (counts negative or summing above B, n_tokens too large),
 * KDA_ERR_NULL, KDA_ERR_ALIGN, KDA_ERR_ORDER (a pending verify of raw
 * projections).
 */
kda_status kda_mixed_step(const kda_shape* shape, const int32_t* roles, const int32_t* tok_start, int32_t n_tokens,
                          int32_t n_decode, int32_t n_spec, int32_t n_prefill, float* state, int64_t* pos,
                          const int32_t* slot_ids, int32_t n_slots, const void* q, const void* k, const void* v,
                          const float* alpha, const float* beta, float* o, kda_log* log, const int32_t* accepted,
                          int32_t* dev_err, void* stream);

/* Human-readable name of a status code (static string). */
const char* kda_status_str(kda_status status);

/* Variant launched by the last successful call on this thread (KDA_VARIANT_*). */
int32_t kda_last_variant(void);

/* KDA_ABI_VERSION of the loaded library. */
int32_t kda_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
