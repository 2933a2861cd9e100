// State-resident KDA kernels for gfx950: decode step, commit (replay of the
// accepted prefix of a verify) and the token-by-token prefill.
//
// Every kernel runs one 64-lane wave per 32-column slice of one
// (sequence, head) state and keeps that slice in registers for as long as it
// needs it (one token for decode, the accepted count for commit, the whole
// prompt for the recurrent prefill).  All of them call kda::token_update with
// the same lane mapping, which is what makes commit bit-identical to repeated
// decode steps.
//
// The decode step streams the fp32 state (read + write, 98.6% of its bytes at
// dk = dv = 128 with bf16 inputs), so it is bound by HBM bandwidth; the loads
// of one wave-wide instruction cover eight full 128-byte lines.
// ("Hyper-optimizing Kimi K3 in vLLM", Part 1, section 4: small-batch decode
// is memory-bound.)

#include <hip/hip_runtime.h>

#include <type_traits>

#include "kda_common.h"
#include "kda_internal.h"

namespace kda {
namespace {

template <typename TIn>
struct StepArgs {
  float* state;
  int64_t* pos;
  const TIn* q;
  const TIn* k;
  const TIn* v;
  const float* alpha;  // decay logits when the inputs are raw projections
  const float* beta;   // beta logits when the inputs are raw projections
  float* o;
  int32_t H;
  float scale;
  float gate_sign;     // raw projections: decay = sigmoid(gate_sign * logit)
  // States in a slot pool: sequence b uses state[slot_ids[b]] and pos[slot_ids[b]].
  const int32_t* slot_ids;
  int32_t n_slots;
  int32_t* dev_err;
};

template <typename TIn>
struct CommitArgs {
  float* state;
  int64_t* pos;
  const TIn* log_k;
  const TIn* log_v;
  const float* log_alpha;
  const float* log_beta;
  const int32_t* accepted;
  int32_t* dev_err;
  const int32_t* log_len;  // per (b, h): rows the pending verify wrote and their form (log_record)
  int32_t H;
  int32_t T;     // tokens of the pending verify
  int32_t Tmax;  // token rows per sequence in the log
  float gate_sign;  // raw logs: decay = sigmoid(gate_sign * logit)
  const int32_t* slot_ids;  // states and positions in a slot pool (null: dense [B])
  int32_t n_slots;
};

template <typename TIn>
struct PrefillArgs {
  float* state;
  int64_t* pos;
  const TIn* q;
  const TIn* k;
  const TIn* v;
  const float* alpha;
  const float* beta;
  float* o;
  const int32_t* ckpt_slots;
  float* slot_states;
  int64_t* slot_pos;
  int32_t* dev_err;
  int32_t H;
  int32_t L;
  int32_t ckpt_every;
  int32_t n_slots;
  float scale;
  float gate_sign;  // raw projections: decay = sigmoid(gate_sign * logit)
  const int32_t* state_slots;  // non-null: states and positions in the slot pool
};

// Waves per workgroup (WPG): the column slices of one (sequence, head) are
// either spread over independent one-wave workgroups (1) or kept together in
// one workgroup on one CU (all slices).  The waves never synchronise either
// way.  Decode and commit pick WPG from the batch: one-wave workgroups start
// faster when there are few of them; whole-state workgroups keep a state's
// reads and writes on one CU.  With non-temporal state traffic the
// whole-state shape measured faster from B = 8 on at H = 32 (1,024 slices:
// 6.86 against 7.19 us per launch at B = 8, 49.6 against 52.2 us at B = 64).
#ifndef KDA_WIDE_WAVES
#define KDA_WIDE_WAVES 1024
#endif
constexpr size_t kWideWaves = KDA_WIDE_WAVES;  // total slices from which whole-state workgroups are used
// Below this many 32-column slices (B <= 3 at H = 32, dv = 128) decode and
// commit run one-wave workgroups of 16 value columns: twice the waves per state, half
// the serial work per wave, the same arithmetic per column (measured 3.33 ->
// 2.95 us per launch at B = 1, 3.71 -> 3.53 at B = 2; at B = 4 it was slower).
#ifndef KDA_NARROW_WAVES
#define KDA_NARROW_WAVES 512
#endif
constexpr size_t kNarrowWaves = KDA_NARROW_WAVES;
// The recurrent prefill loads token t+1's inputs while token t computes (1),
// or loads each token's inputs when it starts (0: fewer live registers).
#ifndef KDA_PREFETCH_NEXT
#define KDA_PREFETCH_NEXT 0
#endif

// Minimum waves per SIMD the register allocator must allow (0: no request).
#ifndef KDA_MIN_WAVES
#define KDA_MIN_WAVES 0
#endif
#if KDA_MIN_WAVES > 0
#define KDA_OCCUPANCY __attribute__((amdgpu_waves_per_eu(KDA_MIN_WAVES)))
#else
#define KDA_OCCUPANCY
#endif

constexpr int kXcds = 8;  // accelerator complex dies on MI355X, each with its own L2

// Value columns per lane NC: 4 (waves of 32 columns) or, for the smallest
// batches' decode, 2 (waves of 16 columns, twice the waves per state).
template <int DV, int WPG, int NC = 4>
constexpr int waves_per_group() {
  return WPG < DV / (kRowGroups * NC) ? WPG : DV / (kRowGroups * NC);
}

// Where a wave sits: its (sequence, head) index and its lane's rows/columns.
template <int DK, int DV, int WPG_ = 1, int NC = 4>
struct Place {
  static constexpr int R = DK / kRowGroups;
  static constexpr int SLICES = DV / (kRowGroups * NC);
  static constexpr int WPG = waves_per_group<DV, WPG_, NC>();
  int bh, b, h, slice, rg, cg, row0, col0, lane;
  __device__ __forceinline__ Place(int H) {
    lane = threadIdx.x & (kWave - 1);
    constexpr int G = SLICES / WPG;  // workgroups per (sequence, head)
    const int x = blockIdx.x;
    if (G > 1 && (gridDim.x % (kXcds * G)) == 0) {
      // Workgroups are handed to the 8 XCDs round-robin by id.  Give the G
      // workgroups of one (sequence, head) ids that are equal mod 8 so they
      // run on one XCD and share its L2 for the per-token inputs.
      const int xcd = x % kXcds, j = x / kXcds;
      slice = (j % G) * WPG + (threadIdx.x >> 6);
      bh = (j / G) * kXcds + xcd;
    } else {
      slice = (x % G) * WPG + (threadIdx.x >> 6);
      bh = x / G;
    }
    b = bh / H;
    h = bh - b * H;
    rg = lane >> 3;
    cg = lane & 7;
    row0 = rg * R;
    col0 = slice * kRowGroups * NC + cg * NC;
  }
  // Offset of this lane's first state element inside a [dk][dv] state.
  __device__ __forceinline__ size_t tile_off() const { return (size_t)row0 * DV + col0; }
};

// PREP: the inputs are raw projections and logits, prepared in the step
// (token_update_prep).  SLOTS: the states and positions live in a slot pool,
// addressed through slot_ids (an id out of range is flagged and skipped).
template <int DK, int DV, typename TIn, int WPG, bool PREP, bool SLOTS, int NC = 4>
__global__ void KDA_OCCUPANCY __launch_bounds__((kWave * waves_per_group<DV, WPG, NC>())) decode_kernel(StepArgs<TIn> a) {
  typedef Place<DK, DV, WPG, NC> P;
  constexpr int R = P::R;
  const P p(a.H);
  int sb = p.b;  // index of the state (and position) this sequence uses
  if constexpr (SLOTS) {
    sb = a.slot_ids[p.b];
    if (sb < 0 || sb >= a.n_slots) {
      if (p.h == 0 && p.slice == 0 && p.lane == 0) atomicOr(a.dev_err, KDA_DEV_ERR_SLOT_ID);
      return;
    }
  }
  const rsrc_t rs = state_rsrc<DK, DV>(a.state + ((size_t)sb * a.H + p.h) * DK * DV);
  const int vo = (int)p.tile_off() * 4;
  float S[R][NC];
  load_tile<R, DV>(rs, vo, S);
  TokenIn<TIn, R, true, NC> in;
  in.load(a.k + (size_t)p.bh * DK + p.row0, a.q + (size_t)p.bh * DK + p.row0,
          a.alpha + (size_t)p.bh * DK + p.row0, a.v + (size_t)p.bh * DV + p.col0, a.beta + p.bh);
  float o[NC];
  if constexpr (PREP)
    in.update_prep(S, a.gate_sign, a.scale, o);
  else
    in.update(S, a.scale, o);
  store_tile<R, DV>(rs, vo, S);
  if (p.rg == 0) {
    if constexpr (NC == 4)
      *reinterpret_cast<float4*>(a.o + (size_t)p.bh * DV + p.col0) = make_float4(o[0], o[1], o[2], o[3]);
    else
      *reinterpret_cast<float2*>(a.o + (size_t)p.bh * DV + p.col0) = make_float2(o[0], o[1]);
  }
  if (p.h == 0 && p.slice == 0 && p.lane == 0) a.pos[sb] += 1;
}

// RAW: the log holds raw projections and logits (decay sigmoid(gate_sign * x)).
template <int DK, int DV, typename TIn, int WPG, bool RAW, int NC = 4>
__global__ void KDA_OCCUPANCY __launch_bounds__((kWave * waves_per_group<DV, WPG, NC>())) commit_kernel(CommitArgs<TIn> a) {
  typedef Place<DK, DV, WPG, NC> P;
  constexpr int R = P::R;
  const P p(a.H);
  int sb = p.b;  // index of the state and position this sequence uses
  if (a.slot_ids) {
    sb = a.slot_ids[p.b];
    if (sb < 0 || sb >= a.n_slots) {
      if (p.h == 0 && p.slice == 0 && p.lane == 0) atomicOr(a.dev_err, KDA_DEV_ERR_SLOT_ID);
      return;
    }
  }
  const int n = a.accepted[p.b];
  if (n < 0 || n > min(a.T, log_rows(a.log_len[p.bh]))) {
    if (p.h == 0 && p.slice == 0 && p.lane == 0) atomicOr(a.dev_err, KDA_DEV_ERR_ACCEPTED);
    return;
  }
  if (n == 0) return;
  const rsrc_t rs = state_rsrc<DK, DV>(a.state + ((size_t)sb * a.H + p.h) * DK * DV);
  const int vo = (int)p.tile_off() * 4;
  float S[R][NC];
  load_tile<R, DV>(rs, vo, S);
  replay_log<DK, DV, TIn, R, RAW>(S, a.log_k, a.log_v, a.log_alpha, a.log_beta, (size_t)p.b * a.Tmax * a.H + p.h,
                                  a.H, n, p.row0, p.col0, a.gate_sign);
  store_tile<R, DV>(rs, vo, S);
  if (p.h == 0 && p.slice == 0 && p.lane == 0) a.pos[sb] += n;
}

// PREP: raw projections and logits, prepared in every step (the decode step
// from raw projections, token by token).
template <int DK, int DV, typename TIn, bool PREP>
__global__ void KDA_OCCUPANCY __launch_bounds__(kWave) prefill_recurrent_kernel(PrefillArgs<TIn> a) {
  typedef Place<DK, DV, 1> P;
  constexpr int R = P::R;
  const P p(a.H);
  const bool owner = p.h == 0 && p.slice == 0 && p.lane == 0;  // the one writer of positions
  int sb = p.b;  // index of the state and position this sequence uses
  if (a.state_slots) {
    sb = a.state_slots[p.b];
    if (sb < 0 || sb >= a.n_slots) {
      if (owner) atomicOr(a.dev_err, KDA_DEV_ERR_SLOT_ID);
      return;
    }
  }
  const int64_t pos0 = owner ? a.pos[sb] : 0;
  const int n_ckpt = a.ckpt_every > 0 ? a.L / a.ckpt_every : 0;
  const rsrc_t rs = state_rsrc<DK, DV>(a.state + ((size_t)sb * a.H + p.h) * DK * DV);
  const int vo = (int)p.tile_off() * 4;
  float S[R][4];
  load_tile<R, DV>(rs, vo, S);
  TokenIn<TIn, R, true> cur, nxt;
  size_t tok = (size_t)p.b * a.L * a.H + p.h;
  if (a.L > 0)
    cur.load(a.k + tok * DK + p.row0, a.q + tok * DK + p.row0, a.alpha + tok * DK + p.row0,
             a.v + tok * DV + p.col0, a.beta + tok);
  for (int t = 0; t < a.L; ++t) {
    const size_t tn = tok + a.H;
    if (t + 1 < a.L)
      nxt.load(a.k + tn * DK + p.row0, a.q + tn * DK + p.row0, a.alpha + tn * DK + p.row0,
               a.v + tn * DV + p.col0, a.beta + tn);
    float o[4];
    if constexpr (PREP)
      cur.update_prep(S, a.gate_sign, a.scale, o);
    else
      cur.update(S, a.scale, o);
    if (p.rg == 0) *reinterpret_cast<float4*>(a.o + tok * DV + p.col0) = make_float4(o[0], o[1], o[2], o[3]);
    if (n_ckpt > 0 && (t + 1) % a.ckpt_every == 0) {
      const int m = (t + 1) / a.ckpt_every - 1;
      const int slot = a.ckpt_slots[(size_t)p.b * n_ckpt + m];
      if (slot >= 0 && slot < a.n_slots) {
        store_tile<R, DV>(state_rsrc<DK, DV>(a.slot_states + ((size_t)slot * a.H + p.h) * DK * DV), vo, S);
        if (owner) a.slot_pos[slot] = pos0 + t + 1;
      } else if (p.slice == 0 && p.lane == 0) {
        atomicOr(a.dev_err, KDA_DEV_ERR_CKPT_SLOT);
      }
    }
    cur = nxt;
    tok = tn;
  }
  store_tile<R, DV>(rs, vo, S);
  if (owner) a.pos[sb] = pos0 + a.L;
}

template <int DK, int DV, int WPG, int NC = 4>
dim3 grid_of(const kda_shape& s) {
  return dim3((unsigned)((size_t)s.B * s.H * (DV / (kRowGroups * NC)) / waves_per_group<DV, WPG, NC>()));
}

// Total one-wave slices of a launch (one per 32 value columns of every state).
template <int DV>
size_t slice_waves(const kda_shape& s) {
  return (size_t)s.B * s.H * (DV / kSliceCols);
}

template <int DK_, int DV_, typename TIn_>
struct Cfg {
  static constexpr int DK = DK_, DV = DV_;
  typedef TIn_ TIn;
};

// Calls f(Cfg<dk, dv, input type>{}) for the shape's instantiation.
template <typename TIn, typename F>
void dispatch_d(const kda_shape& s, F&& f) {
  if (s.dk == 128 && s.dv == 128) f(Cfg<128, 128, TIn>{});
  else if (s.dk == 128 && s.dv == 64) f(Cfg<128, 64, TIn>{});
  else if (s.dk == 64 && s.dv == 128) f(Cfg<64, 128, TIn>{});
  else f(Cfg<64, 64, TIn>{});
}
template <typename F>
void dispatch(const kda_shape& s, F&& f) {
  if (s.in_dtype == KDA_BF16) dispatch_d<bf16_t>(s, f);
  else dispatch_d<float>(s, f);
}

}  // namespace

namespace {

template <bool PREP, bool SLOTS>
hipError_t launch_decode_any(const kda_shape& s, float* state, int64_t* pos, TokenInputs in, float* o,
                             float gate_sign, const int32_t* slot_ids, int32_t n_slots, int32_t* dev_err,
                             hipStream_t st) {
  dispatch(s, [&](auto c) {
    typedef decltype(c) C;
    typedef typename C::TIn TIn;
    constexpr int DK = C::DK, DV = C::DV;
    StepArgs<TIn> a{state, pos,   (const TIn*)in.q, (const TIn*)in.k, (const TIn*)in.v, in.alpha, in.beta, o,
                    s.H,   s.scale, gate_sign,       slot_ids,         n_slots,          dev_err};
    if (slice_waves<DV>(s) >= kWideWaves)
      decode_kernel<DK, DV, TIn, 4, PREP, SLOTS>
          <<<grid_of<DK, DV, 4>(s), kWave * waves_per_group<DV, 4>(), 0, st>>>(a);
    else if (slice_waves<DV>(s) >= kNarrowWaves)
      decode_kernel<DK, DV, TIn, 1, PREP, SLOTS><<<grid_of<DK, DV, 1>(s), kWave, 0, st>>>(a);
    else
      decode_kernel<DK, DV, TIn, 1, PREP, SLOTS, 2><<<grid_of<DK, DV, 1, 2>(s), kWave, 0, st>>>(a);
  });
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const kda_shape& s, float* state, int64_t* pos, TokenInputs in, float* o,
                         hipStream_t st) {
  return launch_decode_any<false, false>(s, state, pos, in, o, 0.f, nullptr, 0, nullptr, st);
}

hipError_t launch_decode_prep(const kda_shape& s, float* state, int64_t* pos, TokenInputs raw, float* o,
                              float gate_sign, hipStream_t st) {
  return launch_decode_any<true, false>(s, state, pos, raw, o, gate_sign, nullptr, 0, nullptr, st);
}

hipError_t launch_decode_slots(const kda_shape& s, const int32_t* slot_ids, float* pool_states, int64_t* pool_pos,
                               int32_t n_slots, TokenInputs in, float* o, int32_t* dev_err, hipStream_t st) {
  return launch_decode_any<false, true>(s, pool_states, pool_pos, in, o, 0.f, slot_ids, n_slots, dev_err, st);
}

hipError_t launch_commit(const kda_shape& s, int32_t T, float* state, int64_t* pos, LogPtrs log,
                         const int32_t* accepted, int32_t* dev_err, int32_t form, hipStream_t st,
                         const int32_t* slot_ids, int32_t n_slots) {
  dispatch(s, [&](auto c) {
    typedef decltype(c) C;
    typedef typename C::TIn TIn;
    constexpr int DK = C::DK, DV = C::DV;
    const float gsign = form == kLogPrepared ? 0.f : (form - kLogRaw == KDA_GATE_SIGMOID ? 1.f : -1.f);
    CommitArgs<TIn> a{state, pos,   (const TIn*)log.k, (const TIn*)log.v, log.alpha, log.beta, accepted, dev_err,
                      log.len, s.H, T,   log.T_max,        gsign,            slot_ids,  n_slots};
    auto go = [&](auto raw) {
      constexpr bool RAW = decltype(raw)::value;
      if (slice_waves<DV>(s) >= kWideWaves)
        commit_kernel<DK, DV, TIn, 4, RAW><<<grid_of<DK, DV, 4>(s), kWave * waves_per_group<DV, 4>(), 0, st>>>(a);
      else if (slice_waves<DV>(s) >= kNarrowWaves)
        commit_kernel<DK, DV, TIn, 1, RAW><<<grid_of<DK, DV, 1>(s), kWave, 0, st>>>(a);
      else
        commit_kernel<DK, DV, TIn, 1, RAW, 2><<<grid_of<DK, DV, 1, 2>(s), kWave, 0, st>>>(a);
    };
    if (form == kLogPrepared)
      go(std::false_type{});
    else
      go(std::true_type{});
  });
  return hipGetLastError();
}

hipError_t launch_prefill_recurrent(const kda_shape& s, int32_t L, float* state, int64_t* pos, TokenInputs in,
                                    float* o, int32_t ckpt_every, const int32_t* ckpt_slots, float* slot_states,
                                    int64_t* slot_pos, int32_t n_slots, int32_t* dev_err, int32_t gate,
                                    hipStream_t st, const int32_t* state_slots) {
  dispatch(s, [&](auto c) {
    typedef decltype(c) C;
    typedef typename C::TIn TIn;
    constexpr int DK = C::DK, DV = C::DV;
    PrefillArgs<TIn> a{state,    pos,     (const TIn*)in.q, (const TIn*)in.k, (const TIn*)in.v, in.alpha, in.beta,
                       o,        ckpt_slots, slot_states,  slot_pos,         dev_err,          s.H,      L,
                       ckpt_every, n_slots, s.scale,       gate == KDA_GATE_SIGMOID ? 1.f : -1.f, state_slots};
    if (gate < 0)
      prefill_recurrent_kernel<DK, DV, TIn, false><<<grid_of<DK, DV, 1>(s), kWave, 0, st>>>(a);
    else
      prefill_recurrent_kernel<DK, DV, TIn, true><<<grid_of<DK, DV, 1>(s), kWave, 0, st>>>(a);
  });
  return hipGetLastError();
}

}  // namespace kda
