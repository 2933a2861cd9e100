// Mixed batches in one launch for gfx950: in one serving step some sequences
// decode one token, some run a speculative round (commit of the accepted
// drafts of their previous round, then the verify of new drafts) and some
// process a segment of their prompt.  One kernel takes all three, so the
// prompt segments' long serial chains run beside the bandwidth-bound decode
// and verify work instead of after it.  ("Hyper-optimizing Kimi K3 in vLLM",
// Part 2: pure decode and mixed batches are different workloads; batch
// shapes decide the kernel choice.)
//
// Every workgroup has the chunked prefill's shape (dv / 16 waves) and takes
// one role from its index:
//   [0, P H)            one (prompt segment, head) each: the chunked MFMA
//                       prefill of kda_prefill_impl.h (chunk 64);
//   [P H, (P + S) H)    one (speculating sequence, head) each: the fused
//                       commit + verify of kda_verify_impl.h with 16 value
//                       columns per wave, its first group's preparation
//                       ahead of the replay;
//   the rest            decode items ((sequence, head) pairs), taken by
//                       groups of dv / 32 waves (32 value columns per wave,
//                       the decode kernel's lane mapping), several items per
//                       group with the next item's loads in flight while the
//                       current one computes.
// Each role's code is the standalone kernel's, with the same lane mapping
// and arithmetic per value column, so states and outputs are bit-identical
// to kda_decode_step, kda_commit_verify and kda_prefill_chunked (chunk 64)
// on the same inputs.  The kernel's register and LDS budget is the
// prefill's (one workgroup per CU), which the decode groups offset by
// keeping two items' state tiles in flight.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>

#include "kda_common.h"
#include "kda_internal.h"
#include "kda_prefill_impl.h"
#include "kda_verify_impl.h"

namespace kda {
namespace {

constexpr int kMixedChunk = 64;  // prompt segments' chunk

// The prompt and speculative roles take their standalone kernels' argument
// blocks, filled on the host (run-time values, as in those kernels: folding
// the unused checkpoint fields to constants measured costlier in registers).
// The decode role reads the token, state, log and count fields of `vf`.
template <typename TIn>
struct MixedArgs {
  PrefillArgs<TIn> pf;  // no checkpoints; state_slots unused (the slot is resolved here)
  VerifyArgs<TIn> vf;   // fused commit + verify; draft_len and slot_ids unused
  const int32_t* roles;      // [B] KDA_ROLE_*
  const int32_t* tok_start;  // [B + 1] first packed token row of each sequence
  const int32_t* slot_ids;   // [B] or null (state b is entry b)
  int32_t B, n_tokens;
  int32_t n_prefill, n_spec, n_decode;
  int32_t items_per_group;  // decode items per group of waves
};

// Batch position of the sequence of rank `rank` (from 0) among those whose
// role is `role`, or -1: one wave scans the roles 64 at a time.  The result
// is wave-uniform.
__device__ __forceinline__ int kth_role(const int32_t* roles, int B, int role, int rank) {
  const int lane = threadIdx.x & (kWave - 1);
  for (int base = 0; base < B; base += kWave) {
    const int i = base + lane;
    const bool hit = i < B && roles[i] == role;
    const uint64_t m = __ballot(hit);
    const int c = __popcll(m);
    if (rank < c) {
      // Set bits of m below this lane: the lane's rank among the hits.
      const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      return __builtin_amdgcn_readfirstlane(base + (int)__builtin_ctzll(__ballot(hit && below == rank)));
    }
    rank -= c;
  }
  return -1;
}

// One sequence of the batch as a role's workgroup sees it.  b < 0: no such
// sequence; ok false: skip it, for the reason in err (a KDA_DEV_ERR_* bit,
// which one designated lane per sequence reports).
struct Seq {
  int b, sb, s0, n, err;
  bool ok;
};

// Finds the sequence of rank `rank` with role `role` and checks its token
// range, state slot and accepted count.
template <typename TIn>
__device__ __forceinline__ Seq find_seq(const MixedArgs<TIn>& a, int role, int rank) {
  Seq s{-1, 0, 0, 0, KDA_DEV_ERR_MIXED, false};
  s.b = kth_role(a.roles, a.B, role, rank);
  if (s.b < 0) return s;
  // Wave-uniform values, kept in scalar registers.
  const int s0 = __builtin_amdgcn_readfirstlane(a.tok_start[s.b]);
  const int s1 = __builtin_amdgcn_readfirstlane(a.tok_start[s.b + 1]);
  if (!(s0 >= 0 && s1 >= s0 && s1 <= a.n_tokens)) return s;
  s.s0 = s0;
  s.n = s1 - s0;
  if (role == KDA_ROLE_DECODE && s.n != 1) return s;
  if (role == KDA_ROLE_SPEC && s.n > a.vf.Tmax) return s;
  s.sb = a.slot_ids ? __builtin_amdgcn_readfirstlane(a.slot_ids[s.b]) : s.b;
  if (s.sb < 0 || s.sb >= a.vf.n_slots) {
    s.err = KDA_DEV_ERR_SLOT_ID;
    return s;
  }
  // Only a speculating sequence commits; a pending count above 0 for any
  // other role would be lost.
  if (role != KDA_ROLE_SPEC && a.vf.T_pend > 0 && __builtin_amdgcn_readfirstlane(a.vf.accepted[s.b]) != 0) {
    s.err = KDA_DEV_ERR_ACCEPTED;
    return s;
  }
  s.err = 0;
  s.ok = true;
  return s;
}

// The batch-wide checks, by one wave: the role counts match the launch, every
// role is known, and idle sequences neither hold an accepted count (nothing
// commits for them) nor keep log rows (their records are cleared, so a later
// commit finds nothing for them).
template <typename TIn>
__device__ void check_batch(const MixedArgs<TIn>& a) {
  const int lane = threadIdx.x & (kWave - 1);
  int c_dec = 0, c_spec = 0, c_pf = 0;
  bool bad_role = false, bad_acc = false;
  for (int base = 0; base < a.B; base += kWave) {
    const int i = base + lane;
    const int r = i < a.B ? a.roles[i] : KDA_ROLE_IDLE;
    c_dec += __popcll(__ballot(r == KDA_ROLE_DECODE));
    c_spec += __popcll(__ballot(r == KDA_ROLE_SPEC));
    c_pf += __popcll(__ballot(r == KDA_ROLE_PREFILL));
    bad_role |= r < KDA_ROLE_IDLE || r > KDA_ROLE_PREFILL;
    const bool idle = i < a.B && r != KDA_ROLE_DECODE && r != KDA_ROLE_SPEC && r != KDA_ROLE_PREFILL;
    if (idle && a.vf.T_pend > 0) bad_acc |= a.vf.accepted[i] != 0;
    if (idle && a.vf.log_len)
      for (int h = 0; h < a.vf.H; ++h) a.vf.log_len[(size_t)i * a.vf.H + h] = log_record(0, kLogPrepared);
  }
  const bool mismatch = c_dec != a.n_decode || c_spec != a.n_spec || c_pf != a.n_prefill;
  const bool any_bad_role = __ballot(bad_role) != 0, any_bad_acc = __ballot(bad_acc) != 0;
  if (lane == 0) {
    if (mismatch || any_bad_role) atomicOr(a.vf.dev_err, KDA_DEV_ERR_MIXED);
    if (any_bad_acc) atomicOr(a.vf.dev_err, KDA_DEV_ERR_ACCEPTED);
  }
}

// N consecutive input values through a buffer resource (uniform base in
// SGPRs, the lane's byte offset vo in one VGPR): a decode group keeps no
// 64-bit lane addresses live across its items.
template <typename TIn, int N>
__device__ __forceinline__ void load_raw_buf(rsrc_t r, int vo, Raw<TIn, N>& x) {
  constexpr int V = sizeof(x.w) / 16;
#pragma unroll
  for (int i = 0; i < V; ++i)
    x.w[i] = __builtin_bit_cast(typename Raw<TIn, N>::vec, __builtin_amdgcn_raw_buffer_load_b128(r, vo, 16 * i, 0));
}
__device__ __forceinline__ void load_v_buf(rsrc_t r, int vo, RawV<bf16_t, 4>& x) {
  x.w = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, vo, 0, 0));
}
__device__ __forceinline__ void load_v_buf(rsrc_t r, int vo, RawV<float, 4>& x) {
  x.w = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, vo, 0, 0));
}

// One decode item: a (sequence, head) pair's state tile and token inputs as
// one lane of its group holds them (the decode kernel's lane mapping).
template <int DK, int DV, typename TIn>
struct DecodeItem {
  static constexpr int R = DK / kRowGroups;
  Seq s;
  int h;
  float S[R][4];
  TokenIn<TIn, R, true, 4> in;
};

// Decode items [first, first + count) of the (decoding sequence rank, head)
// order, by this lane's group of dv / 32 waves.  Two items are in flight:
// item i + 1's state tile is requested right after item i's token inputs,
// so while item i waits for its inputs and computes, the next tile streams
// in (loads return in order, so nothing issued later is waited for).
template <int DK, int DV, typename TIn>
__device__ __forceinline__ void decode_items(const MixedArgs<TIn>& ma, int first, int count) {
  constexpr int R = DK / kRowGroups;
  constexpr int WPI = DV / kSliceCols;  // waves per item
  const VerifyArgs<TIn>& a = ma.vf;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wi = wave % WPI;
  const int rg = lane >> 3, cg = lane & 7;
  const int row0 = rg * R, col0 = wi * kSliceCols + cg * 4;
  const int vo = (row0 * DV + col0) * 4;
  const int end = min(first + count, ma.n_decode * a.H);
  int rank_c = -1;  // the last rank looked up, and its sequence
  Seq seq_c{-1, 0, 0, 0, 0, false};

  auto fetch_state = [&](DecodeItem<DK, DV, TIn>& it, int idx) {
    it.s = Seq{-1, 0, 0, 0, 0, false};
    if (idx >= end) return;
    const int rank = idx / a.H;
    it.h = idx - rank * a.H;
    if (rank != rank_c) {
      seq_c = find_seq(ma, KDA_ROLE_DECODE, rank);
      rank_c = rank;
    }
    it.s = seq_c;
    if (!it.s.ok) return;
    load_tile<R, DV>(state_rsrc<DK, DV>(a.state + ((size_t)it.s.sb * a.H + it.h) * DK * DV), vo, it.S);
  };
  const int vo_k = row0 * (int)sizeof(TIn), vo_a = row0 * 4, vo_v = col0 * (int)sizeof(TIn);
  auto fetch_inputs = [&](DecodeItem<DK, DV, TIn>& it) {
    if (!it.s.ok) return;
    const size_t row = (size_t)it.s.s0 * a.H + it.h;
    load_raw_buf(make_rsrc(a.k + row * DK, DK * sizeof(TIn)), vo_k, it.in.k);
    load_raw_buf(make_rsrc(a.q + row * DK, DK * sizeof(TIn)), vo_k, it.in.q);
    load_raw_buf(make_rsrc(a.alpha + row * DK, DK * 4), vo_a, it.in.a);
    load_v_buf(make_rsrc(a.v + row * DV, DV * sizeof(TIn)), vo_v, it.in.v);
    it.in.beta = a.beta[row];
  };
  auto process = [&](DecodeItem<DK, DV, TIn>& it) {
    if (it.s.err && it.h == 0 && wi == 0 && lane == 0) atomicOr(a.dev_err, it.s.err);
    if (it.s.b < 0) return;
    if (a.log_len && wi == 0 && lane == 0) a.log_len[(size_t)it.s.b * a.H + it.h] = log_record(0, kLogPrepared);
    if (!it.s.ok) return;
    float o[4];
    it.in.update(it.S, a.scale, o);
    // The wide stores take each row's offset in a VGPR (see store_cols);
    // an opaque copy of vo keeps those R sums here instead of hoisted out
    // of the item loop, where they would hold R registers throughout.
    int vs = vo;
    asm volatile("" : "+v"(vs));
    store_tile<R, DV>(state_rsrc<DK, DV>(a.state + ((size_t)it.s.sb * a.H + it.h) * DK * DV), vs, it.S);
    if (rg == 0) {
      const size_t row = (size_t)it.s.s0 * a.H + it.h;
      *reinterpret_cast<float4*>(a.o + row * DV + col0) = make_float4(o[0], o[1], o[2], o[3]);
    }
    if (it.h == 0 && wi == 0 && lane == 0) a.pos[it.s.sb] += 1;
  };

  // fp32 inputs at dk = 128 take twice the registers of bf16 ones: two items
  // in flight would spill, so that case runs one item at a time.
  constexpr bool kTwo = sizeof(TIn) == 2 || DK < 128;
  DecodeItem<DK, DV, TIn> x, y;
  if constexpr (kTwo) {
    fetch_state(x, first);
    for (int idx = first; idx < end; idx += 2) {
      fetch_inputs(x);
      fetch_state(y, idx + 1);
      process(x);
      fetch_inputs(y);
      fetch_state(x, idx + 2);
      process(y);
    }
  } else {
    for (int idx = first; idx < end; ++idx) {
      fetch_state(x, idx);
      fetch_inputs(x);
      process(x);
    }
  }
}

template <int DK, int DV, typename TIn>
__global__ void __launch_bounds__(4 * DV) mixed_kernel(MixedArgs<TIn> a) {
  static_assert(prefill_ct(DV) == 1, "the mixed kernel uses the prefill's one-tile-per-wave shape");
  typedef Smem<DK, kMixedChunk, DV / 16> PfSmem;
  constexpr int kLds = PfSmem::total > (int)sizeof(VerifyLds<DK>) ? PfSmem::total : (int)sizeof(VerifyLds<DK>);
  __shared__ __align__(16) char smem[kLds];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int blk = blockIdx.x;
  if (blk == (int)gridDim.x - 1 && wave == 0) check_batch(a);

  const int H = a.vf.H;
  const int n_pf_wg = a.n_prefill * H, n_spec_wg = a.n_spec * H;
  if (blk < n_pf_wg + n_spec_wg) {
    const bool pf = blk < n_pf_wg;
    const int j = pf ? blk : blk - n_pf_wg;
    const int rank = j / H, h = j - rank * H;
    const Seq s = find_seq(a, pf ? KDA_ROLE_PREFILL : KDA_ROLE_SPEC, rank);
    if (s.err && h == 0 && threadIdx.x == 0) atomicOr(a.vf.dev_err, s.err);
    if (s.b < 0) return;
    int32_t* const rec = a.vf.log_len ? a.vf.log_len + (size_t)s.b * H + h : nullptr;
    if (!s.ok || pf) {
      if (rec && threadIdx.x == 0) *rec = log_record(0, kLogPrepared);
      if (s.ok && s.n > 0) prefill_seq<DK, DV, kMixedChunk, TIn, false>(a.pf, smem, s.b, h, s.sb, (size_t)s.s0, s.n);
      return;
    }
    verify_seq<DK, DV, TIn, true, true, false, true, true>(a.vf, *reinterpret_cast<VerifyLds<DK>*>(smem), s.b, h, s.sb,
                                                     (size_t)s.s0 * H + h, (size_t)s.b * a.vf.Tmax * H + h,
                                                     max(s.n, 1), s.n);
    return;
  }
  // Decode: group grp of this workgroup takes items_per_group consecutive items.
  constexpr int GROUPS = (DV / 16) / (DV / kSliceCols);
  const int grp = wave / (DV / kSliceCols);
  const int g = (blk - n_pf_wg - n_spec_wg) * GROUPS + grp;
  decode_items<DK, DV, TIn>(a, g * a.items_per_group, a.items_per_group);
}

template <int DK, int DV, typename TIn>
void launch_cfg(const MixedArgs<TIn>& a, int n_wg, hipStream_t st) {
  mixed_kernel<DK, DV, TIn><<<dim3(n_wg), dim3(4 * DV), 0, st>>>(a);
}

template <typename TIn>
void launch_shape(const kda_shape& s, const MixedArgs<TIn>& a, int n_wg, hipStream_t st) {
  if (s.dk == 128 && s.dv == 128) launch_cfg<128, 128, TIn>(a, n_wg, st);
  else if (s.dk == 128) launch_cfg<128, 64, TIn>(a, n_wg, st);
  else if (s.dv == 128) launch_cfg<64, 128, TIn>(a, n_wg, st);
  else launch_cfg<64, 64, TIn>(a, n_wg, st);
}

}  // namespace

hipError_t launch_mixed(const kda_shape& s, const MixedBatch& m, float* state, int64_t* pos, const int32_t* slot_ids,
                        int32_t n_slots, TokenInputs in, float* o, const LogPtrs* log, int32_t T_pend,
                        const int32_t* accepted, int32_t* dev_err, hipStream_t st) {
  // Decode items: enough groups to cover the chip once (two groups per
  // workgroup, one workgroup per CU), at least one item per group.
  constexpr int kTargetGroups = 2 * 256;
  const int64_t items = (int64_t)m.n_decode * s.H;
  const int ipg = (int)(items == 0 ? 1 : (items + kTargetGroups - 1) / kTargetGroups);
  const int64_t dec_wg = (items + 2 * ipg - 1) / (2 * ipg);
  // At least one workgroup: the last one also checks the whole batch.
  const int64_t n_wg = std::max<int64_t>(1, (int64_t)(m.n_prefill + m.n_spec) * s.H + dec_wg);
  if (n_wg > INT32_MAX) return hipErrorInvalidValue;
  auto go = [&](auto tag) {
    typedef decltype(tag) TIn;
    const PrefillArgs<TIn> pf{state,   pos,     (const TIn*)in.q, (const TIn*)in.k, (const TIn*)in.v, in.alpha,
                              in.beta, o,       nullptr,          nullptr,          nullptr,          dev_err,
                              s.H,     0,       0,                n_slots,          s.scale,          -1.f,
                              nullptr};
    const VerifyArgs<TIn> vf{state,
                             (const TIn*)in.q,
                             (const TIn*)in.k,
                             (const TIn*)in.v,
                             in.alpha,
                             in.beta,
                             o,
                             log ? (TIn*)log->k : nullptr,
                             log ? (TIn*)log->v : nullptr,
                             log ? log->alpha : nullptr,
                             log ? log->beta : nullptr,
                             s.H,
                             0,
                             log ? log->T_max : 0,
                             s.scale,
                             pos,
                             accepted,
                             dev_err,
                             T_pend,
                             nullptr,
                             log ? log->len : nullptr,
                             0,
                             -1.f,
                             -1.f,
                             nullptr,
                             n_slots};
    const MixedArgs<TIn> a{pf, vf, m.roles, m.tok_start, slot_ids, s.B, m.n_tokens, m.n_prefill, m.n_spec,
                           m.n_decode, ipg};
    launch_shape<TIn>(s, a, (int)n_wg, st);
  };
  if (s.in_dtype == KDA_BF16)
    go(bf16_t{});
  else
    go(float{});
  return hipGetLastError();
}

}  // namespace kda
