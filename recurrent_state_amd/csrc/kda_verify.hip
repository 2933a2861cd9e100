// Speculative verify and the fused commit + verify round: the kernel over a
// batch (one workgroup per (sequence, head)) and its launchers.  The chunk
// form of the verify and the workgroup's code are in kda_verify_impl.h,
// which the mixed-batch kernel shares.

#include <hip/hip_runtime.h>

#include <type_traits>

#include "kda_common.h"
#include "kda_internal.h"
#include "kda_verify_impl.h"

namespace kda {
namespace {

// EARLY (fused round only): the first verify group's preparation runs ahead
// of the replay (verify_seq).
template <int DK, int DV, typename TIn, bool MULTI, bool COMMIT, bool PREP, bool PF, bool EARLY>
__global__ void __launch_bounds__(kWave * DV / (kRowGroups * (PF ? 2 : 4))) verify_chunk_kernel(VerifyArgs<TIn> a) {
  __shared__ __align__(16) VerifyLds<DK> L;
  const int bh = blockIdx.x;
  const int b = bh / a.H, h = bh - b * a.H;
  const int T = a.T;
  int sb = b;  // index of the state (and position) this sequence uses
  if (a.slot_ids) {
    sb = a.slot_ids[b];
    if (sb < 0 || sb >= a.n_slots) {  // uniform over the workgroup: nothing is read or written
      if (h == 0 && threadIdx.x == 0) atomicOr(a.dev_err, KDA_DEV_ERR_SLOT_ID);
      if (threadIdx.x == 0) a.log_len[bh] = log_record(0, kLogPrepared);
      return;
    }
  }
  // Tokens this sequence verifies.
  int Tv = T;
  if (a.draft_len) {
    const int d = a.draft_len[b];
    if (d < 0 || d > T) {
      if (h == 0 && threadIdx.x == 0) atomicOr(a.dev_err, KDA_DEV_ERR_DRAFT_LEN);
      Tv = 0;
    } else {
      Tv = d;
    }
  }
  verify_seq<DK, DV, TIn, MULTI, COMMIT, PREP, PF, EARLY>(a, L, b, h, sb, (size_t)b * T * a.H + h,
                                                   (size_t)b * a.Tmax * a.H + h, T, Tv);
}

// Below this many (sequence, head) pairs a launch is bound by each
// workgroup's serial chain, not by bandwidth: verify (and the fused round)
// run 16 value columns per wave, and the fused round prefetches its replay.
// At and above it the 32-column shape wins (16-column waves up to 4,096
// pairs measured: verify at B = 64 37.6 against 30.5 us, the fused round at
// B = 16 22.0 against 17.6 us; H = 32).
#ifndef KDA_LATENCY_PAIRS
#define KDA_LATENCY_PAIRS 512
#endif
constexpr int kLatencyPairs = KDA_LATENCY_PAIRS;
// The fused round runs its first verify group's preparation ahead of the
// replay when the whole launch fits at two waves per SIMD (256 CUs x 4 SIMDs
// x 2): the registers that work holds through the replay then cost no
// occupancy, and the preparation's loads and LDS work leave the chain.
#ifndef KDA_EARLY_WAVES
#define KDA_EARLY_WAVES (2 * 4 * 256)
#endif
constexpr int kEarlyWaves = KDA_EARLY_WAVES;

template <int DK, int DV, typename TIn, bool COMMIT, bool PREP>
void launch_cfg(const VerifyArgs<TIn>& a, int32_t B, hipStream_t st) {
  const dim3 grid(B * a.H);
  const bool pf_shape = B * a.H < kLatencyPairs;
  const bool early = COMMIT && (int64_t)B * a.H * (DV / (kRowGroups * (pf_shape ? 2 : 4))) <= kEarlyWaves;
  auto go = [&](auto pf, auto ea) {
    constexpr bool PF = decltype(pf)::value, EA = decltype(ea)::value;
    const dim3 block(kWave * DV / (kRowGroups * (PF ? 2 : 4)));
    if (a.T <= kGroup)
      verify_chunk_kernel<DK, DV, TIn, false, COMMIT, PREP, PF, EA><<<grid, block, 0, st>>>(a);
    else
      verify_chunk_kernel<DK, DV, TIn, true, COMMIT, PREP, PF, EA><<<grid, block, 0, st>>>(a);
  };
  auto go_ea = [&](auto pf) {
    if (COMMIT && early)
      go(pf, std::true_type{});
    else
      go(pf, std::false_type{});
  };
  if (pf_shape) {
    go_ea(std::true_type{});
    return;
  }
  go_ea(std::false_type{});
}

template <typename TIn, bool COMMIT, bool PREP>
void launch_shape(const kda_shape& s, const VerifyArgs<TIn>& a, hipStream_t st) {
  if (s.dk == 128 && s.dv == 128) launch_cfg<128, 128, TIn, COMMIT, PREP>(a, s.B, st);
  else if (s.dk == 128) launch_cfg<128, 64, TIn, COMMIT, PREP>(a, s.B, st);
  else if (s.dv == 128) launch_cfg<64, 128, TIn, COMMIT, PREP>(a, s.B, st);
  else launch_cfg<64, 64, TIn, COMMIT, PREP>(a, s.B, st);
}

// gate < 0: prepared inputs; otherwise raw projections with that KDA_GATE_*.
template <typename TIn, bool COMMIT>
void launch_any(const kda_shape& s, int32_t T_pend, int32_t T, const int32_t* draft_len, float* state, int64_t* pos,
                const int32_t* accepted, int32_t* dev_err, TokenInputs in, float* o, LogPtrs log, int32_t gate,
                int32_t pend_gate, const int32_t* slot_ids, int32_t n_slots, hipStream_t st) {
  const VerifyArgs<TIn> a{state,   (const TIn*)in.q, (const TIn*)in.k, (const TIn*)in.v, in.alpha, in.beta, o,
                          (TIn*)log.k, (TIn*)log.v, log.alpha, log.beta, s.H, T, log.T_max, s.scale, pos, accepted,
                          dev_err, T_pend, draft_len, log.len, gate < 0 ? 0 : gate,
                          gate == KDA_GATE_SIGMOID ? 1.f : -1.f, pend_gate == KDA_GATE_SIGMOID ? 1.f : -1.f,
                          slot_ids, n_slots};
  if (gate < 0)
    launch_shape<TIn, COMMIT, false>(s, a, st);
  else
    launch_shape<TIn, COMMIT, true>(s, a, st);
}

}  // namespace

hipError_t launch_verify(const kda_shape& s, int32_t T, const int32_t* draft_len, const float* state, TokenInputs in,
                         float* o, LogPtrs log, int32_t* dev_err, int32_t gate, hipStream_t st,
                         const int32_t* slot_ids, int32_t n_slots) {
  // The verify-only kernel never writes through `state`.
  float* sp = const_cast<float*>(state);
  if (s.in_dtype == KDA_BF16)
    launch_any<bf16_t, false>(s, 0, T, draft_len, sp, nullptr, nullptr, dev_err, in, o, log, gate, -1, slot_ids,
                              n_slots, st);
  else
    launch_any<float, false>(s, 0, T, draft_len, sp, nullptr, nullptr, dev_err, in, o, log, gate, -1, slot_ids,
                             n_slots, st);
  return hipGetLastError();
}

hipError_t launch_commit_verify(const kda_shape& s, int32_t T_pend, int32_t T, const int32_t* draft_len, float* state,
                                int64_t* pos, const int32_t* accepted, int32_t* dev_err, TokenInputs in, float* o,
                                LogPtrs log, int32_t gate, int32_t pend_gate, hipStream_t st,
                                const int32_t* slot_ids, int32_t n_slots) {
  if (s.in_dtype == KDA_BF16)
    launch_any<bf16_t, true>(s, T_pend, T, draft_len, state, pos, accepted, dev_err, in, o, log, gate, pend_gate,
                             slot_ids, n_slots, st);
  else
    launch_any<float, true>(s, T_pend, T, draft_len, state, pos, accepted, dev_err, in, o, log, gate, pend_gate,
                            slot_ids, n_slots, st);
  return hipGetLastError();
}

}  // namespace kda
