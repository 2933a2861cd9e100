// Chunked prompt processing on MFMA: the kernels over a batch of prompts of
// one length (one workgroup per (sequence, head)) and their launchers.  The
// chunk algebra and the single-role workgroup's code are in
// kda_prefill_impl.h, which the mixed-batch kernel shares; at chunk 64 the
// prepared inputs run on the bit-identical form with separate key and value
// waves (kda_prefill_ws.h), and so do raw projections.

#include <hip/hip_runtime.h>

#include <type_traits>

#include "kda_common.h"
#include "kda_internal.h"
#include "kda_prefill_impl.h"
#include "kda_prefill_ws.h"

// 0 keeps every shape on the single-role kernel.
#ifndef KDA_PREFILL_WS
#define KDA_PREFILL_WS 1
#endif
// 0 keeps raw projections on the single-role kernel.
#ifndef KDA_PREFILL_WS_PREP
#define KDA_PREFILL_WS_PREP 1
#endif

namespace kda {
namespace {

template <int DK, int DV, int CH, typename TIn, bool PREP>
__global__ void __launch_bounds__(DV * 4 / prefill_ct(DV)) prefill_chunked_kernel(PrefillArgs<TIn> a) {
  __shared__ __align__(16) char smem[Smem<DK, CH, DV / (16 * prefill_ct(DV))>::total];
  const int bh = blockIdx.x;
  const int b = bh / a.H, h = bh - b * a.H;
  int sb = b;  // index of the state and position this sequence uses
  if (a.state_slots) {
    sb = a.state_slots[b];
    if (sb < 0 || sb >= a.n_slots) {  // uniform over the workgroup
      if (h == 0 && threadIdx.x == 0) atomicOr(a.dev_err, KDA_DEV_ERR_SLOT_ID);
      return;
    }
  }
  prefill_seq<DK, DV, CH, TIn, PREP>(a, smem, b, h, sb, (size_t)b * a.L, a.L);
}

// One workgroup of dv / 16 value waves and ws_key_waves(dk) key waves per (sequence, head).
template <int DK, int DV, int CH, typename TIn, bool PREP>
__global__ void __launch_bounds__(64 * (DV / 16 + ws_key_waves(DK))) prefill_ws_kernel(PrefillArgs<TIn> a) {
  __shared__ __align__(16) char smem[SmemWs<DK, CH>::total];
  const int bh = blockIdx.x;
  const int b = bh / a.H, h = bh - b * a.H;
  int sb = b;
  if (a.state_slots) {
    sb = a.state_slots[b];
    if (sb < 0 || sb >= a.n_slots) {  // uniform over the workgroup
      if (h == 0 && threadIdx.x == 0) atomicOr(a.dev_err, KDA_DEV_ERR_SLOT_ID);
      return;
    }
  }
  prefill_seq_ws<DK, DV, CH, TIn, PREP>(a, smem, b, h, sb, (size_t)b * a.L, a.L);
}

template <int DK, int DV, typename TIn>
hipError_t launch_cfg(const kda_shape& s, int32_t L, int32_t chunk, float* state, int64_t* pos, TokenInputs in,
                      float* o, int32_t ckpt_every, const int32_t* ckpt_slots, float* slot_states, int64_t* slot_pos,
                      int32_t n_slots, int32_t* dev_err, int32_t gate, const int32_t* state_slots, hipStream_t st) {
  PrefillArgs<TIn> a{state,      pos,     (const TIn*)in.q, (const TIn*)in.k, (const TIn*)in.v, in.alpha, in.beta,
                     o,          ckpt_slots, slot_states,  slot_pos,         dev_err,          s.H,      L,
                     ckpt_every, n_slots, s.scale,         gate == KDA_GATE_SIGMOID ? 1.f : -1.f, state_slots};
  const dim3 grid((unsigned)((size_t)s.B * s.H));
  auto go = [&](auto prep) {
    constexpr bool PREP = decltype(prep)::value;
    // Raw projections run on it too (their keys and queries requested a
    // period ahead); chunk 32 keeps the single-role kernel.
    if constexpr (KDA_PREFILL_WS && (DV == 128 || DV == 64) &&
                  (DK == 128 || DK == 64) && (!PREP || KDA_PREFILL_WS_PREP)) {
      if (chunk == 64) {
        prefill_ws_kernel<DK, DV, 64, TIn, PREP><<<grid, 64 * (DV / 16 + ws_key_waves(DK)), 0, st>>>(a);
        return;
      }
    }
    if (chunk == 64)
      prefill_chunked_kernel<DK, DV, 64, TIn, PREP><<<grid, 4 * DV / prefill_ct(DV), 0, st>>>(a);
    else
      prefill_chunked_kernel<DK, DV, 32, TIn, PREP><<<grid, 4 * DV / prefill_ct(DV), 0, st>>>(a);
  };
  if (gate < 0)
    go(std::false_type{});
  else
    go(std::true_type{});
  return hipGetLastError();
}

template <typename TIn>
hipError_t launch_dtype(const kda_shape& s, int32_t L, int32_t chunk, float* state, int64_t* pos, TokenInputs in,
                        float* o, int32_t ckpt_every, const int32_t* ckpt_slots, float* slot_states, int64_t* slot_pos,
                        int32_t n_slots, int32_t* dev_err, int32_t gate, const int32_t* state_slots,
                        hipStream_t st) {
  if (s.dk == 128 && s.dv == 128)
    return launch_cfg<128, 128, TIn>(s, L, chunk, state, pos, in, o, ckpt_every, ckpt_slots, slot_states, slot_pos,
                                     n_slots, dev_err, gate, state_slots, st);
  if (s.dk == 128 && s.dv == 64)
    return launch_cfg<128, 64, TIn>(s, L, chunk, state, pos, in, o, ckpt_every, ckpt_slots, slot_states, slot_pos,
                                    n_slots, dev_err, gate, state_slots, st);
  if (s.dk == 64 && s.dv == 128)
    return launch_cfg<64, 128, TIn>(s, L, chunk, state, pos, in, o, ckpt_every, ckpt_slots, slot_states, slot_pos,
                                    n_slots, dev_err, gate, state_slots, st);
  return launch_cfg<64, 64, TIn>(s, L, chunk, state, pos, in, o, ckpt_every, ckpt_slots, slot_states, slot_pos,
                                 n_slots, dev_err, gate, state_slots, st);
}

}  // namespace

hipError_t launch_prefill_chunked(const kda_shape& s, int32_t L, int32_t chunk, float* state, int64_t* pos,
                                  TokenInputs in, float* o, int32_t ckpt_every, const int32_t* ckpt_slots,
                                  float* slot_states, int64_t* slot_pos, int32_t n_slots, int32_t* dev_err,
                                  int32_t gate, hipStream_t st, const int32_t* state_slots) {
  if (chunk != 32 && chunk != 64) return hipErrorInvalidValue;
  if (s.in_dtype == KDA_BF16)
    return launch_dtype<bf16_t>(s, L, chunk, state, pos, in, o, ckpt_every, ckpt_slots, slot_states, slot_pos,
                                n_slots, dev_err, gate, state_slots, st);
  return launch_dtype<float>(s, L, chunk, state, pos, in, o, ckpt_every, ckpt_slots, slot_states, slot_pos, n_slots,
                             dev_err, gate, state_slots, st);
}

}  // namespace kda
