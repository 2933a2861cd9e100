// Shared device helpers for the KDA recurrent-state kernels (gfx950, wave64).
//
// Thread mapping used by every state-resident kernel (decode, verify, commit,
// recurrent prefill).  One wave owns a 32-column slice of one (sequence, head)
// state S [dk][dv]; lane = 8 * rg + cg with
//   cg in [0, 8): the lane's 4 value columns  col0 = 32 * slice + 4 * cg
//   rg in [0, 8): the lane's R = dk / 8 consecutive key rows  row0 = R * rg
// so each lane keeps R x 4 fp32 state values in registers.  A load of one
// row index by the whole wave touches 8 full 128-byte lines (one per row
// group).  Reductions over the key axis run inside the wave (xor over lane
// bits 3..5), so waves never synchronise with each other and no LDS is used.
// The smallest batches use 16-column slices instead (NC = 2 columns per
// lane: col0 = 16 * slice + 2 * cg): the same rows per lane and the same
// reduction tree, so every column's arithmetic is unchanged.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda.h"

namespace kda {

constexpr int kWave = 64;
constexpr int kSliceCols = 32;  // value columns per wave
constexpr int kRowGroups = 8;   // lanes sharing a column group, each with R rows

typedef uint16_t bf16_t;  // bfloat16 bit pattern

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Raw storage of N consecutive input values (bit-exact copy source for the log).
template <typename TIn, int N>
struct Raw;
template <int N>
struct Raw<bf16_t, N> {
  static_assert(N % 8 == 0, "bf16 rows are moved 16 bytes at a time");
  typedef uint4 vec;
  vec w[N / 8];
};
template <int N>
struct Raw<float, N> {
  static_assert(N % 4 == 0, "f32 rows are moved 16 bytes at a time");
  typedef float4 vec;
  vec w[N / 4];
};

template <typename TIn, int N>
__device__ __forceinline__ void load_raw(const TIn* p, Raw<TIn, N>& r) {
  typedef typename Raw<TIn, N>::vec vec;
  constexpr int V = sizeof(r.w) / 16;
#pragma unroll
  for (int i = 0; i < V; ++i) r.w[i] = reinterpret_cast<const vec*>(p)[i];
}

template <typename TIn, int N>
__device__ __forceinline__ void store_raw(TIn* p, const Raw<TIn, N>& r) {
  typedef typename Raw<TIn, N>::vec vec;
  constexpr int V = sizeof(r.w) / 16;
#pragma unroll
  for (int i = 0; i < V; ++i) reinterpret_cast<vec*>(p)[i] = r.w[i];
}

template <int N>
__device__ __forceinline__ void widen(const Raw<bf16_t, N>& r, float (&x)[N]) {
#pragma unroll
  for (int i = 0; i < N / 8; ++i) {
    const uint32_t a[4] = {r.w[i].x, r.w[i].y, r.w[i].z, r.w[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[8 * i + 2 * j] = bf16_lo(a[j]);
      x[8 * i + 2 * j + 1] = bf16_hi(a[j]);
    }
  }
}

template <int N>
__device__ __forceinline__ void widen(const Raw<float, N>& r, float (&x)[N]) {
#pragma unroll
  for (int i = 0; i < N / 4; ++i) {
    x[4 * i] = r.w[i].x;
    x[4 * i + 1] = r.w[i].y;
    x[4 * i + 2] = r.w[i].z;
    x[4 * i + 3] = r.w[i].w;
  }
}

// Element r of a raw row run, widened to fp32 (r is a compile-time constant
// after unrolling, so this is one shift/mask or a register read).
template <int N>
__device__ __forceinline__ float elem(const Raw<bf16_t, N>& r, int i) {
  const uint4 w = r.w[i / 8];
  const uint32_t x = (i % 8) < 2 ? w.x : (i % 8) < 4 ? w.y : (i % 8) < 6 ? w.z : w.w;
  return (i & 1) ? bf16_hi(x) : bf16_lo(x);
}
template <int N>
__device__ __forceinline__ float elem(const Raw<float, N>& r, int i) {
  const float4 w = r.w[i / 4];
  return (i % 4) == 0 ? w.x : (i % 4) == 1 ? w.y : (i % 4) == 2 ? w.z : w.w;
}

// The lane's NC consecutive value entries (NC = 4, or 2 in the small-batch
// speculative kernels, whose waves own 16 value columns).
template <typename TIn, int NC>
struct RawV;
template <>
struct RawV<bf16_t, 4> {
  typedef uint2 vec;
  vec w;
};
template <>
struct RawV<float, 4> {
  typedef float4 vec;
  vec w;
};
template <>
struct RawV<bf16_t, 2> {
  typedef uint32_t vec;
  vec w;
};
template <>
struct RawV<float, 2> {
  typedef float2 vec;
  vec w;
};
template <typename TIn>
using Raw4 = RawV<TIn, 4>;

template <typename TIn, int NC>
__device__ __forceinline__ void load4(const TIn* p, RawV<TIn, NC>& r) {
  r.w = *reinterpret_cast<const typename RawV<TIn, NC>::vec*>(p);
}
template <typename TIn, int NC>
__device__ __forceinline__ void store4(TIn* p, const RawV<TIn, NC>& r) {
  *reinterpret_cast<typename RawV<TIn, NC>::vec*>(p) = r.w;
}
__device__ __forceinline__ void widen4(const RawV<bf16_t, 4>& r, float (&x)[4]) {
  x[0] = bf16_lo(r.w.x);
  x[1] = bf16_hi(r.w.x);
  x[2] = bf16_lo(r.w.y);
  x[3] = bf16_hi(r.w.y);
}
__device__ __forceinline__ void widen4(const RawV<float, 4>& r, float (&x)[4]) {
  x[0] = r.w.x;
  x[1] = r.w.y;
  x[2] = r.w.z;
  x[3] = r.w.w;
}
__device__ __forceinline__ void widen4(const RawV<bf16_t, 2>& r, float (&x)[2]) {
  x[0] = bf16_lo(r.w);
  x[1] = bf16_hi(r.w);
}
__device__ __forceinline__ void widen4(const RawV<float, 2>& r, float (&x)[2]) {
  x[0] = r.w.x;
  x[1] = r.w.y;
}

// Cross-lane pair exchange on gfx950.  After the swap, a holds the value of
// the lower partner (even 16-lane row, resp. lower 32 lanes) and b the upper
// one, on both partners.  Written as inline assembly because hipcc folds the
// two results of __builtin_amdgcn_permlane{16,32}_swap(x, x) into one (it
// adds the first result to itself).  "s_nop 1" gives the two wait states a
// permlane read needs after a VALU write of its operands.
__device__ __forceinline__ float pair_sum16(float x) {
  float a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return a + b;
}
__device__ __forceinline__ float pair_sum32(float x) {
  float a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return a + b;
}

// Sum over the 8 row groups of a wave (lane bits 3, 4, 5), without LDS:
//   bit 3: DPP rotate of each 16-lane row by 8 (lane i reads lane i ^ 8),
//   bit 4: v_permlane16_swap (odd 16-lane rows exchanged with even rows),
//   bit 5: v_permlane32_swap (upper 32 lanes exchanged with lower 32).
// Every lane ends with the same value for its column group: each stage adds
// the same two operands on both partner lanes (the swaps return the pair in
// a fixed (lower, upper) order), and IEEE addition is commutative.
__device__ __forceinline__ float rowgroup_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128 /* row_ror:8 */,
                                                             0xf, 0xf, false));
  return pair_sum32(pair_sum16(x));
}

// Sum over all 64 lanes: rotations by 8, 4, 2, 1 inside each 16-lane row,
// then the two permlane swaps across rows.
__device__ __forceinline__ float wave_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x124, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x122, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x121, 0xf, 0xf, false));
  return pair_sum32(pair_sum16(x));
}

// lane ^ 16 and lane ^ 32 partners through the LDS crossbar (no LDS memory).
__device__ __forceinline__ float xor16_partner(float x) {
  // ds_swizzle bit mode: and_mask 0x1f, or_mask 0, xor_mask 0x10.
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401f));
}
__device__ __forceinline__ float xor32_partner(float x) {
  const int lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, __builtin_bit_cast(int, x)));
}

// rowgroup_sum for callers with many independent sums: the same additions in
// the same pairs (so bit-identical results), with the cross-row exchanges
// through the crossbar so that the compiler can interleave the sums.
__device__ __forceinline__ float rowgroup_sum_many(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xf, 0xf, false));
  x += xor16_partner(x);
  return x + xor32_partner(x);
}

// Sum over aligned groups of N = 32 or 64 lanes, every lane of a group
// getting the same value.  Across 16-lane rows it exchanges through the LDS
// crossbar (ds_swizzle for lane ^ 16, ds_bpermute for lane ^ 32) rather than
// the inline-assembly swaps above: those are scheduling boundaries, and a
// caller that needs many independent sums (one per token) wants them
// interleaved.  Each stage adds the same two values on both partner lanes
// (in either order; IEEE addition is commutative), so the group agrees.
template <int N>
__device__ __forceinline__ float lane_group_sum(float x) {
  static_assert(N == 32 || N == 64, "lane group");
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x124, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x122, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x121, 0xf, 0xf, false));
  x += xor16_partner(x);
  if (N == 64) x += xor32_partner(x);
  return x;
}

// One token of the gated delta rule on a lane's R x 4 register tile:
//   S1 = Diag(alpha) S;  u = S1^T k;  e = beta (v - u);  S = S1 + k e^T
// and, when WITH_OUT, o = scale (S1^T q + e (k . q)), which equals
// scale * S^T q of the updated state.  k, q and alpha stay in their loaded
// (raw) form and are widened row by row, so no fp32 copy of them is kept
// live next to the state.  Decode, verify, commit and the recurrent prefill
// all call this one function with the same lane mapping, so their states and
// outputs agree bit for bit.
template <int R, bool WITH_OUT, typename TIn, int NC>
__device__ __forceinline__ void token_update(float (&S)[R][NC], const Raw<TIn, R>& kraw, const Raw<float, R>& araw,
                                             const Raw<TIn, R>& qraw, const float (&vc)[NC], float beta,
                                             float scale, float (&o)[NC]) {
  float u[NC], w[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) u[c] = w[c] = 0.f;
  float kq = 0.f;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float kr = elem(kraw, r), ar = elem(araw, r);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const float s1 = ar * S[r][c];
      S[r][c] = s1;
      u[c] = __builtin_fmaf(kr, s1, u[c]);
      if (WITH_OUT) w[c] = __builtin_fmaf(elem(qraw, r), s1, w[c]);
    }
    if (WITH_OUT) kq = __builtin_fmaf(kr, elem(qraw, r), kq);
  }
#pragma unroll
  for (int c = 0; c < NC; ++c) u[c] = rowgroup_sum(u[c]);
  if (WITH_OUT) {
#pragma unroll
    for (int c = 0; c < NC; ++c) w[c] = rowgroup_sum(w[c]);
    kq = rowgroup_sum(kq);
  }
  float e[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) e[c] = beta * (vc[c] - u[c]);
  if (WITH_OUT) {
#pragma unroll
    for (int c = 0; c < NC; ++c) o[c] = scale * __builtin_fmaf(e[c], kq, w[c]);
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float kr = elem(kraw, r);
#pragma unroll
    for (int c = 0; c < NC; ++c) S[r][c] = __builtin_fmaf(kr, e[c], S[r][c]);
  }
}

// 1 / (1 + e^-x): exactly 0 for x = -inf (or far below zero) and exactly 1
// for x = +inf (or far above).
__device__ __forceinline__ float sigmoid_f32(float x) { return __builtin_amdgcn_rcpf(1.f + __expf(-x)); }

// 1 / |x| from the squared norm; a zero vector keeps norm factor 0, so it
// stays zero.  IEEE square root and division: scaling the vector by 2^p
// scales the factor by exactly 2^-p.
__device__ __forceinline__ float inv_norm(float sq) {
  const float r = 1.f / sqrtf(sq);  // computed unconditionally: a select, not a branch
  return sq > 0.f ? r : 0.f;
}

// token_update from raw projections (the input preparation fused into the
// step).  q and k arrive un-normalised, the decay as its logit x (per key
// channel) and beta as its logit.  The step uses
//   k^ = k / |k|, q^ = q / |q|  (L2 norms over the key channels),
//   alpha = sigmoid(gsign * x)  (gsign = -1: exp(-softplus(x)) = 1 / (1 + e^x);
//                                gsign = +1: sigmoid(x)),
//   beta = sigmoid(beta logit),
// and otherwise the same update and output as token_update.  The squared
// norms are reduced in the same pass as S1^T k and S1^T q, and the unit
// vectors enter as factors: u = (S1^T k) / |k|, S = S1 + (k / |k|) e^T,
// o = scale (S1^T q / |q| + e (k . q) / (|k| |q|)).  Without WITH_OUT (the
// replay of logged tokens) q is not touched and the state is the same.
template <int R, bool WITH_OUT, typename TIn, int NC>
__device__ __forceinline__ void token_update_prep(float (&S)[R][NC], const Raw<TIn, R>& kraw,
                                                  const Raw<float, R>& xraw, const Raw<TIn, R>& qraw,
                                                  const float (&vc)[NC], float beta_logit, float gsign, float scale,
                                                  float (&o)[NC]) {
  float u[NC], w[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) u[c] = w[c] = 0.f;
  float kq = 0.f, kk = 0.f, qq = 0.f;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float kr = elem(kraw, r);
    const float ar = sigmoid_f32(gsign * elem(xraw, r));
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const float s1 = ar * S[r][c];
      S[r][c] = s1;
      u[c] = __builtin_fmaf(kr, s1, u[c]);
      if (WITH_OUT) w[c] = __builtin_fmaf(elem(qraw, r), s1, w[c]);
    }
    kk = __builtin_fmaf(kr, kr, kk);
    if (WITH_OUT) {
      const float qr = elem(qraw, r);
      kq = __builtin_fmaf(kr, qr, kq);
      qq = __builtin_fmaf(qr, qr, qq);
    }
  }
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    u[c] = rowgroup_sum(u[c]);
    if (WITH_OUT) w[c] = rowgroup_sum(w[c]);
  }
  kk = rowgroup_sum(kk);
  if (WITH_OUT) {
    kq = rowgroup_sum(kq);
    qq = rowgroup_sum(qq);
  }
  const float rk = inv_norm(kk);
  const float beta = sigmoid_f32(beta_logit);
  float e[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) e[c] = beta * (vc[c] - u[c] * rk);
  if (WITH_OUT) {
    const float rq = inv_norm(qq);
    const float kqn = kq * rk * rq;
#pragma unroll
    for (int c = 0; c < NC; ++c) o[c] = scale * __builtin_fmaf(e[c], kqn, w[c] * rq);
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float kn = elem(kraw, r) * rk;
#pragma unroll
    for (int c = 0; c < NC; ++c) S[r][c] = __builtin_fmaf(kn, e[c], S[r][c]);
  }
}

// State tiles are streamed: each launch reads a state once and writes it once,
// and the next access to it comes a whole model layer (or round) later.  The
// state loads and stores therefore carry the non-temporal hint (bit 0: stores,
// bit 1: loads), which measured 8% faster for decode at B = 64 and 23% at
// B = 16 (H = 32, eight 128 MiB layer states), with commit and verify gaining
// alike.
#ifndef KDA_STATE_NT
#define KDA_STATE_NT 3
#endif
// Cache-policy bits of a buffer instruction for state traffic (2 = nt).
constexpr int kStateLoadAux = (KDA_STATE_NT & 2) ? 2 : 0;
constexpr int kStateStoreAux = (KDA_STATE_NT & 1) ? 2 : 0;
// Buffer-resource access: one SGPR base + range per tensor window, a 32-bit
// lane offset in a VGPR and uniform offsets in SGPRs (or the instruction's
// immediate), so no 64-bit address is kept per lane.  The hardware range
// check covers the lane offset plus the immediate, not the SGPR offset, so
// callers keep every access inside its window.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kRsrcWord3 = 0x00020000;  // raw 32-bit data format

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}

// NC fp32 values as one 16- or 8-byte buffer store (AUX: cache-policy bits).
// The uniform offset `so` is folded into the lane offset and the SGPR offset
// operand left zero: the compiler tracks the hazard of a VALU write to the
// data registers of a wide store (more than 32 bits here, to be safe) only
// when the store has no SGPR offset, and on gfx950 the hazard is real (such
// stores were seen writing the register's next value).  Every buffer store
// wider than 32 bits in this library is written this way.
template <int NC, int AUX>
__device__ __forceinline__ void store_cols(const float (&x)[NC], rsrc_t r, int vo, int so) {
  if constexpr (NC == 4) {
    const u32x4 w = {__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3])};
    __builtin_amdgcn_raw_buffer_store_b128(w, r, vo + so, 0, AUX);
  } else {
    const u32x2 w = {__float_as_uint(x[0]), __float_as_uint(x[1])};
    __builtin_amdgcn_raw_buffer_store_b64(w, r, vo + so, 0, AUX);
  }
}
// NC fp32 values from one 16- or 8-byte buffer load (AUX: cache-policy bits).
template <int NC, int AUX>
__device__ __forceinline__ void load_cols(float (&x)[NC], rsrc_t r, int vo, int so) {
  if constexpr (NC == 4) {
    const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(r, vo, so, AUX);
    x[0] = __uint_as_float(w.x);
    x[1] = __uint_as_float(w.y);
    x[2] = __uint_as_float(w.z);
    x[3] = __uint_as_float(w.w);
  } else {
    const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(r, vo, so, AUX);
    x[0] = __uint_as_float(w.x);
    x[1] = __uint_as_float(w.y);
  }
}

// Window over one (sequence, head) state [dk][dv].
template <int DK, int DV>
__device__ __forceinline__ rsrc_t state_rsrc(const float* state_bh) {
  return make_rsrc(state_bh, (uint32_t)(DK * DV * 4));
}

// A lane's R x NC state tile (rows DV floats apart, NC = 4 or 2 columns) in
// the state window rs, starting at byte offset vo: R buffer accesses that
// share one offset register (the rows are uniform offsets), with the
// non-temporal hint of the state traffic.
template <int R, int DV, int NC>
__device__ __forceinline__ void load_tile(rsrc_t rs, int vo, float (&S)[R][NC]) {
#pragma unroll
  for (int r = 0; r < R; ++r) load_cols<NC, kStateLoadAux>(S[r], rs, vo, r * DV * 4);
}

template <int R, int DV, int NC>
__device__ __forceinline__ void store_tile(rsrc_t rs, int vo, const float (&S)[R][NC]) {
#pragma unroll
  for (int r = 0; r < R; ++r) store_cols<NC, kStateStoreAux>(S[r], rs, vo, r * DV * 4);
}

// The per-token inputs one lane needs, as stored (raw) and widened.
template <typename TIn, int R, bool WITH_Q, int NC = 4>
struct TokenIn {
  Raw<TIn, R> k, q;
  Raw<float, R> a;
  RawV<TIn, NC> v;
  float beta;
  __device__ __forceinline__ void load(const TIn* kp, const TIn* qp, const float* ap, const TIn* vp,
                                       const float* bp) {
    load_raw(kp, k);
    if (WITH_Q) load_raw(qp, q);
    load_raw(ap, a);
    load4(vp, v);
    beta = *bp;
  }
  __device__ __forceinline__ void update(float (&S)[R][NC], float scale, float (&o)[NC]) const {
    float vc[NC];
    widen4(v, vc);
    token_update<R, WITH_Q>(S, k, a, q, vc, beta, scale, o);
  }
  // Raw projections: `a` holds the decay logits and `beta` the beta logit.
  __device__ __forceinline__ void update_prep(float (&S)[R][NC], float gsign, float scale, float (&o)[NC]) const {
    float vc[NC];
    widen4(v, vc);
    token_update_prep<R, WITH_Q>(S, k, a, q, vc, beta, gsign, scale, o);
  }
};

// Replays n logged tokens onto a lane's R x 4 state tile (rows row0..,
// columns col0..): the commit step.  Logged token t of this (sequence, head)
// sits at row tok0 + t * H of the [B][T_max][H] log regions.  RAW = false:
// the log holds prepared inputs (the decode step's update); RAW = true: raw
// projections and logits with decay sigmoid(gsign * logit) (the update of the
// decode step from raw projections).  Commit and the fused commit + verify
// both call this, so their states are bit-identical to n decode steps of the
// matching kind.  Callers pick RAW from the log record before loading any
// state, so each form runs as its own code path.
template <int DK, int DV, typename TIn, int R, bool RAW, int NC = 4>
struct LogReplay {
  const TIn* k;
  const TIn* v;
  const float* alpha;
  const float* beta;
  size_t tok0;
  int H, row0, col0;
  TokenIn<TIn, R, false, NC> cur, nxt;
  __device__ __forceinline__ void load(int t, TokenIn<TIn, R, false, NC>& x) const {
    const size_t tk = tok0 + (size_t)t * H;
    x.load(k + tk * DK + row0, nullptr, alpha + tk * DK + row0, v + tk * DV + col0, beta + tk);
  }
  // Issues the loads of logged token 0 (present whenever a verify is pending),
  // so they can be in flight before the count is known or the state loaded.
  __device__ __forceinline__ void prime() { load(0, cur); }
  // Applies logged tokens 0 .. n-1 (token 0 primed); the loads of token t + 1
  // are issued before token t's update, so each token's memory latency hides
  // behind the previous update.
  __device__ __forceinline__ void run(float (&S)[R][NC], int n, float gsign) {
    for (int t = 0; t < n; ++t) {
      if (t + 1 < n) load(t + 1, nxt);
      float o[NC];
      if constexpr (RAW)
        cur.update_prep(S, gsign, 0.f, o);
      else
        cur.update(S, 0.f, o);
      cur = nxt;
    }
  }
};

template <int DK, int DV, typename TIn, int R, bool RAW, int NC>
__device__ __forceinline__ void replay_log(float (&S)[R][NC], const TIn* log_k, const TIn* log_v,
                                           const float* log_alpha, const float* log_beta, size_t tok0, int H,
                                           int n, int row0, int col0, float gsign) {
  TokenIn<TIn, R, false, NC> cur;
  for (int t = 0; t < n; ++t) {
    const size_t tk = tok0 + (size_t)t * H;
    cur.load(log_k + tk * DK + row0, nullptr, log_alpha + tk * DK + row0, log_v + tk * DV + col0, log_beta + tk);
    float o[NC];
    if constexpr (RAW)
      cur.update_prep(S, gsign, 0.f, o);
    else
      cur.update(S, 0.f, o);
  }
}

// The per-(sequence, head) record of the log: the rows the last verify
// filled (low 16 bits) and the form of the logged inputs (high bits:
// kLogPrepared, or kLogRaw + gate for raw projections; the host keeps the
// same form in kda_log.pending_form to pick the replay kernel).
constexpr int kLogPrepared = 0;
constexpr int kLogRaw = 1;
__host__ __device__ constexpr int log_record(int rows, int form) { return rows | (form << 16); }
__device__ __forceinline__ int log_rows(int rec) { return rec & 0xffff; }

}  // namespace kda
