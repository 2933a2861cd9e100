// Speculative verify for gfx950: T draft tokens from a committed state that
// is read once and never written, in the chunk (WY) form of the same gated
// delta rule, on the vector units.
//
// Unrolling the recurrence over a group of G tokens from the group's start
// state S0 (gamma_t = prod_{r<=t} alpha_r per key channel, products over the
// group only):
//   u_t = S0^T (gamma_t k_t) + sum_{s<t} A_ts e_s,   e_t = beta_t (v_t - u_t)
//   o_t = scale (S0^T (gamma_t q_t) + sum_{s<=t} P_ts e_s)
//   A_ts = sum_i k_s,i k_t,i prod_{s<r<=t} alpha_r,i      (s < t)
//   P_ts = sum_i k_s,i q_t,i prod_{s<r<=t} alpha_r,i      (s <= t)
// and the state after the group is
//   S_G = Diag(gamma_{G-1}) S0 + sum_s Diag(prod_{s<r<G} alpha_r) k_s e_s^T.
// (Chunked form of the per-channel-gated delta rule, written out in the
// appendix on the chunked WY/UT form; the per-token rule is the one the
// "Hyper-optimizing Kimi K3 in vLLM" pages call KDA.)
//
// Only 2 G multiply-adds per state element are needed for a group (the two
// projections S0^T (gamma k) and S0^T (gamma q)), against 4 G for the token
// loop (decay, k projection, q projection, rank-1 update).  Without packed
// fp32 a wave64 FMA costs four cycles, so at T = 4 the token loop's vector
// work is as long as the state's HBM read; this form halves it.  The decay
// products are formed as products of alphas (no division by a cumulative
// product), so gates of 0 are exact.
//
// One workgroup per (sequence, head), dv / 32 waves; wave w owns value
// columns [32 w, 32 w + 32) with the state lane mapping of the other state
// kernels (lane = 8 rg + cg: rows [R rg, R rg + R), columns 4 cg .. 4 cg + 3).
// Small batches use dv / 16 waves of 16 columns (columns 2 cg, 2 cg + 1 of
// the wave's slice): each column's arithmetic is the same, with half the work
// per wave.  Per group of up to four tokens:
//   1. preparation (all waves): gamma_t k_t, gamma_t q_t, the update
//      coefficients and the A / P entries into LDS; wave w takes the tokens
//      t = w (mod waves) and lane l key channels [CPL l, CPL l + CPL);
//   2. projections: each lane multiplies its R x NC state tile into 2 G
//      accumulators per column, then sums over the 8 row groups in-wave
//      (DPP row rotate, v_permlane16_swap, v_permlane32_swap);
//   3. per column: forward substitution for e_t, then o_t;
//   4. when tokens remain: S <- S_G in registers.
// The verify outputs therefore differ from decode-step outputs by rounding
// only; the committed state is always advanced by the commit kernel's token
// loop, which is the decode step's arithmetic.

#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

#include "kda_common.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kGroup = 4;  // tokens per group

template <typename TIn>
struct VerifyArgs {
  float* state;  // written only by the fused commit + verify
  const TIn* q;
  const TIn* k;
  const TIn* v;
  const float* alpha;
  const float* beta;
  float* o;
  TIn* log_k;
  TIn* log_v;
  float* log_alpha;
  float* log_beta;
  int32_t H;
  int32_t T;      // tokens verified by this call
  int32_t Tmax;   // token rows per sequence in the log
  float scale;
  // Fused commit + verify only: commit of the pending T_pend logged tokens.
  int64_t* pos;
  const int32_t* accepted;
  int32_t* dev_err;
  int32_t T_pend;
  // Per-sequence draft lengths (null: all T) and the log's per-(b, h) count
  // of verified rows, which bounds the next commit.
  const int32_t* draft_len;
  int32_t* log_len;
  // Raw projections (verify from raw inputs only): KDA_GATE_* of the decay
  // logits and its sign (decay = sigmoid(gate_sign * logit)).
  int32_t gate;
  float gate_sign;
  float pend_gate_sign;  // fused commit of a raw pending log (PREP): its decay sign
  // States (and, with COMMIT, positions) in a slot pool: sequence b uses
  // state[slot_ids[b]] and pos[slot_ids[b]]; null: the dense [B] arrays.
  const int32_t* slot_ids;
  int32_t n_slots;
};

// Per-group LDS.  Key-channel vectors are stored by row group with a padded
// stride (RP = R + 4 floats): the eight distinct row groups a wave reads in
// one 16-byte load then fall on disjoint banks.
template <int DK>
struct VerifyLds {
  static constexpr int R = DK / kRowGroups;
  static constexpr int RP = R + 4;
  static constexpr int VEC = kRowGroups * RP;
  float kap[kGroup][VEC];  // gamma_t k_t
  float rho[kGroup][VEC];  // gamma_t q_t
  float cof[kGroup][VEC];  // k_s prod_{s<r<G} alpha_r
  float gend[VEC];         // prod_{r<G} alpha_r
  float A[kGroup][kGroup];
  float P[kGroup][kGroup];
  static __device__ __forceinline__ int at(int ch) { return (ch / R) * RP + ch % R; }
};

// N consecutive key channels as stored (N = 1 or 2).
template <typename TIn, int N>
struct Chan;
template <>
struct Chan<bf16_t, 1> {
  uint32_t w;
  __device__ __forceinline__ float operator[](int) const { return bf16_lo(w); }
  __device__ __forceinline__ void load(rsrc_t r, int vo, int so) {
    w = __builtin_amdgcn_raw_buffer_load_b16(r, vo, so, 0);
  }
  __device__ __forceinline__ void store(rsrc_t r, int vo, int so) const {
    __builtin_amdgcn_raw_buffer_store_b16((unsigned short)w, r, vo, so, 0);
  }
};
template <>
struct Chan<bf16_t, 2> {
  uint32_t w;
  __device__ __forceinline__ float operator[](int i) const { return i ? bf16_hi(w) : bf16_lo(w); }
  __device__ __forceinline__ void load(rsrc_t r, int vo, int so) { w = __builtin_amdgcn_raw_buffer_load_b32(r, vo, so, 0); }
  __device__ __forceinline__ void store(rsrc_t r, int vo, int so) const {
    __builtin_amdgcn_raw_buffer_store_b32(w, r, vo, so, 0);
  }
};
template <>
struct Chan<float, 1> {
  uint32_t w;
  __device__ __forceinline__ float operator[](int) const { return __uint_as_float(w); }
  __device__ __forceinline__ void load(rsrc_t r, int vo, int so) { w = __builtin_amdgcn_raw_buffer_load_b32(r, vo, so, 0); }
  __device__ __forceinline__ void store(rsrc_t r, int vo, int so) const {
    __builtin_amdgcn_raw_buffer_store_b32(w, r, vo, so, 0);
  }
};
template <>
struct Chan<float, 2> {
  u32x2 w;
  __device__ __forceinline__ float operator[](int i) const { return __uint_as_float(i ? w.y : w.x); }
  __device__ __forceinline__ void load(rsrc_t r, int vo, int so) { w = __builtin_amdgcn_raw_buffer_load_b64(r, vo, so, 0); }
  __device__ __forceinline__ void store(rsrc_t r, int vo, int so) const {
    __builtin_amdgcn_raw_buffer_store_b64(w, r, vo + so, 0, 0);  // SGPR offset zero: see store_cols
  }
};

// NC consecutive value columns as stored (NC = 4, or 2 in the small-batch
// kernels whose waves own 16 value columns).
template <typename TIn, int NC>
struct ValC;
template <>
struct ValC<bf16_t, 4> {
  u32x2 w;
  __device__ __forceinline__ void load(rsrc_t r, int vo, int so) { w = __builtin_amdgcn_raw_buffer_load_b64(r, vo, so, 0); }
  __device__ __forceinline__ void store(rsrc_t r, int vo, int so) const {
    __builtin_amdgcn_raw_buffer_store_b64(w, r, vo + so, 0, 0);  // SGPR offset zero: see store_cols
  }
  __device__ __forceinline__ void widen(float (&x)[4]) const {
    x[0] = bf16_lo(w.x);
    x[1] = bf16_hi(w.x);
    x[2] = bf16_lo(w.y);
    x[3] = bf16_hi(w.y);
  }
};
template <>
struct ValC<float, 4> {
  u32x4 w;
  __device__ __forceinline__ void load(rsrc_t r, int vo, int so) { w = __builtin_amdgcn_raw_buffer_load_b128(r, vo, so, 0); }
  __device__ __forceinline__ void store(rsrc_t r, int vo, int so) const {
    __builtin_amdgcn_raw_buffer_store_b128(w, r, vo + so, 0, 0);  // SGPR offset zero: see store_cols
  }
  __device__ __forceinline__ void widen(float (&x)[4]) const {
    x[0] = __uint_as_float(w.x);
    x[1] = __uint_as_float(w.y);
    x[2] = __uint_as_float(w.z);
    x[3] = __uint_as_float(w.w);
  }
};
template <>
struct ValC<bf16_t, 2> {
  uint32_t w;
  __device__ __forceinline__ void load(rsrc_t r, int vo, int so) { w = __builtin_amdgcn_raw_buffer_load_b32(r, vo, so, 0); }
  __device__ __forceinline__ void store(rsrc_t r, int vo, int so) const {
    __builtin_amdgcn_raw_buffer_store_b32(w, r, vo, so, 0);
  }
  __device__ __forceinline__ void widen(float (&x)[2]) const {
    x[0] = bf16_lo(w);
    x[1] = bf16_hi(w);
  }
};
template <>
struct ValC<float, 2> {
  u32x2 w;
  __device__ __forceinline__ void load(rsrc_t r, int vo, int so) { w = __builtin_amdgcn_raw_buffer_load_b64(r, vo, so, 0); }
  __device__ __forceinline__ void store(rsrc_t r, int vo, int so) const {
    __builtin_amdgcn_raw_buffer_store_b64(w, r, vo + so, 0, 0);  // SGPR offset zero: see store_cols
  }
  __device__ __forceinline__ void widen(float (&x)[2]) const {
    x[0] = __uint_as_float(w.x);
    x[1] = __uint_as_float(w.y);
  }
};

// Windows over one (sequence, head)'s T tokens: consecutive tokens are H
// rows apart in every [B][T][H][d] tensor.
template <typename TIn, int DK, int DV>
struct Streams {
  rsrc_t k, q, alpha, v, o, log_k, log_v, log_alpha;
  int sk_in, sk_f32, sv_in, sv_f32;  // bytes between consecutive tokens
  __device__ __forceinline__ Streams(const VerifyArgs<TIn>& a, size_t tok0, size_t tok0_log, int T) {
    const size_t span = (size_t)(T - 1) * a.H;  // rows from the first to the last token
    const size_t es = sizeof(TIn);
    k = make_rsrc(a.k + tok0 * DK, (uint32_t)((span * DK + DK) * es));
    q = make_rsrc(a.q + tok0 * DK, (uint32_t)((span * DK + DK) * es));
    alpha = make_rsrc(a.alpha + tok0 * DK, (uint32_t)((span * DK + DK) * 4));
    v = make_rsrc(a.v + tok0 * DV, (uint32_t)((span * DV + DV) * es));
    o = make_rsrc(a.o + tok0 * DV, (uint32_t)((span * DV + DV) * 4));
    log_k = make_rsrc(a.log_k + tok0_log * DK, (uint32_t)((span * DK + DK) * es));
    log_v = make_rsrc(a.log_v + tok0_log * DV, (uint32_t)((span * DV + DV) * es));
    log_alpha = make_rsrc(a.log_alpha + tok0_log * DK, (uint32_t)((span * DK + DK) * 4));
    sk_in = a.H * DK * (int)es;
    sk_f32 = a.H * DK * 4;
    sv_in = a.H * DV * (int)es;
    sv_f32 = a.H * DV * 4;
  }
};

// A no-op for verify_group's `before_barrier` hook.
struct NoHook {
  __device__ __forceinline__ void operator()() const {}
};

// One group of G <= kGroup tokens starting at token t0, from the state tile S
// (rows [R rg, R rg + R) of this lane, columns col0 .. col0 + 3).  MULTI with
// advance: advance S to the state after the group (not needed after the last
// group, whose state is never written).  PREP: the inputs are raw
// projections and logits; they are prepared here (unit q and k, decay and
// beta from their logits, as the decode step from raw projections does) and
// logged raw.
// EARLY: before_barrier() runs between the group's preparation and the
// barrier that ends it, and the group's log rows are written after that
// barrier (the fused round replays the pending rows there, from the same
// log, while the preparation's loads and LDS work are in flight).
template <int DK, int DV, typename TIn, bool MULTI, bool PREP, int NC, bool EARLY = false, typename LoadState,
          typename Hook = NoHook>
__device__ __forceinline__ void verify_group(const VerifyArgs<TIn>& a, const Streams<TIn, DK, DV>& st,
                                             VerifyLds<DK>& L, float (&S)[DK / kRowGroups][NC], int t0, int G,
                                             size_t tok0, size_t tok0_log, int lane, int wave, bool first,
                                             const LoadState& load_state, bool advance,
                                             const Hook& before_barrier = Hook()) {
  constexpr int NW = DV / (kRowGroups * NC);  // waves: each owns 8 NC value columns
  constexpr int QW = (kGroup + NW - 1) / NW;    // preparation tokens per wave
  constexpr int R = DK / kRowGroups;
  constexpr int CPL = DK / kWave;  // key channels per lane in the preparation
  constexpr int RP = VerifyLds<DK>::RP;
  const int rg = lane >> 3, cg = lane & 7;
  const int col0 = wave * kRowGroups * NC + cg * NC;
  const int ch0 = lane * CPL;
  const int kvo_in = ch0 * (int)sizeof(TIn), kvo_f32 = ch0 * 4;
  const int vvo_in = col0 * (int)sizeof(TIn), vvo_f32 = col0 * 4;

  // ---- 1. preparation ---------------------------------------------------
  // Every input load of the group is issued before any use; padding tokens
  // (r >= G) re-read the group's last token and are never used.
  Chan<float, CPL> al[kGroup];
  Chan<TIn, CPL> kk[kGroup];
  ValC<TIn, NC> vv[kGroup];
  Chan<TIn, CPL> qq[QW];  // q of this wave's tokens wave, wave + NW, ...
  float bt[kGroup];
#pragma unroll
  for (int r = 0; r < kGroup; ++r) {
    const int tr = t0 + min(r, G - 1);
    al[r].load(st.alpha, kvo_f32, tr * st.sk_f32);
    kk[r].load(st.k, kvo_in, tr * st.sk_in);
    vv[r].load(st.v, vvo_in, tr * st.sv_in);
    bt[r] = a.beta[tok0 + (size_t)tr * a.H];
  }
#pragma unroll
  for (int j = 0; j < QW; ++j) qq[j].load(st.q, kvo_in, (t0 + min(wave + j * NW, G - 1)) * st.sk_in);
  // The state tile goes last: loads retire in order, so the preparation
  // below waits only for the small input loads while the tile streams in,
  // and the projections consume its rows as they land.
  if (first) {
    __builtin_amdgcn_sched_barrier(0);  // keep the issue order: inputs, then the tile
    load_state(S);
    __builtin_amdgcn_sched_barrier(0);
  }
  // The group's decays, key norm factors and betas as the recurrence uses
  // them (the loaded values themselves unless PREP).
  float av[kGroup][CPL], kn[kGroup], bp[kGroup];
#pragma unroll
  for (int r = 0; r < kGroup; ++r) {
    float k2 = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      if constexpr (PREP) {
        av[r][c] = sigmoid_f32(a.gate_sign * al[r][c]);
        k2 = __builtin_fmaf(kk[r][c], kk[r][c], k2);
      } else {
        av[r][c] = al[r][c];
      }
    }
    if constexpr (PREP) {
      kn[r] = inv_norm(lane_group_sum<64>(k2));
      bp[r] = sigmoid_f32(bt[r]);
    } else {
      kn[r] = 1.f;
      bp[r] = bt[r];
    }
  }
  if (MULTI && !first) __syncthreads();  // the previous group's LDS reads are done
  // This wave's tokens' k and alpha as stored, kept for a deferred log write.
  Chan<TIn, CPL> kt_log[EARLY ? QW : 1];
  Chan<float, CPL> at_log[EARLY ? QW : 1];
#pragma unroll
  for (int j = 0; j < QW; ++j) {
    const int t = wave + j * NW;
    if (t >= G) break;
    const int tt = t0 + t;
    const Chan<TIn, CPL> qt = qq[j];
    // Pick k_t and alpha_t out of the unrolled arrays without dynamic indexing.
    Chan<TIn, CPL> kt = kk[0];
    Chan<float, CPL> at = al[0];
    float knt = kn[0];
#pragma unroll
    for (int r = 1; r < kGroup; ++r)
      if (r == t) {
        kt = kk[r];
        at = al[r];
        knt = kn[r];
      }
    float qnt = 1.f;
    if constexpr (PREP) {
      float q2 = 0.f;
#pragma unroll
      for (int c = 0; c < CPL; ++c) q2 = __builtin_fmaf(qt[c], qt[c], q2);
      qnt = inv_norm(lane_group_sum<64>(q2));
    }
    if constexpr (EARLY) {
      kt_log[j] = kt;
      at_log[j] = at;
    } else {
      kt.store(st.log_k, kvo_in, tt * st.sk_in);
      at.store(st.log_alpha, kvo_f32, tt * st.sk_f32);
    }
    float pA[kGroup], pP[kGroup];
#pragma unroll
    for (int s = 0; s < kGroup; ++s) pA[s] = pP[s] = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const float kv = PREP ? kt[c] * knt : kt[c], qv = PREP ? qt[c] * qnt : qt[c];
      float gam = av[0][c];
#pragma unroll
      for (int r = 1; r < kGroup; ++r)
        if (r <= t) gam *= av[r][c];
      const int ix = VerifyLds<DK>::at(ch0 + c);
      L.kap[t][ix] = kv * gam;
      L.rho[t][ix] = qv * gam;
      if (MULTI && advance) {
        float cof = kv;
#pragma unroll
        for (int r = 1; r < kGroup; ++r)
          if (r > t && r < G) cof *= av[r][c];
        L.cof[t][ix] = cof;
      }
      // Backward over s = t .. 0 with bb = prod_{s<r<=t} alpha_r.
      float bb = 1.f;
#pragma unroll
      for (int s = kGroup - 1; s >= 0; --s) {
        if (s <= t) {
          const float ks = PREP ? kk[s][c] * kn[s] : kk[s][c];
          pP[s] = __builtin_fmaf(qv * ks, bb, pP[s]);
          if (s < t) pA[s] = __builtin_fmaf(kv * ks, bb, pA[s]);
          bb *= av[s][c];
        }
      }
    }
#pragma unroll
    for (int s = 0; s < kGroup; ++s) {
      if (s <= t) {
        const float ps = lane_group_sum<64>(pP[s]);
        const float as = s < t ? lane_group_sum<64>(pA[s]) : 0.f;
        if (lane == 0) {
          L.P[t][s] = ps;
          L.A[t][s] = as;
        }
      }
    }
  }
  if (MULTI && advance && wave == 0) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      float gam = av[0][c];
#pragma unroll
      for (int r = 1; r < kGroup; ++r)
        if (r < G) gam *= av[r][c];
      L.gend[VerifyLds<DK>::at(ch0 + c)] = gam;
    }
  }
  if constexpr (EARLY) {
    before_barrier();
    __syncthreads();  // every wave has replayed the pending rows: the log can be rewritten
#pragma unroll
    for (int j = 0; j < QW; ++j) {
      const int t = wave + j * NW;
      if (t < G) {
        kt_log[j].store(st.log_k, kvo_in, (t0 + t) * st.sk_in);
        at_log[j].store(st.log_alpha, kvo_f32, (t0 + t) * st.sk_f32);
      }
    }
  }
  // Log of v (this wave's columns; row group r writes token r) and beta.
  // (Written out here, not in a helper taking the arrays by reference: the
  // compiler would move such an array to LDS and wait for its loads before
  // issuing the state tile's.)
#pragma unroll
  for (int r = 0; r < kGroup; ++r)
    if (r < G && rg == r) vv[r].store(st.log_v, vvo_in, (t0 + r) * st.sv_in);
  if (wave == 0 && lane < G) {
    float bl = bt[0];
#pragma unroll
    for (int r = 1; r < kGroup; ++r)
      if (lane == r) bl = bt[r];
    a.log_beta[tok0_log + (size_t)(t0 + lane) * a.H] = bl;
  }
  if constexpr (!EARLY) __syncthreads();

  // ---- 2. projections x_t = S0^T kap_t, y_t = S0^T rho_t -----------------
  // Row blocks outermost: each block of four state rows is used by every
  // token of the group and is then dead (single-group case).
  float x[kGroup][NC], y[kGroup][NC];
#pragma unroll
  for (int t = 0; t < kGroup; ++t)
#pragma unroll
    for (int c = 0; c < NC; ++c) x[t][c] = y[t][c] = 0.f;
#pragma unroll
  for (int r4 = 0; r4 < R / 4; ++r4) {
#pragma unroll
    for (int t = 0; t < kGroup; ++t) {
      if (t < G) {
        const float4 kp = *reinterpret_cast<const float4*>(&L.kap[t][rg * RP + 4 * r4]);
        const float4 rp = *reinterpret_cast<const float4*>(&L.rho[t][rg * RP + 4 * r4]);
        const float kq[4] = {kp.x, kp.y, kp.z, kp.w}, rq[4] = {rp.x, rp.y, rp.z, rp.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            x[t][c] = __builtin_fmaf(kq[i], S[4 * r4 + i][c], x[t][c]);
            y[t][c] = __builtin_fmaf(rq[i], S[4 * r4 + i][c], y[t][c]);
          }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kGroup; ++t) {
    if (t < G) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        x[t][c] = rowgroup_sum_many(x[t][c]);
        y[t][c] = rowgroup_sum_many(y[t][c]);
      }
    }
  }

  // ---- 3. forward substitution and outputs, per column ------------------
  float e[kGroup][NC];
#pragma unroll
  for (int t = 0; t < kGroup; ++t) {
    if (t < G) {
      float vc[NC];
      vv[t].widen(vc);
      float o[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        float u = x[t][c];
#pragma unroll
        for (int s = 0; s < t; ++s) u = __builtin_fmaf(L.A[t][s], e[s][c], u);
        e[t][c] = bp[t] * (vc[c] - u);
        float w = y[t][c];
#pragma unroll
        for (int s = 0; s <= t; ++s) w = __builtin_fmaf(L.P[t][s], e[s][c], w);
        o[c] = a.scale * w;
      }
      if (rg == t) {
        store_cols<NC, 0>(o, st.o, vvo_f32, (t0 + t) * st.sv_f32);
      }
    }
  }

  // ---- 4. advance the in-register state --------------------------------
  if (MULTI && advance) {
#pragma unroll
    for (int r4 = 0; r4 < R / 4; ++r4) {
      const float4 g4 = *reinterpret_cast<const float4*>(&L.gend[rg * RP + 4 * r4]);
      const float gq[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int c = 0; c < NC; ++c) S[4 * r4 + i][c] *= gq[i];
#pragma unroll
      for (int s = 0; s < kGroup; ++s) {
        if (s < G) {
          const float4 c4 = *reinterpret_cast<const float4*>(&L.cof[s][rg * RP + 4 * r4]);
          const float cq[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int c = 0; c < NC; ++c) S[4 * r4 + i][c] = __builtin_fmaf(cq[i], e[s][c], S[4 * r4 + i][c]);
        }
      }
    }
  }
}

// MULTI: T may exceed one group (the state is advanced in registers between
// groups); otherwise T <= kGroup and the state dies after the projections.
// COMMIT: first replay the accepted prefix of the pending verify (the commit
// step, with the decode step's token loop), write the committed state and
// position, then verify the new tokens from the state still in registers.
// PF: small batches, where a launch is bound by the latency of one
// workgroup's serial chain, not by bandwidth.  Each wave owns 16 value
// columns instead of 32 (twice the waves per state), and with COMMIT the
// replay keeps the next logged token's loads in flight (double-buffered).
// One (sequence, head) by one workgroup of kWave dv / (8 NC) lanes.  Input
// token t sits at row tok0 + t H of the [tokens][H][d] inputs and outputs
// (the windows cover T_span >= max(Tv, 1) tokens) and at row tok0_log + t H
// of the log; the state and position are entry sb; bh = b H + h indexes
// the log's records.  With COMMIT the accepted prefix of the pending verify
// is replayed first; then the Tv tokens are verified and logged.
template <int DK, int DV, typename TIn, bool MULTI, bool COMMIT, bool PREP, bool PF, bool EARLY = false>
__device__ __forceinline__ void verify_seq(const VerifyArgs<TIn>& a, VerifyLds<DK>& L, int b, int h, int sb,
                                           size_t tok0, size_t tok0_log, int T_span, int Tv) {
  constexpr int R = DK / kRowGroups;
  // Value columns per lane: small batches (PF) split a state over twice as
  // many waves (16 columns each) to halve each wave's serial chain; the
  // arithmetic of every column is the same either way.
  constexpr int NC = PF ? 2 : 4;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rg = lane >> 3, cg = lane & 7;
  const int bh = b * a.H + h;
  const Streams<TIn, DK, DV> st(a, tok0, tok0_log, T_span);

  // The lane's state tile, loaded once.
  float S[R][NC];
  const rsrc_t rs = make_rsrc(a.state + ((size_t)sb * a.H + h) * DK * DV, DK * DV * 4);
  const int row0 = rg * R, col0 = wave * kRowGroups * NC + cg * NC;
  const int svo = (row0 * DV + col0) * 4;
  auto load_state = [&](float (&St)[R][NC]) {
#pragma unroll
    for (int r = 0; r < R; ++r) load_cols<NC, kStateLoadAux>(St[r], rs, svo, r * DV * 4);
  };
  auto no_load = [](float (&)[R][NC]) {};
  if (COMMIT) {
    LogReplay<DK, DV, TIn, R, PREP, NC> rp{a.log_k, a.log_v, a.log_alpha, a.log_beta, tok0_log, a.H, row0, col0};
    if (PF && a.T_pend > 0) rp.prime();  // logged token 0's loads go out ahead of the state tile
    load_state(S);
    // The replay runs with a count of 0 when nothing is to be committed, so
    // the tile has one definition after it (a replay under a branch keeps a
    // second copy of the 64-register tile live for the path that skips it).
    int n = 0;
    if (a.T_pend > 0) {
      n = a.accepted[b];
      if (n < 0 || n > min(a.T_pend, log_rows(a.log_len[bh]))) {
        if (h == 0 && wave == 0 && lane == 0) atomicOr(a.dev_err, KDA_DEV_ERR_ACCEPTED);
        n = 0;
      }
    }
    auto commit = [&]() {
      if constexpr (PF)
        rp.run(S, n, a.pend_gate_sign);
      else
        replay_log<DK, DV, TIn, R, PREP>(S, a.log_k, a.log_v, a.log_alpha, a.log_beta, tok0_log, a.H, n, row0, col0,
                                         a.pend_gate_sign);
      if (n > 0) {
#pragma unroll
        for (int r = 0; r < R; ++r) store_cols<NC, kStateStoreAux>(S[r], rs, svo, r * DV * 4);
        if (h == 0 && wave == 0 && lane == 0) a.pos[sb] += n;
      }
    };
    if (EARLY && Tv > 0) {
      // The first group's preparation (its input loads and LDS work) goes
      // ahead of the replay; the group's barrier then orders every wave's
      // reads of the pending rows and count before the group rewrites them.
      verify_group<DK, DV, TIn, MULTI, PREP, NC, true>(a, st, L, S, 0, min(kGroup, Tv), tok0, tok0_log, lane, wave,
                                                      true, no_load, MULTI && kGroup < Tv, commit);
      if (threadIdx.x == 0) a.log_len[bh] = log_record(Tv, PREP ? kLogRaw + a.gate : kLogPrepared);
      if constexpr (MULTI)
        for (int t0 = kGroup; t0 < Tv; t0 += kGroup)
          verify_group<DK, DV, TIn, true, PREP, NC>(a, st, L, S, t0, min(kGroup, Tv - t0), tok0, tok0_log, lane, wave,
                                                    false, no_load, t0 + kGroup < Tv);
      return;
    }
    commit();
    if (a.T_pend > 0) __syncthreads();  // every wave has read the pending log rows and count before the verify rewrites them
  }
  if (threadIdx.x == 0) a.log_len[bh] = log_record(Tv, PREP ? kLogRaw + a.gate : kLogPrepared);
  if (Tv == 0) return;
  if (COMMIT) {
    if (MULTI) {
      for (int t0 = 0; t0 < Tv; t0 += kGroup)
        verify_group<DK, DV, TIn, true, PREP, NC>(a, st, L, S, t0, min(kGroup, Tv - t0), tok0, tok0_log, lane, wave, t0 == 0,
                                              no_load, t0 + kGroup < Tv);
    } else {
      verify_group<DK, DV, TIn, false, PREP, NC>(a, st, L, S, 0, Tv, tok0, tok0_log, lane, wave, true, no_load, false);
    }
  } else if (MULTI) {
    for (int t0 = 0; t0 < Tv; t0 += kGroup)
      verify_group<DK, DV, TIn, true, PREP, NC>(a, st, L, S, t0, min(kGroup, Tv - t0), tok0, tok0_log, lane, wave, t0 == 0,
                                            load_state, t0 + kGroup < Tv);
  } else {
    verify_group<DK, DV, TIn, false, PREP, NC>(a, st, L, S, 0, Tv, tok0, tok0_log, lane, wave, true, load_state, false);
  }
}

}  // namespace
}  // namespace kda
