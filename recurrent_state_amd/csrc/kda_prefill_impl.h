// Chunked (WY / UT-transform) prompt processing for gfx950 on MFMA.
//
// The pages leave the prefill math to the method; this kernel computes the
// same result as running the gated delta rule token by token (up to
// rounding), chunk by chunk.  For a chunk of n <= CH tokens starting from
// state S (rows = key channels, columns = value channels):
//
//   S~   = Diag(alpha_0) S                          first token's decay, applied up front
//   G_r  = prod_{1 <= s <= r} alpha_s               per key channel (G_0 = 1)
//   Kt   = k * G,  Qt = q * G,  Kh = k / G,  Kb = k * G_{n-1} / G
//   A    = strictly-lower(Diag(beta) Kt Kh^T)       (CH x CH)
//   P    = lower-with-diagonal(Qt Kh^T)             (CH x CH)
//   T    = (I + A)^-1 Diag(beta)
//   E    = T (V - Kt S~)                            (CH x dv)
//   O    = scale (Qt S~ + P E)
//   S'   = Diag(G_{n-1}) S~ + Kb^T E
//
// Kt Kh^T only ever forms the ratios G_r / G_i = prod_{i < s <= r} alpha_s
// (<= 1), but Kh itself grows as 1 / G.  Leaving the first token's decay out
// of G (it goes into S~) keeps a one-token chunk free of any division, and a
// chunk is cut short where some channel's G would drop below kMinDecay
// (2^-96): the chunk ends before that token and the next chunk starts there.
// So every factor stays within fp32 range and every gate in [0, 1] is
// handled exactly; gates that decay by less than 2^96 over a full chunk, in
// every channel, never shorten a chunk.
//
// One workgroup owns one (sequence, head) for the whole prompt and walks
// its chunks in order; wave w of the workgroup (dv / 16 waves) owns value
// columns [16 w, 16 w + 16) of the state, which stays in registers in the
// MFMA accumulator layout across chunks.  With two waves per SIMD, one
// wave's MFMA and LDS latency hides behind the other's work.  The key-side products (Kt, Qt, Kh, Kb,
// A, P, T) are shared by the waves through LDS.
//
// Precision: every contraction runs on v_mfma_f32_16x16x32_bf16 with fp32
// operands split as x = hi + lo (two bf16), and x*y ~ hi*hi + hi*lo + lo*hi
// accumulated in fp32 (the three-product bf16 scheme of Henry, Tang and
// Heinecke, "Leveraging the bfloat16 Artificial Intelligence Datatype For
// Higher-Precision Computations", ARITH 2019): about 2^-16 relative error
// per product instead of bf16's 2^-9.  The inverses of the 16 x 16 diagonal
// blocks of I + A are fp32 VALU.
//
// Operand layouts (16x16x32 bf16, verified on gfx950): lane l holds
//   A[m = l & 15][k = 8 (l >> 4) + e],  B[k = 8 (l >> 4) + e][n = l & 15],
//   D[m = 4 (l >> 4) + r][n = l & 15],  e < 8, r < 4.
// The contraction index k may be permuted consistently in A and B; this
// kernel uses k-slot e of lane group g = l >> 4 for index
//   pi(g, e) = 4 g + e (e < 4),  16 + 4 g + (e - 4) (e >= 4)
// inside each 32-wide k block, which turns two stacked D tiles (rows 0..15
// and 16..31 of the block) directly into a B operand.  The LDS planes store
// every k block in that slot order (column c at kpos(c)), so an operand is
// one aligned 16-byte LDS read per plane.

#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

#include "kda_common.h"
#include "kda_internal.h"

namespace kda {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;

struct Op {  // one MFMA operand as hi and lo bf16 parts
  bf16x8_t hi, lo;
};

__device__ __forceinline__ f32x4_t mfma(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// c += a * b with both operands split: hi*hi + hi*lo + lo*hi.
__device__ __forceinline__ f32x4_t mfma3(const Op& a, const Op& b, f32x4_t c) {
  c = mfma(a.lo, b.hi, c);
  c = mfma(a.hi, b.lo, c);
  return mfma(a.hi, b.hi, c);
}

__device__ __forceinline__ uint32_t bf16_bits(__bf16 h) { return (uint32_t)__builtin_bit_cast(uint16_t, h); }

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;

// Two fp32 values -> one packed bf16 pair (a in the low half), rounded to
// nearest even by one packed conversion instruction.
__device__ __forceinline__ uint32_t cvt2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// fp32 pair -> packed hi and lo bf16 pairs (round to nearest even both times):
// hi = bf16(x), lo = bf16(x - hi).  Written with packed conversions (two per
// pair); converting each value on its own costs twice the instructions.
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = cvt2(a, b);
  lo = cvt2(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}

__device__ __forceinline__ __bf16 split_hi(float x, __bf16& lo) {
  const __bf16 h = (__bf16)x;
  lo = (__bf16)(x - (float)h);
  return h;
}

// B operand from two stacked D tiles (rows 0..15 and 16..31 of a k block).
__device__ __forceinline__ Op op_from_tiles(const f32x4_t& t0, const f32x4_t& t1) {
  uint32_t h0, h1, h2, h3, l0, l1, l2, l3;
  split2(t0[0], t0[1], h0, l0);
  split2(t0[2], t0[3], h1, l1);
  split2(t1[0], t1[1], h2, l2);
  split2(t1[2], t1[3], h3, l3);
  const u32x4_t h = {h0, h1, h2, h3}, l = {l0, l1, l2, l3};
  return Op{__builtin_bit_cast(bf16x8_t, h), __builtin_bit_cast(bf16x8_t, l)};
}

// op_from_tiles(t0, t1) from op_from_tiles(t0, zero): the t0 half (words
// 0 and 1 of each part) is taken as it is, only t1 is split.
__device__ __forceinline__ Op op_with_upper(const Op& lower, const f32x4_t& t1) {
  u32x4_t h = __builtin_bit_cast(u32x4_t, lower.hi), l = __builtin_bit_cast(u32x4_t, lower.lo);
  uint32_t h2, h3, l2, l3;
  split2(t1[0], t1[1], h2, l2);
  split2(t1[2], t1[3], h3, l3);
  h[2] = h2;
  h[3] = h3;
  l[2] = l2;
  l[3] = l3;
  return Op{__builtin_bit_cast(bf16x8_t, h), __builtin_bit_cast(bf16x8_t, l)};
}

// Storage position of column c in a plane row: inside each 32-wide k block,
// slot e of lane group g (logical column pi(g, e)) sits at 8 g + e.
__device__ __forceinline__ int kpos(int c) { return (c & ~31) + 8 * ((c & 15) >> 2) + 4 * ((c & 31) >> 4) + (c & 3); }

// A (or B) operand read from a row-major bf16 plane: row `row`, lane group
// g's eight slots of the k block starting at logical column c0 = 32 kb + 4 g
// (logical columns c0..c0+3 and c0+16..c0+19), stored contiguously at
// 32 kb + 8 g.
__device__ __forceinline__ bf16x8_t plane_op(const bf16_t* plane, int row, int rs, int c0) {
  return *reinterpret_cast<const bf16x8_t*>(plane + row * rs + c0 + (c0 & 31));
}

__device__ __forceinline__ Op plane_op2(const bf16_t* hi, const bf16_t* lo, int row, int rs, int c0) {
  return Op{plane_op(hi, row, rs, c0), plane_op(lo, row, rs, c0)};
}

// Global accesses go through buffer resources (make_rsrc): each lane
// supplies one VGPR offset and per-access constants go in the SGPR offset
// operand, so a 64-element register tile spread over many rows costs one
// address VGPR.  The hardware range check does not cover the SGPR offset, so
// every access below is kept inside its window by explicit guards; the window
// size is a backstop.
__device__ __forceinline__ float ld_f32(rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}
__device__ __forceinline__ void st_f32(rsrc_t r, float v, int voff, int soff) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v), r, voff, soff, 0);
}
// Two consecutive input elements as loaded (bf16: one packed dword; f32: two
// dwords), widened when used.
template <typename TIn>
struct Pair2;
template <>
struct Pair2<bf16_t> {
  uint32_t w;
  __device__ __forceinline__ void load(rsrc_t r, int voff) { w = __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0); }
  __device__ __forceinline__ float lo() const { return bf16_lo(w); }
  __device__ __forceinline__ float hi() const { return bf16_hi(w); }
};
template <>
struct Pair2<float> {
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  u32x2 w;  // one 8-byte load (a vector result type keeps the load full width)
  __device__ __forceinline__ void load(rsrc_t r, int voff) { w = __builtin_amdgcn_raw_buffer_load_b64(r, voff, 0, 0); }
  __device__ __forceinline__ float lo() const { return __uint_as_float(w.x); }
  __device__ __forceinline__ float hi() const { return __uint_as_float(w.y); }
};
// One input element as loaded.
template <typename TIn>
struct One;
template <>
struct One<bf16_t> {
  uint32_t w;
  __device__ __forceinline__ void load(rsrc_t r, int voff) { w = __builtin_amdgcn_raw_buffer_load_b16(r, voff, 0, 0); }
  __device__ __forceinline__ float get() const { return bf16_lo(w); }
};
template <>
struct One<float> {
  float w;
  __device__ __forceinline__ void load(rsrc_t r, int voff) { w = ld_f32(r, voff, 0); }
  __device__ __forceinline__ float get() const { return w; }
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
  // Non-null: sequence b's state and position are slot state_slots[b] of the
  // pool (slot_states / slot_pos, n_slots); a bad id skips the sequence.
  const int32_t* state_slots;
};

// LDS layout of one workgroup (bytes).  Region R2 holds Kh during the A/P
// products and then P (hi/lo) plus the fp32 diagonal 16 x 16 blocks of A;
// R3 holds M (hi/lo): the strictly lower off-diagonal blocks of A and, on
// the diagonal, the inverses (I + A_jj)^-1.
template <int DK, int CH, int NW>
struct Smem {
  // Row strides (elements) of 16-byte aligned rows.  A wave reads an
  // operand as rows l & 15 at 16-byte column group l >> 4; on gfx950 that is
  // free of bank conflicts when the row stride is 8 mod 16 dwords, and
  // 2-way conflicted at 4 mod 8 dwords (measured).  The Kt/Qt planes, the
  // most-read operand, get the conflict-free stride; the others the 8-element
  // pad that fits the 160 KiB budget.
  static constexpr int RS_Q = DK + 16;  // Kt / Qt planes
  static constexpr int RS_K = DK + 8;   // Kh planes
  static constexpr int RS_C = CH + 8;   // token-indexed planes (Kb^T, M, P)
  static constexpr int NB = CH / 16;   // 16-token blocks per chunk
  static constexpr int NG = (64 * NW) / (DK / 2);  // token groups in the preparation phase
  static constexpr int KQ_PLANE = 2 * CH * RS_Q;   // elements per KQ plane
  static constexpr int KH_PLANE = CH * RS_K;
  static constexpr int KB_PLANE = DK * RS_C;
  static constexpr int CC_PLANE = CH * RS_C;
  static constexpr int off_kq = 0;
  static constexpr int off_kb = off_kq + 2 * KQ_PLANE * 2;
  static constexpr int off_r2 = off_kb + 2 * KB_PLANE * 2;
  static constexpr int r2_a = 2 * KH_PLANE * 2;
  // Diagonal blocks of A, fp32 and transposed (column i of a block is a
  // contiguous row of RS_D floats).  A block takes 16 RS_D + 4 floats: the
  // 4-float skew puts the same column of the NB blocks in different banks,
  // as the inverse reads them in one instruction.
  static constexpr int RS_D = 20;
  static constexpr int DSTRIDE = 16 * RS_D + 4;
  static constexpr int DIAG = NB * DSTRIDE;  // floats of the diagonal blocks
  static constexpr int r2_b = 2 * CC_PLANE * 2 + DIAG * 4;
  static constexpr int off_r3 = off_r2 + (r2_a > r2_b ? r2_a : r2_b);
  static constexpr int total = off_r3 + 2 * CC_PLANE * 2;
  // beta (CH floats), G_{n-1} and alpha_0 (DK floats each) and one int per
  // wave live in the 16 unused bytes at the end of each row of the Kb^T hi
  // plane (4 floats per row).
  static_assert(CH + 2 * DK + NW <= 4 * DK && (RS_C - CH) * 2 == 16, "misc values must fit the Kb row padding");
  // Token-group decay products, only live between the two passes
  // of the preparation: they borrow the M region, which is written later.
  static constexpr int off_tot = off_r3;
  static_assert(NG * DK * 4 <= 2 * CC_PLANE * 2, "decay-product scratch must fit the M region");
  static_assert(total <= 163840, "LDS budget exceeded");
  static_assert(off_kb % 16 == 0 && r2_a % 16 == 0 && off_r3 % 16 == 0 && (RS_Q * 2) % 16 == 0 &&
                    (KQ_PLANE * 2) % 16 == 0 && (KB_PLANE * 2) % 16 == 0 && (KH_PLANE * 2) % 16 == 0 &&
                    (CC_PLANE * 2) % 16 == 0 && (RS_K * 2) % 16 == 0 && (RS_C * 2) % 16 == 0,
                "16-byte aligned planes and rows");
};

// Lower-triangular tile (mt, nt), nt <= mt < 4, of triangular index ii.
__device__ __forceinline__ void tri_tile(int ii, int& mt, int& nt) {
  mt = ii >= 6 ? 3 : ii >= 3 ? 2 : ii >= 1 ? 1 : 0;
  nt = ii - mt * (mt + 1) / 2;
}

// PREP: q, k arrive un-normalised and the decay and beta as logits; the
// preparation phase normalises q and k (one full-wave sum per token: a wave
// holds every key channel of its tokens) and applies the gates, and the rest
// of the chunk is the prepared kernel's.
// 16-column tiles of the state per wave.  A wave reads each LDS operand of
// its value-side products once and applies it to all of its tiles.  Two
// tiles per wave (four waves at dv = 128) halve the LDS reads per matrix
// instruction but measured much slower (2.40 against 1.82 ms at B = 8,
// L = 8192): the chunk's chain is bound by latency, which eight waves hide
// better than four, not by LDS bandwidth.  One tile per wave is the default.
#ifndef KDA_PREFILL_CT
#define KDA_PREFILL_CT 1
#endif
// dv = 64 keeps one tile per wave: with two its two waves would each prepare
// twice the tokens, beyond the register file.
constexpr int prefill_ct(int DV) { return DV >= 128 ? KDA_PREFILL_CT : 1; }

// Smallest in-chunk decay product G a chunk may hold in any key channel:
// 1 / G then stays below 2^96, far inside the fp32 (and bf16) range, and the
// hi/lo split of k G keeps its precision for all but negligible components.
constexpr float kMinDecay = 0x1p-96f;

// The whole prompt of one (sequence, head), run by one workgroup of
// 64 dv / (16 prefill_ct(dv)) lanes: n_tok tokens, token t at row
// (tok0 + t) H + h of the [tokens][H][d] inputs and outputs; the state and
// position are entry sb of a.state and a.pos; due checkpoints (a.ckpt_every
// > 0) take their slots from row b of a.ckpt_slots.  smem points to the
// workgroup's Smem<DK, CH, waves>::total bytes of LDS.
template <int DK, int DV, int CH, typename TIn, bool PREP>
__device__ __forceinline__ void prefill_seq(const PrefillArgs<TIn>& a, char* smem, int b, int h, int sb, size_t tok0,
                                            int n_tok) {
  constexpr int CT = prefill_ct(DV);  // 16-column state tiles per wave
  constexpr int NW = DV / (16 * CT);  // waves; wave w owns value columns [16 CT w, 16 CT (w + 1))
  constexpr int NT = 64 * NW;        // threads
  constexpr int NB = CH / 16;        // 16-token blocks
  constexpr int KB = DK / 32;        // 32-channel k blocks
  constexpr int MT = DK / 16;        // channel tiles of the state
  constexpr int CP = DK / 2;         // channel pairs
  typedef Smem<DK, CH, NW> L;
  constexpr int NG = L::NG;
  constexpr int TPG = CH / NG;       // tokens per preparation group
  static_assert(NT % CP == 0 && CH % NG == 0 && TPG % 2 == 0, "preparation mapping");
  static_assert(CH == 32 || CH == 64, "chunk");

  bf16_t* kq_hi = reinterpret_cast<bf16_t*>(smem + L::off_kq);
  bf16_t* kq_lo = kq_hi + L::KQ_PLANE;
  bf16_t* kb_hi = reinterpret_cast<bf16_t*>(smem + L::off_kb);
  bf16_t* kb_lo = kb_hi + L::KB_PLANE;
  bf16_t* kh_hi = reinterpret_cast<bf16_t*>(smem + L::off_r2);
  bf16_t* kh_lo = kh_hi + L::KH_PLANE;
  bf16_t* p_hi = reinterpret_cast<bf16_t*>(smem + L::off_r2);
  bf16_t* p_lo = p_hi + L::CC_PLANE;
  float* adiag = reinterpret_cast<float*>(smem + L::off_r2 + 2 * L::CC_PLANE * 2);
  bf16_t* m_hi = reinterpret_cast<bf16_t*>(smem + L::off_r3);
  bf16_t* m_lo = m_hi + L::CC_PLANE;
  // beta_t at misc(t), G_n of channel c at misc(CH + c): the Kb^T row padding.
  auto misc = [&](int v) -> float& {
    return *reinterpret_cast<float*>(smem + L::off_kb + (v >> 2) * (L::RS_C * 2) + CH * 2 + (v & 3) * 4);
  };
  // misc(v) .. misc(v + 3) for v = 0 mod 4: one 16-byte read (one row's padding).
  auto misc4 = [&](int v) -> float4 {
    return *reinterpret_cast<const float4*>(smem + L::off_kb + (v >> 2) * (L::RS_C * 2) + CH * 2);
  };
  float* stot = reinterpret_cast<float*>(smem + L::off_tot);

  const bool owner = h == 0 && threadIdx.x == 0;  // the one writer of positions
  const int64_t pos0 = owner ? a.pos[sb] : 0;
  const int n_ckpt = a.ckpt_every > 0 ? n_tok / a.ckpt_every : 0;
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};

  // State columns of this wave in the accumulator layout:
  // st[ct][mt][r] = S[16 mt + 4 g + r][16 CT wave + 16 ct + l16], at byte
  // tile_voff + (16 mt + r) DV 4 + 64 ct.
  f32x4_t st[CT][MT];
  const int tile_voff = ((4 * ((threadIdx.x & 63) >> 4)) * DV + 16 * CT * (threadIdx.x >> 6) + (threadIdx.x & 15)) * 4;
  const rsrc_t rs_state = make_rsrc(a.state + ((size_t)sb * a.H + h) * DK * DV, DK * DV * 4);
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) st[ct][mt][r] = ld_f32(rs_state, tile_voff, (16 * mt + r) * DV * 4 + 64 * ct);

  const int rowk = a.H * DK, rowv = a.H * DV;  // elements between consecutive tokens
  // Nominal length of the chunk starting at token t: CH tokens, fewer at the
  // end of the prompt, and never past the next checkpoint boundary.
  const int ck_end = n_ckpt * a.ckpt_every;  // last checkpointed token position
  auto nominal = [&](int t) {
    int m = min(CH, n_tok - t);
    if (t < ck_end) m = min(m, (t / a.ckpt_every + 1) * a.ckpt_every - t);
    return m;
  };

  // Every global input load of a chunk (alpha, k, q, beta and this wave's
  // value tile) is issued one chunk ahead, before the previous chunk's value
  // phase, so its memory latency hides behind that phase.  Thread (cp, tg)
  // owns key channels 2 cp, 2 cp + 1 for tokens [tg TPG, tg TPG + TPG); a
  // padding row reads the chunk's last valid row (always inside the window)
  // and is replaced when used (alpha by 1, the others by 0).
  Pair2<float> ra[TPG];
  Pair2<TIn> rk[TPG], rq[TPG];
  float rb;  // beta of token tg TPG + (cp mod TPG): one load per lane instead of TPG identical ones
  One<TIn> rv[CT][NB][4];
  auto issue_loads = [&](int t_b, int nn, int tid_) {
    const size_t r0 = (tok0 + t_b) * a.H + h;
    const rsrc_t wk = make_rsrc(a.k + r0 * DK, ((nn - 1) * rowk + DK) * sizeof(TIn));
    const rsrc_t wq = make_rsrc(a.q + r0 * DK, ((nn - 1) * rowk + DK) * sizeof(TIn));
    const rsrc_t wa = make_rsrc(a.alpha + r0 * DK, ((nn - 1) * rowk + DK) * 4);
    const rsrc_t wb = make_rsrc(a.beta + r0, ((nn - 1) * a.H + 1) * 4);
    const rsrc_t wv = make_rsrc(a.v + r0 * DV, ((nn - 1) * rowv + DV) * sizeof(TIn));
    const int cp_ = tid_ % CP, tg_ = tid_ / CP;
    const int g_ = (tid_ & 63) >> 4, col_ = 16 * CT * (tid_ >> 6) + (tid_ & 15);
#pragma unroll
    for (int i = 0; i < TPG; ++i) {
      const int rc = min(tg_ * TPG + i, nn - 1);
      const int vo = rc * rowk + 2 * cp_;
      ra[i].load(wa, vo * 4);
      rk[i].load(wk, vo * (int)sizeof(TIn));
      rq[i].load(wq, vo * (int)sizeof(TIn));
    }
    rb = ld_f32(wb, min(tg_ * TPG + cp_ % TPG, nn - 1) * a.H * 4, 0);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int mt = 0; mt < NB; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int rc = min(16 * mt + 4 * g_ + r, nn - 1);
          rv[ct][mt][r].load(wv, (rc * rowv + col_ + 16 * ct) * (int)sizeof(TIn));
        }
  };
  int n_next = n_tok > 0 ? nominal(0) : 0;
  if (n_tok > 0) issue_loads(0, n_next, threadIdx.x);

  for (int t_base = 0; t_base < n_tok;) {
    // Lane coordinates are re-derived from an opaque copy of the thread id
    // in every chunk: otherwise the compiler hoists every LDS address of the
    // loop body out of the chunk loop and keeps them all live in registers.
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g = lane >> 4;
    int n = n_next;  // valid tokens in this chunk (cut short below if a decay is too strong); rows n.. are padding
    const size_t row0 = (tok0 + t_base) * a.H + h;  // [B][L][H] row index of the chunk's first token
    const rsrc_t rs_o = make_rsrc(a.o + row0 * DV, ((n - 1) * rowv + DV) * 4);

    // ---- Phase 1: cumulative decay and the decayed key/query planes -----
    const int cp = tid % CP, tg = tid / CP;
    const int c0 = 2 * cp;
    float al0[TPG], al1[TPG], k0[TPG], k1[TPG], q0[TPG], q1[TPG];
    float vv[CT][NB][4];
#pragma unroll
    for (int i = 0; i < TPG; ++i) {
      const bool pad = tg * TPG + i >= n;
      float x0 = ra[i].lo(), x1 = ra[i].hi();
      if constexpr (PREP) {
        x0 = sigmoid_f32(a.gate_sign * x0);
        x1 = sigmoid_f32(a.gate_sign * x1);
      }
      al0[i] = pad ? 1.f : x0;  // padding tokens do not decay
      al1[i] = pad ? 1.f : x1;
      k0[i] = pad ? 0.f : rk[i].lo();
      k1[i] = pad ? 0.f : rk[i].hi();
      q0[i] = pad ? 0.f : rq[i].lo();
      q1[i] = pad ? 0.f : rq[i].hi();
    }
    if constexpr (PREP) {
      // The CP lanes of token group tg (an aligned group of 32 or 64 lanes)
      // hold all DK key channels of its tokens, two per lane.  The 2 TPG
      // sums are independent, so they are formed together and interleave.
      float sk[TPG], sq[TPG];
#pragma unroll
      for (int i = 0; i < TPG; ++i) {
        sk[i] = lane_group_sum<CP>(__builtin_fmaf(k0[i], k0[i], k1[i] * k1[i]));
        sq[i] = lane_group_sum<CP>(__builtin_fmaf(q0[i], q0[i], q1[i] * q1[i]));
      }
#pragma unroll
      for (int i = 0; i < TPG; ++i) {
        const float rk_ = inv_norm(sk[i]), rq_ = inv_norm(sq[i]);
        k0[i] *= rk_;
        k1[i] *= rk_;
        q0[i] *= rq_;
        q1[i] *= rq_;
      }
    }
    // Token 0's decay is applied to the state before the chunk's products
    // (S~ = Diag(alpha_0) S), so it stays out of G.
    if (tg == 0) {
      misc(CH + DK + c0) = al0[0];
      misc(CH + DK + c0 + 1) = al1[0];
      al0[0] = al1[0] = 1.f;
    }
    {
      // Pass A: per-channel running products of alpha within the token group
      // (the cumulative decay itself: one multiply per token instead of a
      // logarithm and two exponentials); the group totals are combined
      // through LDS.
      float g0[TPG], g1[TPG];
      float s0 = 1.f, s1 = 1.f;
#pragma unroll
      for (int i = 0; i < TPG; ++i) {
        s0 *= al0[i];
        s1 *= al1[i];
        g0[i] = s0;
        g1[i] = s1;
      }
      stot[tg * DK + c0] = s0;
      stot[tg * DK + c0 + 1] = s1;
      if (cp < TPG) misc(tg * TPG + cp) = tg * TPG + cp < n ? (PREP ? sigmoid_f32(rb) : rb) : 0.f;  // padding: beta 0
      __syncthreads();
      float off0 = 1.f, off1 = 1.f, gn0 = 1.f, gn1 = 1.f;
#pragma unroll
      for (int j = 0; j < NG; ++j) {
        const float t0 = stot[j * DK + c0], t1 = stot[j * DK + c0 + 1];
        if (j < tg) {
          off0 *= t0;
          off1 *= t1;
        }
        gn0 *= t0;
        gn1 *= t1;
      }
      // Every wave holds every key channel (CP lanes per token group), so each
      // wave reaches the same decision from the same group totals.  G is
      // monotone in r, so the whole chunk is safe when G_{n-1} >= kMinDecay in
      // every channel.
      if (__any(gn0 < kMinDecay || gn1 < kMinDecay)) {
        // Cut the chunk before the first token r whose G_r < kMinDecay in some
        // channel (r >= 1: G_0 = 1).  Tokens from there on become padding and
        // start the next chunk.
        int f = n;
#pragma unroll
        for (int i = TPG - 1; i >= 0; --i) {
          const int r = tg * TPG + i;
          if (r < n && (off0 * g0[i] < kMinDecay || off1 * g1[i] < kMinDecay)) f = r;
        }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) f = min(f, __shfl_xor(f, m));
        if (lane == 0) *reinterpret_cast<int*>(&misc(CH + 2 * DK + wave)) = f;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < NW; ++w) f = min(f, *reinterpret_cast<const int*>(&misc(CH + 2 * DK + w)));
        n = __builtin_amdgcn_readfirstlane(f);  // equal in every lane
        // The lanes holding token n - 1 publish G_{n-1} of their channels.
#pragma unroll
        for (int i = 0; i < TPG; ++i)
          if (tg * TPG + i == n - 1) {
            misc(CH + c0) = off0 * g0[i];
            misc(CH + c0 + 1) = off1 * g1[i];
          }
        __syncthreads();
        gn0 = misc(CH + c0);
        gn1 = misc(CH + c0 + 1);
#pragma unroll
        for (int i = 0; i < TPG; ++i)
          if (tg * TPG + i >= n) k0[i] = k1[i] = q0[i] = q1[i] = 0.f;
        if (cp < TPG && tg * TPG + cp >= n) misc(tg * TPG + cp) = 0.f;
      } else if (tg == 0) {
        misc(CH + c0) = gn0;
        misc(CH + c0 + 1) = gn1;
      }
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int mt = 0; mt < NB; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) vv[ct][mt][r] = 16 * mt + 4 * g + r < n ? rv[ct][mt][r].get() : 0.f;
      // Pass B: the decayed planes; Kb goes to transposed planes two tokens at a time.
      // Kb = Kh G_{n-1} (no third factor per element).
      const float egn0 = gn0, egn1 = gn1;
      const int pc = kpos(c0);  // storage column of the channel pair (c0, c0 + 1)
      uint32_t kbh0 = 0, kbl0 = 0, kbh1 = 0, kbl1 = 0;
#pragma unroll
      for (int i = 0; i < TPG; ++i) {
        const int tr = tg * TPG + i;
        const float e0 = off0 * g0[i], e1 = off1 * g1[i];  // gamma of token tr
        const float ie0 = __builtin_amdgcn_rcpf(e0), ie1 = __builtin_amdgcn_rcpf(e1);
        uint32_t hi, lo;
        split2(k0[i] * e0, k1[i] * e1, hi, lo);  // Kt
        *reinterpret_cast<uint32_t*>(kq_hi + tr * L::RS_Q + pc) = hi;
        *reinterpret_cast<uint32_t*>(kq_lo + tr * L::RS_Q + pc) = lo;
        split2(q0[i] * e0, q1[i] * e1, hi, lo);  // Qt
        *reinterpret_cast<uint32_t*>(kq_hi + (CH + tr) * L::RS_Q + pc) = hi;
        *reinterpret_cast<uint32_t*>(kq_lo + (CH + tr) * L::RS_Q + pc) = lo;
        // Padding rows: zero (their G may be below kMinDecay, even 0).
        const float kh0 = tr < n ? k0[i] * ie0 : 0.f, kh1 = tr < n ? k1[i] * ie1 : 0.f;
        split2(kh0, kh1, hi, lo);  // Kh
        *reinterpret_cast<uint32_t*>(kh_hi + tr * L::RS_K + pc) = hi;
        *reinterpret_cast<uint32_t*>(kh_lo + tr * L::RS_K + pc) = lo;
        __bf16 l0, l1;
        const __bf16 h0 = split_hi(kh0 * egn0, l0), h1 = split_hi(kh1 * egn1, l1);
        const int sh = (i & 1) * 16;
        kbh0 |= bf16_bits(h0) << sh;
        kbl0 |= bf16_bits(l0) << sh;
        kbh1 |= bf16_bits(h1) << sh;
        kbl1 |= bf16_bits(l1) << sh;
        if (i & 1) {
          const int pt = kpos(tr - 1);  // storage column of the token pair (tr - 1, tr)
          *reinterpret_cast<uint32_t*>(kb_hi + c0 * L::RS_C + pt) = kbh0;
          *reinterpret_cast<uint32_t*>(kb_lo + c0 * L::RS_C + pt) = kbl0;
          *reinterpret_cast<uint32_t*>(kb_hi + (c0 + 1) * L::RS_C + pt) = kbh1;
          *reinterpret_cast<uint32_t*>(kb_lo + (c0 + 1) * L::RS_C + pt) = kbl1;
          kbh0 = kbl0 = kbh1 = kbl1 = 0;
        }
      }
    }
    __syncthreads();

    // ---- Phase 2: A = Diag(beta) Kt Kh^T and P = Qt Kh^T (lower tiles) ---
    // Tile list: index i < NA are A tiles (mt, nt), nt <= mt < NB; the next
    // NA are P tiles (NB + mt, nt).  Waves take tiles round-robin.  Each tile
    // is formed transposed (Kh as the A operand), so lane (g, l16) holds
    // row 16 mt + l16, columns 16 nt + 4 g .. + 3 of the tile: four
    // consecutive slots of a plane row, written hi and lo with one 8-byte
    // store each.
    constexpr int NA = NB * (NB + 1) / 2;
    constexpr int MAXT = (2 * NA + NW - 1) / NW;
    constexpr bool EVEN = (2 * NA) % NW == 0;  // every wave has MAXT tiles
    f32x4_t at[MAXT];
#pragma unroll
    for (int s_ = 0; s_ < MAXT; ++s_) {
      const int i = wave + s_ * NW;
      at[s_] = zero4;
      if (EVEN || i < 2 * NA) {
        int mt, nt;
        tri_tile(i < NA ? i : i - NA, mt, nt);
        const int row = (i < NA ? 0 : CH) + 16 * mt + l16;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const int k0_ = 32 * kb + 4 * g;
          at[s_] = mfma3(plane_op2(kh_hi, kh_lo, 16 * nt + l16, L::RS_K, k0_), plane_op2(kq_hi, kq_lo, row, L::RS_Q, k0_),
                         at[s_]);
        }
      }
    }
    __syncthreads();  // Kh is dead from here on; P and the diagonal blocks of A take its place
#pragma unroll
    for (int s_ = 0; s_ < MAXT; ++s_) {
      const int i = wave + s_ * NW;
      if (EVEN || i < 2 * NA) {
        int mt, nt;
        tri_tile(i < NA ? i : i - NA, mt, nt);
        const int tr = 16 * mt + l16;  // row token of this lane
        const int c0 = 16 * nt + 4 * g;  // its first column token
        float v4[4];
        if (i < NA) {  // wave-uniform branch
          const float bta = misc(tr);
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = c0 + e < tr ? at[s_][e] * bta : 0.f;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = c0 + e <= tr ? at[s_][e] : 0.f;
        }
        if (i < NA && mt == nt) {
          float* aj = adiag + mt * L::DSTRIDE;
#pragma unroll
          for (int e = 0; e < 4; ++e) aj[(4 * g + e) * L::RS_D + l16] = v4[e];
        } else {
          uint32_t h0, l0, h1, l1;
          split2(v4[0], v4[1], h0, l0);
          split2(v4[2], v4[3], h1, l1);
          bf16_t* dh = (i < NA ? m_hi : p_hi) + tr * L::RS_C + kpos(c0);
          bf16_t* dl = (i < NA ? m_lo : p_lo) + tr * L::RS_C + kpos(c0);
          *reinterpret_cast<uint2*>(dh) = make_uint2(h0, h1);
          *reinterpret_cast<uint2*>(dl) = make_uint2(l0, l1);
        }
      }
    }
    // Upper tiles inside a 32-token k block are read (against zero operands)
    // by the P E product and the block solve: make them zero in P and M.
    for (int i = wave; i < NB / 2; i += NW) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tr = 32 * i + 4 * g + r, tc = 32 * i + 16 + l16;
        p_hi[tr * L::RS_C + kpos(tc)] = 0;
        p_lo[tr * L::RS_C + kpos(tc)] = 0;
        m_hi[tr * L::RS_C + kpos(tc)] = 0;
        m_lo[tr * L::RS_C + kpos(tc)] = 0;
      }
    }
    __syncthreads();

    // ---- Phase 3: diagonal blocks X_jj = (I + A_jj)^-1 into M ------------
    // The last wave (it has the fewest A/P tiles) inverts every block at
    // once: lane 16 j + c forms column c of block j by right-looking
    // elimination in fp32 (x = e_c; for each i, column i of A_jj times x_i
    // is subtracted from the rows below i), so the chain is one multiply-add
    // per step; the columns are broadcast reads of the transposed copy.  The
    // block goes to M (1 on the diagonal, 0 above) as hi/lo.
    if (wave == NW - 1 && lane < 16 * NB) {
      const int j = lane >> 4, cc = lane & 15;
      const float* aj = adiag + j * L::DSTRIDE;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = r == cc ? 1.f : 0.f;
#pragma unroll
      for (int i = 0; i < 15; ++i) {
#pragma unroll
        for (int q = (i + 1) / 4; q < 4; ++q) {
          const float4 c4 = *reinterpret_cast<const float4*>(aj + i * L::RS_D + 4 * q);
          const float cv[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (4 * q + e > i) x[4 * q + e] = __builtin_fmaf(-cv[e], x[i], x[4 * q + e]);
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        __bf16 lo;
        const __bf16 hi = split_hi(x[r], lo);
        m_hi[(16 * j + r) * L::RS_C + kpos(16 * j + cc)] = __builtin_bit_cast(bf16_t, hi);
        m_lo[(16 * j + r) * L::RS_C + kpos(16 * j + cc)] = __builtin_bit_cast(bf16_t, lo);
      }
    }
    // No barrier here: the next loads and the X product below read only
    // registers and the Kt/Qt planes, so the other waves run them while the
    // last one inverts the blocks.  The barrier after the X product orders
    // the M writes before their reads.

    // The chunk's end, taken after the possible cut above (whose branch the
    // compiler cannot prove uniform): readfirstlane keeps it, the next
    // chunk's length and every buffer resource formed from them in scalar
    // registers.
    const int t_end = __builtin_amdgcn_readfirstlane(t_base + n);
    if (t_end < n_tok) {
      n_next = nominal(t_end);
      issue_loads(t_end, n_next, tid);
    }

    // ---- Phase 4: value side for this wave's CT tiles of 16 columns ------
    // Every LDS operand below is read once and used for all CT tiles.
    // 4a: S~ = Diag(alpha_0) S.
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const float4 a4 = misc4(CH + DK + 16 * mt + 4 * g);
      const float a0[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) st[ct][mt][r] *= a0[r];
    }
    // 4b: X = Kt S~ in the accumulator layout (lane: tokens 16 mt + 4 g + r,
    // column l16), and Qt S~ transposed into ot: with the state as the first
    // operand and the Qt plane as the second, lane (g, l16) holds columns
    // 4 g .. 4 g + 3 of token 16 mt + l16 (an accumulator tile is a valid
    // operand of either side, transposed), so the outputs leave as one
    // 16-byte store per token block instead of four 4-byte ones.
    f32x4_t xs[CT][NB], ot[CT][NB];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int mt = 0; mt < NB; ++mt) xs[ct][mt] = ot[ct][mt] = zero4;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      Op sop[CT];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) sop[ct] = op_from_tiles(st[ct][2 * kb], st[ct][2 * kb + 1]);
      const int k0_ = 32 * kb + 4 * g;
#pragma unroll
      for (int mt = 0; mt < NB; ++mt) {
        const Op kop = plane_op2(kq_hi, kq_lo, 16 * mt + l16, L::RS_Q, k0_);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) xs[ct][mt] = mfma3(kop, sop[ct], xs[ct][mt]);
      }
#pragma unroll
      for (int mt = 0; mt < NB; ++mt) {
        const Op qop = plane_op2(kq_hi, kq_lo, CH + 16 * mt + l16, L::RS_Q, k0_);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) ot[ct][mt] = mfma3(sop[ct], qop, ot[ct][mt]);
      }
    }
    __syncthreads();  // the diagonal blocks of M are complete
    // 4c/4d: R = V - Kt S~, then E = (I + A)^-1 Diag(beta) R by 16-token blocks:
    //   E_i = X_ii (beta_i R_i - sum_{j<i} A_ij E_j).
    // E is kept only as MFMA B operands eop[ct][kb] (32-token k blocks); while
    // block 2 kb + 1 is pending, eop[ct][kb] holds E_{2kb} and zeros.  The sum
    // runs over whole k blocks of M: the zero half adds nothing.
    Op eop[CT][NB / 2];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      f32x4_t z[CT];
      const float4 b4 = misc4(16 * i + 4 * g);
      const float bt4[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) z[ct][r] = bt4[r] * (vv[ct][i][r] - xs[ct][i][r]);
      if (i > 0) {
        f32x4_t cs[CT];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) cs[ct] = zero4;
#pragma unroll
        for (int kb = 0; kb <= (i - 1) / 2; ++kb) {
          const Op mop = plane_op2(m_hi, m_lo, 16 * i + l16, L::RS_C, 32 * kb + 4 * g);
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) cs[ct] = mfma3(mop, eop[ct][kb], cs[ct]);
        }
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) z[ct] -= cs[ct];
      }
      const Op ax = plane_op2(m_hi, m_lo, 16 * i + l16, L::RS_C, 32 * (i / 2) + 4 * g);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const f32x4_t e = mfma3(ax, (i & 1) ? op_from_tiles(zero4, z[ct]) : op_from_tiles(z[ct], zero4), zero4);
        xs[ct][i] = e;  // R_i is dead: keep E_i until its k block is complete
        eop[ct][i / 2] = (i & 1) ? op_with_upper(eop[ct][i / 2], e) : op_from_tiles(e, zero4);
      }
    }
    // 4e: O = scale (Qt S~ + P E), transposed like ot: (P E)^T = E^T P^T
    // takes E's operand as the first factor and the P plane rows as the
    // second.  Padding tokens (n..CH-1) need no test: their offsets start at
    // or past the end of rs_o's range, so the buffer unit drops those stores
    // (a per-lane branch here costs the kernel its registers).  The lane's
    // offset is laundered so that one register serves every token block.
    int ovo = (l16 * rowv + 16 * CT * wave + 4 * g) * 4;
    asm volatile("" : "+v"(ovo));
#pragma unroll
    for (int mt = 0; mt < NB; ++mt) {
#pragma unroll
      for (int kb = 0; kb <= mt / 2; ++kb) {
        const Op pop = plane_op2(p_hi, p_lo, 16 * mt + l16, L::RS_C, 32 * kb + 4 * g);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) ot[ct][mt] = mfma3(eop[ct][kb], pop, ot[ct][mt]);
      }
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const float o4[4] = {a.scale * ot[ct][mt][0], a.scale * ot[ct][mt][1], a.scale * ot[ct][mt][2],
                             a.scale * ot[ct][mt][3]};
        store_cols<4, 0>(o4, rs_o, ovo, (16 * mt * rowv + 16 * ct) * 4);
      }
    }
    // 4f: S = Diag(G_{n-1}) S~ + Kb^T E.
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const float4 g4 = misc4(CH + 16 * mt + 4 * g);
      const float gn4[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) st[ct][mt][r] *= gn4[r];
#pragma unroll
      for (int kb = 0; kb < NB / 2; ++kb) {
        const Op bop = plane_op2(kb_hi, kb_lo, 16 * mt + l16, L::RS_C, 32 * kb + 4 * g);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) st[ct][mt] = mfma3(bop, eop[ct][kb], st[ct][mt]);
      }
    }
    // Checkpoint at the end of this chunk when one is due (chunks never
    // cross a checkpoint boundary).
    if (t_end <= ck_end && t_end % a.ckpt_every == 0) {
      const int m = t_end / a.ckpt_every - 1;
      const int slot = a.ckpt_slots[(size_t)b * n_ckpt + m];
      if (slot >= 0 && slot < a.n_slots) {
        const rsrc_t rs_slot = make_rsrc(a.slot_states + ((size_t)slot * a.H + h) * DK * DV, DK * DV * 4);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) st_f32(rs_slot, st[ct][mt][r], tile_voff, (16 * mt + r) * DV * 4 + 64 * ct);
        if (owner) a.slot_pos[slot] = pos0 + t_end;
      } else if (tid == 0) {
        atomicOr(a.dev_err, KDA_DEV_ERR_CKPT_SLOT);
      }
    }
    __syncthreads();  // the next chunk rewrites every LDS region
    t_base = t_end;
  }

#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) st_f32(rs_state, st[ct][mt][r], tile_voff, (16 * mt + r) * DV * 4 + 64 * ct);
  if (owner) a.pos[sb] = pos0 + n_tok;
}

}  // namespace
}  // namespace kda
