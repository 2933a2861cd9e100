// Chunked prompt processing with the key side and the value side of each
// chunk on different waves (chunk 64; dk and dv 64 or 128).  The comments
// below count the waves of dk = dv = 128: eight of each role.
//
// The chunk algebra is the one of kda_prefill_impl.h, operation for
// operation: every product, split and sum below is formed from the same
// operands in the same order, so this kernel's outputs, states and
// checkpoints are bit-identical to the single-role kernel's.  (Raw
// projections are prepared by the key waves: each sums
// its 16 channels' part of a token's squared norms and the key waves' parts
// are added after the first barrier, an order the single-role kernel's full-wave
// sums do not share, so that form agrees with it to rounding.)  What changes
// is who does the work and when.  The key-side products of a chunk (the
// cumulative decays, the Kt / Qt / Kh / Kb^T planes, the A and P tiles and
// the inverses of the diagonal blocks of I + A) do not depend on the state.
// Eight key waves (each owning 16 key channels) build them for chunk c
// while eight value waves (one per 16 state columns, holding the state in
// registers) finish chunk c - 1; each SIMD runs two of each, the key waves'
// vector arithmetic and LDS writes beside the value waves' matrix work.
// The split keeps both roles within 128 registers (four waves per SIMD)
// without spills.
//
// One period of the loop handles the key side of chunk c and the value
// side of chunk c - 1; it has four workgroup barriers, and each role does
// the following between them (the LDS region each step reads or writes is
// named after the step; the default build does all of Kt S~ and (Qt S~)^T
// in I3 and gives every tile to the key waves):
//
//   interval  value waves                          key waves
//   I1        E and outputs of c - 1 (M, P, beta)  cumulative decay of c, cut vote, alpha_0
//   I2        state update of c - 1 (Kb^T, G),     chunk length; Kt / Qt planes; Kh into
//             checkpoint                           the P / M region
//   I3        S~ = Diag(alpha_0) S; Kt S~, Qt S~   Kb^T, beta, G; A and P tiles (Kh,
//             (Kt / Qt); value loads of c          Kt / Qt); one diagonal block each
//                                                  (key waves 0..3), inverted
//   I4        (optionally: last k blocks of the    A and P tiles into M and P; inverses into M
//             products, a P tile)
//
// Each region is written only after the barrier that ends its last read of
// the previous chunk: Kt / Qt (read in I3 and I4) are rewritten in I2 of
// the next period; the P / M region (read in I1) takes Kh in I2 and P / M in
// I4, after the A / P products have read Kh (I3); Kb^T and its row padding
// (read in I2) are rewritten in I3.  Each of key waves 0..3 forms and
// inverts one diagonal block of A in its own part of the fp32 diagonal
// region, so that needs no barrier.  Both roles run the same number of
// periods, from values both read from LDS, so their barriers pair up.

#pragma once

#include "kda_prefill_impl.h"

// k blocks of the value waves' Kt S~ and (Qt S~)^T products done in I3; the
// rest run in I4, beside the key waves' write-back.
#ifndef KDA_PREFILL_WS_XS
#define KDA_PREFILL_WS_XS 4
#endif
// Key waves request a chunk's inputs one period ahead (1) or in its own period
// (0).  The decays and betas go ahead only for prepared bf16 inputs: fp32 keys
// and queries take twice the registers, and raw projections need their
// keys and queries early; both hold only those ahead.
#ifndef KDA_PREFILL_WS_PREFETCH
#define KDA_PREFILL_WS_PREFETCH 1
#endif

namespace kda {
namespace {

// LDS layout (bytes).  The Kt / Qt planes, the Kb^T planes (whose row
// padding holds beta, G_{n-1}, alpha_0 and the cut votes), the region that
// holds Kh and then P and M, and one key wave's fp32 diagonal blocks.
template <int DK, int CH>
struct SmemWs {
  static constexpr int RS_Q = DK + 16;  // Kt / Qt planes (conflict-free stride, as in Smem)
  // Every plane takes the conflict-free row stride (8 mod 16 dwords); the
  // single-role kernel's layout has room for it only in the Kt / Qt planes.
  static constexpr int RS_K = DK + 16;  // Kh planes
  static constexpr int RS_C = CH + 16;  // token-indexed planes (Kb^T, M, P)
  static constexpr int NB = CH / 16;
  static constexpr int KQ_PLANE = 2 * CH * RS_Q;
  static constexpr int KH_PLANE = CH * RS_K;
  static constexpr int KB_PLANE = DK * RS_C;
  static constexpr int CC_PLANE = CH * RS_C;
  static constexpr int off_kq = 0;
  static constexpr int off_kb = off_kq + 2 * KQ_PLANE * 2;
  static constexpr int off_r2 = off_kb + 2 * KB_PLANE * 2;
  static constexpr int r2_kh = 2 * KH_PLANE * 2;
  static constexpr int r2_pm = 4 * CC_PLANE * 2;  // P hi, P lo, M hi, M lo
  static constexpr int RS_D = 20;                 // diagonal blocks: as in Smem
  static constexpr int DSTRIDE = 16 * RS_D + 4;
  static constexpr int off_diag = off_r2 + (r2_kh > r2_pm ? r2_kh : r2_pm);
  static constexpr int total = off_diag + NB * DSTRIDE * 4;
  // Slots of the misc values (floats; the votes are ints).
  static constexpr int M_BETA = 0, M_GN = CH, M_A0 = CH + DK, M_VOTE = CH + 2 * DK;
  static_assert(M_VOTE + DK / 8 <= 4 * DK && (RS_C - CH) * 2 >= 16, "misc values must fit the Kb^T row padding");
  static_assert(total <= 163840, "LDS budget exceeded");
  static_assert(off_kb % 16 == 0 && off_r2 % 16 == 0 && off_diag % 16 == 0 && (KQ_PLANE * 2) % 16 == 0 &&
                    (KB_PLANE * 2) % 16 == 0 && (KH_PLANE * 2) % 16 == 0 && (CC_PLANE * 2) % 16 == 0,
                "16-byte aligned planes");
};

// P tiles formed by each value wave (1), or none (0: the key waves form all).
#ifndef KDA_PREFILL_WS_VALUE_TILES
#define KDA_PREFILL_WS_VALUE_TILES 0
#endif
// Key channels per key wave.
#ifndef KDA_PREFILL_WS_KEY_CHANNELS
#define KDA_PREFILL_WS_KEY_CHANNELS 16
#endif
// Key waves per workgroup.
constexpr int ws_key_waves(int DK) { return DK / KDA_PREFILL_WS_KEY_CHANNELS; }

// Tiles of A and P (chunk 64): entries 0..5 are A's strictly lower blocks
// (mt, nt), nt < mt; entries 6..15 the P blocks (mt, nt), nt <= mt, in
// tri_tile order; entries 16..19 A's diagonal blocks.  With value-wave
// tiles, value wave v takes entry 16 - NV + v; key wave kw takes diagonal
// block kw (entry 16 + kw) if kw < 4, and entries kw, kw + NK, ... below the
// value waves' entries.
__device__ __forceinline__ void ws_tile(int i, bool& is_a, int& mt, int& nt) {
  if (i >= 16) {
    is_a = true;
    mt = nt = i - 16;
  } else if (i < 6) {
    is_a = true;
    mt = i >= 3 ? 3 : i >= 1 ? 2 : 1;
    nt = i - mt * (mt - 1) / 2;
  } else {
    is_a = false;
    tri_tile(i - 6, mt, nt);
  }
}

// Sum over aligned groups of 8 lanes, every lane of a group getting it:
// partners lane ^ 1 and lane ^ 2 (quad permutes), then the other quad of the
// group (half-row mirror).
__device__ __forceinline__ float lane8_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xb1, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4e, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xf, 0xf, false));
  return x;
}

// Lane i of each aligned group of 8 lanes, to every lane of the group
// (ds_swizzle bit mode: source lane (lane & 0x18) | i of each 32-lane half).
// i must fold to a constant.
__device__ __forceinline__ float lane8_bcast(float x, int i) {
  const int v = __builtin_bit_cast(int, x);
  int r;
  switch (i & 7) {
    case 0: r = __builtin_amdgcn_ds_swizzle(v, 0x18 | (0 << 5)); break;
    case 1: r = __builtin_amdgcn_ds_swizzle(v, 0x18 | (1 << 5)); break;
    case 2: r = __builtin_amdgcn_ds_swizzle(v, 0x18 | (2 << 5)); break;
    case 3: r = __builtin_amdgcn_ds_swizzle(v, 0x18 | (3 << 5)); break;
    case 4: r = __builtin_amdgcn_ds_swizzle(v, 0x18 | (4 << 5)); break;
    case 5: r = __builtin_amdgcn_ds_swizzle(v, 0x18 | (5 << 5)); break;
    case 6: r = __builtin_amdgcn_ds_swizzle(v, 0x18 | (6 << 5)); break;
    default: r = __builtin_amdgcn_ds_swizzle(v, 0x18 | (7 << 5)); break;
  }
  return __builtin_bit_cast(float, r);
}

// The whole prompt of one (sequence, head), run by one workgroup of
// 64 (dv / 16 + ws_key_waves(dk)) lanes; arguments as for prefill_seq.
// PREP: raw projections and logits, prepared by the key
// waves (see the key role).
template <int DK, int DV, int CH, typename TIn, bool PREP = false>
__device__ __forceinline__ void prefill_seq_ws(const PrefillArgs<TIn>& a, char* smem, int b, int h, int sb,
                                               size_t tok0, int n_tok) {
  static_assert((DK == 128 || DK == 64) && CH == 64 && DV % 16 == 0, "shape");
  constexpr int NV = DV / 16;   // value waves: wave v owns value columns [16 v, 16 v + 16)
  constexpr int NK = ws_key_waves(DK);  // key waves: key wave kw owns channels [CPW kw, CPW kw + CPW)
  constexpr int CPW = DK / NK;         // key channels per key wave
  constexpr int PPW = CPW / 2;         // channel pairs per key wave
  constexpr int TPL = CH * PPW / 64;   // tokens per key lane
  constexpr int NB = CH / 16;   // 16-token blocks
  constexpr int KB = DK / 32;   // 32-channel k blocks
  constexpr int MT = DK / 16;   // channel tiles of the state
  constexpr int TPG = 8;        // tokens per decay sub-group (the single-role kernel's groups)
  constexpr int NSG = CH / TPG; // sub-groups per chunk
  constexpr int SGL = TPL / TPG;  // sub-groups per key lane
  static_assert(TPL % TPG == 0 && 64 % PPW == 0 && NK >= 2, "key-wave mapping");
  typedef SmemWs<DK, CH> L;
  constexpr int VT = KDA_PREFILL_WS_VALUE_TILES;  // P tiles per value wave (0 or 1)
  static_assert(VT == 0 || VT == 1, "value-wave tiles");

  bf16_t* kq_hi = reinterpret_cast<bf16_t*>(smem + L::off_kq);
  bf16_t* kq_lo = kq_hi + L::KQ_PLANE;
  bf16_t* kb_hi = reinterpret_cast<bf16_t*>(smem + L::off_kb);
  bf16_t* kb_lo = kb_hi + L::KB_PLANE;
  bf16_t* kh_hi = reinterpret_cast<bf16_t*>(smem + L::off_r2);
  bf16_t* kh_lo = kh_hi + L::KH_PLANE;
  bf16_t* p_hi = reinterpret_cast<bf16_t*>(smem + L::off_r2);
  bf16_t* p_lo = p_hi + L::CC_PLANE;
  bf16_t* m_hi = p_lo + L::CC_PLANE;
  bf16_t* m_lo = m_hi + L::CC_PLANE;
  float* adiag = reinterpret_cast<float*>(smem + L::off_diag);
  auto misc = [&](int v) -> float& {
    return *reinterpret_cast<float*>(smem + L::off_kb + (v >> 2) * (L::RS_C * 2) + CH * 2 + (v & 3) * 4);
  };
  auto misc4 = [&](int v) -> float4 {
    return *reinterpret_cast<const float4*>(smem + L::off_kb + (v >> 2) * (L::RS_C * 2) + CH * 2);
  };
  auto vote = [&](int kw) -> int& { return *reinterpret_cast<int*>(&misc(L::M_VOTE + kw)); };
  // The key waves' parts of a token's squared norm (raw projections): one
  // float per key wave in the row padding of the Kt (row t: k of token t) or
  // Qt (row CH + t: q) hi plane, which no product reads.
  static_assert((L::RS_Q - DK) * 2 >= NK * 4 && (L::RS_Q * 2) % 16 == 0 && (DK * 2) % 16 == 0, "norm parts");
  auto norm_part = [&](int row) -> float* { return reinterpret_cast<float*>(kq_hi + row * L::RS_Q + DK); };
  // The chunk length agreed after the votes (every wave reads the same four).
  auto voted_length = [&]() {
    int n = vote(0);
#pragma unroll
    for (int kw = 1; kw < NK; ++kw) n = min(n, vote(kw));
    return __builtin_amdgcn_readfirstlane(n);
  };

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rowk = a.H * DK, rowv = a.H * DV;  // elements between consecutive tokens
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};

  if (wave < NV) {
    // ===================== value waves =====================
    const bool owner = h == 0 && threadIdx.x == 0;  // the one writer of positions
    const int64_t pos0 = owner ? a.pos[sb] : 0;
    const int n_ckpt = a.ckpt_every > 0 ? n_tok / a.ckpt_every : 0;
    const int ck_end = n_ckpt * a.ckpt_every;
    // st[mt][r] = S[16 mt + 4 g + r][16 wave + l16], at byte tile_voff + (16 mt + r) DV 4.
    f32x4_t st[MT];
    const int tile_voff = ((4 * ((threadIdx.x & 63) >> 4)) * DV + 16 * wave + (threadIdx.x & 15)) * 4;
    const rsrc_t rs_state = make_rsrc(a.state + ((size_t)sb * a.H + h) * DK * DV, DK * DV * 4);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) st[mt][r] = ld_f32(rs_state, tile_voff, (16 * mt + r) * DV * 4);

    f32x4_t xs[NB], ot[NB];  // Kt S~ (then E) and (Qt S~)^T of the chunk in flight
    Op eop[NB / 2];          // E as B operands, from the solve to the state update
    f32x4_t pt_v;            // this wave's tile of P, from I3 to I4
    One<TIn> rv[NB][4];      // this wave's value tile of the chunk in flight
    // k blocks kb0 .. kb1 - 1 of Kt S~ and (Qt S~)^T: the first XS in I3, the
    // rest in I4, where the key waves write their tiles back.
    constexpr int XS = KDA_PREFILL_WS_XS;
    auto x_blocks = [&](int kb0, int kb1, int l16, int g) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        if (kb < kb0 || kb >= kb1) continue;
        const Op sop = op_from_tiles(st[2 * kb], st[2 * kb + 1]);
        const int k0_ = 32 * kb + 4 * g;
#pragma unroll
        for (int mt = 0; mt < NB; ++mt)
          xs[mt] = mfma3(plane_op2(kq_hi, kq_lo, 16 * mt + l16, L::RS_Q, k0_), sop, xs[mt]);
#pragma unroll
        for (int mt = 0; mt < NB; ++mt)
          ot[mt] = mfma3(sop, plane_op2(kq_hi, kq_lo, CH + 16 * mt + l16, L::RS_Q, k0_), ot[mt]);
      }
    };
    int t_k = 0;             // first token of the chunk whose key side runs this period
    int t_prev = 0, n_prev = 0;
    bool prev = false;       // a chunk awaits its solve, outputs and state update
    for (;;) {
      const bool have = t_k < n_tok;
      if (!have && !prev) break;
      int tid = threadIdx.x;
      asm volatile("" : "+v"(tid));
      const int lane = tid & 63, l16 = lane & 15, g = lane >> 4;

      // ---- I1: E and the outputs of the previous chunk ----
      if (prev) {
        float vv[NB][4];
        if (n_prev == CH) {  // no padding rows
#pragma unroll
          for (int mt = 0; mt < NB; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) vv[mt][r] = rv[mt][r].get();
        } else {
#pragma unroll
          for (int mt = 0; mt < NB; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) vv[mt][r] = 16 * mt + 4 * g + r < n_prev ? rv[mt][r].get() : 0.f;
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          const float4 b4 = misc4(L::M_BETA + 16 * i + 4 * g);
          const float bt4[4] = {b4.x, b4.y, b4.z, b4.w};
          f32x4_t z;
#pragma unroll
          for (int r = 0; r < 4; ++r) z[r] = bt4[r] * (vv[i][r] - xs[i][r]);
          if (i > 0) {
            f32x4_t cs = zero4;
#pragma unroll
            for (int kb = 0; kb <= (i - 1) / 2; ++kb)
              cs = mfma3(plane_op2(m_hi, m_lo, 16 * i + l16, L::RS_C, 32 * kb + 4 * g), eop[kb], cs);
            z -= cs;
          }
          const Op ax = plane_op2(m_hi, m_lo, 16 * i + l16, L::RS_C, 32 * (i / 2) + 4 * g);
          const f32x4_t e = mfma3(ax, (i & 1) ? op_from_tiles(zero4, z) : op_from_tiles(z, zero4), zero4);
          xs[i] = e;
          eop[i / 2] = (i & 1) ? op_from_tiles(xs[i - 1], e) : op_from_tiles(e, zero4);
        }
        const size_t row0 = (tok0 + t_prev) * a.H + h;
        const rsrc_t rs_o = make_rsrc(a.o + row0 * DV, ((n_prev - 1) * rowv + DV) * 4);
        // Padding tokens' offsets start at or past the end of rs_o's range:
        // the buffer unit drops those stores.
        int ovo = (l16 * rowv + 16 * wave + 4 * g) * 4;
        asm volatile("" : "+v"(ovo));
#pragma unroll
        for (int mt = 0; mt < NB; ++mt) {
#pragma unroll
          for (int kb = 0; kb <= mt / 2; ++kb)
            ot[mt] = mfma3(eop[kb], plane_op2(p_hi, p_lo, 16 * mt + l16, L::RS_C, 32 * kb + 4 * g), ot[mt]);
          const float o4[4] = {a.scale * ot[mt][0], a.scale * ot[mt][1], a.scale * ot[mt][2], a.scale * ot[mt][3]};
          store_cols<4, 0>(o4, rs_o, ovo, 16 * mt * rowv * 4);
        }
      }
      __syncthreads();  // B1

      // ---- I2: state update and checkpoint of the previous chunk ----
      const int n_k = have ? voted_length() : 0;
      if (prev) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const float4 g4 = misc4(L::M_GN + 16 * mt + 4 * g);
          const float gn4[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) st[mt][r] *= gn4[r];
#pragma unroll
          for (int kb = 0; kb < NB / 2; ++kb)
            st[mt] = mfma3(plane_op2(kb_hi, kb_lo, 16 * mt + l16, L::RS_C, 32 * kb + 4 * g), eop[kb], st[mt]);
        }
        const int t_end = t_prev + n_prev;
        if (t_end <= ck_end && t_end % a.ckpt_every == 0) {
          const int m = t_end / a.ckpt_every - 1;
          const int slot = a.ckpt_slots[(size_t)b * n_ckpt + m];
          if (slot >= 0 && slot < a.n_slots) {
            const rsrc_t rs_slot = make_rsrc(a.slot_states + ((size_t)slot * a.H + h) * DK * DV, DK * DV * 4);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
              for (int r = 0; r < 4; ++r) st_f32(rs_slot, st[mt][r], tile_voff, (16 * mt + r) * DV * 4);
            if (owner) a.slot_pos[slot] = pos0 + t_end;
          } else if (tid == 0) {
            atomicOr(a.dev_err, KDA_DEV_ERR_CKPT_SLOT);
          }
        }
      }
      __syncthreads();  // B2

      // ---- I3: S~ = Diag(alpha_0) S, then Kt S~ and (Qt S~)^T; value loads ----
      if (have) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const float4 a4 = misc4(L::M_A0 + 16 * mt + 4 * g);
          const float a0[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) st[mt][r] *= a0[r];
        }
#pragma unroll
        for (int mt = 0; mt < NB; ++mt) xs[mt] = ot[mt] = zero4;
        x_blocks(0, XS, l16, g);
        // This wave's tile of P.
        pt_v = zero4;
        if (VT) {
          bool is_a;
          int mt, nt;
          ws_tile(16 - NV + wave, is_a, mt, nt);
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            const int k0_ = 32 * kb + 4 * g;
            pt_v = mfma3(plane_op2(kh_hi, kh_lo, 16 * nt + l16, L::RS_K, k0_),
                         plane_op2(kq_hi, kq_lo, CH + 16 * mt + l16, L::RS_Q, k0_), pt_v);
          }
        }
        // The value tile of this chunk, used by its solve in I1 of the next
        // period; issued after the products so that its registers are free
        // during them.  Padding rows lie past the end of the window (the
        // buffer unit returns zero) and are replaced by zero when used; one
        // chained offset register, as for the key inputs.
        const size_t r0 = (tok0 + t_k) * a.H + h;
        const rsrc_t wv = make_rsrc(a.v + r0 * DV, ((n_k - 1) * rowv + DV) * sizeof(TIn));
        int vo = (4 * g * rowv + 16 * wave + l16) * (int)sizeof(TIn);
#pragma unroll
        for (int mt = 0; mt < NB; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            asm volatile("" : "+v"(vo));
            rv[mt][r].load(wv, vo);
            vo += (r < 3 ? 1 : 13) * rowv * (int)sizeof(TIn);  // next row: 16 mt + 4 g + r + 1, or the next block
          }
      }
      __syncthreads();  // B3
      // ---- I4: the rest of Kt S~ and (Qt S~)^T; this wave's tile of P into the P planes ----
      if (have) x_blocks(XS, KB, l16, g);
      if (have && VT) {
        bool is_a;
        int mt, nt;
        ws_tile(16 - NV + wave, is_a, mt, nt);
        const int tr = 16 * mt + l16, ct0 = 16 * nt + 4 * g;
        float v4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = ct0 + e <= tr ? pt_v[e] : 0.f;
        uint32_t h0, l0, h1, l1;
        split2(v4[0], v4[1], h0, l0);
        split2(v4[2], v4[3], h1, l1);
        *reinterpret_cast<uint2*>(p_hi + tr * L::RS_C + kpos(ct0)) = make_uint2(h0, h1);
        *reinterpret_cast<uint2*>(p_lo + tr * L::RS_C + kpos(ct0)) = make_uint2(l0, l1);
      }
      __syncthreads();  // B4
      prev = have;
      if (have) {
        t_prev = t_k;
        n_prev = n_k;
        t_k += n_k;
      }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) st_f32(rs_state, st[mt][r], tile_voff, (16 * mt + r) * DV * 4);
    if (owner) a.pos[sb] = pos0 + n_tok;
  } else {
    // ===================== key waves =====================
    // Lane (p, j) of key wave kw: key channels c0 = CPW kw + 2 p and c0 + 1
    // (p = lane mod PPW) for the TPL tokens [TPL j, TPL j + TPL)
    // (j = lane / PPW), which are the decay sub-groups SGL j ... SGL j + SGL - 1.
    const int kw = wave - NV;
    const int n_ckpt = a.ckpt_every > 0 ? n_tok / a.ckpt_every : 0;
    const int ck_end = n_ckpt * a.ckpt_every;
    auto nominal = [&](int t) {
      int m = min(CH, n_tok - t);
      if (t < ck_end) m = min(m, (t / a.ckpt_every + 1) * a.ckpt_every - t);
      return m;
    };
    // With bf16 inputs a chunk's inputs are requested one period ahead: its
    // decays and betas in I2 of the chunk before (once that chunk's length is
    // voted and its decays are consumed), its keys and queries after that
    // chunk's plane pass, into registers that are free from then on.  The
    // loads are issued on every path, empty past the last chunk, so the
    // compiler's wait counts let each wait cover only the loads it needs
    // (with the requests under a branch, the waits after the join also
    // covered the requests just issued).  Otherwise the decays are requested
    // at the start of the chunk's own I1 and the keys and queries once the
    // decays are consumed.
    // Padding rows lie past the end of the window, where the buffer unit
    // returns zero (their values are replaced anyway).  Each load's lane
    // offset is the previous one plus a row, passed through an opaque copy
    // so that the compiler keeps one offset register instead of sixteen.
    // kPfKQ: keys and queries a period ahead; kPfA: decays and betas too.
    // Raw projections need a chunk's keys and queries at the start of its I1
    // (their norms), so they run only with kPfKQ; their decays are requested
    // at the start of I1, where the norm parts are formed while they arrive
    // (held from I2 on, they pushed the key role past 128 registers).  Prepared
    // fp32 inputs do the same: their keys and queries take twice the
    // registers, and with the decays also held ahead that form spilled.
    constexpr bool kPfKQ = KDA_PREFILL_WS_PREFETCH;
    constexpr bool kPfA = kPfKQ && !PREP && sizeof(TIn) == 2;
    static_assert(!PREP || (kPfKQ && (NK == 8 || NK == 4) && PPW == TPL), "raw projections on the key waves");
    Pair2<float> ra[TPL];
    Pair2<TIn> rk[TPL], rq[TPL];
    float rb = 0.f;       // beta of token `lane`
    float rb_next = 0.f;  // the same for the next chunk (requested a period ahead)
    auto issue_alpha = [&](int t_b, int nn, int lane_, float& rb_dst) {
      const size_t r0 = (tok0 + t_b) * a.H + h;
      // nn = 0 (past the last chunk): an empty window, every load returns 0.
      const rsrc_t wa = make_rsrc(a.alpha + r0 * DK, nn > 0 ? ((nn - 1) * rowk + DK) * 4 : 0);
      int vo = (TPL * (lane_ / PPW) * rowk + CPW * kw + 2 * (lane_ % PPW)) * 4;
#pragma unroll
      for (int i = 0; i < TPL; ++i) {
        asm volatile("" : "+v"(vo));
        ra[i].load(wa, vo);
        vo += rowk * 4;
      }
      {
        const rsrc_t wb = make_rsrc(a.beta + r0, nn > 0 ? ((nn - 1) * a.H + 1) * 4 : 0);
        rb_dst = ld_f32(wb, min(lane_, nn - 1) * a.H * 4, 0);
      }
    };
    auto issue_kq = [&](int t_b, int nn, int lane_) {
      const size_t r0 = (tok0 + t_b) * a.H + h;
      const uint32_t bytes = nn > 0 ? ((nn - 1) * rowk + DK) * sizeof(TIn) : 0;
      const rsrc_t wk = make_rsrc(a.k + r0 * DK, bytes);
      const rsrc_t wq = make_rsrc(a.q + r0 * DK, bytes);
      int vo = (TPL * (lane_ / PPW) * rowk + CPW * kw + 2 * (lane_ % PPW)) * (int)sizeof(TIn);
#pragma unroll
      for (int i = 0; i < TPL; ++i) {
        asm volatile("" : "+v"(vo));
        rk[i].load(wk, vo);
        rq[i].load(wq, vo);
        vo += rowk * (int)sizeof(TIn);
      }
    };
    int t_k = 0;
    int n_nom = n_tok > 0 ? nominal(0) : 0;  // nominal length of the chunk at t_k
    if (kPfA && n_tok > 0) issue_alpha(0, n_nom, threadIdx.x & 63, rb_next);
    if (kPfKQ && n_tok > 0) issue_kq(0, n_nom, threadIdx.x & 63);
    while (t_k < n_tok) {
      int tid = threadIdx.x;
      asm volatile("" : "+v"(tid));
      const int lane = tid & 63, l16 = lane & 15, g = lane >> 4;
      const int p_ = lane % PPW, j = lane / PPW, c0 = CPW * kw + 2 * p_;

      // ---- I1: cumulative decay within the sub-groups, cut vote, alpha_0 ----
      float g0[TPL], g1[TPL];          // running products within each sub-group
      float off0[SGL], off1[SGL];      // decay before each of the lane's sub-groups
      float gn0 = 1.f, gn1 = 1.f;      // G_{n-1} of the two channels
      {
        if constexpr (kPfA)
          rb = rb_next;
        else
          issue_alpha(t_k, n_nom, lane, rb);
        float al0[TPL], al1[TPL];
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
          const bool pad = TPL * j + i >= n_nom;
          float x0 = ra[i].lo(), x1 = ra[i].hi();
          if constexpr (PREP) {
            x0 = sigmoid_f32(a.gate_sign * x0);
            x1 = sigmoid_f32(a.gate_sign * x1);
          }
          al0[i] = pad ? 1.f : x0;  // padding tokens do not decay
          al1[i] = pad ? 1.f : x1;
        }
        if constexpr (PREP) {
          // This wave's part (its 16 key channels) of the squared norms of
          // each token's k and q; lane p of token group j writes token
          // TPL j + p's into the row padding of the Kt / Qt hi planes, and
          // every wave sums the eight parts after the barrier.
          float sk[TPL], sq[TPL];
#pragma unroll
          for (int i = 0; i < TPL; ++i) {
            const float k0 = rk[i].lo(), k1 = rk[i].hi(), q0 = rq[i].lo(), q1 = rq[i].hi();
            sk[i] = lane8_sum(__builtin_fmaf(k0, k0, k1 * k1));
            sq[i] = lane8_sum(__builtin_fmaf(q0, q0, q1 * q1));
          }
          float mk = sk[0], mq = sq[0];
#pragma unroll
          for (int i = 1; i < TPL; ++i)
            if (p_ == i) {
              mk = sk[i];
              mq = sq[i];
            }
          norm_part(TPL * j + p_)[kw] = mk;
          norm_part(CH + TPL * j + p_)[kw] = mq;
        }
        // Token 0's decay goes into S~ = Diag(alpha_0) S, not into G.
        if (j == 0) {
          misc(L::M_A0 + c0) = al0[0];
          misc(L::M_A0 + c0 + 1) = al1[0];
          al0[0] = al1[0] = 1.f;
        }
        float s0[SGL], s1[SGL];
#pragma unroll
        for (int u = 0; u < SGL; ++u) {
          s0[u] = 1.f;
          s1[u] = 1.f;
#pragma unroll
          for (int i = 0; i < TPG; ++i) {
            s0[u] *= al0[TPG * u + i];
            s1[u] *= al1[TPG * u + i];
            g0[TPG * u + i] = s0[u];
            g1[TPG * u + i] = s1[u];
          }
        }
        // Sub-group totals of this channel pair, in sub-group order: sub-group
        // SGL jj + u sits in lane p + PPW jj.
        float t0[NSG], t1[NSG];
#pragma unroll
        for (int jj = 0; jj < NSG / SGL; ++jj)
#pragma unroll
          for (int u = 0; u < SGL; ++u) {
            t0[SGL * jj + u] = __shfl(s0[u], p_ + PPW * jj);
            t1[SGL * jj + u] = __shfl(s1[u], p_ + PPW * jj);
          }
#pragma unroll
        for (int u = 0; u < SGL; ++u) {
          off0[u] = 1.f;
          off1[u] = 1.f;
#pragma unroll
          for (int s = 0; s < NSG; ++s)
            if (s < SGL * j + u) {
              off0[u] *= t0[s];
              off1[u] *= t1[s];
            }
        }
#pragma unroll
        for (int s = 0; s < NSG; ++s) {
          gn0 *= t0[s];
          gn1 *= t1[s];
        }
        // Cut vote: the first token r whose G_r drops below kMinDecay in one
        // of this wave's channels (G is monotone in r), else the nominal length.
        int f = n_nom;
        if (__any(gn0 < kMinDecay || gn1 < kMinDecay)) {
#pragma unroll
          for (int i = TPL - 1; i >= 0; --i) {
            const int r = TPL * j + i;
            if (r < n_nom && (off0[i / TPG] * g0[i] < kMinDecay || off1[i / TPG] * g1[i] < kMinDecay)) f = r;
          }
#pragma unroll
          for (int m = 32; m >= 1; m >>= 1) f = min(f, __shfl_xor(f, m));
        }
        if (lane == 0) vote(kw) = f;
        if constexpr (!kPfKQ) issue_kq(t_k, n_nom, lane);
      }
      __syncthreads();  // B1

      // ---- I2: chunk length; Kt and Qt planes; Kh ----
      int n = n_nom;
      float kh0[TPL], kh1[TPL];
      {
        n = voted_length();
        if (n < n_nom) {
          // The lane holding token n - 1 of each channel pair gives G_{n-1}.
          const int i1 = (n - 1) % TPL, src = p_ + PPW * ((n - 1) / TPL);
          float e0 = 0.f, e1 = 0.f;
#pragma unroll
          for (int i = 0; i < TPL; ++i)
            if (i == i1) {
              e0 = off0[i / TPG] * g0[i];
              e1 = off1[i / TPG] * g1[i];
            }
          gn0 = __shfl(e0, src);
          gn1 = __shfl(e1, src);
        }
        // The next chunk starts where this one ends: its decays and betas go
        // out now (ra is free once the decay pass has run), its keys and
        // queries after the plane pass below.  Past the last chunk the
        // windows are empty: the loads are issued anyway (they return 0 and
        // read nothing), so that the wait counts are the same on every path.
        const int t_next = t_k + n;
        const int n_next = t_next < n_tok ? nominal(t_next) : 0;
        // Lane p forms 1 / |k| and 1 / |q| of token TPL j + p from the key
        // waves' parts (PREP); the plane pass takes each token's pair from the
        // lane that holds it, as it reaches the token.
        float ik = 0.f, iq = 0.f;
        if constexpr (PREP) {
          const float4 a0 = *reinterpret_cast<const float4*>(norm_part(TPL * j + p_));
          const float4 b0 = *reinterpret_cast<const float4*>(norm_part(CH + TPL * j + p_));
          float sk = (a0.x + a0.y) + (a0.z + a0.w), sq = (b0.x + b0.y) + (b0.z + b0.w);
          if constexpr (NK == 8) {
            const float4 a1 = *reinterpret_cast<const float4*>(norm_part(TPL * j + p_) + 4);
            const float4 b1 = *reinterpret_cast<const float4*>(norm_part(CH + TPL * j + p_) + 4);
            sk += (a1.x + a1.y) + (a1.z + a1.w);
            sq += (b1.x + b1.y) + (b1.z + b1.w);
          }
          ik = inv_norm(sk);
          iq = inv_norm(sq);
        }
        if (kPfA) issue_alpha(t_next, n_next, lane, rb_next);
        const int pc = kpos(c0);
        // A full chunk has no padding rows: its copy of the loop drops the tests.
        auto planes = [&](auto full) {
          constexpr bool FULL = decltype(full)::value;
#pragma unroll
          for (int i = 0; i < TPL; ++i) {
            const int tr = TPL * j + i;
            const bool valid = FULL || tr < n;
            float k0 = valid ? rk[i].lo() : 0.f, k1 = valid ? rk[i].hi() : 0.f;
            float q0 = valid ? rq[i].lo() : 0.f, q1 = valid ? rq[i].hi() : 0.f;
            if constexpr (PREP) {
              const float nk = lane8_bcast(ik, i), nq = lane8_bcast(iq, i);  // from lane p = i of the group
              k0 *= nk;
              k1 *= nk;
              q0 *= nq;
              q1 *= nq;
            }
            const float e0 = off0[i / TPG] * g0[i], e1 = off1[i / TPG] * g1[i];  // G of token tr
            const float ie0 = __builtin_amdgcn_rcpf(e0), ie1 = __builtin_amdgcn_rcpf(e1);
            uint32_t hi, lo;
            split2(k0 * e0, k1 * e1, hi, lo);  // Kt
            *reinterpret_cast<uint32_t*>(kq_hi + tr * L::RS_Q + pc) = hi;
            *reinterpret_cast<uint32_t*>(kq_lo + tr * L::RS_Q + pc) = lo;
            split2(q0 * e0, q1 * e1, hi, lo);  // Qt
            *reinterpret_cast<uint32_t*>(kq_hi + (CH + tr) * L::RS_Q + pc) = hi;
            *reinterpret_cast<uint32_t*>(kq_lo + (CH + tr) * L::RS_Q + pc) = lo;
            kh0[i] = valid ? k0 * ie0 : 0.f;  // padding rows: zero (their G may be 0)
            kh1[i] = valid ? k1 * ie1 : 0.f;
            split2(kh0[i], kh1[i], hi, lo);  // Kh
            *reinterpret_cast<uint32_t*>(kh_hi + tr * L::RS_K + pc) = hi;
            *reinterpret_cast<uint32_t*>(kh_lo + tr * L::RS_K + pc) = lo;
          }
        };
        if (n == CH)
          planes(std::true_type{});
        else
          planes(std::false_type{});
        if (kPfKQ) issue_kq(t_next, n_next, lane);
      }
      __syncthreads();  // B2

      // ---- I3: Kb^T, beta, G; next loads; A and P tiles; diagonal blocks ----
      constexpr int KT = 16 - NV * VT;  // tiles of the key waves other than the diagonal blocks
      static_assert(NV <= 10, "value waves take P tiles only");
      static_assert(NK >= NB, "at most one diagonal block per key wave");
      const bool has_diag = kw < NB;
      constexpr int MAXT = 1 + (KT + NK - 1) / NK;  // slots per key wave
      f32x4_t at[MAXT];
      float xinv[16];
      {
        // Kb = Kh G_{n-1}, into the transposed planes two tokens at a time.
#pragma unroll
        for (int i = 0; i < TPL; i += 2) {
          uint32_t bh0, bl0, bh1, bl1;
          split2(kh0[i] * gn0, kh0[i + 1] * gn0, bh0, bl0);  // channel c0, tokens i and i + 1
          split2(kh1[i] * gn1, kh1[i + 1] * gn1, bh1, bl1);
          const int pt = kpos(TPL * j + i);  // storage column of the token pair
          *reinterpret_cast<uint32_t*>(kb_hi + c0 * L::RS_C + pt) = bh0;
          *reinterpret_cast<uint32_t*>(kb_lo + c0 * L::RS_C + pt) = bl0;
          *reinterpret_cast<uint32_t*>(kb_hi + (c0 + 1) * L::RS_C + pt) = bh1;
          *reinterpret_cast<uint32_t*>(kb_lo + (c0 + 1) * L::RS_C + pt) = bl1;
        }
        if (j == 0) {
          misc(L::M_GN + c0) = gn0;
          misc(L::M_GN + c0 + 1) = gn1;
        }
        const float beta_l = lane < n ? (PREP ? sigmoid_f32(rb) : rb) : 0.f;  // beta of token `lane` (padding: 0)
        if (kw == 0) misc(L::M_BETA + lane) = beta_l;

        // Slot 0 of key wave kw is diagonal block kw of A, the other slots
        // its share of the remaining tiles.  One loop for every key wave (two
        // differently shaped branches of matrix products would be merged and
        // run by all of them).
#pragma unroll
        for (int s = 0; s < MAXT; ++s) {
          const int i = s == 0 ? 16 + kw : kw + NK * (s - 1);
          at[s] = zero4;
          if (s == 0 ? has_diag : i < KT) {
            bool is_a;
            int mt, nt;
            ws_tile(i, is_a, mt, nt);
            const int row = (is_a ? 0 : CH) + 16 * mt + l16;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
              const int k0_ = 32 * kb + 4 * g;
              at[s] = mfma3(plane_op2(kh_hi, kh_lo, 16 * nt + l16, L::RS_K, k0_),
                            plane_op2(kq_hi, kq_lo, row, L::RS_Q, k0_), at[s]);
            }
          }
        }
        if (has_diag) {
          // Diagonal block kw of A (fp32, transposed, into this wave's own part
          // of the diagonal region) and its inverse: lane cc (every group of 16
          // lanes does the same) forms column cc by right-looking elimination.
          {
            const float bta = __shfl(beta_l, 16 * kw + l16);  // beta of this lane's row token
            float* aj = adiag + kw * L::DSTRIDE;
#pragma unroll
            for (int e = 0; e < 4; ++e) aj[(4 * g + e) * L::RS_D + l16] = 4 * g + e < l16 ? at[0][e] * bta : 0.f;
          }
          const int cc = lane & 15;
          const float* aj = adiag + kw * L::DSTRIDE;
#pragma unroll
          for (int r = 0; r < 16; ++r) xinv[r] = r == cc ? 1.f : 0.f;
#pragma unroll
          for (int i = 0; i < 15; ++i) {
#pragma unroll
            for (int q = (i + 1) / 4; q < 4; ++q) {
              const float4 c4 = *reinterpret_cast<const float4*>(aj + i * L::RS_D + 4 * q);
              const float cv[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (4 * q + e > i) xinv[4 * q + e] = __builtin_fmaf(-cv[e], xinv[i], xinv[4 * q + e]);
            }
          }
        }
      }
      __syncthreads();  // B3

      // ---- I4: A and P tiles into M and P, the inverses into M's diagonal ----
      {
#pragma unroll
        for (int s = 1; s < MAXT; ++s) {
          const int i = kw + NK * (s - 1);
          if (i < KT) {
            bool is_a;
            int mt, nt;
            ws_tile(i, is_a, mt, nt);
            const int tr = 16 * mt + l16;   // row token of this lane
            const int ct0 = 16 * nt + 4 * g;  // its first column token
            float v4[4];
            if (is_a) {
              const float bta = misc(L::M_BETA + tr);
#pragma unroll
              for (int e = 0; e < 4; ++e) v4[e] = ct0 + e < tr ? at[s][e] * bta : 0.f;
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e) v4[e] = ct0 + e <= tr ? at[s][e] : 0.f;
            }
            uint32_t h0, l0, h1, l1;
            split2(v4[0], v4[1], h0, l0);
            split2(v4[2], v4[3], h1, l1);
            bf16_t* dh = (is_a ? m_hi : p_hi) + tr * L::RS_C + kpos(ct0);
            bf16_t* dl = (is_a ? m_lo : p_lo) + tr * L::RS_C + kpos(ct0);
            *reinterpret_cast<uint2*>(dh) = make_uint2(h0, h1);
            *reinterpret_cast<uint2*>(dl) = make_uint2(l0, l1);
          }
        }
        // Upper tiles inside a 32-token k block are read against zero
        // operands by the P E product and the block solve: zero them.
        if (kw < NB / 2) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int tr = 32 * kw + 4 * g + r, tc = 32 * kw + 16 + l16;
            p_hi[tr * L::RS_C + kpos(tc)] = 0;
            p_lo[tr * L::RS_C + kpos(tc)] = 0;
            m_hi[tr * L::RS_C + kpos(tc)] = 0;
            m_lo[tr * L::RS_C + kpos(tc)] = 0;
          }
        }
        // The inverse of diagonal block kw: every group of 16 lanes holds all
        // of it (lane cc column cc); group q writes rows 4 q .. 4 q + 3.
        const int cc = lane & 15, q = lane >> 4;
#pragma unroll
        for (int e = 0; e < 4 && kw < NB; ++e) {
          float x = xinv[e];
#pragma unroll
          for (int qq = 1; qq < 4; ++qq)
            if (q == qq) x = xinv[4 * qq + e];
          __bf16 lo;
          const __bf16 hi = split_hi(x, lo);
          const int idx = (16 * kw + 4 * q + e) * L::RS_C + kpos(16 * kw + cc);
          m_hi[idx] = __builtin_bit_cast(bf16_t, hi);
          m_lo[idx] = __builtin_bit_cast(bf16_t, lo);
        }
      }
      __syncthreads();  // B4
      t_k = __builtin_amdgcn_readfirstlane(t_k + n);
      if (t_k < n_tok) n_nom = nominal(t_k);
    }
    // The value waves' last period (solve, outputs and state update of the
    // last chunk) has its four barriers too.
    if (n_tok > 0)
      for (int i = 0; i < 4; ++i) __syncthreads();
  }
}

}  // namespace
}  // namespace kda
