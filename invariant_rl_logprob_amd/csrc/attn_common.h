// Pieces of the attention arithmetic shared by every attention kernel (GQA and MLA,
// decode and prefill), so that one query row's value is produced by one sequence of
// instructions whichever kernel computes it.
#pragma once

#include <utility>

#include "common.h"

namespace ril {

// Zero the bf16 elements j >= n_valid of a lane's 8-element vector.
__device__ __forceinline__ u32x4 keep_first(u32x4 v, int n_valid) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t lo = (2 * w < n_valid) ? 0x0000ffffu : 0u;
    const uint32_t hi = (2 * w + 1 < n_valid) ? 0xffff0000u : 0u;
    v[w] &= (lo | hi);
  }
  return v;
}

// Offset (elements) of K(t, d) inside one 16-token page block laid out so that an
// MFMA A-operand of S^T = K Q^T is one 16-byte load per lane:
//   (d/32)*512 + ((d%32)/8)*128 + ((t%8)/4)*64 + (t/8)*32 + (t%4)*8 + d%8
__device__ __forceinline__ int k_page_offset(int t, int d) {
  return (d >> 5) * 512 + ((d & 31) >> 3) * 128 + ((t & 7) >> 2) * 64 + (t >> 3) * 32 + (t & 3) * 8 + (d & 7);
}

// The online-softmax update of one 64-token tile for this lane's column.
//   s[mb][i]: fp32 q.k of token tile_start + 32(mb/2) + 8(lane/16) + 4(mb%2) + i
//             (the S^T MFMA output layout, M-block mb = 2kc + h)
//   pos     : the column's query position (tokens after it are masked)
// Produces the bf16 P^T operands of the two 32-token PV steps (k-slot j of lane group
// g <-> token 32kc + 8g + j), the rescale factor alpha = exp2(m - m'), and the new (m, l).
// MASK = false: the caller knows every token of the tile is at or before pos (the mask
// would keep every score), so the selects are left out; the values are the same.
template <bool MASK = true>
__device__ __forceinline__ void tile_softmax(f32x4 (&s)[4], int tile_start, int pos, float cscale,
                                             float m, float l, bf16x8 (&pop)[2], float &alpha,
                                             float &m_new, float &l_new) {
  const int grp = (threadIdx.x & 63) >> 4;
  float tmax = neg_inf();
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = tile_start + 32 * (mb >> 1) + 8 * grp + 4 * (mb & 1) + i;
      const float x = s[mb][i] * cscale;
      s[mb][i] = (!MASK || tok <= pos) ? x : neg_inf();
      tmax = fmaxf(tmax, s[mb][i]);
    }
  }
  tmax = max_groups(tmax);
  m_new = fmaxf(m, tmax);
  const float m_use = (m_new == neg_inf()) ? 0.f : m_new;
  alpha = exp2f_hw(m - m_use);
  float rs = 0.f;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) s[mb][i] = exp2f_hw(s[mb][i] - m_use);
    const float r = ((s[mb][0] + s[mb][1]) + s[mb][2]) + s[mb][3];
    rs = (mb == 0) ? r : rs + r;
  }
  rs = sum_groups(rs);
  l_new = __builtin_fmaf(l, alpha, rs);
#pragma unroll
  for (int kc = 0; kc < 2; ++kc) {
    u32x4 w;
    w[0] = pack2(s[2 * kc][0], s[2 * kc][1]);
    w[1] = pack2(s[2 * kc][2], s[2 * kc][3]);
    w[2] = pack2(s[2 * kc + 1][0], s[2 * kc + 1][1]);
    w[3] = pack2(s[2 * kc + 1][2], s[2 * kc + 1][3]);
    pop[kc] = as_bf16x8(w);
  }
}

// merged <- merge(merged, split): the one merge rule of every split-KV attention.
template <int N>
__device__ __forceinline__ void merge_state(float &M, float &L, float (&O)[N], float ms, float ls,
                                            const float (&os)[N]) {
  const float mn = fmaxf(M, ms);
  const float a = exp2f_hw(M - mn);
  const float b = exp2f_hw(ms - mn);
  L = __builtin_fmaf(L, a, ls * b);
#pragma unroll
  for (int j = 0; j < N; ++j) O[j] = __builtin_fmaf(O[j], a, os[j] * b);
  M = mn;
}

// Split merge over stored fp32 partials, split 0 first then left to right; lane owns
// PER consecutive dims.  Writes bf16(O / L).  Shared by every decode-style attention.
// The loads of CH splits are issued together before they are folded (in the same order),
// so a row's splits cost one memory latency per CH splits rather than one each.
template <int D>
__device__ __forceinline__ void merge_partials(const float *__restrict__ part_o,
                                               const float *__restrict__ part_ml, long base, int ns,
                                               bf16_t *__restrict__ op) {
  constexpr int PER = D / 64;
  constexpr int CH = PER <= 2 ? 8 : 4;
  const int lane = threadIdx.x & 63;
  float M = 0.f, L = 0.f;
  float O[PER];
  for (int s0 = 0; s0 < ns; s0 += CH) {
    float ms[CH], ls[CH], os[CH][PER];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const long s = base + min(s0 + c, ns - 1);  // past the last split: a repeat, not folded
      ms[c] = part_ml[s * 2];
      ls[c] = part_ml[s * 2 + 1];
#pragma unroll
      for (int j = 0; j < PER; ++j) os[c][j] = part_o[s * D + lane * PER + j];
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      if (s0 + c >= ns) break;
      if (s0 + c == 0) {
        M = ms[0];
        L = ls[0];
#pragma unroll
        for (int j = 0; j < PER; ++j) O[j] = os[0][j];
      } else {
        merge_state<PER>(M, L, O, ms[c], ls[c], os[c]);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) op[lane * PER + j] = f2bf(__fdiv_rn(O[j], L));
}

// ---------------------------------------------------------------------------
// The tile routine shared by decode and prefill
// ---------------------------------------------------------------------------

// Half of a 64-token tile in MFMA operand registers (D/8 16-byte values per lane):
// either its K half or its V half.
//   K half, r[mb*(D/32) + c]  : A operand of S^T = K Q^T for M-block mb = 2kc + h,
//                               dims 32c .. 32c+31; row r <-> token 32kc + 8(r/4) + 4h + r%4
//   V half, r[kc*(D/16) + db] : A operand of o^T += V^T P^T for 32-token step kc, dims
//                               16db .. 16db+15; k-slot 8(lane/16) + j <-> token 32kc + 8(lane/16) + j
template <int D>
struct Half {
  u32x4 r[D / 8];
};

// Operand loads from global memory or from an LDS copy of the same page blocks.
struct FromGlobal {
  static __device__ __forceinline__ u32x4 ld(const bf16_t *p) { return ld16(p); }
};
// Global loads with the nontemporal (streaming) cache policy, for data read once per call.
struct NtGlobal {
  static __device__ __forceinline__ u32x4 ld(const bf16_t *p) {
    return __builtin_nontemporal_load((const u32x4 __attribute__((address_space(1))) *)(p));
  }
};
struct FromLds {
  static __device__ __forceinline__ u32x4 ld(const bf16_t *p) {
    return *(const __attribute__((address_space(3))) u32x4 *)(p);
  }
};
// LDS reads the compiler does not track: the waitcnt pass would otherwise make every LDS
// read wait for all direct-to-LDS copies in flight (it cannot tell which LDS bytes they
// write), serialising the copy pipeline.  The caller orders them after the copies they
// read (its own vmcnt wait + barrier) and calls lds_settle before using the values.
struct FromLdsUntracked {
  static __device__ __forceinline__ u32x4 ld(const bf16_t *p) {
    u32x4 r;
    const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) bf16_t *)p;
    asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(a));
    return r;
  }
};

// ---------------------------------------------------------------------------
// FP8 (OCP E4M3) KV pages (Bitwise-consistent RL post, section 4.2: FP8 storage, one write
// path, one dequantizing read shared by every phase).  A page block (16 tokens, one kv
// head) is 32*D bytes: K then V, 16*D bytes each, one byte per value, laid out so that a
// 16-byte load holds two MFMA operands:
//   K (t, d) -> 2*((d/64)*512 + ((d%32)/8)*128 + ((t%8)/4)*64 + (t/8)*32 + (t%4)*8)
//               + ((d/32)%2)*8 + d%8                 (chunks c = 2j and 2j+1 side by side)
//   V (t, d) -> 16*D + (t/8)*8*D + ((d/32)*16 + d%16)*16 + ((d/16)%2)*8 + t%8
//                                                    (dims d and d+16 side by side)
// The stored code is e4m3(x * 2^-s) (nearest even, magnitudes past 448 saturating, NaN
// kept with its sign) with s a model constant per tensor; the value read back is
// code * 2^s, which bf16 holds exactly, so dequantization adds no rounding (the 2^s is
// applied outside the MFMA operands: see fp8_operand).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int k_page_offset8(int t, int d) {
  return 2 * ((d >> 6) * 512 + ((d & 31) >> 3) * 128 + ((t & 7) >> 2) * 64 + (t >> 3) * 32 + (t & 3) * 8) +
         ((d >> 5) & 1) * 8 + (d & 7);
}
__device__ __forceinline__ int v_page_offset8(int t, int d, int D) {
  return 16 * D + (t >> 3) * 8 * D + ((d >> 5) * 16 + (d & 15)) * 16 + ((d >> 4) & 1) * 8 + (t & 7);
}

// Eight E4M3 codes (two words) -> one bf16 MFMA operand holding the codes' values (exact:
// the fp32 decode is exact for every code and the values are bf16 values).
//
// The scales 2^s are not applied here.  K's multiplies the softmax constant (scores =
// (q . code) * (c * 2^s_k)) and V's multiplies the fp32 output state once, before it is
// stored (decode partials) or divided (prefill).  A power of two commutes with every fp32
// rounding between those points, so this equals attending over code * 2^s (outside the
// subnormal and overflow ranges of fp32), and prefill and decode fold them identically.
// One v_cvt_scalef32_pk_bf16_fp8 per two codes, scale 1: the codes' values land in bf16
// directly (checked on every code, NaNs included, against decoding to fp32 and rounding to
// bf16: the same bits; half the instructions).
__device__ __forceinline__ u32x4 fp8_operand(uint32_t w0, uint32_t w1) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true));
  return r;
}

// Raw FP8 half-tile: D/16 16-byte values per lane, each two operands of the bf16 Half.
//   K: r[mb*(D/64) + j] = operands (mb, c = 2j) and (mb, 2j+1)
//   V: r[kc*(D/32) + j] = operands (kc, db = 2j) and (kc, 2j+1)
template <int D>
struct Half8 {
  u32x4 r[D / 16];
};

template <int D>
__device__ __forceinline__ void dequant_k(const Half8<D> &raw, Half<D> &t) {
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int j = 0; j < D / 64; ++j) {
      const u32x4 w = raw.r[mb * (D / 64) + j];
      t.r[mb * (D / 32) + 2 * j] = fp8_operand(w[0], w[1]);
      t.r[mb * (D / 32) + 2 * j + 1] = fp8_operand(w[2], w[3]);
    }
}

template <int D>
__device__ __forceinline__ void dequant_v(const Half8<D> &raw, Half<D> &t) {
#pragma unroll
  for (int kc = 0; kc < 2; ++kc)
#pragma unroll
    for (int j = 0; j < D / 32; ++j) {
      const u32x4 w = raw.r[kc * (D / 32) + j];
      t.r[kc * (D / 16) + 2 * j] = fp8_operand(w[0], w[1]);
      t.r[kc * (D / 16) + 2 * j + 1] = fp8_operand(w[2], w[3]);
    }
}

// pg8[k]: byte address of the FP8 K block of the tile's k-th page (V at +16*D bytes).
template <int D, typename Mem = FromGlobal>
__device__ __forceinline__ void load_k8(Half8<D> &t, const uint8_t *const (&pg8)[4]) {
  const int lane = threadIdx.x & 63;
  const int grp = lane >> 4, r16 = lane & 15;
  const int rq = r16 >> 2, ri = r16 & 3;
#pragma unroll
  for (int kc = 0; kc < 2; ++kc)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint8_t *kb = pg8[2 * kc + (rq >> 1)] + 2 * (grp * 128 + h * 64 + (rq & 1) * 32 + ri * 8);
#pragma unroll
      for (int j = 0; j < D / 64; ++j)
        t.r[(2 * kc + h) * (D / 64) + j] = Mem::ld(reinterpret_cast<const bf16_t *>(kb + j * 1024));
    }
}

template <int D, typename Mem = FromGlobal>
__device__ __forceinline__ void load_v8(Half8<D> &t, const uint8_t *const (&pg8)[4]) {
  const int lane = threadIdx.x & 63;
  const int grp = lane >> 4, r16 = lane & 15;
#pragma unroll
  for (int kc = 0; kc < 2; ++kc) {
    const uint8_t *vb = pg8[2 * kc + (grp >> 1)] + 16 * D + (grp & 1) * (8 * D) + r16 * 16;
#pragma unroll
    for (int j = 0; j < D / 32; ++j) t.r[kc * (D / 32) + j] = Mem::ld(reinterpret_cast<const bf16_t *>(vb + j * 256));
  }
}

// pg[k]: K block of the tile's k-th page (its V block follows at +16*D).
template <int D, typename Mem = FromGlobal>
__device__ __forceinline__ void load_k(Half<D> &t, const bf16_t *const (&pg)[4]) {
  const int lane = threadIdx.x & 63;
  const int grp = lane >> 4, r16 = lane & 15;
  const int rq = r16 >> 2, ri = r16 & 3;
#pragma unroll
  for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const bf16_t *kb = pg[2 * kc + (rq >> 1)] + grp * 128 + h * 64 + (rq & 1) * 32 + ri * 8;
#pragma unroll
      for (int c = 0; c < D / 32; ++c) t.r[(2 * kc + h) * (D / 32) + c] = Mem::ld(kb + c * 512);
    }
  }
}

template <int D, typename Mem = FromGlobal>
__device__ __forceinline__ void load_v(Half<D> &t, const bf16_t *const (&pg)[4]) {
  const int lane = threadIdx.x & 63;
  const int grp = lane >> 4, r16 = lane & 15;
#pragma unroll
  for (int kc = 0; kc < 2; ++kc) {
    const bf16_t *vb = pg[2 * kc + (grp >> 1)] + 16 * D + (grp & 1) * (8 * D) + r16 * 8;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) t.r[kc * (D / 16) + db] = Mem::ld(vb + db * 128);
  }
}

// Wait for this wave's untracked LDS reads; each value passes through an empty asm after
// the wait, so no use of it can be scheduled before the wait.
template <int D>
__device__ __forceinline__ void lds_settle(Half<D> &t) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: );
#pragma unroll
  for (int i = 0; i < D / 8; ++i) asm volatile("" : "+v"(t.r[i]));
}

// First half of the tile update for the 16 query rows (MFMA columns) of this wave:
// scores from the K half, then the online-softmax step (tile_softmax).
//   qop : B operand of S^T = K Q^T (lane: column lane%16, dims 32c + 8(lane/16) ..)
//   pos : this lane's column's query position (-1: padding column)
// The q.k MFMA chains of one tile: s[mb] = sum over c = 0, 1, ... of K_mb,c Q_c^T.
template <int D>
__device__ __forceinline__ void attn_score_mfma(const Half<D> &k, const bf16x8 (&qop)[D / 32], f32x4 (&s)[4]) {
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < D / 32; ++c) acc = mfma(as_bf16x8(k.r[mb * (D / 32) + c]), qop[c], acc);
    s[mb] = acc;
  }
}

// The same chains from an FP8 half-tile, each operand dequantized (fp8_operand, exact)
// just before its MFMA: operand (mb, c = 2j) is words 0-1 of raw r[mb*(D/64) + j], c = 2j+1
// words 2-3 -- the operands dequant_k would produce, in the same order, without holding a
// dequantized tile in registers.
template <int D>
__device__ __forceinline__ void attn_score_mfma8(const Half8<D> &k, const bf16x8 (&qop)[D / 32], f32x4 (&s)[4]) {
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < D / 64; ++j) {
      const u32x4 w = k.r[mb * (D / 64) + j];
      acc = mfma(as_bf16x8(fp8_operand(w[0], w[1])), qop[2 * j], acc);
      acc = mfma(as_bf16x8(fp8_operand(w[2], w[3])), qop[2 * j + 1], acc);
    }
    s[mb] = acc;
  }
}

template <int D, bool MASK = true>
__device__ __forceinline__ void attn_scores(const Half<D> &k, int tile_start, const bf16x8 (&qop)[D / 32],
                                            int pos, float cscale, float m, float l, bf16x8 (&pop)[2],
                                            float &alpha, float &m_new, float &l_new) {
  f32x4 s[4];
  attn_score_mfma<D>(k, qop, s);
  tile_softmax<MASK>(s, tile_start, pos, cscale, m, l, pop, alpha, m_new, l_new);
}

// Second half: o = o * alpha + MFMA(bf16 P, V), two 32-token steps in token order.
//   vbound : V values of tokens >= vbound are read as 0 (beyond any column's context)
// State per lane = its column's (m, l) and o^T[16db + 4(lane/16) + i].
// MAYBE_INACTIVE: some column may have pos < tile_start; such columns keep their state.
// VMASK = false: the caller knows the tile ends at or before vbound, so no V value needs
// zeroing.
template <int D, bool MAYBE_INACTIVE, bool VMASK, typename VOp>
__device__ __forceinline__ void attn_values_op(VOp vop, int tile_start, int pos, int vbound,
                                               const bf16x8 (&pop)[2], float alpha, float m_new, float l_new,
                                               float &m, float &l, f32x4 (&o)[D / 16]) {
  const int grp = (threadIdx.x & 63) >> 4;
  // o is rescaled and accumulated in place on every path (one register set for o, so
  // the callers' variants need no copies); inactive columns get their old state back.
  f32x4 keep[D / 16];
  if (MAYBE_INACTIVE) {
#pragma unroll
    for (int db = 0; db < D / 16; ++db) keep[db] = o[db];
  }
#pragma unroll
  for (int db = 0; db < D / 16; ++db) o[db] = o[db] * alpha;
#pragma unroll
  for (int kc = 0; kc < 2; ++kc) {
    const int n_valid = vbound - (tile_start + 32 * kc + 8 * grp);
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      u32x4 vv = vop(kc, db);
      if (VMASK && n_valid < 8) vv = keep_first(vv, n_valid);
      o[db] = mfma(as_bf16x8(vv), pop[kc], o[db]);
    }
  }
  if (MAYBE_INACTIVE) {
    const bool act = tile_start <= pos;
    m = act ? m_new : m;
    l = act ? l_new : l;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
#pragma unroll
      for (int i = 0; i < 4; ++i) o[db][i] = act ? o[db][i] : keep[db][i];
    }
  } else {
    m = m_new;
    l = l_new;
  }
}

template <int D, bool MAYBE_INACTIVE, bool VMASK = true>
__device__ __forceinline__ void attn_values(const Half<D> &v, int tile_start, int pos, int vbound,
                                            const bf16x8 (&pop)[2], float alpha, float m_new, float l_new,
                                            float &m, float &l, f32x4 (&o)[D / 16]) {
  attn_values_op<D, MAYBE_INACTIVE, VMASK>([&](int kc, int db) { return v.r[kc * (D / 16) + db]; }, tile_start,
                                           pos, vbound, pop, alpha, m_new, l_new, m, l, o);
}

// The same from an FP8 half-tile: operand (kc, db) is dequantized just before its MFMA
// (db = 2j: words 0-1 of raw r[kc*(D/32) + j], db = 2j+1: words 2-3, as dequant_v lays them).
template <int D, bool MAYBE_INACTIVE, bool VMASK = true>
__device__ __forceinline__ void attn_values8(const Half8<D> &v, int tile_start, int pos, int vbound,
                                             const bf16x8 (&pop)[2], float alpha, float m_new, float l_new,
                                             float &m, float &l, f32x4 (&o)[D / 16]) {
  attn_values_op<D, MAYBE_INACTIVE, VMASK>(
      [&](int kc, int db) {
        const u32x4 w = v.r[kc * (D / 32) + (db >> 1)];
        return (db & 1) ? fp8_operand(w[2], w[3]) : fp8_operand(w[0], w[1]);
      },
      tile_start, pos, vbound, pop, alpha, m_new, l_new, m, l, o);
}

// One whole 64-token tile update (both halves).
template <int D, bool MAYBE_INACTIVE>
__device__ __forceinline__ void attn_tile(const Half<D> &k, const Half<D> &v, int tile_start,
                                          const bf16x8 (&qop)[D / 32], int pos, int vbound,
                                          float cscale, float &m, float &l, f32x4 (&o)[D / 16]) {
  bf16x8 pop[2];
  float alpha, m_new, l_new;
  attn_scores<D>(k, tile_start, qop, pos, cscale, m, l, pop, alpha, m_new, l_new);
  attn_values<D, MAYBE_INACTIVE>(v, tile_start, pos, vbound, pop, alpha, m_new, l_new, m, l, o);
}

template <int D>
__device__ __forceinline__ void load_qop(bf16x8 (&qop)[D / 32], const bf16_t *qrow, bool ok) {
  const int grp = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    u32x4 v = ld16(qrow + c * 32 + grp * 8);
    if (!ok) v = u32x4{0u, 0u, 0u, 0u};
    qop[c] = as_bf16x8(v);
  }
}

// K block base of page slot `idx` of the split (0 .. 4*tiles-1): a wave-uniform readlane.
__device__ __forceinline__ const bf16_t *page_base(const bf16_t *pool, int pid_lane, int idx, int Hkv,
                                                   int g, int D) {
  const int p = __builtin_amdgcn_readlane(pid_lane, idx);
  return pool + ((long)p * Hkv + g) * (32 * D);
}

template <int D>
__device__ __forceinline__ void tile_pages(const bf16_t *(&pg)[4], const bf16_t *pool, int pid_lane,
                                           int tile, int Hkv, int g) {
#pragma unroll
  for (int k = 0; k < 4; ++k) pg[k] = page_base(pool, pid_lane, 4 * tile + k, Hkv, g, D);
}


}  // namespace ril
