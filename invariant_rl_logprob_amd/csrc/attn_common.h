// Pieces of the attention arithmetic shared by every attention kernel (GQA and MLA,
// decode and prefill), so that one query row's value is produced by one sequence of
// instructions whichever kernel computes it.
#pragma once

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
      s[mb][i] = (tok <= pos) ? x : neg_inf();
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
template <int D>
__device__ __forceinline__ void merge_partials(const float *__restrict__ part_o,
                                               const float *__restrict__ part_ml, long base, int ns,
                                               bf16_t *__restrict__ op) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x & 63;
  float M = part_ml[base * 2], L = part_ml[base * 2 + 1];
  float O[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) O[j] = part_o[base * D + lane * PER + j];
  for (int s = 1; s < ns; ++s) {
    float os[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) os[j] = part_o[(base + s) * D + lane * PER + j];
    merge_state<PER>(M, L, O, part_ml[(base + s) * 2], part_ml[(base + s) * 2 + 1], os);
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) op[lane * PER + j] = f2bf(__fdiv_rn(O[j], L));
}

}  // namespace ril
