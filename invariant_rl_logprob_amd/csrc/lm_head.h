// What every lm-head kernel shares: the K order of a vocabulary tile and the tile's
// softmax partials, so the bf16 and the W8A8 heads reduce their logits identically.
#pragma once

#include "common.h"

namespace ril {

// Every output column accumulates its K steps in the order r, r+1, ..., nk-1, 0, ..., r-1
// with r = (37 * tile) mod nk: one order per column, chosen by the column's tile alone
// (never by the batch, M or the grid), which spreads the tiles' concurrent weight reads
// over the HBM channels instead of having every tile read the same K offset at once.
__device__ __forceinline__ int lm_rot(int tile, int nk) { return (37 * tile) % nk; }

// S11 epilogue: the logits acc of one 256-column vocabulary tile (wave w owns columns
// 64w .. 64w+63 as four 16-column MFMA blocks, column 16nb + lane%16; rows in the MFMA
// output layout, 16*MB per workgroup) become, per row, the tile max and
//   s_t = ((S_0 + S_1) + S_2) + S_3,  S_w = xor-butterfly over 16 lanes of
//         (((e_0 + e_1) + e_2) + e_3),  e = exp2((l - max) * log2 e)
// written to part[row, tile] as (max, s_t), and the target's logit if the target falls
// in the tile.  Rows past M are computed and dropped: they never touch a row's tree.
template <int MB>
__device__ __forceinline__ void lm_tile_epilogue(const f32x4 (&acc)[MB][4], float (&red)[4][16 * MB], int tile,
                                                 int m0, int M, int V, const int32_t *__restrict__ target,
                                                 float *__restrict__ part, float *__restrict__ tgt_logit,
                                                 int n_vt) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int grp = lane >> 4, r16 = lane & 15;
  const int c0 = tile * kVocabTile + wave * 64;
  bool cval[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) cval[nb] = (c0 + 16 * nb + r16) < V;
  // tile max per row
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float mx = neg_inf();
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) mx = fmaxf(mx, cval[nb] ? acc[mb][nb][i] : neg_inf());
      mx = max16(mx);
      if (r16 == 0) red[wave][16 * mb + 4 * grp + i] = mx;
    }
  }
  __syncthreads();
  float mt[MB][4];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * mb + 4 * grp + i;
      mt[mb][i] = fmaxf(fmaxf(red[0][r], red[1][r]), fmaxf(red[2][r], red[3][r]));
    }
  __syncthreads();
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float e[4];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        e[nb] = cval[nb] ? exp2f_hw((acc[mb][nb][i] - mt[mb][i]) * kLog2e) : 0.f;
      float sm = ((e[0] + e[1]) + e[2]) + e[3];
      sm = sum16(sm);
      if (r16 == 0) red[wave][16 * mb + 4 * grp + i] = sm;
    }
  }
  __syncthreads();
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * mb + 4 * grp + i;
      const int row = m0 + r;
      if (row >= M) continue;
      if (wave == 0 && r16 == 0) {
        const float st = ((red[0][r] + red[1][r]) + red[2][r]) + red[3][r];
        part[((long)row * n_vt + tile) * 2] = mt[mb][i];
        part[((long)row * n_vt + tile) * 2 + 1] = st;
      }
      const int tg = target[row];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        if (cval[nb] && c0 + 16 * nb + r16 == tg) tgt_logit[row] = acc[mb][nb][i];
    }
  }
}

}  // namespace ril
