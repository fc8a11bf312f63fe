// What every lm-head kernel shares: the K order of a vocabulary tile and the tile's
// softmax partials, so the bf16 and the W8A8 heads reduce their logits identically.
#pragma once

#include "common.h"

namespace ril {

// Every output column accumulates its K steps in the order r, r+1, ..., nk-1, 0, ..., r-1
// with r = (37 * (tile / 8)) mod nk: one order per column, chosen by the column's tile
// alone (never by the batch, M or the grid).  Groups of 8 consecutive vocabulary tiles
// share r, so workgroups on 8 tiles of a group read the same activation K slice at the same
// time (one fetch into L2 serves all of them); different groups start at different K
// offsets, which spreads the concurrent weight reads of a decode step over the HBM
// channels instead of having every tile read the same K offset at once.
__device__ __forceinline__ int lm_rot(int tile, int nk) { return (37 * (tile >> 3)) % nk; }

// S11 epilogue: the logits acc of one 256-column vocabulary tile (the wave of column group
// cg owns columns 64cg .. 64cg+63 as four 16-column MFMA blocks, column 16nb + lane%16;
// rows in the MFMA output layout, 16*MB from m0; the four waves of a row group share red:
// red[0] holds the per-wave row maxima, red[1] the per-wave row sums) become, per row,
// the tile max and
//   s_t = ((S_0 + S_1) + S_2) + S_3,  S_w = xor-butterfly over 16 lanes of
//         (((e_0 + e_1) + e_2) + e_3),  e = exp2((l - max) * log2 e)
// written to part[row, tile] as (max, s_t), and the target's logit if the target falls
// in the tile.  Rows past M are computed and dropped: they never touch a row's tree.
// The tile max is read back from red where it is needed rather than held per row, which
// keeps the epilogue's registers few at large MB.
// Every wave of the workgroup calls it (it synchronises the workgroup).
template <int MB>
__device__ __forceinline__ void lm_tile_epilogue(const f32x4 (&acc)[MB][4], float (&red)[2][4][16 * MB], int cg,
                                                 int tile, int m0, int M, int V, const int32_t *__restrict__ target,
                                                 float *__restrict__ part, float *__restrict__ tgt_logit,
                                                 int n_vt) {
  const int lane = threadIdx.x & 63;
  const int grp = lane >> 4, r16 = lane & 15;
  const int c0 = tile * kVocabTile + cg * 64;
  bool cval[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) cval[nb] = (c0 + 16 * nb + r16) < V;
  auto tile_max = [&](int r) { return fmaxf(fmaxf(red[0][0][r], red[0][1][r]), fmaxf(red[0][2][r], red[0][3][r])); };
  // this wave's max per row
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float mx = neg_inf();
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) mx = fmaxf(mx, cval[nb] ? acc[mb][nb][i] : neg_inf());
      mx = max16(mx);
      if (r16 == 0) red[0][cg][16 * mb + 4 * grp + i] = mx;
    }
  }
  __syncthreads();
  // this wave's sum per row against the tile max
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float mt = tile_max(16 * mb + 4 * grp + i);
      float e[4];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) e[nb] = cval[nb] ? exp2f_hw((acc[mb][nb][i] - mt) * kLog2e) : 0.f;
      float sm = ((e[0] + e[1]) + e[2]) + e[3];
      sm = sum16(sm);
      if (r16 == 0) red[1][cg][16 * mb + 4 * grp + i] = sm;
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
      if (cg == 0 && r16 == 0) {
        const float st = ((red[1][0][r] + red[1][1][r]) + red[1][2][r]) + red[1][3][r];
        part[((long)row * n_vt + tile) * 2] = tile_max(r);
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
