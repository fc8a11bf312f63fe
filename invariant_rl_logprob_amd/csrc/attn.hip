// Paged GQA attention with a fixed KV split (S5, S8, S9, S10).
//
// The split is a model constant in tokens (the zero-mismatch-rl README, key-features
// table: fixed-split attention), never derived from the batch, the context or the GPU,
// so the rollout's split-KV decode and the trainer's prefill run one reduction tree
// (Bitwise-consistent RL post, section 2: phase consistency; section 4.2: one read
// path shared by prefill, decode and the trainer).
//
// Per query row (one q head at one position p), the value is defined by:
//   for each split s = 0 .. floor(p / S), tokens [sS, min(p+1, (s+1)S)):
//     state (m, l, o) = (-inf, 0, 0)
//     for each 64-token tile of the split, in order (one call of attn_tile):
//       x_j = fp32(q . k_j) * c   (c = scale * log2 e; one MFMA chain over D in 32-wide steps)
//       x_j = -inf for j > p;  m' = max(m, max_j x_j);  a = exp2(m - m');  p_j = exp2(x_j - m')
//       l = fma(l, a, sum_j p_j)    (fixed tree: lane-local, then xor 16, xor 32)
//       o = o * a + MFMA(bf16(p), V)  (two 32-token MFMA steps, in token order)
//   merged = split 0;  for s >= 1: merged = merge(merged, split s)   (merge_state)
//   out = bf16(O / L)   (IEEE divide)
// Decode computes each split in its own workgroup and stores the fp32 state (a
// lossless store); a second kernel merges.  Prefill keeps both the split state and the
// merged state in registers and merges at each split boundary.  Both execute exactly
// the sequence above for every row; only the MFMA column a row occupies differs, and an
// MFMA output element depends on its own row and column operands alone.
//
// KV page (16 tokens, one kv head) = K block then V block, each 16*D bf16, laid out so
// each MFMA operand is one 16-byte load per lane:
//   K (t, d) -> (d/32)*512 + ((d%32)/8)*128 + ((t%8)/4)*64 + (t/8)*32 + (t%4)*8 + d%8
//   V (t, d) -> (t/8)*8D + d*8 + t%8
// A page of the pool holds all kv heads: page p, kv head g starts at (p*Hkv + g)*32D.
#include "attn_common.h"
#include "kernels.h"

namespace ril {

// ---------------------------------------------------------------------------
// S5: KV write (shared by prefill, decode and the history writer)
// ---------------------------------------------------------------------------

// One thread per (token, kv head, 8-dim group).  mode 0: packed prefill tokens (cu,
// start_pos); mode 1: decode rows (token r is row r at position ctx_len[r]-1).
template <int D>
__global__ __launch_bounds__(256) void kv_write_kernel(
    const bf16_t *__restrict__ k, const bf16_t *__restrict__ v, int row_stride, int n_tok,
    int mode, const int32_t *__restrict__ cu, const int32_t *__restrict__ start_pos, int n_seqs,
    const int32_t *__restrict__ ctx_len, const int32_t *__restrict__ page_table, int page_stride,
    bf16_t *__restrict__ pool, int n_pages, int Hkv) {
  const int per_tok = Hkv * (D / 8);
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long)n_tok * per_tok) return;
  const int j = (int)(idx / per_tok);
  const int rem = (int)(idx % per_tok);
  const int g = rem / (D / 8);
  const int d0 = (rem % (D / 8)) * 8;
  int seq, pos;
  if (mode == 0) {
    seq = locate_seq(cu, n_seqs, j);
    pos = start_pos[seq] + (j - cu[seq]);
  } else {
    seq = j;
    pos = ctx_len[j] - 1;
  }
  if (pos < 0 || pos / kPage >= page_stride) return;  // the attention marks the row NaN
  const int pid = page_table[(long)seq * page_stride + pos / kPage];
  if ((unsigned)pid >= (unsigned)n_pages) return;
  bf16_t *kb = pool + ((long)pid * Hkv + g) * (32 * D);
  bf16_t *vb = kb + 16 * D;
  const int t = pos % kPage;
  const u32x4 kv8 = ld16(k + (long)j * row_stride + g * D + d0);
  st16(kb + k_page_offset(t, d0), kv8);
  const u32x4 vv8 = ld16(v + (long)j * row_stride + g * D + d0);
  bf16_t *vt = vb + (t / 8) * (8 * D) + t % 8;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    vt[(d0 + 2 * w) * 8] = (bf16_t)(vv8[w] & 0xffffu);
    vt[(d0 + 2 * w + 1) * 8] = (bf16_t)(vv8[w] >> 16);
  }
}

// ---------------------------------------------------------------------------
// The tile routine shared by decode and prefill
// ---------------------------------------------------------------------------

// One 64-token tile of K and V in MFMA operand registers (16-byte loads per lane).
//   k[2kc+h][c] : A operand of S^T = K Q^T for M-block (kc, h), dims 32c .. 32c+31;
//                 row r <-> token 32kc + 8(r/4) + 4h + r%4
//   v[kc][db]   : A operand of o^T += V^T P^T for 32-token step kc, dims 16db .. 16db+15;
//                 k-slot 8(lane/16) + j <-> token 32kc + 8(lane/16) + j
template <int D>
struct KVTile {
  u32x4 k[4][D / 32];
  u32x4 v[2][D / 16];
};

// pg[k]: K block of the tile's k-th page (its V block follows at +16*D).
template <int D>
__device__ __forceinline__ void load_tile(KVTile<D> &t, const bf16_t *const (&pg)[4]) {
  const int lane = threadIdx.x & 63;
  const int grp = lane >> 4, r16 = lane & 15;
  const int rq = r16 >> 2, ri = r16 & 3;
#pragma unroll
  for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const bf16_t *kb = pg[2 * kc + (rq >> 1)] + grp * 128 + h * 64 + (rq & 1) * 32 + ri * 8;
#pragma unroll
      for (int c = 0; c < D / 32; ++c) t.k[2 * kc + h][c] = ld16(kb + c * 512);
    }
  }
#pragma unroll
  for (int kc = 0; kc < 2; ++kc) {
    const bf16_t *vb = pg[2 * kc + (grp >> 1)] + 16 * D + (grp & 1) * (8 * D) + r16 * 8;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) t.v[kc][db] = ld16(vb + db * 128);
  }
}

// One 64-token KV tile for the 16 query rows (MFMA columns) of this wave.
//   qop     : B operand of S^T = K Q^T (lane: column lane%16, dims 32c + 8(lane/16) ..)
//   pos     : this lane's column's query position (-1: padding column)
//   vbound  : V values of tokens >= vbound are read as 0 (beyond any column's context)
// State per lane = its column's (m, l) and o^T[16db + 4(lane/16) + i].
// MAYBE_INACTIVE: some column may have pos < tile_start; such columns keep their state.
template <int D, bool MAYBE_INACTIVE>
__device__ __forceinline__ void attn_tile(const KVTile<D> &t, int tile_start,
                                          const bf16x8 (&qop)[D / 32], int pos, int vbound,
                                          float cscale, float &m, float &l, f32x4 (&o)[D / 16]) {
  const int lane = threadIdx.x & 63;
  const int grp = lane >> 4;
  f32x4 s[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < D / 32; ++c) acc = mfma(as_bf16x8(t.k[mb][c]), qop[c], acc);
    s[mb] = acc;
  }
  bf16x8 pop[2];
  float alpha, m_new, l_new;
  tile_softmax(s, tile_start, pos, cscale, m, l, pop, alpha, m_new, l_new);
  f32x4 on[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) on[db] = o[db] * alpha;
#pragma unroll
  for (int kc = 0; kc < 2; ++kc) {
    const int n_valid = vbound - (tile_start + 32 * kc + 8 * grp);
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      u32x4 vv = t.v[kc][db];
      if (n_valid < 8) vv = keep_first(vv, n_valid);
      on[db] = mfma(as_bf16x8(vv), pop[kc], on[db]);
    }
  }
  if (MAYBE_INACTIVE) {
    const bool act = tile_start <= pos;
    m = act ? m_new : m;
    l = act ? l_new : l;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
#pragma unroll
      for (int i = 0; i < 4; ++i) o[db][i] = act ? on[db][i] : o[db][i];
    }
  } else {
    m = m_new;
    l = l_new;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) o[db] = on[db];
  }
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

// Page ids of one split, one per lane: lane i holds the id of page index
// min(first + i, last) of the sequence (the clamp keeps reads in bounds; tokens beyond
// the context are masked).  Returns whether any id in range lies outside the pool.
__device__ __forceinline__ bool split_pages(const int32_t *pt, int first, int last, int n_pages,
                                            int &pid) {
  const int lane = threadIdx.x & 63;
  int p = pt[min(first + lane, last)];
  const bool bad = (unsigned)p >= (unsigned)n_pages;
  pid = bad ? 0 : p;
  return __any(bad);
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

// ---------------------------------------------------------------------------
// S8: decode split kernel.  grid (max splits, Hkv, rows), one wave each.  The next
// tile's K/V loads are issued before the current tile is computed.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void attn_decode_split_kernel(
    const bf16_t *__restrict__ q, int q_row_stride, const int32_t *__restrict__ ctx_len,
    const int32_t *__restrict__ page_table, int page_stride, const bf16_t *__restrict__ pool,
    int n_pages, int Hkv, int G, int split_tokens, int ctx_bound, float cscale,
    float *__restrict__ part_o, float *__restrict__ part_ml, int max_splits) {
  const int split = blockIdx.x, g = blockIdx.y, row = blockIdx.z;
  const int lane = threadIdx.x;
  const int ctx = ctx_len[row];
  const int s0 = split * split_tokens;
  if (ctx < 1 || ctx > ctx_bound || s0 >= ctx) return;
  const int Hq = Hkv * G;
  const int n = lane & 15, grp = lane >> 4;
  const bool col_ok = n < G;
  const int s1 = min(ctx, s0 + split_tokens);
  const int n_tiles = (s1 - s0 + kTile - 1) / kTile;
  int pid;
  const bool bad = split_pages(page_table + (long)row * page_stride, s0 / kPage, (ctx - 1) / kPage,
                               n_pages, pid);
  KVTile<D> buf0, buf1;
  const bf16_t *pg[4];
  tile_pages<D>(pg, pool, pid, 0, Hkv, g);
  load_tile<D>(buf0, pg);
  bf16x8 qop[D / 32];
  load_qop<D>(qop, q + (long)row * q_row_stride + (g * G + (col_ok ? n : 0)) * D, col_ok);
  float m = neg_inf(), l = 0.f;
  f32x4 o[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int t = 0; t < n_tiles; t += 2) {
    if (t + 1 < n_tiles) {
      tile_pages<D>(pg, pool, pid, t + 1, Hkv, g);
      load_tile<D>(buf1, pg);
    }
    attn_tile<D, false>(buf0, s0 + t * kTile, qop, ctx - 1, ctx, cscale, m, l, o);
    if (t + 1 < n_tiles) {
      if (t + 2 < n_tiles) {
        tile_pages<D>(pg, pool, pid, t + 2, Hkv, g);
        load_tile<D>(buf0, pg);
      }
      attn_tile<D, false>(buf1, s0 + (t + 1) * kTile, qop, ctx - 1, ctx, cscale, m, l, o);
    }
  }
  if (bad) l = __builtin_nanf("");
  if (!col_ok) return;
  const long base = ((long)row * Hq + g * G + n) * max_splits + split;
  float *po = part_o + base * D + grp * 4;
#pragma unroll
  for (int db = 0; db < D / 16; ++db) *reinterpret_cast<f32x4 *>(po + db * 16) = o[db];
  if (grp == 0) {
    part_ml[base * 2] = m;
    part_ml[base * 2 + 1] = l;
  }
}

// ---------------------------------------------------------------------------
// S9: decode merge kernel.  grid (Hq, rows), one wave; lane owns D/64 dims.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void attn_decode_merge_kernel(
    const int32_t *__restrict__ ctx_len, int ctx_bound, int split_tokens, int Hq, int max_splits,
    const float *__restrict__ part_o, const float *__restrict__ part_ml, bf16_t *__restrict__ out) {
  constexpr int PER = D / 64;
  const int h = blockIdx.x, row = blockIdx.y, lane = threadIdx.x;
  const int ctx = ctx_len[row];
  bf16_t *op = out + ((long)row * Hq + h) * D + lane * PER;
  if (ctx < 1 || ctx > ctx_bound) {
#pragma unroll
    for (int j = 0; j < PER; ++j) op[j] = (bf16_t)0x7fc0u;
    return;
  }
  const int ns = (ctx + split_tokens - 1) / split_tokens;
  merge_partials<D>(part_o, part_ml, ((long)row * Hq + h) * max_splits, ns, op - lane * PER);
}

// ---------------------------------------------------------------------------
// S10: prefill attention.  grid (block bound, Hkv), one wave per 16 query columns
// (16/G tokens x G heads of one sequence).  Splits and tiles run in order; the split
// state and the merged state both stay in registers.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void attn_prefill_kernel(
    const bf16_t *__restrict__ q, int q_row_stride, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ start_pos, int n_seqs, const int32_t *__restrict__ page_table,
    int page_stride, const bf16_t *__restrict__ pool, int n_pages, int Hkv, int G,
    int split_tokens, int ctx_bound, float cscale, bf16_t *__restrict__ out) {
  const int g = blockIdx.y;
  const int lane = threadIdx.x;
  const int tpb = 16 / G;
  // Block -> (sequence, first token): wave-wide prefix sum of per-sequence block counts.
  int remaining = blockIdx.x, seq = -1, tok0 = 0;
  for (int base = 0; base < n_seqs; base += 64) {
    const int i = base + lane;
    const int nb = (i < n_seqs) ? (cu[i + 1] - cu[i] + tpb - 1) / tpb : 0;
    int incl = nb;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(incl, off, 64);
      if (lane >= off) incl += t;
    }
    const int total = __shfl(incl, 63, 64);
    if (remaining < total) {
      const unsigned long long mask = __ballot(incl > remaining);
      const int first = __ffsll((long long)mask) - 1;
      const int excl = __shfl(incl - nb, first, 64);
      seq = base + first;
      tok0 = (remaining - excl) * tpb;
      break;
    }
    remaining -= total;
  }
  if (seq < 0) return;
  const int Hq = Hkv * G;
  const int n_tok = cu[seq + 1] - cu[seq];
  const int sp = start_pos[seq];
  const int n = lane & 15, grp = lane >> 4;
  const int tl = n / G, hh = n % G;
  const bool col_ok = tok0 + tl < n_tok;
  const long j = cu[seq] + tok0 + (col_ok ? tl : 0);
  const int pos = col_ok ? sp + tok0 + tl : -1;
  const int tok_hi = min(tok0 + tpb, n_tok);
  const int p_max = sp + tok_hi - 1, p_min = sp + tok0;
  bf16_t *op = out + (j * Hq + g * G + hh) * D + grp * 4;
  if (sp < 0 || p_max + 1 > ctx_bound || (p_max / kPage) >= page_stride) {
    if (col_ok) {
#pragma unroll
      for (int db = 0; db < D / 16; ++db)
        for (int i = 0; i < 4; ++i) op[db * 16 + i] = (bf16_t)0x7fc0u;
    }
    return;
  }
  bf16x8 qop[D / 32];
  load_qop<D>(qop, q + j * q_row_stride + (g * G + hh) * D, col_ok);
  float M = neg_inf(), L = 0.f;
  float O[D / 4];
#pragma unroll
  for (int e = 0; e < D / 4; ++e) O[e] = 0.f;
  const int32_t *pt = page_table + (long)seq * page_stride;
  const int last_page = p_max / kPage;
  bool bad = false;
  const int n_splits = p_max / split_tokens + 1;
  KVTile<D> tile;
  for (int si = 0; si < n_splits; ++si) {
    const int s0 = si * split_tokens;
    const int s1 = min(p_max + 1, s0 + split_tokens);
    int pid;
    bad |= split_pages(pt, s0 / kPage, last_page, n_pages, pid);
    float m = neg_inf(), l = 0.f;
    f32x4 o[D / 16];
#pragma unroll
    for (int db = 0; db < D / 16; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int t0 = s0; t0 < s1; t0 += kTile) {
      const bf16_t *pg[4];
      tile_pages<D>(pg, pool, pid, (t0 - s0) / kTile, Hkv, g);
      load_tile<D>(tile, pg);
      if (t0 <= p_min)
        attn_tile<D, false>(tile, t0, qop, pos, p_max + 1, cscale, m, l, o);
      else
        attn_tile<D, true>(tile, t0, qop, pos, p_max + 1, cscale, m, l, o);
    }
    if (s0 <= pos) {
      float os[D / 4];
#pragma unroll
      for (int db = 0; db < D / 16; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) os[db * 4 + i] = o[db][i];
      if (si == 0) {
        M = m;
        L = l;
#pragma unroll
        for (int e = 0; e < D / 4; ++e) O[e] = os[e];
      } else {
        merge_state<D / 4>(M, L, O, m, l, os);
      }
    }
  }
  if (bad) L = __builtin_nanf("");
  if (!col_ok) return;
#pragma unroll
  for (int db = 0; db < D / 16; ++db) {
    uint32_t w0 = pack2(__fdiv_rn(O[db * 4 + 0], L), __fdiv_rn(O[db * 4 + 1], L));
    uint32_t w1 = pack2(__fdiv_rn(O[db * 4 + 2], L), __fdiv_rn(O[db * 4 + 3], L));
    *reinterpret_cast<uint2 *>(op + db * 16) = make_uint2(w0, w1);
  }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------

hipError_t launch_kv_write(const KvWriteArgs &a, hipStream_t st) {
  const long total = (long)a.n_tok * a.Hkv * (a.D / 8);
  if (total == 0) return hipSuccess;
  const int threads = 256;
  const unsigned blocks = (unsigned)((total + threads - 1) / threads);
  if (a.D == 128)
    hipLaunchKernelGGL(kv_write_kernel<128>, dim3(blocks), dim3(threads), 0, st, a.k, a.v,
                       a.row_stride, a.n_tok, a.mode, a.cu, a.start_pos, a.n_seqs, a.ctx_len,
                       a.page_table, a.page_stride, a.pool, a.n_pages, a.Hkv);
  else
    hipLaunchKernelGGL(kv_write_kernel<64>, dim3(blocks), dim3(threads), 0, st, a.k, a.v,
                       a.row_stride, a.n_tok, a.mode, a.cu, a.start_pos, a.n_seqs, a.ctx_len,
                       a.page_table, a.page_stride, a.pool, a.n_pages, a.Hkv);
  return hipGetLastError();
}

hipError_t launch_attn_split(const AttnDecodeArgs &a, hipStream_t st) {
  const int n_split_grid = (a.ctx_bound + a.split_tokens - 1) / a.split_tokens;
  dim3 grid(n_split_grid, a.Hkv, a.n_rows);
  if (a.D == 128)
    hipLaunchKernelGGL(attn_decode_split_kernel<128>, grid, dim3(64), 0, st, a.q, a.q_row_stride,
                       a.ctx_len, a.page_table, a.page_stride, a.pool, a.n_pages, a.Hkv, a.G,
                       a.split_tokens, a.ctx_bound, a.cscale, a.part_o, a.part_ml, a.max_splits);
  else
    hipLaunchKernelGGL(attn_decode_split_kernel<64>, grid, dim3(64), 0, st, a.q, a.q_row_stride,
                       a.ctx_len, a.page_table, a.page_stride, a.pool, a.n_pages, a.Hkv, a.G,
                       a.split_tokens, a.ctx_bound, a.cscale, a.part_o, a.part_ml, a.max_splits);
  return hipGetLastError();
}

hipError_t launch_attn_merge(const AttnDecodeArgs &a, hipStream_t st) {
  dim3 grid(a.Hkv * a.G, a.n_rows);
  if (a.D == 128)
    hipLaunchKernelGGL(attn_decode_merge_kernel<128>, grid, dim3(64), 0, st, a.ctx_len, a.ctx_bound,
                       a.split_tokens, a.Hkv * a.G, a.max_splits, a.part_o, a.part_ml, a.out);
  else
    hipLaunchKernelGGL(attn_decode_merge_kernel<64>, grid, dim3(64), 0, st, a.ctx_len, a.ctx_bound,
                       a.split_tokens, a.Hkv * a.G, a.max_splits, a.part_o, a.part_ml, a.out);
  return hipGetLastError();
}

hipError_t launch_attn_prefill(const AttnPrefillArgs &a, hipStream_t st) {
  const int tpb = 16 / a.G;
  const int blocks = (a.n_tok + tpb - 1) / tpb + a.n_seqs;
  dim3 grid(blocks, a.Hkv);
  if (a.D == 128)
    hipLaunchKernelGGL(attn_prefill_kernel<128>, grid, dim3(64), 0, st, a.q, a.q_row_stride, a.cu,
                       a.start_pos, a.n_seqs, a.page_table, a.page_stride, a.pool, a.n_pages,
                       a.Hkv, a.G, a.split_tokens, a.ctx_bound, a.cscale, a.out);
  else
    hipLaunchKernelGGL(attn_prefill_kernel<64>, grid, dim3(64), 0, st, a.q, a.q_row_stride, a.cu,
                       a.start_pos, a.n_seqs, a.page_table, a.page_stride, a.pool, a.n_pages,
                       a.Hkv, a.G, a.split_tokens, a.ctx_bound, a.cscale, a.out);
  return hipGetLastError();
}

}  // namespace ril
