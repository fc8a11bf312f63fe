// Absorbed multi-head latent attention (MLA) over a paged latent cache, dense and over
// an indexer's top-k selection (S5, S8, S9).
//
// Every head reads the same cached latent row per token: 512 latent dims + 64 rope
// dims (576 bf16).  Scores use all 576 dims; values are the first 512 (the absorbed
// form of the Bitwise-consistent RL post, section 3: MLA compresses KV before caching).
//
// The split is a model constant and splits merge left to right, as for GQA.  Decode
// runs one workgroup per (row, split, group of 64 heads): 4 waves, wave w owning heads
// 64*group + 16w .. +15 as its MFMA columns (one wave per SIMD: the 512-wide fp32
// accumulator of 16 heads takes 128 registers per lane).  The trainer-side recompute
// runs the very same kernels with one "row" per query token (context = position + 1),
// after writing the chunk's latents: prefill and decode are one code path.
//
// Dense: a split covers `split_tokens` consecutive positions in 64-token tiles.
// Sparse: a split covers `split_tokens` consecutive entries of the row's selection list
// (positions in descending order, -1 last: the list order is the accumulation order,
// post section 4.3), in 64-entry tiles gathered from their pages.
//
// Latent page (16 tokens) = one 16 x 576 block in the K-operand layout of attn_common.h
// (k_page_offset); a sparse page also holds the 16 tokens' fp32 indexer keys after it.
// Per 64-token tile the workgroup puts the tile into LDS in the same layout (73,728 B)
// and writes a transposed copy of the 512 value dims, V^T[d][token] with a 72-element
// row (73,728 B), so both MFMA operands are 16-byte LDS reads.  Entries at or beyond
// the row's bound are written as 0 into V^T; their scores are masked.
#include <algorithm>

#include "attn_common.h"
#include "kernels.h"

namespace ril {

constexpr int kMlaDqk = 576, kMlaDv = 512;
constexpr int kMlaPage = kPage * kMlaDqk;     // 9216 elements: one page's latent block
constexpr int kVtRow = 72;                    // 64 tokens + 8 pad (bank spread)
constexpr int kMlaThreads = 256;              // 4 waves x 16 heads (H % 64 == 0)
constexpr int kTileUnits = 4 * kMlaPage / 8;  // 4608 16-byte units per tile

// ---------------------------------------------------------------------------
// S5 for MLA: one thread per (token, 16-byte unit): 72 latent units, then (sparse)
// 32 units of the fp32 indexer key at page + 9216 elements + 256 * t elements.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void mla_kv_write_kernel(
    const bf16_t *__restrict__ c, int row_stride, const float *__restrict__ kidx, int n_tok, int mode,
    const int32_t *__restrict__ cu, const int32_t *__restrict__ start_pos, int n_seqs,
    const int32_t *__restrict__ ctx_len, const int32_t *__restrict__ page_table, int page_stride,
    bf16_t *__restrict__ pool, int page_elems, int n_pages) {
  const int per_tok = kMlaDqk / 8 + (kidx ? 32 : 0);
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long)n_tok * per_tok) return;
  const int j = (int)(idx / per_tok);
  const int u = (int)(idx % per_tok);
  int seq, pos;
  if (mode == 0) {
    seq = locate_seq(cu, n_seqs, j);
    pos = start_pos[seq] + (j - cu[seq]);
  } else {
    seq = j;
    pos = ctx_len[j] - 1;
  }
  if (pos < 0 || pos / kPage >= page_stride) return;
  const int pid = page_table[(long)seq * page_stride + pos / kPage];
  if ((unsigned)pid >= (unsigned)n_pages) return;
  bf16_t *page = pool + (long)pid * page_elems;
  const int t = pos % kPage;
  if (u < kMlaDqk / 8) {
    st16(page + k_page_offset(t, u * 8), ld16(c + (long)j * row_stride + u * 8));
  } else {
    const int w = u - kMlaDqk / 8;  // 4 floats per unit
    st16(page + kMlaPage + t * 256 + w * 8, ld16(kidx + (long)j * 128 + w * 4));
  }
}

// Row r of a launch -> (sequence, context, q/output row).  mode 0: decode rows;
// mode 1: packed prefill tokens row0 + r, each attending to its own prefix.
__device__ __forceinline__ void mla_row(int mode, int r, int row0, const int32_t *ctx_len,
                                        const int32_t *cu, const int32_t *start_pos, int n_seqs,
                                        int &seq, int &ctx, long &qrow) {
  if (mode == 0) {
    seq = r;
    ctx = ctx_len[r];
    qrow = r;
  } else {
    const int j = row0 + r;
    seq = locate_seq(cu, n_seqs, j);
    ctx = start_pos[seq] + (j - cu[seq]) + 1;
    qrow = j;
  }
}

// ---------------------------------------------------------------------------
// Tile routines (LDS operands), shared by the dense and the sparse split kernels
// ---------------------------------------------------------------------------

__device__ __forceinline__ void mla_load_q(bf16x8 (&qop)[kMlaDqk / 32], const bf16_t *q, long qrow, int H,
                                           int head, bool col_ok) {
  const int grp = (threadIdx.x & 63) >> 4;
  const bf16_t *qp = q + (qrow * H + (col_ok ? head : 0)) * (long)kMlaDqk + grp * 8;
#pragma unroll
  for (int c = 0; c < kMlaDqk / 32; ++c) {
    u32x4 v = ld16(qp + c * 32);
    if (!col_ok) v = u32x4{0u, 0u, 0u, 0u};
    qop[c] = as_bf16x8(v);
  }
}

// S^T = K Q^T for the 64-token tile in LDS (K layout, 4 virtual pages).
__device__ __forceinline__ void mla_tile_scores(f32x4 (&s)[4], const bf16_t *kt,
                                                const bf16x8 (&qop)[kMlaDqk / 32]) {
  const int lane = threadIdx.x & 63, grp = lane >> 4, r16 = lane & 15;
  const int rq = r16 >> 2, ri = r16 & 3;
#pragma unroll
  for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const bf16_t *kb = kt + (2 * kc + (rq >> 1)) * kMlaPage + grp * 128 + h * 64 + (rq & 1) * 32 + ri * 8;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < kMlaDqk / 32; ++c)
        acc = mfma(as_bf16x8(*reinterpret_cast<const u32x4 *>(kb + c * 512)), qop[c], acc);
      s[2 * kc + h] = acc;
    }
  }
}

// o^T = o^T * alpha + V^T P^T with V^T from LDS.
__device__ __forceinline__ void mla_tile_values(f32x4 (&o)[kMlaDv / 16], const bf16_t *vt,
                                                const bf16x8 (&pop)[2], float alpha) {
  const int lane = threadIdx.x & 63, grp = lane >> 4, r16 = lane & 15;
#pragma unroll
  for (int db = 0; db < kMlaDv / 16; ++db) {
    f32x4 acc = o[db] * alpha;
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const u32x4 vv = *reinterpret_cast<const u32x4 *>(vt + (16 * db + r16) * kVtRow + 32 * kc + 8 * grp);
      acc = mfma(as_bf16x8(vv), pop[kc], acc);
    }
    o[db] = acc;
  }
}

// V^T[d][token] for d < 512 from the K-layout tile in LDS; tile rows with index
// >= n_live are written as 0.
__device__ __forceinline__ void mla_tile_transpose(const bf16_t *kt, bf16_t *vt, int n_live) {
  for (int u = threadIdx.x; u < kTileUnits; u += kMlaThreads) {
    const int p = u / (kMlaPage / 8), e = (u % (kMlaPage / 8)) * 8;
    const int dc = e >> 9, g = (e >> 7) & 3, h = (e >> 6) & 1, th = (e >> 5) & 1, i = (e >> 3) & 3;
    const int d0 = 32 * dc + 8 * g;
    if (d0 >= kMlaDv) continue;
    const int tok = 16 * p + 8 * th + 4 * h + i;
    u32x4 v = *reinterpret_cast<const u32x4 *>(kt + p * kMlaPage + e);
    if (tok >= n_live) v = u32x4{0u, 0u, 0u, 0u};
    bf16_t *dst = vt + d0 * kVtRow + tok;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      dst[(2 * w) * kVtRow] = (bf16_t)(v[w] & 0xffffu);
      dst[(2 * w + 1) * kVtRow] = (bf16_t)(v[w] >> 16);
    }
  }
}

__device__ __forceinline__ void mla_store_partial(float *part_o, float *part_ml, long base,
                                                  const f32x4 (&o)[kMlaDv / 16], float m, float l) {
  const int grp = (threadIdx.x & 63) >> 4;
  float *po = part_o + base * kMlaDv + grp * 4;
#pragma unroll
  for (int db = 0; db < kMlaDv / 16; ++db) *reinterpret_cast<f32x4 *>(po + db * 16) = o[db];
  if (grp == 0) {
    part_ml[base * 2] = m;
    part_ml[base * 2 + 1] = l;
  }
}

// ---------------------------------------------------------------------------
// S8, dense: grid (splits, H/64, rows), 256 threads.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void mla_split_kernel(
    const bf16_t *__restrict__ q, int mode, int row0, const int32_t *__restrict__ ctx_len,
    const int32_t *__restrict__ cu, const int32_t *__restrict__ start_pos, int n_seqs,
    const int32_t *__restrict__ page_table, int page_stride, const bf16_t *__restrict__ pool, int page_elems,
    int n_pages, int H, int split_tokens, int ctx_bound, float cscale, float *__restrict__ part_o,
    float *__restrict__ part_ml, int max_splits) {
  __shared__ bf16_t kt[4 * kMlaPage];
  __shared__ bf16_t vt[kMlaDv * kVtRow];
  const int split = blockIdx.x, hg = blockIdx.y, r = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, r16 = lane & 15;
  int seq, ctx;
  long qrow;
  mla_row(mode, r, row0, ctx_len, cu, start_pos, n_seqs, seq, ctx, qrow);
  const int s0 = split * split_tokens;
  if (ctx < 1 || ctx > ctx_bound || s0 >= ctx) return;  // uniform over the workgroup
  const int s1 = min(ctx, s0 + split_tokens);
  const int n_tiles = (s1 - s0 + kTile - 1) / kTile;
  // page ids of the split: lane i of every wave holds page index s0/16 + i (+64 in pidB)
  const int32_t *pt = page_table + (long)seq * page_stride;
  const int first = s0 / kPage, last = (ctx - 1) / kPage;
  int pidA = pt[min(first + lane, last)], pidB = pt[min(first + 64 + lane, last)];
  bool bad = (unsigned)pidA >= (unsigned)n_pages || (unsigned)pidB >= (unsigned)n_pages;
  pidA = ((unsigned)pidA < (unsigned)n_pages) ? pidA : 0;
  pidB = ((unsigned)pidB < (unsigned)n_pages) ? pidB : 0;
  bad = __syncthreads_or(bad);
  const int head = 64 * hg + 16 * wave + r16;
  const bool col_ok = head < H;
  bf16x8 qop[kMlaDqk / 32];
  mla_load_q(qop, q, qrow, H, head, col_ok);
  // A tile = 4 pages = 72 blocks of 64 16-byte units; block b lies in page b/18.  Wave w
  // issues blocks w, w+4, ...: each is one direct-to-LDS load (lane i -> 16 bytes at
  // kt + 512*b + 8*i), so no registers hold the tile in flight.
  constexpr int kBlocks = 4 * kMlaPage / 512;  // 72
  auto issue = [&](int t) {
    for (int b = wave; b < kBlocks; b += kMlaThreads / 64) {
      const int p = b / (kMlaPage / 512);
      const int idx = 4 * t + p;
      const int pid = idx < 64 ? __builtin_amdgcn_readlane(pidA, idx) : __builtin_amdgcn_readlane(pidB, idx - 64);
      const bf16_t *src = pool + (long)pid * page_elems + (b % (kMlaPage / 512)) * 512 + lane * 8;
      __builtin_amdgcn_global_load_lds(src, kt + b * 512, 16, 0, 0);
    }
  };
  float m = neg_inf(), l = 0.f;
  f32x4 o[kMlaDv / 16];
#pragma unroll
  for (int db = 0; db < kMlaDv / 16; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  issue(0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  mla_tile_transpose(kt, vt, ctx - s0);
  __syncthreads();
  for (int t = 0; t < n_tiles; ++t) {
    const int t0 = s0 + t * kTile;
    f32x4 s[4];
    mla_tile_scores(s, kt, qop);
    __syncthreads();  // every wave has read the K tile: refill it while PV runs
    if (t + 1 < n_tiles) issue(t + 1);
    bf16x8 pop[2];
    float alpha, m_new, l_new;
    tile_softmax(s, t0, ctx - 1, cscale, m, l, pop, alpha, m_new, l_new);
    mla_tile_values(o, vt, pop, alpha);
    m = m_new;
    l = l_new;
    if (t + 1 < n_tiles) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();  // next K tile landed; every wave is done with V^T
      mla_tile_transpose(kt, vt, ctx - (t0 + kTile));
      __syncthreads();
    }
  }
  if (bad) l = __builtin_nanf("");
  if (!col_ok) return;
  mla_store_partial(part_o, part_ml, ((long)r * H + head) * max_splits + split, o, m, l);
}

// ---------------------------------------------------------------------------
// S8, sparse: grid (splits of the selection, H/64, rows), 256 threads.  Tile entries
// are gathered from their pages into LDS (K layout), then the dense tile routines run
// with the entry index in place of the position.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void mla_sparse_split_kernel(
    const bf16_t *__restrict__ q, int mode, int row0, const int32_t *__restrict__ ctx_len,
    const int32_t *__restrict__ cu, const int32_t *__restrict__ start_pos, int n_seqs,
    const int32_t *__restrict__ page_table, int page_stride, const bf16_t *__restrict__ pool, int page_elems,
    int n_pages, int H, const int32_t *__restrict__ sel, int topk, int split_entries, int ctx_bound,
    float cscale, float *__restrict__ part_o, float *__restrict__ part_ml, int max_splits) {
  __shared__ bf16_t kt[4 * kMlaPage];
  __shared__ bf16_t vt[kMlaDv * kVtRow];
  const int split = blockIdx.x, hg = blockIdx.y, r = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, r16 = lane & 15;
  int seq, ctx;
  long qrow;
  mla_row(mode, r, row0, ctx_len, cu, start_pos, n_seqs, seq, ctx, qrow);
  const int n_sel = min(ctx, topk);
  const int e0 = split * split_entries;
  if (ctx < 1 || ctx > ctx_bound || e0 >= n_sel) return;  // uniform over the workgroup
  const int e1 = min(n_sel, e0 + split_entries);
  const int n_tiles = (e1 - e0 + kTile - 1) / kTile;
  const int32_t *pt = page_table + (long)seq * page_stride;
  const int32_t *rsel = sel + (long)r * topk;
  const int head = 64 * hg + 16 * wave + r16;
  const bool col_ok = head < H;
  bf16x8 qop[kMlaDqk / 32];
  mla_load_q(qop, q, qrow, H, head, col_ok);
  float m = neg_inf(), l = 0.f;
  f32x4 o[kMlaDv / 16];
#pragma unroll
  for (int db = 0; db < kMlaDv / 16; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  bool bad = false;
  for (int t = 0; t < n_tiles; ++t) {
    const int t0 = e0 + t * kTile;
    __syncthreads();  // every wave is done with the previous tile
    // unit u: entry u / 72 of the tile, latent dims 8 * (u % 72) .. +7
    for (int u = threadIdx.x; u < kTileUnits; u += kMlaThreads) {
      const int e = u / (kMlaDqk / 8), d0 = (u % (kMlaDqk / 8)) * 8;
      const int entry = t0 + e;
      const int pos = entry < n_sel ? rsel[entry] : -1;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (pos >= 0 && pos < ctx) {
        const int pid = pt[pos / kPage];
        if ((unsigned)pid < (unsigned)n_pages)
          v = ld16(pool + (long)pid * page_elems + k_page_offset(pos % kPage, d0));
        else
          bad = true;
      } else if (entry < n_sel) {
        bad = true;  // a listed entry that is not a position of the row
      }
      *reinterpret_cast<u32x4 *>(kt + (e >> 4) * kMlaPage + k_page_offset(e & 15, d0)) = v;
    }
    __syncthreads();
    mla_tile_transpose(kt, vt, n_sel - t0);
    __syncthreads();
    f32x4 s[4];
    mla_tile_scores(s, kt, qop);
    bf16x8 pop[2];
    float alpha, m_new, l_new;
    tile_softmax(s, t0, n_sel - 1, cscale, m, l, pop, alpha, m_new, l_new);
    mla_tile_values(o, vt, pop, alpha);
    m = m_new;
    l = l_new;
  }
  bad = __syncthreads_or(bad);
  if (bad) l = __builtin_nanf("");
  if (!col_ok) return;
  mla_store_partial(part_o, part_ml, ((long)r * H + head) * max_splits + split, o, m, l);
}

// ---------------------------------------------------------------------------
// S9 for MLA: grid (H, rows), one wave; writes out[qrow][h][0..511].  The number of
// splits is that of the row's positions (dense) or of its selection (sparse).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void mla_merge_kernel(
    int mode, int row0, const int32_t *__restrict__ ctx_len, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ start_pos, int n_seqs, int ctx_bound, int split_tokens, int topk, int H,
    int max_splits, const float *__restrict__ part_o, const float *__restrict__ part_ml,
    bf16_t *__restrict__ out) {
  const int h = blockIdx.x, r = blockIdx.y, lane = threadIdx.x;
  int seq, ctx;
  long qrow;
  mla_row(mode, r, row0, ctx_len, cu, start_pos, n_seqs, seq, ctx, qrow);
  bf16_t *op = out + (qrow * H + h) * kMlaDv;
  if (ctx < 1 || ctx > ctx_bound) {
#pragma unroll
    for (int j = 0; j < kMlaDv / 64; ++j) op[lane * (kMlaDv / 64) + j] = (bf16_t)0x7fc0u;
    return;
  }
  const int n = topk > 0 ? min(ctx, topk) : ctx;
  const int ns = (n + split_tokens - 1) / split_tokens;
  merge_partials<kMlaDv>(part_o, part_ml, ((long)r * H + h) * max_splits, ns, op);
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------

hipError_t launch_mla_kv_write(const MlaKvWriteArgs &a, hipStream_t st) {
  const long total = (long)a.n_tok * (kMlaDqk / 8 + (a.kidx ? 32 : 0));
  if (total == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((total + 255) / 256);
  hipLaunchKernelGGL(mla_kv_write_kernel, dim3(blocks), dim3(256), 0, st, a.c, a.row_stride, a.kidx, a.n_tok,
                     a.mode, a.cu, a.start_pos, a.n_seqs, a.ctx_len, a.page_table, a.page_stride, a.pool,
                     a.page_elems, a.n_pages);
  return hipGetLastError();
}

hipError_t launch_mla_split(const MlaAttnArgs &a, hipStream_t st) {
  if (a.n_rows == 0) return hipSuccess;
  if (a.sel) {
    const int n_bound = std::min(a.ctx_bound, a.topk);
    dim3 grid((n_bound + a.split_tokens - 1) / a.split_tokens, a.H / 64, a.n_rows);
    hipLaunchKernelGGL(mla_sparse_split_kernel, grid, dim3(kMlaThreads), 0, st, a.q, a.mode, a.row0, a.ctx_len,
                       a.cu, a.start_pos, a.n_seqs, a.page_table, a.page_stride, a.pool, a.page_elems,
                       a.n_pages, a.H, a.sel, a.topk, a.split_tokens, a.ctx_bound, a.cscale, a.part_o,
                       a.part_ml, a.max_splits);
  } else {
    dim3 grid((a.ctx_bound + a.split_tokens - 1) / a.split_tokens, a.H / 64, a.n_rows);
    hipLaunchKernelGGL(mla_split_kernel, grid, dim3(kMlaThreads), 0, st, a.q, a.mode, a.row0, a.ctx_len, a.cu,
                       a.start_pos, a.n_seqs, a.page_table, a.page_stride, a.pool, a.page_elems, a.n_pages,
                       a.H, a.split_tokens, a.ctx_bound, a.cscale, a.part_o, a.part_ml, a.max_splits);
  }
  return hipGetLastError();
}

hipError_t launch_mla_merge(const MlaAttnArgs &a, hipStream_t st) {
  if (a.n_rows == 0) return hipSuccess;
  hipLaunchKernelGGL(mla_merge_kernel, dim3(a.H, a.n_rows), dim3(64), 0, st, a.mode, a.row0, a.ctx_len, a.cu,
                     a.start_pos, a.n_seqs, a.ctx_bound, a.split_tokens, a.sel ? a.topk : 0, a.H,
                     a.max_splits, a.part_o, a.part_ml, a.out);
  return hipGetLastError();
}

}  // namespace ril
