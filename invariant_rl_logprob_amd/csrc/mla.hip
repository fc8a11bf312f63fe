// Absorbed multi-head latent attention (MLA) over a paged latent cache (S5, S8, S9).
//
// Every head reads the same cached latent row per token: 512 latent dims + 64 rope
// dims (576 bf16).  Scores use all 576 dims; values are the first 512 (the absorbed
// form of the Bitwise-consistent RL post, section 3: MLA compresses KV before caching).
//
// The split is a model constant in tokens and splits merge left to right, as for GQA.
// Decode runs one workgroup per (row, split, group of 64 heads): 4 waves, wave w owning
// heads 64*group + 16w .. +15 as its MFMA columns (one wave per SIMD: the 512-wide fp32
// accumulator of 16 heads takes 128 registers per lane).  The trainer-side recompute runs the very same two kernels with
// one "row" per query token (context = its position + 1), after writing the chunk's
// latents: prefill and decode are one code path, not two that agree.
//
// Latent page (16 tokens) = one 16 x 576 block in the K-operand layout of attn_common.h
// (k_page_offset).  Per 64-token tile the workgroup copies the four pages into LDS once
// (73,728 B) and writes a transposed copy of the 512 value dims, V^T[d][token] with a
// 72-element row (73,728 B), so both MFMA operands are 16-byte LDS reads.  Tokens at
// or beyond the row's context are written as 0 into V^T; their scores are masked.
#include <algorithm>

#include "attn_common.h"
#include "kernels.h"

namespace ril {

constexpr int kMlaDqk = 576, kMlaDv = 512;
constexpr int kMlaPage = kPage * kMlaDqk;  // 9216 elements
constexpr int kVtRow = 72;                 // 64 tokens + 8 pad (bank spread)
constexpr int kMlaThreads = 256;                         // 4 waves x 16 heads (H % 64 == 0)

// ---------------------------------------------------------------------------
// S5 for MLA: one thread per (token, 8-dim group) writes 16 bytes.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void mla_kv_write_kernel(
    const bf16_t *__restrict__ c, int row_stride, int n_tok, int mode, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ start_pos, int n_seqs, const int32_t *__restrict__ ctx_len,
    const int32_t *__restrict__ page_table, int page_stride, bf16_t *__restrict__ pool, int n_pages) {
  constexpr int per_tok = kMlaDqk / 8;
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long)n_tok * per_tok) return;
  const int j = (int)(idx / per_tok);
  const int d0 = (int)(idx % per_tok) * 8;
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
  st16(pool + (long)pid * kMlaPage + k_page_offset(pos % kPage, d0), ld16(c + (long)j * row_stride + d0));
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
// S8 for MLA: grid (splits, H/64, rows), 256 threads.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void mla_split_kernel(
    const bf16_t *__restrict__ q, int mode, int row0, const int32_t *__restrict__ ctx_len,
    const int32_t *__restrict__ cu, const int32_t *__restrict__ start_pos, int n_seqs,
    const int32_t *__restrict__ page_table, int page_stride, const bf16_t *__restrict__ pool,
    int n_pages, int H, int split_tokens, int ctx_bound, float cscale, float *__restrict__ part_o,
    float *__restrict__ part_ml, int max_splits) {
  __shared__ bf16_t kt[4 * kMlaPage];
  __shared__ bf16_t vt[kMlaDv * kVtRow];
  const int split = blockIdx.x, hg = blockIdx.y, r = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int grp = lane >> 4, r16 = lane & 15;
  constexpr int nthr = kMlaThreads;
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
  // query operand: column = head 64*hg + 16*wave + r16
  const int head = 64 * hg + 16 * wave + r16;
  const bool col_ok = head < H;
  bf16x8 qop[kMlaDqk / 32];
  {
    const bf16_t *qp = q + (qrow * H + (col_ok ? head : 0)) * (long)kMlaDqk + grp * 8;
#pragma unroll
    for (int c = 0; c < kMlaDqk / 32; ++c) {
      u32x4 v = ld16(qp + c * 32);
      if (!col_ok) v = u32x4{0u, 0u, 0u, 0u};
      qop[c] = as_bf16x8(v);
    }
  }
  // A tile = 4 pages = 72 blocks of 64 16-byte units; block b lies in page b/18.  Wave w
  // issues blocks w, w+4, ...: each is one direct-to-LDS load (lane i -> 16 bytes at
  // kt + 512*b + 8*i), so no registers hold the tile in flight.
  constexpr int kBlocks = 4 * kMlaPage / 512;  // 72
  auto issue = [&](int t) {
    for (int b = wave; b < kBlocks; b += nthr / 64) {
      const int p = b / (kMlaPage / 512);
      const int idx = 4 * t + p;
      const int pid = idx < 64 ? __builtin_amdgcn_readlane(pidA, idx) : __builtin_amdgcn_readlane(pidB, idx - 64);
      const bf16_t *src = pool + (long)pid * kMlaPage + (b % (kMlaPage / 512)) * 512 + lane * 8;
      __builtin_amdgcn_global_load_lds(src, kt + b * 512, 16, 0, 0);
    }
  };
  // V^T[d][token] for d < 512 from the K-layout tile in LDS; tokens at or beyond the
  // context are written as 0.
  auto transpose = [&](int t) {
    const int t0 = s0 + t * kTile;
    for (int u = tid; u < 4 * kMlaPage / 8; u += nthr) {
      const int p = u / (kMlaPage / 8), e = (u % (kMlaPage / 8)) * 8;
      const int dc = e >> 9, g = (e >> 7) & 3, h = (e >> 6) & 1, th = (e >> 5) & 1, i = (e >> 3) & 3;
      const int d0 = 32 * dc + 8 * g;
      if (d0 >= kMlaDv) continue;
      const int tok = 16 * p + 8 * th + 4 * h + i;
      u32x4 v = *reinterpret_cast<const u32x4 *>(kt + p * kMlaPage + e);
      if (t0 + tok >= ctx) v = u32x4{0u, 0u, 0u, 0u};
      bf16_t *dst = vt + d0 * kVtRow + tok;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        dst[(2 * w) * kVtRow] = (bf16_t)(v[w] & 0xffffu);
        dst[(2 * w + 1) * kVtRow] = (bf16_t)(v[w] >> 16);
      }
    }
  };
  float m = neg_inf(), l = 0.f;
  f32x4 o[kMlaDv / 16];
#pragma unroll
  for (int db = 0; db < kMlaDv / 16; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int rq = r16 >> 2, ri = r16 & 3;
  issue(0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  transpose(0);
  __syncthreads();
  for (int t = 0; t < n_tiles; ++t) {
    const int t0 = s0 + t * kTile;
    f32x4 s[4];
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
    __syncthreads();  // every wave has read the K tile: refill it while PV runs
    if (t + 1 < n_tiles) issue(t + 1);
    bf16x8 pop[2];
    float alpha, m_new, l_new;
    tile_softmax(s, t0, ctx - 1, cscale, m, l, pop, alpha, m_new, l_new);
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
    m = m_new;
    l = l_new;
    if (t + 1 < n_tiles) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();  // next K tile landed; every wave is done with V^T
      transpose(t + 1);
      __syncthreads();
    }
  }
  if (bad) l = __builtin_nanf("");
  if (!col_ok) return;
  const long base = ((long)r * H + head) * max_splits + split;
  float *po = part_o + base * kMlaDv + grp * 4;
#pragma unroll
  for (int db = 0; db < kMlaDv / 16; ++db) *reinterpret_cast<f32x4 *>(po + db * 16) = o[db];
  if (grp == 0) {
    part_ml[base * 2] = m;
    part_ml[base * 2 + 1] = l;
  }
}

// ---------------------------------------------------------------------------
// S9 for MLA: grid (H, rows), one wave; writes out[qrow][h][0..511].
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void mla_merge_kernel(
    int mode, int row0, const int32_t *__restrict__ ctx_len, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ start_pos, int n_seqs, int ctx_bound, int split_tokens, int H,
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
  const int ns = (ctx + split_tokens - 1) / split_tokens;
  merge_partials<kMlaDv>(part_o, part_ml, ((long)r * H + h) * max_splits, ns, op);
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------

hipError_t launch_mla_kv_write(const MlaKvWriteArgs &a, hipStream_t st) {
  const long total = (long)a.n_tok * (kMlaDqk / 8);
  if (total == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((total + 255) / 256);
  hipLaunchKernelGGL(mla_kv_write_kernel, dim3(blocks), dim3(256), 0, st, a.c, a.row_stride, a.n_tok, a.mode,
                     a.cu, a.start_pos, a.n_seqs, a.ctx_len, a.page_table, a.page_stride, a.pool, a.n_pages);
  return hipGetLastError();
}

hipError_t launch_mla_split(const MlaAttnArgs &a, hipStream_t st) {
  if (a.n_rows == 0) return hipSuccess;
  dim3 grid((a.ctx_bound + a.split_tokens - 1) / a.split_tokens, (a.H + 63) / 64, a.n_rows);
  hipLaunchKernelGGL(mla_split_kernel, grid, dim3(kMlaThreads), 0, st, a.q, a.mode, a.row0, a.ctx_len,
                     a.cu, a.start_pos, a.n_seqs, a.page_table, a.page_stride, a.pool, a.n_pages, a.H,
                     a.split_tokens, a.ctx_bound, a.cscale, a.part_o, a.part_ml, a.max_splits);
  return hipGetLastError();
}

hipError_t launch_mla_merge(const MlaAttnArgs &a, hipStream_t st) {
  if (a.n_rows == 0) return hipSuccess;
  hipLaunchKernelGGL(mla_merge_kernel, dim3(a.H, a.n_rows), dim3(64), 0, st, a.mode, a.row0, a.ctx_len, a.cu,
                     a.start_pos, a.n_seqs, a.ctx_bound, a.split_tokens, a.H, a.max_splits, a.part_o,
                     a.part_ml, a.out);
  return hipGetLastError();
}

}  // namespace ril
