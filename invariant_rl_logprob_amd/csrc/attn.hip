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
template <int D>
__device__ __forceinline__ void attn_scores(const Half<D> &k, int tile_start, const bf16x8 (&qop)[D / 32],
                                            int pos, float cscale, float m, float l, bf16x8 (&pop)[2],
                                            float &alpha, float &m_new, float &l_new) {
  f32x4 s[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < D / 32; ++c) acc = mfma(as_bf16x8(k.r[mb * (D / 32) + c]), qop[c], acc);
    s[mb] = acc;
  }
  tile_softmax(s, tile_start, pos, cscale, m, l, pop, alpha, m_new, l_new);
}

// Second half: o = o * alpha + MFMA(bf16 P, V), two 32-token steps in token order.
//   vbound : V values of tokens >= vbound are read as 0 (beyond any column's context)
// State per lane = its column's (m, l) and o^T[16db + 4(lane/16) + i].
// MAYBE_INACTIVE: some column may have pos < tile_start; such columns keep their state.
template <int D, bool MAYBE_INACTIVE>
__device__ __forceinline__ void attn_values(const Half<D> &v, int tile_start, int pos, int vbound,
                                            const bf16x8 (&pop)[2], float alpha, float m_new, float l_new,
                                            float &m, float &l, f32x4 (&o)[D / 16]) {
  const int grp = (threadIdx.x & 63) >> 4;
  f32x4 on[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) on[db] = o[db] * alpha;
#pragma unroll
  for (int kc = 0; kc < 2; ++kc) {
    const int n_valid = vbound - (tile_start + 32 * kc + 8 * grp);
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      u32x4 vv = v.r[kc * (D / 16) + db];
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

// ---------------------------------------------------------------------------
// S8: decode split kernel, one wave per (row, kv head, split).  The 1-D grid lists the
// work longest first, so the hardware dispatcher fills the machine with full splits and
// ends on the short ones: slots [0, n_sg*R*Hkv) are the full splits, split-major (the
// kv heads of one page adjacent); then for c = n_cls .. 1 one slot per (row, kv head)
// whose partial last split has c tiles.  Slots with no such work exit at once.  Which
// wave computes a split never changes its arithmetic.  K/V loads run up to two tiles
// ahead of the tile being computed.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void attn_decode_split_kernel(
    const bf16_t *__restrict__ q, int q_row_stride, const int32_t *__restrict__ ctx_len,
    const int32_t *__restrict__ page_table, int page_stride, const bf16_t *__restrict__ pool,
    int n_pages, int Hkv, int G, int split_tokens, int ctx_bound, int n_rows, int n_sg, float cscale,
    float *__restrict__ part_o, float *__restrict__ part_ml, int max_splits) {
  const int lane = threadIdx.x;
  const int per_s = Hkv * n_rows;
  const int b = blockIdx.x;
  const bool full = b < n_sg * per_s;
  const int rem = full ? b % per_s : (b - n_sg * per_s) % per_s;
  const int row = rem / Hkv, g = rem % Hkv;
  const int cls = full ? 0 : split_tokens / kTile - (b - n_sg * per_s) / per_s;
  const int n = lane & 15, grp = lane >> 4;
  const bool col_ok = n < G;
  const int32_t *pt = page_table + (long)row * page_stride;
  // Loads that do not depend on the context length are issued together with it.
  const int ctx = ctx_len[row];
  int split = full ? b / per_s : 0;
  int p_raw = full ? pt[min(split * (split_tokens / kPage) + lane, page_stride - 1)] : 0;
  bf16x8 qop[D / 32];
  load_qop<D>(qop, q + (long)row * q_row_stride + (g * G + (col_ok ? n : 0)) * D, col_ok);
  if (ctx < 1 || ctx > ctx_bound) return;
  if (full) {
    if ((split + 1) * split_tokens > ctx) return;
  } else {
    const int tail = ctx % split_tokens;
    if (tail == 0 || (tail + kTile - 1) / kTile != cls) return;
    split = ctx / split_tokens;
    p_raw = pt[min(split * (split_tokens / kPage) + lane, page_stride - 1)];
  }
  const int Hq = Hkv * G;
  const int s0 = split * split_tokens;
  const int s1 = min(ctx, s0 + split_tokens);
  const int n_tiles = (s1 - s0 + kTile - 1) / kTile;
  // lane i: id of page s0/16 + i when that page holds context, else page 0 (its tokens
  // are masked); an id outside the pool marks the row NaN.
  const bool in_ctx = s0 / kPage + lane <= (ctx - 1) / kPage;
  const bool bad_lane = in_ctx && (unsigned)p_raw >= (unsigned)n_pages;
  const int pid = (in_ctx && !bad_lane) ? p_raw : 0;
  const bool bad = __any(bad_lane);
  // Five half-tile slots: while the scores of tile t run, the V half of t and both halves
  // of t+1 and the K half of t+2 are in flight (64 KB per wave for D = 128).
  // Half-tile h (K of tile h/2 if h is even, else its V) lives in slot h % 5.
  Half<D> ring[5];
  const bf16_t *pg[4];
  tile_pages<D>(pg, pool, pid, 0, Hkv, g);
  load_k<D>(ring[0], pg);
  load_v<D>(ring[1], pg);
  if (n_tiles > 1) {
    tile_pages<D>(pg, pool, pid, 1, Hkv, g);
    load_k<D>(ring[2], pg);
    load_v<D>(ring[3], pg);
  }
  float m = neg_inf(), l = 0.f;
  f32x4 o[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int t0 = 0; t0 < n_tiles; t0 += 5) {
#pragma unroll
    for (int j = 0; j < 5; ++j) {
      const int t = t0 + j;
      if (t < n_tiles) {
        const bool ahead = t + 2 < n_tiles;
        if (ahead) {
          tile_pages<D>(pg, pool, pid, t + 2, Hkv, g);
          load_k<D>(ring[(2 * j + 4) % 5], pg);  // the slot of V(t-1), already consumed
        }
        bf16x8 pop[2];
        float alpha, m_new, l_new;
        attn_scores<D>(ring[(2 * j) % 5], s0 + t * kTile, qop, ctx - 1, cscale, m, l, pop, alpha, m_new,
                       l_new);
        if (ahead) load_v<D>(ring[(2 * j) % 5], pg);  // the slot of K(t), just consumed
        attn_values<D, false>(ring[(2 * j + 1) % 5], s0 + t * kTile, ctx - 1, ctx, pop, alpha, m_new, l_new,
                              m, l, o);
      }
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
// S10: prefill attention.  grid (workgroup bound, Hkv); a workgroup of NW waves covers
// QT = NW*(16/G) consecutive query tokens of one sequence for one kv head, wave w owning
// one block of 16 MFMA columns (16/G tokens x G heads).  The workgroup walks the 64-token
// KV tiles of its context in order.  Each tile is copied once into LDS by direct-to-LDS
// loads spread over the waves, NBUF-1 tiles ahead of the tile being computed, and read
// by every wave.  Per column the arithmetic is the decode chain exactly: the same
// attn_scores / attn_values per tile, a fresh state per split and merge_state at each
// split's end, with per-column predication (MAYBE_INACTIVE) for tiles and splits past
// the column's position.  Split and merged states stay in registers.
// ---------------------------------------------------------------------------
// LDS slot of one page block (K then V, 16*D bf16 each), padded by 128 bytes so the two
// pages one K-operand load touches fall on different banks.
template <int D>
constexpr int lds_page() { return 32 * D + 64; }

// s_waitcnt vmcnt(N): wait until at most N vector-memory operations of this wave are
// outstanding (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N == 0 || N == 2 || N == 4 || N == 8, "add the count");
  if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else if constexpr (N == 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
  else if constexpr (N == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
}

template <int D, int NW, int NBUF>
__global__ __launch_bounds__(512) void attn_prefill_kernel(
    const bf16_t *__restrict__ q, int q_row_stride, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ start_pos, int n_seqs, const int32_t *__restrict__ page_table,
    int page_stride, const bf16_t *__restrict__ pool, int n_pages, int Hkv, int G,
    int split_tokens, int ctx_bound, float cscale, bf16_t *__restrict__ out) {
  static_assert(NW >= 1 && NW <= 8, "at most 512 threads (the launch bound)");
  static_assert(NBUF >= 2 && NBUF <= 4, "tiles in flight");
  constexpr int kSlot = lds_page<D>();
  constexpr int kPieces = 32 * D / 512;       // 1 KB pieces per page block
  static_assert((4 * kPieces) % NW == 0, "every wave copies the same number of pieces");
  constexpr int kPer = 4 * kPieces / NW;      // pieces (= vector-memory ops) per wave per tile
  __shared__ __attribute__((aligned(16))) bf16_t kv[NBUF][4 * kSlot];
  const int g = blockIdx.y;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int tpb = 16 / G;
  const int QT = NW * tpb;
  // Block -> (sequence, first token): wave-wide prefix sum of per-sequence block counts
  // (every wave computes the same answer).
  int remaining = blockIdx.x, seq = -1, tok0 = 0;
  for (int base = 0; base < n_seqs; base += 64) {
    const int i = base + lane;
    const int nb = (i < n_seqs) ? (cu[i + 1] - cu[i] + QT - 1) / QT : 0;
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
      tok0 = (remaining - excl) * QT;
      break;
    }
    remaining -= total;
  }
  if (seq < 0) return;  // the same for the whole workgroup
  // wave-uniform values kept in scalar registers (the page-table reads below are then
  // scalar loads, which never wait on the vector-memory counter of the tile copies)
  seq = __builtin_amdgcn_readfirstlane(seq);
  tok0 = __builtin_amdgcn_readfirstlane(tok0);
  const int Hq = Hkv * G;
  const int n_tok = __builtin_amdgcn_readfirstlane(cu[seq + 1] - cu[seq]);
  const int sp = __builtin_amdgcn_readfirstlane(start_pos[seq]);
  const int n = lane & 15, grp = lane >> 4;
  const int hh = n % G;
  const int wtok0 = tok0 + wave * tpb;  // first token of this wave
  const int tok = wtok0 + n / G;
  const bool col_ok = tok < n_tok;
  const long jrow = cu[seq] + (col_ok ? tok : 0);
  const int pos = col_ok ? sp + tok : -1;
  bf16_t *op = out + (jrow * Hq + g * G + hh) * D + grp * 4;
  const int p_max = sp + min(tok0 + QT, n_tok) - 1;  // the workgroup's last position
  if (sp < 0 || p_max + 1 > ctx_bound || (p_max / kPage) >= page_stride) {
    if (col_ok) {
#pragma unroll
      for (int db = 0; db < D / 16; ++db)
        for (int i = 0; i < 4; ++i) op[db * 16 + i] = (bf16_t)0x7fc0u;
    }
    return;
  }
  const int w_min = sp + wtok0;                             // this wave's first position
  const int w_max = sp + min(wtok0 + tpb, n_tok) - 1;       // and last (< w_min if none)
  bf16x8 qop[D / 32];
  load_qop<D>(qop, q + jrow * q_row_stride + (g * G + hh) * D, col_ok);

  const int32_t *pt = page_table + (long)seq * page_stride;
  const int last_page = p_max / kPage;
  const int n_tiles = p_max / kTile + 1;
  bool bad = false;
  // Wave w copies pieces w, w+NW, ... of tile T (piece pc: page block pc/kPieces of the
  // tile, 1 KB number pc%kPieces) into buffer T%NBUF: exactly kPer loads per wave per
  // tile, whatever the tile (a page past the context is read from page 0; its tokens
  // are masked), so the vmcnt arithmetic below is exact.  The page ids are wave-uniform
  // scalar loads of the table (indexes clamped to the context's last page, so every read
  // stays inside the sequence's row), fetched one iteration before the copy.
  auto fetch_ids = [&](int T, int (&raw)[kPer]) {
#pragma unroll
    for (int u = 0; u < kPer; ++u) raw[u] = pt[min(4 * T + (wave + u * NW) / kPieces, last_page)];
  };
  auto copy_tile = [&](int T, const int (&raw)[kPer]) {
    bf16_t *buf = &kv[T % NBUF][0];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int pc = wave + u * NW;
      const int P = 4 * T + pc / kPieces;
      const bool b = P <= last_page && (unsigned)raw[u] >= (unsigned)n_pages;
      bad |= b;
      const int pid = (P <= last_page && !b) ? raw[u] : 0;
      const int j = pc % kPieces;
      const bf16_t *src = pool + ((long)pid * Hkv + g) * (32 * D) + j * 512 + lane * 8;
      bf16_t *dst = buf + (pc / kPieces) * kSlot + j * 512;
      __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
    }
  };
  int idn[kPer];
  for (int T = 0; T < NBUF - 1 && T < n_tiles; ++T) {
    fetch_ids(T, idn);
    copy_tile(T, idn);
  }
  if (NBUF - 1 < n_tiles) fetch_ids(NBUF - 1, idn);

  float M = neg_inf(), L = 0.f, m = neg_inf(), l = 0.f;
  float O[D / 4];
  f32x4 o[D / 16];
#pragma unroll
  for (int e = 0; e < D / 4; ++e) O[e] = 0.f;
  for (int T = 0; T < n_tiles; ++T) {
    // tile T landed (at most `ahead` later tiles still in flight), then the barrier:
    // every wave's pieces are visible and every wave is done with tile T-1's buffer
    const int ahead = min(NBUF - 2, n_tiles - 1 - T);
    if (ahead >= 2) wait_vmem<2 * kPer>();
    else if (ahead == 1) wait_vmem<kPer>();
    else wait_vmem<0>();
    __syncthreads();
    if (T + NBUF - 1 < n_tiles) {
      copy_tile(T + NBUF - 1, idn);
      if (T + NBUF < n_tiles) fetch_ids(T + NBUF, idn);
    }
    const int t0 = T * kTile;
    const int s0 = t0 - t0 % split_tokens;
    if (t0 == s0) {
      m = neg_inf();
      l = 0.f;
#pragma unroll
      for (int db = 0; db < D / 16; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (t0 <= w_max) {
      const bf16_t *pg[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) pg[k] = &kv[T % NBUF][k * kSlot];
      Half<D> hk;
      load_k<D, FromLdsUntracked>(hk, pg);
      lds_settle<D>(hk);
      bf16x8 pop[2];
      float alpha, m_new, l_new;
      attn_scores<D>(hk, t0, qop, pos, cscale, m, l, pop, alpha, m_new, l_new);
      Half<D> hv;
      load_v<D, FromLdsUntracked>(hv, pg);
      lds_settle<D>(hv);
      if (t0 <= w_min)
        attn_values<D, false>(hv, t0, pos, p_max + 1, pop, alpha, m_new, l_new, m, l, o);
      else
        attn_values<D, true>(hv, t0, pos, p_max + 1, pop, alpha, m_new, l_new, m, l, o);
    }
    // end of a split: fold its state into the merged state of every column it reached
    if (t0 + kTile >= min(s0 + split_tokens, p_max + 1) && s0 <= pos) {
      float os[D / 4];
#pragma unroll
      for (int db = 0; db < D / 16; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) os[db * 4 + i] = o[db][i];
      if (s0 == 0) {
        M = m;
        L = l;
#pragma unroll
        for (int e = 0; e < D / 4; ++e) O[e] = os[e];
      } else {
        merge_state<D / 4>(M, L, O, m, l, os);
      }
    }
  }
  // a page id outside the pool seen by any wave marks the whole workgroup's rows NaN
  if (__syncthreads_or(bad)) L = __builtin_nanf("");
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
  if (a.n_rows == 0) return hipSuccess;
  const int n_sg = a.ctx_bound / a.split_tokens;  // full splits a row can have
  const long slots = (long)(n_sg + a.split_tokens / kTile) * a.Hkv * a.n_rows;
  if (slots > 0x7fffffffL) return hipErrorInvalidValue;
  dim3 grid((unsigned)slots);
  if (a.D == 128)
    hipLaunchKernelGGL(attn_decode_split_kernel<128>, grid, dim3(64), 0, st, a.q, a.q_row_stride,
                       a.ctx_len, a.page_table, a.page_stride, a.pool, a.n_pages, a.Hkv, a.G,
                       a.split_tokens, a.ctx_bound, a.n_rows, n_sg, a.cscale, a.part_o, a.part_ml,
                       a.max_splits);
  else
    hipLaunchKernelGGL(attn_decode_split_kernel<64>, grid, dim3(64), 0, st, a.q, a.q_row_stride,
                       a.ctx_len, a.page_table, a.page_stride, a.pool, a.n_pages, a.Hkv, a.G,
                       a.split_tokens, a.ctx_bound, a.n_rows, n_sg, a.cscale, a.part_o, a.part_ml,
                       a.max_splits);
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

constexpr int kPrefillNcb = 1, kPrefillWaves = 8;

hipError_t launch_attn_prefill(const AttnPrefillArgs &a, hipStream_t st) {
  constexpr int NW = 8, NBUF = 4;
  const int QT = NW * (16 / a.G);
  const long blocks = (long)(a.n_tok + QT - 1) / QT + a.n_seqs;  // bound on sum of ceil(n_s / QT)
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  dim3 grid((unsigned)blocks, a.Hkv);
  if (a.D == 128)
    hipLaunchKernelGGL((attn_prefill_kernel<128, NW, NBUF>), grid, dim3(64 * NW), 0, st, a.q, a.q_row_stride,
                       a.cu, a.start_pos, a.n_seqs, a.page_table, a.page_stride, a.pool, a.n_pages,
                       a.Hkv, a.G, a.split_tokens, a.ctx_bound, a.cscale, a.out);
  else
    hipLaunchKernelGGL((attn_prefill_kernel<64, NW, NBUF>), grid, dim3(64 * NW), 0, st, a.q, a.q_row_stride,
                       a.cu, a.start_pos, a.n_seqs, a.page_table, a.page_stride, a.pool, a.n_pages,
                       a.Hkv, a.G, a.split_tokens, a.ctx_bound, a.cscale, a.out);
  return hipGetLastError();
}

}  // namespace ril
