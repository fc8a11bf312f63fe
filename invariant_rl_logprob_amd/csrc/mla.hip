// Absorbed multi-head latent attention (MLA) over a paged latent cache, dense and over
// an indexer's top-k selection (S5, S8, S9).
//
// Every head reads the same cached latent row per token: 512 latent dims + 64 rope
// dims (576 bf16).  Scores use all 576 dims; values are the first 512 (the absorbed
// form of the Bitwise-consistent RL post, section 3: MLA compresses KV before caching).
//
// The split is a model constant and splits merge left to right, as for GQA.  Decode
// runs one workgroup per (row, split, group of 64 heads): 8 waves in 4 pairs, pair p
// owning heads 64*group + 16p .. +15 as its MFMA columns.  The pair's first wave
// computes the scores and the online-softmax step and hands P and the rescale factor to
// its partner through LDS; each wave of the pair then accumulates half of the 512 value
// dims (a column's o^T elements are independent, so the split of dims changes no bits).  The trainer-side recompute
// runs the very same kernels with one "row" per query token (context = position + 1),
// after writing the chunk's latents: prefill and decode are one code path.
//
// Dense: a split covers `split_tokens` consecutive positions in 64-token tiles.
// Sparse: a split covers `split_tokens` consecutive entries of the row's selection list
// (positions in descending order, -1 last: the list order is the accumulation order,
// post section 4.3), in 64-entry tiles gathered from their pages.
//
// Latent page (16 tokens), dense kind: one 16 x 576 block in the K-operand layout of
// attn_common.h (k_page_offset), so a tile's copy moves whole pages in that order.
// Sparse kind: the 16 rows token-major (element (t, d) at 576 t + d), then the 16 tokens'
// fp32 indexer keys: a selected token is gathered alone, and its 1152 bytes are then
// 9 whole cache lines (in the K layout they spread over 72 lines, 16 bytes of each).
// Per 64-token tile the workgroup copies the tile into LDS (double-buffered: the next
// tile is copied while the current one is computed) in the K layout up to a swizzle of
// its 16-byte units: LDS unit u of a page slot holds K-layout unit mla_swz(u).
// Score operands are 16-byte LDS reads.  Value operands come from the same tile through
// gfx950's transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group, lane i
// receives element i%4 of the 8-byte chunks addressed by lanes 4e + i/4, e = 0..3, so
// lanes pointing at 4 consecutive dims of 4 tokens hand each lane one dim of those 4
// tokens -- the V^T operand -- with no transposed copy.  Value entries at or beyond the
// row's bound are zeroed in the operand; their scores are masked.
#include <algorithm>
#include <utility>

#include "attn_common.h"
#include "kernels.h"

namespace ril {

constexpr int kMlaDqk = 576, kMlaDv = 512;
constexpr int kMlaPage = kPage * kMlaDqk;     // 9216 elements: one page's latent block
constexpr int kMlaSlot = kMlaPage + 64;       // LDS slot of a page: +128 B spreads the banks
constexpr int kMlaThreads = 512;              // 4 pairs of waves x 16 heads (H % 64 == 0)

// Within a page slot, 16-byte unit u sits at LDS unit mla_swz(u) (an involution: when
// bit 4, the parity of the 8-dim group, is set, it flips bits 2 and 3, the token half and
// the token quad within the page).  Without it the value operands' transposing reads,
// which take four tokens of each of two adjacent 8-dim groups per 16 lanes, read 256
// bytes apart: two-way LDS bank conflicts.  Of the maps that XOR one of bits 0-4 into
// others, this is the one under which both those reads and the score reads (16 bytes
// per lane, two page slots) run free of bank conflicts on gfx950's LDS (measured with
// its bank-conflict counter); flipping bit 3 alone cleared the value reads but made the
// score reads conflict two-way.  The map acts on bits 0-4 only, so adding 32 or more
// units to a unit adds the same to its place.
__device__ __forceinline__ int mla_swz(int u) { return u ^ (((u >> 4) & 1) * 12); }

// FP8 latent pages (Bitwise-consistent RL post, section 4.2: FP8 storage, one write path,
// one dequantizing read for every phase): a page's latent block is 16 x 576 E4M3 codes,
// token-major (code of (t, d) at byte 576 t + d, 9216 bytes), each the code of
// c * 2^-s (nearest even, magnitudes past 448 saturating, NaN kept with its sign) for the
// model's one latent scale exponent s; the sparse kind's fp32 indexer keys follow at byte
// 9216.  Every read takes the codes' values (exact in bf16) as the MFMA operands and
// applies 2^s outside them, as the GQA FP8 cache does: the scores' softmax constant
// carries it, and the fp32 value state is multiplied by it once, before the split's
// partial is stored.  A power of two commutes with every fp32 rounding in between, so
// this is attention over code * 2^s (outside fp32's subnormal and overflow ranges), the
// same in every phase.  Token-major keeps each token's codes in whole 16-byte units, so
// the sparse kind gathers a selected token with 16-byte copies.
constexpr int kMla8Page = kPage * kMlaDqk;  // 9216 bytes of codes per page
constexpr int kMla8Tile = kTile * kMlaDqk;  // 36864 bytes: one tile's codes

// ---------------------------------------------------------------------------
// S5 for MLA: one thread per (token, 16-byte unit) of the page: 72 latent units (bf16:
// K layout for the dense kind, token-major for the sparse kind) or 36 (FP8 codes,
// token-major), then (sparse) 32 units of the fp32 indexer key, token t's at byte
// latent_bytes + 512 t of the page.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void mla_kv_write_kernel(
    const bf16_t *__restrict__ c, int row_stride, const float *__restrict__ kidx, int n_tok, int mode,
    const int32_t *__restrict__ cu, const int32_t *__restrict__ start_pos, int n_seqs,
    const int32_t *__restrict__ ctx_len, const int32_t *__restrict__ page_table, int page_stride,
    bf16_t *__restrict__ pool, int page_elems, int n_pages, bool fp8, float inv_scale, bool token_major) {
  const int n_lat = fp8 ? kMlaDqk / 16 : kMlaDqk / 8;
  const int per_tok = n_lat + (kidx ? 32 : 0);
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
  uint8_t *page8 = reinterpret_cast<uint8_t *>(page);
  const int t = pos % kPage;
  if (u < n_lat) {
    const bf16_t *src = c + (long)j * row_stride;
    if (!fp8) {
      st16(page + (token_major ? t * kMlaDqk + u * 8 : k_page_offset(t, u * 8)), ld16(src + u * 8));
    } else {
      const u32x4 a = ld16(src + u * 16), b = ld16(src + u * 16 + 8);
      u32x4 codes;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t x = w < 2 ? a[2 * w] : b[2 * w - 4], y = w < 2 ? a[2 * w + 1] : b[2 * w - 3];
        const uint32_t lo = fp8_codes2(bf2f((bf16_t)(x & 0xffffu)) * inv_scale, bf2f((bf16_t)(x >> 16)) * inv_scale);
        const uint32_t hi = fp8_codes2(bf2f((bf16_t)(y & 0xffffu)) * inv_scale, bf2f((bf16_t)(y >> 16)) * inv_scale);
        codes[w] = lo | (hi << 16);
      }
      st16(page8 + t * kMlaDqk + u * 16, codes);
    }
  } else {
    const int w = u - n_lat;  // 4 floats per unit
    st16(page8 + (fp8 ? kMla8Page : 2 * kMlaPage) + t * 512 + w * 16, ld16(kidx + (long)j * 128 + w * 4));
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


// S^T = K Q^T for the 64-token tile in LDS (K layout, 4 page slots).  K step outermost:
// each step's four M-block operands are read while the previous step's MFMAs run; every
// accumulator still runs c = 0, 1, ... in order.  M-block mb of step c sits at byte
// (mb/2)*2*slot + (mb%2)*128 + c*1024 from this lane's base.
constexpr int kSlotBytes = 2 * kMlaSlot;
__device__ __forceinline__ void mla_tile_scores(f32x4 (&s)[4], const bf16_t *kt,
                                                const bf16x8 (&qop)[kMlaDqk / 32]) {
  const int lane = threadIdx.x & 63, grp = lane >> 4, r16 = lane & 15;
  const int rq = r16 >> 2, ri = r16 & 3;
  // this lane's page unit for M blocks 0/2 (token quad 0) and 1/3 (quad 1), swizzled
  const int u0 = grp * 16 + (rq & 1) * 4 + ri;
  const uint32_t slot = lds_addr(kt) + 2 * (rq >> 1) * kMlaSlot;
  const uint32_t base0 = slot + 16 * mla_swz(u0), base1 = slot + 16 * mla_swz(u0 + 8);
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) s[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4 a[2][4];
  auto issue = [&](auto cc) {
    constexpr int C = decltype(cc)::value;
    a[C & 1][0] = lds_rd128<C * 1024>(base0);
    a[C & 1][1] = lds_rd128<C * 1024>(base1);
    a[C & 1][2] = lds_rd128<C * 1024 + 2 * kSlotBytes>(base0);
    a[C & 1][3] = lds_rd128<C * 1024 + 2 * kSlotBytes>(base1);
  };
  issue(std::integral_constant<int, 0>{});
  static_for<kMlaDqk / 32>([&](auto cc) {
    constexpr int C = decltype(cc)::value;
    if constexpr (C + 1 < kMlaDqk / 32) {
      issue(std::integral_constant<int, C + 1>{});
      lds_wait<4>();
    } else {
      lds_wait<0>();
    }
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      settle(a[C & 1][mb]);
      s[mb] = mfma(as_bf16x8(a[C & 1][mb]), qop[C], s[mb]);
    }
  });
}

// The pair's exchange goes through LDS with untracked stores and loads and an asm barrier
// that waits for LDS operations only: a compiler-visible LDS access or __syncthreads
// would also wait for the next tile's copy in flight (vmcnt(0)) in the middle of a tile.
__device__ __forceinline__ void lds_wr32(uint32_t addr, float v) {
  asm volatile("ds_write_b32 %0, %1" ::"v"(addr), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_wr128(uint32_t addr, u32x4 v) {
  asm volatile("ds_write_b128 %0, %1" ::"v"(addr), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// V^T operands for the value dims 256*half .. +255: block b (dims 16b ..) of the 32-token
// step kc.  Lane (group g, i = lane % 16) gets V[32kc + 8g + j][256*half + 16b + i],
// j = 0..7, by two transposing reads (tokens +0..3 from base 0, +4..7 from base 1: the
// swizzle makes their distance lane-dependent); the block adds 512*b bytes (the swizzle
// does not depend on it) and the step 2 page slots.  Entries j >= n_valid read as 0.
struct MlaVBase {
  uint32_t b0, b1;
};
__device__ __forceinline__ MlaVBase mla_v_base(const bf16_t *kt, int half) {
  const int lane = threadIdx.x & 63, grp = lane >> 4, i = lane & 15;
  const int tok = 8 * grp + (i >> 2);
  const int e = k_page_offset(tok & 15, 256 * half + 4 * (i & 3));  // element; tokens +4..7: +64
  const uint32_t slot = lds_addr(kt) + 2 * (tok >> 4) * kMlaSlot;
  const int u = e >> 3, sub = 2 * (e & 7);  // unit, byte within it
  return MlaVBase{slot + 16 * mla_swz(u) + sub, slot + 16 * mla_swz(u + 8) + sub};
}
template <int B, int KC>
__device__ __forceinline__ void mla_v_issue(u32x2 (&r)[2], MlaVBase base) {
  r[0] = lds_rdtr<512 * B + 2 * kSlotBytes * KC>(base.b0);
  r[1] = lds_rdtr<512 * B + 2 * kSlotBytes * KC>(base.b1);
}
__device__ __forceinline__ bf16x8 mla_v_take(u32x2 (&r)[2], int n_valid) {
  settle(r[0]);
  settle(r[1]);
  u32x4 v = {r[0].x, r[0].y, r[1].x, r[1].y};
  if (n_valid < 8) v = keep_first(v, n_valid);  // entries at or beyond the bound read as 0
  return as_bf16x8(v);
}

// o^T = o^T * alpha + V^T P^T for value dims 256*half .. +255.  MASK: some entries of the
// tile are at or beyond the bound (n_live < 64).  The next dim block's operands are read
// while this block's two MFMAs run.  (alpha = 1 for every column of the wave -- no new
// maximum -- leaves o unchanged bit for bit, so the products are skipped then.)
template <bool MASK>
__device__ __forceinline__ void mla_tile_values(f32x4 (&o)[kMlaDv / 32], const bf16_t *kt, int half,
                                                const bf16x8 (&pop)[2], float alpha, int n_live) {
  const int grp = (threadIdx.x & 63) >> 4;
  const int nv0 = MASK ? n_live - 8 * grp : 8, nv1 = MASK ? n_live - (32 + 8 * grp) : 8;
  const MlaVBase base = mla_v_base(kt, half);
  if (__any(alpha != 1.f)) {
#pragma unroll
    for (int b = 0; b < kMlaDv / 32; ++b) o[b] = o[b] * alpha;
  }
  // token step 0 for every dim block, then step 1: a block's two MFMAs are 16 apart, so
  // the second never waits for the first (per element: rescale, step 0, step 1)
  u32x2 r[2][2];
  mla_v_issue<0, 0>(r[0], base);
  static_for<2 * (kMlaDv / 32)>([&](auto ii) {
    constexpr int I = decltype(ii)::value, KC = I / (kMlaDv / 32), B = I % (kMlaDv / 32);
    if constexpr (I + 1 < 2 * (kMlaDv / 32)) {
      constexpr int KN = (I + 1) / (kMlaDv / 32), BN = (I + 1) % (kMlaDv / 32);
      mla_v_issue<BN, KN>(r[(I + 1) & 1], base);
      lds_wait<2>();
    } else {
      lds_wait<0>();
    }
    o[B] = mfma(mla_v_take(r[I & 1], KC == 0 ? nv0 : nv1), pop[KC], o[B]);
  });
}

// This wave's half of the split's o (dims 256*half ..), and (m, l) from the scoring wave.
__device__ __forceinline__ void mla_store_partial(float *part_o, float *part_ml, long base, int half,
                                                  const f32x4 (&o)[kMlaDv / 32], float m, float l) {
  const int grp = (threadIdx.x & 63) >> 4;
  float *po = part_o + base * kMlaDv + 256 * half + grp * 4;
#pragma unroll
  for (int b = 0; b < kMlaDv / 32; ++b) *reinterpret_cast<f32x4 *>(po + b * 16) = o[b];
  if (half == 0 && grp == 0) {
    part_ml[base * 2] = m;
    part_ml[base * 2 + 1] = l;
  }
}

// K-layout unit v (16 bytes, 0 .. 1151) of a page block -> (token t, first dim d0): the
// inverse of k_page_offset.
__device__ __forceinline__ void mla_unit_td(int v, int &t, int &d0) {
  const int c = v >> 6, g = (v >> 4) & 3, a = (v >> 3) & 1, bq = (v >> 2) & 1, cc = v & 3;
  t = 8 * bq + 4 * a + cc;
  d0 = 32 * c + 8 * g;
}

// ---------------------------------------------------------------------------
// S8: grid (splits, H/64, rows), 512 threads; SPARSE: splits of the row's selection.
// Per tile: the scoring wave of each pair computes the scores of its 16 heads and the
// online-softmax step and hands P and alpha over; both waves of the pair accumulate their
// half of the value dims.  Tile t+1 is copied into the other LDS buffer (72 direct-to-LDS
// loads of 1 KB, 9 per wave, each filling 64 consecutive LDS units of one page slot with
// the swizzled page units) while tile t is computed.  Sparse: each wave holds, one entry per lane, the positions of
// the tile after next and the page ids of the next tile, so no copy waits on a lookup.
// ---------------------------------------------------------------------------
template <bool SPARSE>
__global__ __launch_bounds__(512) void mla_split_kernel(
    const bf16_t *__restrict__ q, int mode, int row0, const int32_t *__restrict__ ctx_len,
    const int32_t *__restrict__ cu, const int32_t *__restrict__ start_pos, int n_seqs,
    const int32_t *__restrict__ page_table, int page_stride, const bf16_t *__restrict__ pool, int page_elems,
    int n_pages, int H, const int32_t *__restrict__ sel, int topk, int split_tokens, int ctx_bound,
    float cscale, float *__restrict__ part_o, float *__restrict__ part_ml, int max_splits) {
  __shared__ __attribute__((aligned(16))) bf16_t kt[2][4 * kMlaSlot];
  __shared__ u32x4 xp[4][2][64];  // P^T operands handed from each pair's scoring wave
  __shared__ float xa[4][64];     // and its rescale factor, per lane
  const int split = blockIdx.x, hg = blockIdx.y, r = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, r16 = lane & 15;
  const int pair = wave & 3, half = wave >> 2;  // waves p and p+4 share SIMD p
  int seq, ctx;
  long qrow;
  mla_row(mode, r, row0, ctx_len, cu, start_pos, n_seqs, seq, ctx, qrow);
  const int n_all = SPARSE ? min(ctx, topk) : ctx;  // positions, or selected entries
  const int s0 = split * split_tokens;
  if (ctx < 1 || ctx > ctx_bound || s0 >= n_all) return;  // uniform over the workgroup
  const int s1 = min(n_all, s0 + split_tokens);
  const int n_tiles = (s1 - s0 + kTile - 1) / kTile;
  const int32_t *pt = page_table + (long)seq * page_stride;
  const int32_t *rsel = SPARSE ? sel + (long)r * topk : nullptr;
  bool bad = false;
  // dense: page ids of the split, lane i holding page index s0/16 + i (+64 in pidB);
  // pages past the context read as page 0 (their tokens are masked)
  int pidA = 0, pidB = 0;
  // sparse: per lane = entry of a tile: position (-1: none) and page id
  int pos1 = -1, pid1 = 0, pos2 = -1;
  auto entry_pos = [&](int t) {  // position of entry `lane` of tile t
    const int e = s0 + t * kTile + lane;
    int p = -1;
    if (t < n_tiles && e < n_all) {
      p = rsel[e];
      if (p < 0 || p >= ctx) {
        bad = true;  // a listed entry that is not a position of the row
        p = -1;
      }
    }
    return p;
  };
  auto entry_pid = [&](int p) {
    if (p < 0) return 0;
    const int id = pt[p / kPage];
    const bool b = (unsigned)id >= (unsigned)n_pages;
    bad |= b;
    return b ? 0 : id;
  };
  if (!SPARSE) {
    const int first = s0 / kPage, last = (ctx - 1) / kPage;
    const int a = first + lane, b = first + 64 + lane;
    pidA = pt[min(a, last)];
    pidB = pt[min(b, last)];
    bad = (a <= last && (unsigned)pidA >= (unsigned)n_pages) || (b <= last && (unsigned)pidB >= (unsigned)n_pages);
    pidA = (a <= last && (unsigned)pidA < (unsigned)n_pages) ? pidA : 0;
    pidB = (b <= last && (unsigned)pidB < (unsigned)n_pages) ? pidB : 0;
  } else {
    pos1 = entry_pos(0);
    pid1 = entry_pid(pos1);
    pos2 = entry_pos(1);
  }
  const int head = 64 * hg + 16 * pair + r16;
  const bool col_ok = head < H;
  bf16x8 qop[kMlaDqk / 32];
  if (half == 0) mla_load_q(qop, q, qrow, H, head, col_ok);

  // copy tile t into buffer t&1: wave w copies page slot w % 4, its 1 KB pieces w / 4,
  // w / 4 + 2, ... (LDS unit 64 j + lane of the slot takes page unit mla_swz(64 j + lane))
  constexpr int kPieces = kMlaPage / 512;  // 18 per page slot
  const int my_ps = wave & 3, j0 = wave >> 2;
  const int lane_unit = mla_swz(lane);     // dense: the swizzle stays within a piece
  auto copy_tile = [&](int t) {
    bf16_t *buf = &kt[t & 1][0] + my_ps * kMlaSlot;
    if (!SPARSE) {
      const int idx = 4 * t + my_ps;  // page index within the split (< 128), uniform
      const int pid = idx < 64 ? __builtin_amdgcn_readlane(pidA, idx) : __builtin_amdgcn_readlane(pidB, idx - 64);
      const bf16_t *page = pool + (long)pid * page_elems;  // uniform: one scalar base per tile
      const int off = lane_unit * 8 + j0 * 512;
#pragma unroll
      for (int i = 0; i < kPieces / 2; ++i)
        __builtin_amdgcn_global_load_lds(page + (off + i * 1024), buf + j0 * 512 + i * 1024, 16, 0, 0);
    } else {
#pragma unroll 1
      for (int i = 0; i < kPieces / 2; ++i) {
        const int j = j0 + 2 * i;
        int tt, d0;
        mla_unit_td(mla_swz(64 * j + lane), tt, d0);
        const int e = 16 * my_ps + tt;  // entry of the tile
        const int p = __shfl(pos1, e, 64), id = __shfl(pid1, e, 64);
        const bf16_t *src = pool + (long)id * page_elems + (p >= 0 ? (p % kPage) * kMlaDqk + d0 : 0);
        __builtin_amdgcn_global_load_lds(src, buf + j * 512, 16, 0, 0);
      }
    }
  };
  const uint32_t xp_lane = lds_addr(&xp[pair][0][0]) + 16 * lane, xa_lane = lds_addr(&xa[pair][0]) + 4 * lane;
  float m = neg_inf(), l = 0.f;
  f32x4 o[kMlaDv / 32];
#pragma unroll
  for (int b = 0; b < kMlaDv / 32; ++b) o[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  copy_tile(0);
  for (int t = 0; t < n_tiles; ++t) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's pieces of tile t landed
    __syncthreads();  // every piece of tile t is visible; every wave is done with tile t-1
    if (t + 1 < n_tiles) {
      if (SPARSE) {
        pid1 = entry_pid(pos2);  // positions of tile t+1 were read last iteration
        pos1 = pos2;
        pos2 = entry_pos(t + 2);
      }
      copy_tile(t + 1);
    }
    const int t0 = s0 + t * kTile;
    const bf16_t *tile = &kt[t & 1][0];
    bf16x8 pop[2];
    float alpha;
    if (half == 0) {
      f32x4 s[4];
      mla_tile_scores(s, tile, qop);
      float m_new, l_new;
      tile_softmax(s, t0, n_all - 1, cscale, m, l, pop, alpha, m_new, l_new);
      m = m_new;
      l = l_new;
      lds_wr128(xp_lane, __builtin_bit_cast(u32x4, pop[0]));
      lds_wr128(xp_lane + 1024, __builtin_bit_cast(u32x4, pop[1]));
      lds_wr32(xa_lane, alpha);
    }
    lds_barrier();  // P and alpha of every pair are in LDS
    if (half == 1) {
      u32x4 p0 = lds_rd128<0>(xp_lane), p1 = lds_rd128<1024>(xp_lane);
      int a = lds_rd32<0>(xa_lane);
      lds_wait<0>();
      settle(p0);
      settle(p1);
      settle(a);
      pop[0] = as_bf16x8(p0);
      pop[1] = as_bf16x8(p1);
      alpha = __builtin_bit_cast(float, a);
    }
    const int n_live = n_all - t0;
    if (n_live >= kTile)
      mla_tile_values<false>(o, tile, half, pop, alpha, n_live);
    else
      mla_tile_values<true>(o, tile, half, pop, alpha, n_live);
  }
  bad = __syncthreads_or(bad);
  if (bad) l = __builtin_nanf("");
  if (!col_ok) return;
  mla_store_partial(part_o, part_ml, ((long)r * H + head) * max_splits + split, half, o, m, l);
}

// ---------------------------------------------------------------------------
// S8 over FP8 latent pages: the same grid, waves, tile routines and order as
// mla_split_kernel, with the tile dequantized into LDS before it is used.  Each tile's
// codes (36 KB) are copied two tiles ahead into a 2-slot ring by direct-to-LDS loads (36
// pieces of 1 KB: wave w copies pieces w, w + 8, ..), then all 512 threads turn them
// into the bf16 tile in the K layout and swizzle mla_split_kernel reads (the codes'
// values, exact), and the scores and values run on it unchanged, with 2^s in the
// softmax constant and on the stored state.  Per tile: wait for this wave's pieces of the tile,
// barrier (the codes are in, every wave is done with the previous bf16 tile),
// dequantize, barrier (the bf16 tile is in, the codes' slot is free), copy tile t + 2
// into that slot, compute.
// ---------------------------------------------------------------------------
template <int OFF>
__device__ __forceinline__ u32x2 lds_rd64(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "LDS offset field");
  u32x2 r;
  asm volatile("ds_read_b64 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
template <int OFF>
__device__ __forceinline__ void lds_wr128(uint32_t addr, u32x4 v) {
  static_assert(OFF >= 0 && OFF < 65536, "LDS offset field");
  asm volatile("ds_write_b128 %0, %1 offset:%2" ::"v"(addr), "v"(v), "i"(OFF) : "memory");
}

template <bool SPARSE>
__global__ __launch_bounds__(512) void mla_split_fp8_kernel(
    const bf16_t *__restrict__ q, int mode, int row0, const int32_t *__restrict__ ctx_len,
    const int32_t *__restrict__ cu, const int32_t *__restrict__ start_pos, int n_seqs,
    const int32_t *__restrict__ page_table, int page_stride, const uint8_t *__restrict__ pool, int page_bytes,
    int n_pages, int H, const int32_t *__restrict__ sel, int topk, int split_tokens, int ctx_bound,
    float cscale, float scale, float *__restrict__ part_o, float *__restrict__ part_ml, int max_splits) {
  __shared__ __attribute__((aligned(16))) bf16_t kt[4 * kMlaSlot];   // the tile, dequantized
  __shared__ __attribute__((aligned(16))) uint8_t k8[2][kMla8Tile];  // codes of the next tiles
  __shared__ u32x4 xp[4][2][64];
  __shared__ float xa[4][64];
  const int split = blockIdx.x, hg = blockIdx.y, r = blockIdx.z;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63, r16 = lane & 15;
  const int pair = wave & 3, half = wave >> 2;
  int seq, ctx;
  long qrow;
  mla_row(mode, r, row0, ctx_len, cu, start_pos, n_seqs, seq, ctx, qrow);
  const int n_all = SPARSE ? min(ctx, topk) : ctx;
  const int s0 = split * split_tokens;
  if (ctx < 1 || ctx > ctx_bound || s0 >= n_all) return;  // uniform over the workgroup
  const int s1 = min(n_all, s0 + split_tokens);
  const int n_tiles = (s1 - s0 + kTile - 1) / kTile;
  const int32_t *pt = page_table + (long)seq * page_stride;
  const int32_t *rsel = SPARSE ? sel + (long)r * topk : nullptr;
  bool bad = false;
  int pidA = 0, pidB = 0;  // dense: page ids of the split (lane i: page s0/16 + i, +64)
  int pos_c = -1, pid_c = 0, pos_n = -1;  // sparse, per lane = entry: the tile to copy next, the one after
  auto entry_pos = [&](int t) {
    const int e = s0 + t * kTile + lane;
    int p = -1;
    if (t < n_tiles && e < n_all) {
      p = rsel[e];
      if (p < 0 || p >= ctx) {
        bad = true;
        p = -1;
      }
    }
    return p;
  };
  auto entry_pid = [&](int p) {
    if (p < 0) return 0;
    const int id = pt[p / kPage];
    const bool b = (unsigned)id >= (unsigned)n_pages;
    bad |= b;
    return b ? 0 : id;
  };
  if (!SPARSE) {
    const int first = s0 / kPage, last = (ctx - 1) / kPage;
    const int a = first + lane, b = first + 64 + lane;
    pidA = pt[min(a, last)];
    pidB = pt[min(b, last)];
    bad = (a <= last && (unsigned)pidA >= (unsigned)n_pages) || (b <= last && (unsigned)pidB >= (unsigned)n_pages);
    pidA = (a <= last && (unsigned)pidA < (unsigned)n_pages) ? pidA : 0;
    pidB = (b <= last && (unsigned)pidB < (unsigned)n_pages) ? pidB : 0;
  } else {
    pos_c = entry_pos(0);
    pid_c = entry_pid(pos_c);
  }
  const int head = 64 * hg + 16 * pair + r16;
  const bool col_ok = head < H;
  bf16x8 qop[kMlaDqk / 32];
  if (half == 0) mla_load_q(qop, q, qrow, H, head, col_ok);

  // copy tile t's codes into slot t & 1: piece i (1 KB) = bytes 1024 i .. of the tile;
  // dense: page i / 9 of the tile, its bytes 1024 (i % 9) ..; sparse: 16-byte unit
  // u = 64 i + lane is chunk u % 36 of entry u / 36
  constexpr int kPieces8 = kMla8Tile / 1024;  // 36
  auto copy_tile = [&](int t) {
    uint8_t *buf = &k8[t & 1][0];
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      const int i = wave + 8 * k;
      if (k < 4 || wave < kPieces8 - 32) {
        const uint8_t *src;
        if (!SPARSE) {
          const int idx = 4 * t + i / 9;  // page index within the split (< 128), uniform
          const int pid = idx < 64 ? __builtin_amdgcn_readlane(pidA, idx) : __builtin_amdgcn_readlane(pidB, idx - 64);
          src = pool + (long)pid * page_bytes + (i % 9) * 1024 + lane * 16;
        } else {
          const int u = 64 * i + lane, e = u / 36, ch = u - 36 * e;
          const int p = __shfl(pos_c, e, 64), id = __shfl(pid_c, e, 64);
          src = pool + (long)id * page_bytes + (p >= 0 ? (p % kPage) * kMlaDqk + ch * 16 : 0);
        }
        __builtin_amdgcn_global_load_lds((void *)src, (void *)(buf + i * 1024), 16, 0, 0);
      }
    }
  };
  // dequantize slot t & 1 into kt: thread i converts units (i & 127) + 128 k, k = 0..8,
  // of page slot i / 128 (K layout: the unit holds dims d0 .. d0 + 7 of one token t of
  // the slot, whose codes sit at byte 576 (16 slot + t) + d0 of the staged tile).  Adding
  // 128 to a unit adds 64 to d0 and 2048 bytes to its swizzled LDS place, so the nine
  // reads and writes share one address each with immediate offsets.
  uint32_t dq_src, dq_dst;
  {
    const int ps = threadIdx.x >> 7, u0 = threadIdx.x & 127;
    int tt, d0;
    mla_unit_td(u0, tt, d0);
    dq_src = (16 * ps + tt) * kMlaDqk + d0;
    dq_dst = lds_addr(kt) + ps * (2 * kMlaSlot) + 16 * mla_swz(u0);
  }
  auto dequant = [&](int t) {
    const uint32_t src = lds_addr(&k8[t & 1][0]) + dq_src;
    u32x2 c[9];
    static_for<9>([&](auto k_) { c[decltype(k_)::value] = lds_rd64<64 * decltype(k_)::value>(src); });
    lds_wait<0>();
    static_for<9>([&](auto k_) {
      constexpr int k = decltype(k_)::value;
      settle(c[k]);
      lds_wr128<2048 * k>(dq_dst, fp8_operand(c[k][0], c[k][1]));
    });
  };
  const uint32_t xp_lane = lds_addr(&xp[pair][0][0]) + 16 * lane, xa_lane = lds_addr(&xa[pair][0]) + 4 * lane;
  float m = neg_inf(), l = 0.f;
  f32x4 o[kMlaDv / 32];
#pragma unroll
  for (int b = 0; b < kMlaDv / 32; ++b) o[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  copy_tile(0);
  if (SPARSE) {
    pos_c = entry_pos(1);
    pid_c = entry_pid(pos_c);
  }
  if (n_tiles > 1) copy_tile(1);
  if (SPARSE) pos_n = entry_pos(2);
  for (int t = 0; t < n_tiles; ++t) {
    // this wave's pieces of tile t have landed (those of tile t + 1, issued later, may not)
    if (t + 1 < n_tiles) {
      if (wave < kPieces8 - 32) wait_vmem<5>(); else wait_vmem<4>();
    } else {
      wait_vmem<0>();
    }
    asm volatile("s_barrier" ::: "memory");
    if (SPARSE && t + 2 < n_tiles) pid_c = entry_pid(pos_n);  // tile t + 2's pages, used below
    dequant(t);
    lds_barrier();  // the bf16 tile is complete; slot t & 1 is free
    if (t + 2 < n_tiles) {
      if (SPARSE) pos_c = pos_n;
      copy_tile(t + 2);
      if (SPARSE) pos_n = entry_pos(t + 3);
    }
    const int t0 = s0 + t * kTile;
    bf16x8 pop[2];
    float alpha;
    if (half == 0) {
      f32x4 sc[4];
      mla_tile_scores(sc, kt, qop);
      float m_new, l_new;
      tile_softmax(sc, t0, n_all - 1, cscale, m, l, pop, alpha, m_new, l_new);
      m = m_new;
      l = l_new;
      lds_wr128(xp_lane, __builtin_bit_cast(u32x4, pop[0]));
      lds_wr128(xp_lane + 1024, __builtin_bit_cast(u32x4, pop[1]));
      lds_wr32(xa_lane, alpha);
    }
    lds_barrier();
    if (half == 1) {
      u32x4 p0 = lds_rd128<0>(xp_lane), p1 = lds_rd128<1024>(xp_lane);
      int a = lds_rd32<0>(xa_lane);
      lds_wait<0>();
      settle(p0);
      settle(p1);
      settle(a);
      pop[0] = as_bf16x8(p0);
      pop[1] = as_bf16x8(p1);
      alpha = __builtin_bit_cast(float, a);
    }
    const int n_live = n_all - t0;
    if (n_live >= kTile)
      mla_tile_values<false>(o, kt, half, pop, alpha, n_live);
    else
      mla_tile_values<true>(o, kt, half, pop, alpha, n_live);
  }
  bad = __syncthreads_or(bad);
  if (bad) l = __builtin_nanf("");
  if (!col_ok) return;
#pragma unroll
  for (int b = 0; b < kMlaDv / 32; ++b) o[b] = o[b] * scale;  // 2^s: exact
  mla_store_partial(part_o, part_ml, ((long)r * H + head) * max_splits + split, half, o, m, l);
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
  const long total = (long)a.n_tok * ((a.fp8 ? kMlaDqk / 16 : kMlaDqk / 8) + (a.kidx ? 32 : 0));
  if (total == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((total + 255) / 256);
  hipLaunchKernelGGL(mla_kv_write_kernel, dim3(blocks), dim3(256), 0, st, a.c, a.row_stride, a.kidx, a.n_tok,
                     a.mode, a.cu, a.start_pos, a.n_seqs, a.ctx_len, a.page_table, a.page_stride, a.pool,
                     a.page_elems, a.n_pages, a.fp8, a.inv_scale, a.token_major);
  return hipGetLastError();
}

hipError_t launch_mla_split(const MlaAttnArgs &a, hipStream_t st) {
  if (a.n_rows == 0) return hipSuccess;
  if (a.fp8) {
    if (!a.sel && a.split_tokens > 2048) return hipErrorInvalidValue;  // two 64-page id registers
    const int n_bound = a.sel ? std::min(a.ctx_bound, a.topk) : a.ctx_bound;
    dim3 grid((n_bound + a.split_tokens - 1) / a.split_tokens, a.H / 64, a.n_rows);
    const uint8_t *pool = reinterpret_cast<const uint8_t *>(a.pool);
    if (a.sel)
      hipLaunchKernelGGL(mla_split_fp8_kernel<true>, grid, dim3(kMlaThreads), 0, st, a.q, a.mode, a.row0,
                         a.ctx_len, a.cu, a.start_pos, a.n_seqs, a.page_table, a.page_stride, pool,
                         2 * a.page_elems, a.n_pages, a.H, a.sel, a.topk, a.split_tokens, a.ctx_bound,
                         a.cscale * a.scale, a.scale, a.part_o, a.part_ml, a.max_splits);
    else
      hipLaunchKernelGGL(mla_split_fp8_kernel<false>, grid, dim3(kMlaThreads), 0, st, a.q, a.mode, a.row0,
                         a.ctx_len, a.cu, a.start_pos, a.n_seqs, a.page_table, a.page_stride, pool,
                         2 * a.page_elems, a.n_pages, a.H, nullptr, 0, a.split_tokens, a.ctx_bound,
                         a.cscale * a.scale, a.scale, a.part_o, a.part_ml, a.max_splits);
    return hipGetLastError();
  }
  if (a.sel) {
    const int n_bound = std::min(a.ctx_bound, a.topk);
    dim3 grid((n_bound + a.split_tokens - 1) / a.split_tokens, a.H / 64, a.n_rows);
    hipLaunchKernelGGL(mla_split_kernel<true>, grid, dim3(kMlaThreads), 0, st, a.q, a.mode, a.row0, a.ctx_len,
                       a.cu, a.start_pos, a.n_seqs, a.page_table, a.page_stride, a.pool, a.page_elems,
                       a.n_pages, a.H, a.sel, a.topk, a.split_tokens, a.ctx_bound, a.cscale, a.part_o,
                       a.part_ml, a.max_splits);
  } else {
    if (a.split_tokens > 2048) return hipErrorInvalidValue;  // two 64-page id registers
    dim3 grid((a.ctx_bound + a.split_tokens - 1) / a.split_tokens, a.H / 64, a.n_rows);
    hipLaunchKernelGGL(mla_split_kernel<false>, grid, dim3(kMlaThreads), 0, st, a.q, a.mode, a.row0, a.ctx_len,
                       a.cu, a.start_pos, a.n_seqs, a.page_table, a.page_stride, a.pool, a.page_elems,
                       a.n_pages, a.H, nullptr, 0, a.split_tokens, a.ctx_bound, a.cscale, a.part_o,
                       a.part_ml, a.max_splits);
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
