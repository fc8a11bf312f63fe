// Paged GQA prefill attention (S10): the trainer's recompute, and any mixed batch of
// prefill chunks and one-token decode segments.  Every query row runs the decode chain
// of attn.hip exactly (same tile routine, split boundaries and merge rule, from
// attn_common.h), with its states held in registers (Bitwise-consistent RL post,
// section 2: phase consistency; section 4.2: one read path shared by prefill, decode
// and the trainer).
//
// Two kernels, the same per-column arithmetic: attn_prefill2_kernel (bf16 cache: two
// 16-column blocks per wave, each LDS operand read feeding both) and attn_prefill_kernel
// (FP8 cache: one block per wave, the codes dequantized per operand).
#include <type_traits>

#include "attn_common.h"
#include "kernels.h"

namespace ril {

// ---------------------------------------------------------------------------
// S10: prefill attention over the FP8 cache.  grid (workgroup bound, Hkv); a workgroup of NW waves covers
// QT = NW*(16/G) consecutive query tokens of one sequence for one kv head, wave w owning
// one block of 16 MFMA columns (16/G tokens x G heads).  The workgroup walks the 64-token
// KV tiles of its context in order.  Each tile is copied once into LDS by direct-to-LDS
// loads spread over the waves, NBUF-1 tiles ahead of the tile being computed, and read
// by every wave.  Per column the arithmetic is the decode chain exactly: the same
// attn_scores / attn_values per tile, a fresh state per split and merge_state at each
// split's end, with per-column predication (MAYBE_INACTIVE) for tiles and splits past
// the column's position.  Split and merged states stay in registers.
// ---------------------------------------------------------------------------
// LDS slot of one page block in bytes (K then V, 16*D values each, 2 bytes per value in
// bf16 and 1 in FP8), padded by 128 bytes so the two pages one K-operand load touches fall
// on different banks.
template <int D, bool FP8>
constexpr int lds_page_bytes() { return (FP8 ? 32 * D : 64 * D) + 128; }

template <int D, int NW, int NBUF, bool FP8>
__global__ __launch_bounds__(512) void attn_prefill_kernel(
    const bf16_t *__restrict__ q, int q_row_stride, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ start_pos, int n_seqs, const int32_t *__restrict__ page_table,
    int page_stride, const bf16_t *__restrict__ pool, int n_pages, int Hkv, int G,
    int split_tokens, int ctx_bound, float cscale, bf16_t *__restrict__ out, float k_scale, float v_scale) {
  static_assert(NW >= 1 && NW <= 8, "at most 512 threads (the launch bound)");
  static_assert(NBUF >= 2 && NBUF <= 4, "tiles in flight");
  constexpr int kSlotB = lds_page_bytes<D, FP8>();
  constexpr int kPageB = FP8 ? 32 * D : 64 * D;  // bytes of one page block in the pool
  constexpr int kPieces = kPageB / 1024;         // 1 KB pieces per page block
  static_assert((4 * kPieces) % NW == 0, "every wave copies the same number of pieces");
  constexpr int kPer = 4 * kPieces / NW;         // pieces (= vector-memory ops) per wave per tile
  __shared__ __attribute__((aligned(16))) uint8_t kv[NBUF][4 * kSlotB];
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
    uint8_t *buf = &kv[T % NBUF][0];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int pc = wave + u * NW;
      const int P = 4 * T + pc / kPieces;
      const bool b = P <= last_page && (unsigned)raw[u] >= (unsigned)n_pages;
      bad |= b;
      const int pid = (P <= last_page && !b) ? raw[u] : 0;
      const int j = pc % kPieces;
      const uint8_t *src = reinterpret_cast<const uint8_t *>(pool) + ((long)pid * Hkv + g) * kPageB + j * 1024 +
                           lane * 16;
      uint8_t *dst = buf + (pc / kPieces) * kSlotB + j * 1024;
      __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
    }
  };
  int idn[kPer];
  for (int T = 0; T < NBUF - 1 && T < n_tiles; ++T) {
    fetch_ids(T, idn);
    copy_tile(T, idn);
  }
  if (NBUF - 1 < n_tiles) fetch_ids(NBUF - 1, idn);

  // This lane's LDS byte addresses of its K and V operands in buffer 0 (the Half / Half8
  // layouts of load_k / load_v / load_k8 / load_v8 over the 4 page slots); every read adds
  // a constant offset.  FP8 reads bring two operands' codes, dequantized in registers.
  const int r16 = lane & 15, rq = r16 >> 2, ri = r16 & 3;
  const uint32_t kv0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)&kv[0][0];
  const uint32_t kbase = kv0 + (rq >> 1) * kSlotB + 2 * (grp * 128 + (rq & 1) * 32 + ri * 8);  // both layouts
  const uint32_t vbase = FP8 ? kv0 + (grp >> 1) * kSlotB + 16 * D + (grp & 1) * (8 * D) + r16 * 16
                             : kv0 + (grp >> 1) * kSlotB + 2 * (16 * D + (grp & 1) * (8 * D) + r16 * 8);
  using Raw = std::conditional_t<FP8, Half8<D>, Half<D>>;
  auto lds_tile_k = [&](Raw &t, uint32_t base) {
    if constexpr (FP8) {
      static_for<2>([&](auto kc_) {
        static_for<2>([&](auto h_) {
          static_for<D / 64>([&](auto j_) {
            constexpr int kc = decltype(kc_)::value, h = decltype(h_)::value, j = decltype(j_)::value;
            t.r[(2 * kc + h) * (D / 64) + j] = lds_rd128<2 * kc * kSlotB + h * 128 + j * 1024>(base);
          });
        });
      });
    } else {
      static_for<2>([&](auto kc_) {
        static_for<2>([&](auto h_) {
          static_for<D / 32>([&](auto c_) {
            constexpr int kc = decltype(kc_)::value, h = decltype(h_)::value, c = decltype(c_)::value;
            t.r[(2 * kc + h) * (D / 32) + c] = lds_rd128<2 * kc * kSlotB + 2 * (h * 64 + c * 512)>(base);
          });
        });
      });
    }
  };
  auto lds_tile_v = [&](Raw &t, uint32_t base) {
    if constexpr (FP8) {
      static_for<2>([&](auto kc_) {
        static_for<D / 32>([&](auto j_) {
          constexpr int kc = decltype(kc_)::value, j = decltype(j_)::value;
          t.r[kc * (D / 32) + j] = lds_rd128<2 * kc * kSlotB + j * 256>(base);
        });
      });
    } else {
      static_for<2>([&](auto kc_) {
        static_for<D / 16>([&](auto db_) {
          constexpr int kc = decltype(kc_)::value, db = decltype(db_)::value;
          t.r[kc * (D / 16) + db] = lds_rd128<2 * kc * kSlotB + 2 * db * 128>(base);
        });
      });
    }
  };

  float M = neg_inf(), L = 0.f, m = neg_inf(), l = 0.f;
  float O[D / 4];
  f32x4 o[D / 16];
#pragma unroll
  for (int e = 0; e < D / 4; ++e) O[e] = 0.f;
#pragma unroll
  for (int db = 0; db < D / 16; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
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
    if (t0 <= w_max) {
      const uint32_t boff = (uint32_t)(T % NBUF) * (4 * kSlotB);
      Half<D> hk, hv;
      Raw rk, rv;
      lds_tile_k(rk, kbase + boff);
      lds_wait<0>();
#pragma unroll
      for (int i = 0; i < (int)(sizeof(Raw) / 16); ++i) settle(rk.r[i]);
      if constexpr (FP8) dequant_k<D>(rk, hk);
      else hk = rk;
      f32x4 sc[4];
      attn_score_mfma<D>(hk, qop, sc);
      lds_tile_v(rv, vbase + boff);  // lands while the softmax runs
      bf16x8 pop[2];
      float alpha, m_new, l_new;
      // Uniform shortcuts that leave every value unchanged: no causal select when the whole
      // tile is at or before the wave's first position, no V zeroing before the last tile.
      if (t0 + kTile - 1 <= w_min)
        tile_softmax<false>(sc, t0, pos, cscale, m, l, pop, alpha, m_new, l_new);
      else
        tile_softmax<true>(sc, t0, pos, cscale, m, l, pop, alpha, m_new, l_new);
      lds_wait<0>();
#pragma unroll
      for (int i = 0; i < (int)(sizeof(Raw) / 16); ++i) settle(rv.r[i]);
      if constexpr (FP8) dequant_v<D>(rv, hv);
      else hv = rv;
      if (t0 > w_min)
        attn_values<D, true>(hv, t0, pos, p_max + 1, pop, alpha, m_new, l_new, m, l, o);
      else if (t0 + kTile > p_max + 1)
        attn_values<D, false, true>(hv, t0, pos, p_max + 1, pop, alpha, m_new, l_new, m, l, o);
      else
        attn_values<D, false, false>(hv, t0, pos, p_max + 1, pop, alpha, m_new, l_new, m, l, o);
    }
    // end of a split: fold its state into the merged state of every column it reached,
    // then start the next split from the empty state
    if (t0 + kTile >= min(s0 + split_tokens, p_max + 1)) {
      if (s0 <= pos) {
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
      m = neg_inf();
      l = 0.f;
#pragma unroll
      for (int db = 0; db < D / 16; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  // a page id outside the pool seen by any wave marks the whole workgroup's rows NaN
  if (__syncthreads_or(bad)) L = __builtin_nanf("");
  if (!col_ok) return;
  if (FP8) {  // the V scale, on the fp32 state (exact), as the decode partials get it
#pragma unroll
    for (int e = 0; e < D / 4; ++e) O[e] = O[e] * v_scale;
  }
#pragma unroll
  for (int db = 0; db < D / 16; ++db) {
    uint32_t w0 = pack2(__fdiv_rn(O[db * 4 + 0], L), __fdiv_rn(O[db * 4 + 1], L));
    uint32_t w1 = pack2(__fdiv_rn(O[db * 4 + 2], L), __fdiv_rn(O[db * 4 + 3], L));
    *reinterpret_cast<uint2 *>(op + db * 16) = make_uint2(w0, w1);
  }
}

// ---------------------------------------------------------------------------
// S10 with two MFMA column blocks per wave (bf16 cache).  The grid, the block ->
// (sequence, first token) map, the tile copies and the LDS layout are those of
// attn_prefill_kernel; a wave owns 2 x 16 columns (2 x 16/G tokens x G heads), so a
// workgroup covers QT = NW * 32/G tokens and every K or V operand read from LDS feeds one
// MFMA of each block (half the LDS reads per MFMA).  Operands stream from LDS through a
// ring of AHEAD reads in flight instead of a whole tile in registers.  Per column the
// arithmetic is attn_prefill_kernel's, i.e. the decode chain: s[mb] = the MFMAs of K steps
// c = 0, 1, ... in order from zero, tile_softmax, o = o * alpha then the MFMAs of the
// tile's two 32-token steps, merge_state at each split's end.  Tiles wholly at or before
// the wave's first position run both blocks together without masks (every mask would
// keep every value there); the at most two tiles that reach past it run each block alone
// with every mask on (causal select, inactive columns keep their state, V past the
// workgroup's last position read as 0): the same values as the shortcut forms.
// ---------------------------------------------------------------------------
template <int D, int NW, int NBUF>
__global__ __launch_bounds__(512) void attn_prefill2_kernel(
    const bf16_t *__restrict__ q, int q_row_stride, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ start_pos, int n_seqs, const int32_t *__restrict__ page_table,
    int page_stride, const bf16_t *__restrict__ pool, int n_pages, int Hkv, int G,
    int split_tokens, int ctx_bound, float cscale, bf16_t *__restrict__ out) {
  static_assert(NW >= 1 && NW <= 8, "at most 512 threads (the launch bound)");
  static_assert(NBUF >= 2 && NBUF <= 4, "tiles in flight");
  constexpr int kSlotB = lds_page_bytes<D, false>();
  constexpr int kPageB = 64 * D;
  constexpr int kPieces = kPageB / 1024;
  static_assert((4 * kPieces) % NW == 0, "every wave copies the same number of pieces");
  constexpr int kPer = 4 * kPieces / NW;
  constexpr int KC = D / 32, DB = D / 16;  // K steps of a score chain, value dim blocks
  constexpr int AHEAD = 4, SLOTS = AHEAD + 1;
  static_assert(AHEAD <= 4 * KC && AHEAD <= 2 * DB, "ring deeper than a phase");
  __shared__ __attribute__((aligned(16))) uint8_t kv[NBUF][4 * kSlotB];
  const int g = blockIdx.y;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int tpb = 16 / G;
  const int QT = NW * 2 * tpb;
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
  seq = __builtin_amdgcn_readfirstlane(seq);
  tok0 = __builtin_amdgcn_readfirstlane(tok0);
  const int Hq = Hkv * G;
  const int n_tok = __builtin_amdgcn_readfirstlane(cu[seq + 1] - cu[seq]);
  const int sp = __builtin_amdgcn_readfirstlane(start_pos[seq]);
  const int n = lane & 15, grp = lane >> 4;
  const int hh = n % G;
  // block b of wave w: tokens tok0 + b * NW * tpb + w * tpb .. + tpb - 1, so a segment of
  // at most NW * tpb tokens leaves every wave's block 1 empty (those waves then run block 0
  // alone, as many busy waves as with one block per wave)
  auto first_tok = [&](int b) { return tok0 + b * NW * tpb + wave * tpb; };
  int pos[2];
  bool col_ok[2];
  long jrow[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int tok = first_tok(b) + n / G;
    col_ok[b] = tok < n_tok;
    jrow[b] = cu[seq] + (col_ok[b] ? tok : 0);
    pos[b] = col_ok[b] ? sp + tok : -1;
  }
  const int p_max = sp + min(tok0 + QT, n_tok) - 1;  // the workgroup's last position
  if (sp < 0 || p_max + 1 > ctx_bound || (p_max / kPage) >= page_stride) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      bf16_t *op = out + (jrow[b] * Hq + g * G + hh) * D + grp * 4;
      if (col_ok[b]) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
          for (int i = 0; i < 4; ++i) op[db * 16 + i] = (bf16_t)0x7fc0u;
      }
    }
    return;
  }
  const int w_min = sp + first_tok(0);  // this wave's first position
  int w_min_b[2], w_max_b[2];           // each block's first and last position (last < first: none)
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    w_min_b[b] = sp + first_tok(b);
    w_max_b[b] = sp + min(first_tok(b) + tpb, n_tok) - 1;
  }
  bf16x8 qop[2][KC];
#pragma unroll
  for (int b = 0; b < 2; ++b) load_qop<D>(qop[b], q + jrow[b] * q_row_stride + (g * G + hh) * D, col_ok[b]);

  const int32_t *pt = page_table + (long)seq * page_stride;
  const int last_page = p_max / kPage;
  const int n_tiles = p_max / kTile + 1;
  bool bad = false;
  // the copies of attn_prefill_kernel: wave w copies pieces w, w+NW, ... of tile T
  auto fetch_ids = [&](int T, int (&raw)[kPer]) {
#pragma unroll
    for (int u = 0; u < kPer; ++u) raw[u] = pt[min(4 * T + (wave + u * NW) / kPieces, last_page)];
  };
  auto copy_tile = [&](int T, const int (&raw)[kPer]) {
    uint8_t *buf = &kv[T % NBUF][0];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int pc = wave + u * NW;
      const int P = 4 * T + pc / kPieces;
      const bool b = P <= last_page && (unsigned)raw[u] >= (unsigned)n_pages;
      bad |= b;
      const int pid = (P <= last_page && !b) ? raw[u] : 0;
      const int j = pc % kPieces;
      const uint8_t *src = reinterpret_cast<const uint8_t *>(pool) + ((long)pid * Hkv + g) * kPageB + j * 1024 +
                           lane * 16;
      uint8_t *dst = buf + (pc / kPieces) * kSlotB + j * 1024;
      __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
    }
  };
  // PF = NBUF - 2 tiles are copied ahead (not NBUF - 1): a lagging wave (below) still
  // reads tile T-1 while tile T is current, so the copy issued at tile T may only take
  // the buffer of tile T-2.
  constexpr int PF = NBUF - 2;
  int idn[kPer];
  for (int T = 0; T < PF && T < n_tiles; ++T) {
    fetch_ids(T, idn);
    copy_tile(T, idn);
  }
  if (PF < n_tiles) fetch_ids(PF, idn);

  // this lane's LDS byte addresses of its K and V operands in buffer 0 (the layouts of
  // attn_prefill_kernel); K operand (mb, c) and V operand (kc, db) add constant offsets
  const int r16 = lane & 15, rq = r16 >> 2, ri = r16 & 3;
  const uint32_t kv0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)&kv[0][0];
  const uint32_t kbase = kv0 + (rq >> 1) * kSlotB + 2 * (grp * 128 + (rq & 1) * 32 + ri * 8);
  const uint32_t vbase = kv0 + (grp >> 1) * kSlotB + 2 * (16 * D + (grp & 1) * (8 * D) + r16 * 8);

  float M[2], L[2], m[2], l[2];
  float O[2][D / 4];
  f32x4 o[2][DB];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    M[b] = neg_inf();
    L[b] = 0.f;
    m[b] = neg_inf();
    l[b] = 0.f;
#pragma unroll
    for (int e = 0; e < D / 4; ++e) O[b][e] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[b][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // S^T = K Q^T of blocks B0 .. B0+NB-1: K operand (mb, c) read once (operands in c-major
  // order, AHEAD in flight), one MFMA per block; each chain runs c = 0, 1, ... from zero.
  auto scores = [&](auto b0_, auto nb_, uint32_t base, f32x4 (&s)[2][4]) {
    constexpr int B0 = decltype(b0_)::value, NB = decltype(nb_)::value, NOPS = 4 * KC;
    static_for<NB>([&](auto bb) {
      constexpr int B = B0 + decltype(bb)::value;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) s[B][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    });
    u32x4 a[SLOTS];
    auto issue = [&](auto ii) {
      constexpr int I = decltype(ii)::value, c = I / 4, mb = I % 4;
      a[I % SLOTS] = lds_rd128<2 * (mb >> 1) * kSlotB + 2 * ((mb & 1) * 64 + c * 512)>(base);
    };
    static_for<AHEAD>(issue);
    static_for<NOPS>([&](auto ii) {
      constexpr int I = decltype(ii)::value, c = I / 4, mb = I % 4;
      if constexpr (I + AHEAD < NOPS) {
        issue(std::integral_constant<int, I + AHEAD>{});
        lds_wait<AHEAD>();
      } else {
        lds_wait<NOPS - 1 - I>();
      }
      settle(a[I % SLOTS]);
      static_for<NB>([&](auto bb) {
        constexpr int B = B0 + decltype(bb)::value;
        s[B][mb] = mfma(as_bf16x8(a[I % SLOTS]), qop[B][c], s[B][mb]);
      });
    });
  };
  // V operand (kc, db), kc-major; the first AHEAD are issued by v_head (before the softmax)
  auto v_issue = [&](auto ii, u32x4 (&v)[SLOTS], uint32_t base) {
    constexpr int I = decltype(ii)::value, kc = I / DB, db = I % DB;
    v[I % SLOTS] = lds_rd128<2 * kc * kSlotB + 2 * db * 128>(base);
  };
  auto v_head = [&](u32x4 (&v)[SLOTS], uint32_t base) {
    static_for<AHEAD>([&](auto ii) { v_issue(ii, v, base); });
  };
  // o = o * alpha + V^T P^T for blocks B0 .. B0+NB-1, every column active and no V entry
  // past the bound (V operand read once, one MFMA per block; per element the rescale,
  // then the kc = 0 and kc = 1 MFMAs).
  auto values = [&](auto b0_, auto nb_, u32x4 (&v)[SLOTS], uint32_t base, const bf16x8 (&pop)[2][2],
                    const float (&alpha)[2], const float (&m_new)[2], const float (&l_new)[2]) {
    constexpr int B0 = decltype(b0_)::value, NB = decltype(nb_)::value, NOPS = 2 * DB;
    static_for<NB>([&](auto bb) {
      constexpr int B = B0 + decltype(bb)::value;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[B][db] = o[B][db] * alpha[B];
    });
    static_for<NOPS>([&](auto ii) {
      constexpr int I = decltype(ii)::value, kc = I / DB, db = I % DB;
      if constexpr (I + AHEAD < NOPS) {
        v_issue(std::integral_constant<int, I + AHEAD>{}, v, base);
        lds_wait<AHEAD>();
      } else {
        lds_wait<NOPS - 1 - I>();
      }
      settle(v[I % SLOTS]);
      static_for<NB>([&](auto bb) {
        constexpr int B = B0 + decltype(bb)::value;
        o[B][db] = mfma(as_bf16x8(v[I % SLOTS]), pop[B][kc], o[B][db]);
      });
    });
    static_for<NB>([&](auto bb) {
      constexpr int B = B0 + decltype(bb)::value;
      m[B] = m_new[B];
      l[B] = l_new[B];
    });
  };
  // The same step for block B alone with the masks of the tiles that reach past the wave's
  // first position: columns whose position is before the tile keep their state, and V
  // entries at or past vbound read as 0 (the MAYBE_INACTIVE and VMASK forms).  The dims
  // run in NPART parts (kc = 0 and 1 of a part's blocks, then the next part), so only a
  // part's old state is held; per element the order is unchanged.
  auto values_masked = [&](auto b_, const bf16x8 (&pop)[2][2], const float (&alpha)[2], const float (&m_new)[2],
                           const float (&l_new)[2], uint32_t base, int t0, int vbound) {
    constexpr int B = decltype(b_)::value;
    constexpr int NPART = DB, DPP = 1, NOPS = 2 * DPP;
    const bool act = t0 <= pos[B];
    static_for<NPART>([&](auto pp) {
      constexpr int P = decltype(pp)::value;
      f32x4 keep[DPP];
#pragma unroll
      for (int j = 0; j < DPP; ++j) {
        keep[j] = o[B][P * DPP + j];
        o[B][P * DPP + j] = o[B][P * DPP + j] * alpha[B];
      }
      u32x4 v[NOPS];
      static_for<NOPS>([&](auto ii) {
        constexpr int I = decltype(ii)::value, kc = I / DPP, db = P * DPP + I % DPP;
        v[I] = lds_rd128<2 * kc * kSlotB + 2 * db * 128>(base);
      });
      lds_wait<0>();
      static_for<NOPS>([&](auto ii) {
        constexpr int I = decltype(ii)::value, kc = I / DPP, db = P * DPP + I % DPP;
        settle(v[I]);
        u32x4 vv = v[I];
        const int n_valid = vbound - (t0 + 32 * kc + 8 * grp);
        if (n_valid < 8) vv = keep_first(vv, n_valid);
        o[B][db] = mfma(as_bf16x8(vv), pop[B][kc], o[B][db]);
      });
#pragma unroll
      for (int j = 0; j < DPP; ++j) {
#pragma unroll
        for (int i = 0; i < 4; ++i) o[B][P * DPP + j][i] = act ? o[B][P * DPP + j][i] : keep[j][i];
      }
    });
    m[B] = act ? m_new[B] : m[B];
    l[B] = act ? l_new[B] : l[B];
  };

  // tile T landed (at most `ahead` later tiles still in flight), then the barrier: every
  // wave's pieces are visible and every wave is done with tile T-1's buffer; then the copy
  // of tile T+NBUF-1.  Returns the tile's LDS byte offset.
  auto next_tile = [&](int T) {
    const int ahead = min(PF - 1, n_tiles - 1 - T);
    if (ahead >= 2) wait_vmem<2 * kPer>();
    else if (ahead == 1) wait_vmem<kPer>();
    else wait_vmem<0>();
    __syncthreads();
    if (T + PF < n_tiles) {
      copy_tile(T + PF, idn);
      if (T + PF + 1 < n_tiles) fetch_ids(T + PF + 1, idn);
    }
    return (uint32_t)(T % NBUF) * (4 * kSlotB);
  };
  // end of a split: fold its state into the merged state of every column it reached,
  // then start the next split from the empty state
  auto split_end = [&](int t0) {
    const int s0 = t0 - t0 % split_tokens;
    if (t0 + kTile >= min(s0 + split_tokens, p_max + 1)) {
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        if (s0 <= pos[b]) {
          float os[D / 4];
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) os[db * 4 + i] = o[b][db][i];
          if (s0 == 0) {
            M[b] = m[b];
            L[b] = l[b];
#pragma unroll
            for (int e = 0; e < D / 4; ++e) O[b][e] = os[e];
          } else {
            merge_state<D / 4>(M[b], L[b], O[b], m[b], l[b], os);
          }
        }
        m[b] = neg_inf();
        l[b] = 0.f;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[b][db] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  };
  // Tiles wholly at or before the wave's first position (every barrier of the workgroup is
  // still taken once per tile by every wave: the two loops together run n_tiles steps).
  // The second wave of each SIMD (waves NW/2 ..) runs half a tile behind the first: after
  // a barrier it first finishes the value step of the previous tile, so while one wave
  // of a SIMD is in its softmax the other issues MFMAs.  Per column the steps and their
  // order are unchanged.
  const int n_fast = min(n_tiles, (w_min + 1) / kTile);
  int T = 0;
  if (w_max_b[1] < w_min_b[1]) {
    // block 1 holds no token of the sequence (a short segment): block 0 alone
    for (; T < n_fast; ++T) {
      const uint32_t boff = next_tile(T);
      const int t0 = T * kTile;
      f32x4 s[2][4];
      bf16x8 pop[2][2];
      float alpha[2], m_new[2], l_new[2];
      u32x4 v[SLOTS];
      scores(std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{}, kbase + boff, s);
      v_head(v, vbase + boff);
      tile_softmax<false>(s[0], t0, pos[0], cscale, m[0], l[0], pop[0], alpha[0], m_new[0], l_new[0]);
      values(std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{}, v, vbase + boff, pop, alpha,
             m_new, l_new);
      split_end(t0);
    }
  } else if (wave < NW / 2) {
    for (; T < n_fast; ++T) {
      const uint32_t boff = next_tile(T);
      const int t0 = T * kTile;
      f32x4 s[2][4];
      bf16x8 pop[2][2];
      float alpha[2], m_new[2], l_new[2];
      u32x4 v[SLOTS];
      scores(std::integral_constant<int, 0>{}, std::integral_constant<int, 2>{}, kbase + boff, s);
      v_head(v, vbase + boff);  // lands while the softmax runs
#pragma unroll
      for (int b = 0; b < 2; ++b)
        tile_softmax<false>(s[b], t0, pos[b], cscale, m[b], l[b], pop[b], alpha[b], m_new[b], l_new[b]);
      values(std::integral_constant<int, 0>{}, std::integral_constant<int, 2>{}, v, vbase + boff, pop, alpha,
             m_new, l_new);
      split_end(t0);
    }
  } else {
    bf16x8 pop[2][2];
    float alpha[2], m_new[2], l_new[2];
    uint32_t pboff = 0;
    for (; T < n_fast; ++T) {
      const uint32_t boff = next_tile(T);
      const int t0 = T * kTile;
      if (T > 0) {  // the value step of tile T-1 (its buffer is kept while tile T is current)
        u32x4 v[SLOTS];
        v_head(v, vbase + pboff);
        values(std::integral_constant<int, 0>{}, std::integral_constant<int, 2>{}, v, vbase + pboff, pop, alpha,
               m_new, l_new);
        split_end(t0 - kTile);
      }
      f32x4 s[2][4];
      scores(std::integral_constant<int, 0>{}, std::integral_constant<int, 2>{}, kbase + boff, s);
#pragma unroll
      for (int b = 0; b < 2; ++b)
        tile_softmax<false>(s[b], t0, pos[b], cscale, m[b], l[b], pop[b], alpha[b], m_new[b], l_new[b]);
      pboff = boff;
    }
    if (n_fast > 0) {
      u32x4 v[SLOTS];
      v_head(v, vbase + pboff);
      values(std::integral_constant<int, 0>{}, std::integral_constant<int, 2>{}, v, vbase + pboff, pop, alpha,
             m_new, l_new);
      split_end((n_fast - 1) * kTile);
    }
  }
  // the rest: each block alone with every mask, while the tile reaches one of its positions
  for (; T < n_tiles; ++T) {
    const uint32_t boff = next_tile(T);
    const int t0 = T * kTile;
    static_for<2>([&](auto bb) {
      constexpr int B = decltype(bb)::value;
      if (t0 <= w_max_b[B] && w_max_b[B] >= w_min_b[B]) {
        f32x4 s[2][4];
        bf16x8 pop[2][2];
        float alpha[2], m_new[2], l_new[2];
        scores(std::integral_constant<int, B>{}, std::integral_constant<int, 1>{}, kbase + boff, s);
        tile_softmax<true>(s[B], t0, pos[B], cscale, m[B], l[B], pop[B], alpha[B], m_new[B], l_new[B]);
        values_masked(bb, pop, alpha, m_new, l_new, vbase + boff, t0, p_max + 1);
      }
    });
    split_end(t0);
  }
  if (__syncthreads_or(bad)) {
#pragma unroll
    for (int b = 0; b < 2; ++b) L[b] = __builtin_nanf("");
  }
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    if (!col_ok[b]) continue;
    bf16_t *op = out + (jrow[b] * Hq + g * G + hh) * D + grp * 4;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      uint32_t w0 = pack2(__fdiv_rn(O[b][db * 4 + 0], L[b]), __fdiv_rn(O[b][db * 4 + 1], L[b]));
      uint32_t w1 = pack2(__fdiv_rn(O[b][db * 4 + 2], L[b]), __fdiv_rn(O[b][db * 4 + 3], L[b]));
      *reinterpret_cast<uint2 *>(op + db * 16) = make_uint2(w0, w1);
    }
  }
}

hipError_t launch_attn_prefill(const AttnPrefillArgs &a, hipStream_t st) {
  constexpr int NW = 8, NBUF = 4;
  const int QT = NW * (16 / a.G);
  const long blocks = (long)(a.n_tok + QT - 1) / QT + a.n_seqs;  // bound on sum of ceil(n_s / QT)
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  dim3 grid((unsigned)blocks, a.Hkv);
#define RIL_PF(D_, F_)                                                                                            \
  hipLaunchKernelGGL((attn_prefill_kernel<D_, NW, NBUF, F_>), grid, dim3(64 * NW), 0, st, a.q, a.q_row_stride, a.cu, \
                     a.start_pos, a.n_seqs, a.page_table, a.page_stride, a.pool, a.n_pages, a.Hkv, a.G,             \
                     a.split_tokens, a.ctx_bound, a.kv_fp8 ? a.cscale * a.k_scale : a.cscale, a.out, a.k_scale, \
                     a.v_scale)
#define RIL_PF2(D_)                                                                                               \
  hipLaunchKernelGGL((attn_prefill2_kernel<D_, NW, NBUF>), grid2, dim3(64 * NW), 0, st, a.q, a.q_row_stride, a.cu,    \
                     a.start_pos, a.n_seqs, a.page_table, a.page_stride, a.pool, a.n_pages, a.Hkv, a.G,             \
                     a.split_tokens, a.ctx_bound, a.cscale, a.out)
  // bf16 cache: two column blocks per wave (twice the tokens per workgroup)
  const long blocks2 = (long)(a.n_tok + 2 * QT - 1) / (2 * QT) + a.n_seqs;
  dim3 grid2((unsigned)blocks2, a.Hkv);
  if (a.D == 128) {
    if (a.kv_fp8) RIL_PF(128, true); else RIL_PF2(128);
  } else {
    if (a.kv_fp8) RIL_PF(64, true); else RIL_PF2(64);
  }
#undef RIL_PF
#undef RIL_PF2
  return hipGetLastError();
}

}  // namespace ril
