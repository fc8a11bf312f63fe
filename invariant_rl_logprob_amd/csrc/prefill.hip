// Paged GQA prefill attention (S10): the trainer's recompute, and any mixed batch of
// prefill chunks and one-token decode segments.  Every query row runs the decode chain
// of attn.hip exactly (same tile routine, split boundaries and merge rule, from
// attn_common.h), with its states held in registers (Bitwise-consistent RL post,
// section 2: phase consistency; section 4.2: one read path shared by prefill, decode
// and the trainer).
#include <type_traits>

#include "attn_common.h"
#include "kernels.h"

namespace ril {

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
  if (a.D == 128) {
    if (a.kv_fp8) RIL_PF(128, true); else RIL_PF(128, false);
  } else {
    if (a.kv_fp8) RIL_PF(64, true); else RIL_PF(64, false);
  }
#undef RIL_PF
  return hipGetLastError();
}

}  // namespace ril
