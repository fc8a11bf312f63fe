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
#include <type_traits>

#include "attn_common.h"
#include "kernels.h"
#include "norm.h"

namespace ril {

// ---------------------------------------------------------------------------
// S5: KV write (shared by prefill, decode and the history writer)
// ---------------------------------------------------------------------------

// One thread per (token, kv head, 8-dim group).  mode 0: packed prefill tokens (cu,
// start_pos); mode 1: decode rows (token r is row r at position ctx_len[r]-1).
template <int D, bool FP8>
__global__ __launch_bounds__(256) void kv_write_kernel(
    const bf16_t *__restrict__ k, const bf16_t *__restrict__ v, int row_stride, int n_tok,
    int mode, const int32_t *__restrict__ cu, const int32_t *__restrict__ start_pos, int n_seqs,
    const int32_t *__restrict__ ctx_len, const int32_t *__restrict__ page_table, int page_stride,
    bf16_t *__restrict__ pool, int n_pages, int Hkv, float k_inv_scale, float v_inv_scale) {
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
  if constexpr (FP8) {
    uint8_t *pb = reinterpret_cast<uint8_t *>(pool) + ((long)pid * Hkv + g) * (32 * D);
    const int t = pos % kPage;
    const u32x4 kv8 = ld16(k + (long)j * row_stride + g * D + d0);
    const u32x4 vv8 = ld16(v + (long)j * row_stride + g * D + d0);
    uint32_t kw[2];
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const uint32_t lo = fp8_codes2(bf2f((bf16_t)(kv8[2 * w] & 0xffffu)) * k_inv_scale,
                                     bf2f((bf16_t)(kv8[2 * w] >> 16)) * k_inv_scale);
      const uint32_t hi = fp8_codes2(bf2f((bf16_t)(kv8[2 * w + 1] & 0xffffu)) * k_inv_scale,
                                     bf2f((bf16_t)(kv8[2 * w + 1] >> 16)) * k_inv_scale);
      kw[w] = lo | (hi << 16);
    }
    *reinterpret_cast<uint2 *>(pb + k_page_offset8(t, d0)) = make_uint2(kw[0], kw[1]);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t c2 = fp8_codes2(bf2f((bf16_t)(vv8[w] & 0xffffu)) * v_inv_scale,
                                     bf2f((bf16_t)(vv8[w] >> 16)) * v_inv_scale);
      pb[v_page_offset8(t, d0 + 2 * w, D)] = (uint8_t)(c2 & 0xffu);
      pb[v_page_offset8(t, d0 + 2 * w + 1, D)] = (uint8_t)(c2 >> 8);
    }
    return;
  }
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
// S8: decode split kernel, one wave per (row, kv head, split).  The 1-D grid lists the
// work longest first, so the hardware dispatcher fills the machine with full splits and
// ends on the short ones: slots [0, n_sg*R*Hkv) are the full splits, split-major (the
// kv heads of one page adjacent); then for c = n_cls .. 1 one slot per (row, kv head)
// whose partial last split has c tiles.  Slots with no such work exit at once.  Which
// wave computes a split never changes its arithmetic.  K/V loads run up to two tiles
// ahead of the tile being computed, with the nontemporal (streaming) cache policy: each
// byte of the cache is read exactly once per step, and letting it displace other lines
// from the L2 and the memory-side cache cost 8% of the kernel's time.  The bf16 and FP8
// entry points below share this body; the FP8 one runs two waves per SIMD.
// ---------------------------------------------------------------------------
template <int D, bool FP8>
__device__ __forceinline__ void attn_decode_split(
    const bf16_t *__restrict__ q, int q_row_stride, const int32_t *__restrict__ ctx_len,
    const int32_t *__restrict__ page_table, int page_stride, const bf16_t *__restrict__ pool,
    int n_pages, int Hkv, int G, int split_tokens, int ctx_bound, int n_rows, int n_sg, float cscale,
    float *__restrict__ part_o, float *__restrict__ part_ml, int max_splits, float k_scale, float v_scale) {
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
  // Ring of NR = 2*LA + 1 half-tile slots.  bf16: LA = 2 tiles ahead, one wave per SIMD:
  // while the scores of tile t run, the V half of t, both halves of t+1 and the K half of
  // t+2 are in flight (64 KB per wave for D = 128).  FP8: slots hold the codes, each
  // operand dequantized just before its MFMA (no dequantized tile held in registers), and
  // the ring is one tile ahead (3 slots, 16 KB in flight per wave) so that two waves fit
  // each SIMD without spilling: 131 -> 118 us for the 64-row step, where two waves with
  // the 5-slot ring spilled (148 us) and deeper rings at one wave were slower.  Half-tile
  // h (K of tile h/2 if h is even, else its V) lives in slot h % NR.
  constexpr int LA = FP8 ? 1 : 2, NR = 2 * LA + 1;
  using Slot = std::conditional_t<FP8, Half8<D>, Half<D>>;
  Slot ring[NR];
  const bf16_t *pg[4];
  const uint8_t *pg8[4];
  auto pages = [&](int tile) {
    if constexpr (FP8) {
      const uint8_t *p8 = reinterpret_cast<const uint8_t *>(pool);
#pragma unroll
      for (int k = 0; k < 4; ++k)
        pg8[k] = p8 + ((long)__builtin_amdgcn_readlane(pid, 4 * tile + k) * Hkv + g) * (32 * D);
    } else {
      tile_pages<D>(pg, pool, pid, tile, Hkv, g);
    }
  };
  auto ldk = [&](Slot &sl) {
    if constexpr (FP8) load_k8<D, NtGlobal>(sl, pg8);
    else load_k<D, NtGlobal>(sl, pg);
  };
  auto ldv = [&](Slot &sl) {
    if constexpr (FP8) load_v8<D, NtGlobal>(sl, pg8);
    else load_v<D, NtGlobal>(sl, pg);
  };
#pragma unroll
  for (int u = 0; u < LA; ++u) {
    if (u < n_tiles) {
      pages(u);
      ldk(ring[2 * u]);
      ldv(ring[2 * u + 1]);
    }
  }
  float m = neg_inf(), l = 0.f;
  f32x4 o[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int t0 = 0; t0 < n_tiles; t0 += NR) {
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      const int t = t0 + j;
      if (t < n_tiles) {
        const bool ahead = t + LA < n_tiles;
        if (ahead) {
          pages(t + LA);
          ldk(ring[(2 * j + 2 * LA) % NR]);  // the slot of V(t-1), already consumed
        }
        bf16x8 pop[2];
        float alpha, m_new, l_new;
        if constexpr (FP8) {
          f32x4 s[4];
          attn_score_mfma8<D>(ring[(2 * j) % NR], qop, s);
          tile_softmax(s, s0 + t * kTile, ctx - 1, cscale, m, l, pop, alpha, m_new, l_new);
        } else {
          attn_scores<D>(ring[(2 * j) % NR], s0 + t * kTile, qop, ctx - 1, cscale, m, l, pop, alpha, m_new,
                         l_new);
        }
        if (ahead) ldv(ring[(2 * j) % NR]);  // the slot of K(t), just consumed
        if constexpr (FP8) {
          attn_values8<D, false>(ring[(2 * j + 1) % NR], s0 + t * kTile, ctx - 1, ctx, pop, alpha, m_new, l_new,
                                 m, l, o);
        } else {
          attn_values<D, false>(ring[(2 * j + 1) % NR], s0 + t * kTile, ctx - 1, ctx, pop, alpha, m_new, l_new,
                                m, l, o);
        }
      }
    }
  }
  if (FP8) {  // the V scale, on the fp32 state (exact)
#pragma unroll
    for (int db = 0; db < D / 16; ++db) o[db] = o[db] * v_scale;
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

#define RIL_SPLIT_PARAMS                                                                                      \
  const bf16_t *__restrict__ q, int q_row_stride, const int32_t *__restrict__ ctx_len,                         \
      const int32_t *__restrict__ page_table, int page_stride, const bf16_t *__restrict__ pool, int n_pages,     \
      int Hkv, int G, int split_tokens, int ctx_bound, int n_rows, int n_sg, float cscale,                      \
      float *__restrict__ part_o, float *__restrict__ part_ml, int max_splits, float k_scale, float v_scale
#define RIL_SPLIT_ARGS                                                                                         \
  q, q_row_stride, ctx_len, page_table, page_stride, pool, n_pages, Hkv, G, split_tokens, ctx_bound, n_rows, n_sg, \
      cscale, part_o, part_ml, max_splits, k_scale, v_scale
template <int D>
__global__ __launch_bounds__(64) void attn_decode_split_kernel(RIL_SPLIT_PARAMS) {
  attn_decode_split<D, false>(RIL_SPLIT_ARGS);
}
template <int D>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_decode_split_fp8_kernel(
    RIL_SPLIT_PARAMS) {
  attn_decode_split<D, true>(RIL_SPLIT_ARGS);
}
#undef RIL_SPLIT_PARAMS
#undef RIL_SPLIT_ARGS

// ---------------------------------------------------------------------------
// One head's split merge by a half-wave (lane hl of 32 owns dims hl*D/32 ..): the loads of
// CH splits issued together, folded split 0 first, then left to right -- merge_partials'
// order and merge_state's arithmetic per element; writes bf16(O / L) to dst (the lane's
// first dim).  A whole wave thus merges two heads, each lane with 16-byte loads.
// ---------------------------------------------------------------------------
template <int D, int CH>
__device__ __forceinline__ void merge_head_halfwave(const float *__restrict__ part_o,
                                                    const float *__restrict__ part_ml, long base, int ns,
                                                    bf16_t *dst, int hl) {
  constexpr int PER = D / 32;
  float M = 0.f, L = 0.f, O[PER];
  for (int s0 = 0; s0 < ns; s0 += CH) {
    float ms[CH], ls[CH], os[CH][PER];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const long sidx = base + min(s0 + c, ns - 1);  // past the last split: a repeat, not folded
      ms[c] = part_ml[sidx * 2];
      ls[c] = part_ml[sidx * 2 + 1];
#pragma unroll
      for (int j = 0; j < PER; ++j) os[c][j] = part_o[sidx * D + hl * PER + j];
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      if (s0 + c >= ns) break;
      if (s0 + c == 0) {
        M = ms[0];
        L = ls[0];
#pragma unroll
        for (int j = 0; j < PER; ++j) O[j] = os[0][j];
      } else {
        merge_state<PER>(M, L, O, ms[c], ls[c], os[c]);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) dst[j] = f2bf(__fdiv_rn(O[j], L));
}

// ---------------------------------------------------------------------------
// S9: decode merge kernel.  grid (ceil(Hq / 2), rows), one wave: its half-waves merge
// heads 2x and 2x + 1.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void attn_decode_merge_kernel(
    const int32_t *__restrict__ ctx_len, int ctx_bound, int split_tokens, int Hq, int max_splits,
    const float *__restrict__ part_o, const float *__restrict__ part_ml, bf16_t *__restrict__ out) {
  constexpr int PER = D / 32;
  const int lane = threadIdx.x, hl = lane & 31, h = 2 * blockIdx.x + (lane >> 5), row = blockIdx.y;
  if (h >= Hq) return;
  const int ctx = ctx_len[row];
  bf16_t *op = out + ((long)row * Hq + h) * D + hl * PER;
  if (ctx < 1 || ctx > ctx_bound) {
#pragma unroll
    for (int j = 0; j < PER; ++j) op[j] = (bf16_t)0x7fc0u;
    return;
  }
  const int ns = (ctx + split_tokens - 1) / split_tokens;
  merge_head_halfwave<D, 16>(part_o, part_ml, ((long)row * Hq + h) * max_splits, ns, op, hl);
}

// ---------------------------------------------------------------------------
// S9 + S3 for decode rows whose attention output goes straight into the final RMSNorm
// (no output projection, no MLP block): grid (rows), 16 waves.  The half-waves merge the
// row's heads in turn (the merge kernel's arithmetic) into LDS and the attention output;
// then wave 0 normalises the row (rmsnorm_row, the RMSNorm kernel's arithmetic on the
// same bf16 values).  One launch instead of two.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(1024) void attn_merge_norm_kernel(
    const int32_t *__restrict__ ctx_len, int ctx_bound, int split_tokens, int Hq, int max_splits,
    const float *__restrict__ part_o, const float *__restrict__ part_ml, bf16_t *__restrict__ out,
    const bf16_t *__restrict__ gain, float eps, bf16_t *__restrict__ z, int ldz) {
  constexpr int PER = D / 32;
  __shared__ __attribute__((aligned(16))) bf16_t xr[kMergeNormMaxD];
  const int row = blockIdx.x, wave = threadIdx.x >> 6, lane = threadIdx.x & 63, nw = blockDim.x >> 6;
  const int hl = lane & 31, hw = lane >> 5;
  const int d = Hq * D;
  const int ctx = ctx_len[row];
  const bool ok = ctx >= 1 && ctx <= ctx_bound;
  const int ns = ok ? (ctx + split_tokens - 1) / split_tokens : 0;
  for (int h0 = 2 * wave; h0 < Hq; h0 += 2 * nw) {
    const int h = h0 + hw;
    if (h >= Hq) continue;
    bf16_t *xh = xr + h * D + hl * PER;
    if (!ok) {
#pragma unroll
      for (int j = 0; j < PER; ++j) xh[j] = (bf16_t)0x7fc0u;
      continue;
    }
    merge_head_halfwave<D, 8>(part_o, part_ml, ((long)row * Hq + h) * max_splits, ns, xh, hl);
  }
  __syncthreads();
  bf16_t *orow = out + (long)row * d;
  for (int e = threadIdx.x; e < d / 8; e += blockDim.x) st16(orow + e * 8, *reinterpret_cast<const u32x4 *>(xr + e * 8));
  if (wave == 0) {
    bf16_t *zr = z + (long)row * ldz;
    rmsnorm_row([&](int e) { return *reinterpret_cast<const u32x4 *>(xr + e * 8); },
                [&](int e, u32x4 o, u32x4) { st16(zr + e * 8, o); }, d, gain, eps, false);
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
  const float ki = 1.f / a.k_scale, vi = 1.f / a.v_scale;  // powers of two: exact
#define RIL_KVW(D_, F_)                                                                                  \
  hipLaunchKernelGGL((kv_write_kernel<D_, F_>), dim3(blocks), dim3(threads), 0, st, a.k, a.v, a.row_stride, \
                     a.n_tok, a.mode, a.cu, a.start_pos, a.n_seqs, a.ctx_len, a.page_table, a.page_stride,  \
                     a.pool, a.n_pages, a.Hkv, ki, vi)
  if (a.D == 128) {
    if (a.kv_fp8) RIL_KVW(128, true); else RIL_KVW(128, false);
  } else {
    if (a.kv_fp8) RIL_KVW(64, true); else RIL_KVW(64, false);
  }
#undef RIL_KVW
  return hipGetLastError();
}

hipError_t launch_attn_split(const AttnDecodeArgs &a, hipStream_t st) {
  if (a.n_rows == 0) return hipSuccess;
  const int n_sg = a.ctx_bound / a.split_tokens;  // full splits a row can have
  const long slots = (long)(n_sg + a.split_tokens / kTile) * a.Hkv * a.n_rows;
  if (slots > 0x7fffffffL) return hipErrorInvalidValue;
  dim3 grid((unsigned)slots);
#define RIL_SPLIT(K_)                                                                                          \
  hipLaunchKernelGGL(K_, grid, dim3(64), 0, st, a.q, a.q_row_stride, a.ctx_len, a.page_table, a.page_stride, a.pool, \
                     a.n_pages, a.Hkv, a.G, a.split_tokens, a.ctx_bound, a.n_rows, n_sg,                          \
                     a.kv_fp8 ? a.cscale * a.k_scale : a.cscale, a.part_o, a.part_ml, a.max_splits, a.k_scale,   \
                     a.v_scale)
  if (a.D == 128) {
    if (a.kv_fp8) RIL_SPLIT(attn_decode_split_fp8_kernel<128>); else RIL_SPLIT(attn_decode_split_kernel<128>);
  } else {
    if (a.kv_fp8) RIL_SPLIT(attn_decode_split_fp8_kernel<64>); else RIL_SPLIT(attn_decode_split_kernel<64>);
  }
#undef RIL_SPLIT
  return hipGetLastError();
}

hipError_t launch_attn_merge(const AttnDecodeArgs &a, hipStream_t st) {
  dim3 grid((a.Hkv * a.G + 1) / 2, a.n_rows);
  if (a.D == 128)
    hipLaunchKernelGGL(attn_decode_merge_kernel<128>, grid, dim3(64), 0, st, a.ctx_len, a.ctx_bound,
                       a.split_tokens, a.Hkv * a.G, a.max_splits, a.part_o, a.part_ml, a.out);
  else
    hipLaunchKernelGGL(attn_decode_merge_kernel<64>, grid, dim3(64), 0, st, a.ctx_len, a.ctx_bound,
                       a.split_tokens, a.Hkv * a.G, a.max_splits, a.part_o, a.part_ml, a.out);
  return hipGetLastError();
}

hipError_t launch_attn_merge_norm(const AttnDecodeArgs &a, const bf16_t *gain, float eps, bf16_t *z, int ldz,
                                  hipStream_t st) {
  if (a.n_rows == 0) return hipSuccess;
  if (a.Hkv * a.G * a.D > kMergeNormMaxD) return hipErrorInvalidValue;
  if (a.D == 128)
    hipLaunchKernelGGL(attn_merge_norm_kernel<128>, dim3(a.n_rows), dim3(1024), 0, st, a.ctx_len, a.ctx_bound,
                       a.split_tokens, a.Hkv * a.G, a.max_splits, a.part_o, a.part_ml, a.out, gain, eps, z, ldz);
  else
    hipLaunchKernelGGL(attn_merge_norm_kernel<64>, dim3(a.n_rows), dim3(1024), 0, st, a.ctx_len, a.ctx_bound,
                       a.split_tokens, a.Hkv * a.G, a.max_splits, a.part_o, a.part_ml, a.out, gain, eps, z, ldz);
  return hipGetLastError();
}

}  // namespace ril
