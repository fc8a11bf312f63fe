// W8A8 block-FP8 lm-head (Bitwise-consistent RL post, section 4.1: the deployment GEMM
// is W8A8 with block-FP8 weights, and the trainer quantizes its bf16 weights to block
// FP8 by the deployment rule and calls the same GEMM, one accumulation order for every M).
//
// Quantization (both operands, OCP E4M3 codes with E8M0 power-of-two scales):
//   activations: per row, per group of 128 consecutive K values;
//   weights:     per block of 128 vocabulary columns x 128 K values;
//   scale 2^e, e the smallest integer >= -127 with amax <= 448 * 2^e (0 for an all-zero
//   group; the E8M0 NaN code 255 for a group holding an infinity or NaN); the code of x
//   is e4m3(x * 2^-e), nearest even, which never leaves the E4M3 range.
// Product: one v_mfma_scale_f32_16x16x128_f8f6f4 per 128-wide K step and 16 x 16 block,
// its E8M0 operands the row's and the weight block's scales, accumulating in fp32 in the
// lm-head's fixed per-column K order (lm_rot).  A row's logits depend on its own codes,
// its scales and the column's order only, never on M, the batch or the grid.
#include "common.h"
#include "kernels.h"
#include "lm_head.h"

namespace ril {

typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ i32x8 cat8(u32x4 lo, u32x4 hi) {
  return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// D += A B^T over one 128-wide K step with per-lane E8M0 scales (biased exponents in the
// low byte of sa, sb).  A lane's 32 code bytes are row (column) lane%16 at K offsets
// 32*(lane/16) + 0..31; the hardware groups the K values into four 32-wide scale blocks
// that straddle lane groups, which does not matter here: all four of a row's lanes carry
// the same scale.
__device__ __forceinline__ f32x4 mfma_fp8(i32x8 a, i32x8 b, f32x4 c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

// Biased E8M0 exponent of a group from the bits of its largest magnitude (a
// non-negative float): 127 + max(e, -127), e the smallest integer with amax <= 448 * 2^e
// (amax = m 2^E with 1 <= m < 2 needs e = E - 8, or E - 7 when m > 1.75); 127 for 0;
// 255 (NaN) when amax is not finite.
__device__ __forceinline__ int e8m0_of_amax(uint32_t u) {
  if (u >= 0x7f800000u) return 255;
  if (u == 0) return 127;
  const int ef = (int)(u >> 23);                 // 0 for subnormals: clamped below
  const int e = ef - 135 + ((u & 0x7fffffu) > 0x600000u ? 1 : 0);
  return 127 + (e < -127 ? -127 : e);
}

// ---------------------------------------------------------------------------
// Activation quantization: Z [M, K] bf16 (row stride ldz) -> A8 [M, K] codes and
// ea [M, K/128] biased exponents.  16 lanes per group, 8 values per lane.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void quant_rows_fp8_kernel(const bf16_t *__restrict__ Z, int ldz, int M,
                                                             int K, uint8_t *__restrict__ A8,
                                                             int32_t *__restrict__ ea) {
  const int nk = K >> 7;
  const long gidx = (long)blockIdx.x * 256 + threadIdx.x;
  const long g = gidx >> 4;  // group (row, kb); every lane of a 16-lane group shares it
  const int part = (int)(gidx & 15);
  const bool live = g < (long)M * nk;
  const int row = live ? (int)(g / nk) : 0, kb = live ? (int)(g % nk) : 0;
  u32x4 v = u32x4{0u, 0u, 0u, 0u};
  if (live) v = ld16(Z + (long)row * ldz + kb * 128 + part * 8);
  // largest magnitude as bits: integer order of |bf16| bits is value order, NaN above inf
  uint32_t mag = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    mag = max(mag, v[j] & 0x7fffu);
    mag = max(mag, (v[j] >> 16) & 0x7fffu);
  }
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) mag = max(mag, (uint32_t)__shfl_xor((int)mag, off, 64));
  const int be = e8m0_of_amax(mag << 16);
  const int sh = be == 255 ? 0 : 127 - be;  // multiply by 2^-e (exact: no overflow, see above)
  uint32_t w[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const uint32_t lo = fp8_codes2(__builtin_ldexpf(bf2f((bf16_t)(v[2 * j] & 0xffffu)), sh),
                                   __builtin_ldexpf(bf2f((bf16_t)(v[2 * j] >> 16)), sh));
    const uint32_t hi = fp8_codes2(__builtin_ldexpf(bf2f((bf16_t)(v[2 * j + 1] & 0xffffu)), sh),
                                   __builtin_ldexpf(bf2f((bf16_t)(v[2 * j + 1] >> 16)), sh));
    w[j] = lo | (hi << 16);
  }
  if (live) {
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    *(u32x2_t __attribute__((address_space(1))) *)(A8 + (long)row * K + kb * 128 + part * 8) = u32x2_t{w[0], w[1]};
    if (part == 0) ea[(long)row * nk + kb] = be;
  }
}

// ---------------------------------------------------------------------------
// Weight packing.  Exponents: ew [2 * n_vt, K/128] biased, one per 128 x 128 block
// (columns past V count as zero).  Codes, per vocabulary tile, per 128-wide K step, one
// contiguous 32 KB piece: the step's B operands of the tile's sixteen 16-column MFMA
// blocks in lane order, each lane's 32 bytes split in two 16-byte halves 1 KB apart, so
// every weight load of a wave is one contiguous 1 KB and a workgroup's reads of a step
// are one 32 KB run (measured: the full-rate streaming pattern; blocks kept apart by the
// K extent read about 10% slower):
//   W(c, k) -> ((c/256) * (K/128) + k/128) * 32768 + ((c%256)/16) * 2048
//              + ((k%32)/16) * 1024 + (((k%128)/32) * 16 + c%16) * 16 + k%16
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void pack_fp8_exp_kernel(const bf16_t *__restrict__ src, int V, int K,
                                                           int32_t *__restrict__ ew) {
  __shared__ uint32_t red[4];
  const int b = blockIdx.x, kb = blockIdx.y, nk = K >> 7;
  const int r = threadIdx.x >> 1, half = threadIdx.x & 1;
  const long c = (long)b * 128 + r;
  uint32_t mag = 0;
  if (c < V) {
    const bf16_t *p = src + c * K + kb * 128 + half * 64;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const u32x4 v = ld16(p + q * 8);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        mag = max(mag, v[j] & 0x7fffu);
        mag = max(mag, (v[j] >> 16) & 0x7fffu);
      }
    }
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) mag = max(mag, (uint32_t)__shfl_xor((int)mag, off, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mag;
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t m = max(max(red[0], red[1]), max(red[2], red[3]));
    ew[(long)b * nk + kb] = e8m0_of_amax(m << 16);
  }
}

__global__ __launch_bounds__(256) void pack_fp8_codes_kernel(const bf16_t *__restrict__ src, int V, int K,
                                                             const int32_t *__restrict__ ew,
                                                             uint8_t *__restrict__ dst, long n_pieces) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n_pieces) return;
  const int nk = K >> 7;
  const int lane = (int)(i & 63), h = (int)((i >> 6) & 1), blk = (int)((i >> 7) & 15);
  const long ts = i >> 11;  // tile * nk + step
  const int step = (int)(ts % nk);
  const long c = (ts / nk) * 256 + blk * 16 + (lane & 15);
  const int k = step * 128 + (lane >> 4) * 32 + h * 16;
  u32x4 out = u32x4{0u, 0u, 0u, 0u};
  if (c < V) {
    const int be = ew[(c >> 7) * nk + step];
    const int sh = be == 255 ? 0 : 127 - be;
    const u32x4 v0 = ld16(src + c * K + k), v1 = ld16(src + c * K + k + 8);
    uint32_t hw[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      hw[j] = fp8_codes2(__builtin_ldexpf(bf2f((bf16_t)(v0[j] & 0xffffu)), sh),
                         __builtin_ldexpf(bf2f((bf16_t)(v0[j] >> 16)), sh));
      hw[4 + j] = fp8_codes2(__builtin_ldexpf(bf2f((bf16_t)(v1[j] & 0xffffu)), sh),
                             __builtin_ldexpf(bf2f((bf16_t)(v1[j] >> 16)), sh));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = hw[2 * j] | (hw[2 * j + 1] << 16);
  }
  st16(dst + i * 16, out);
}

// ---------------------------------------------------------------------------
// The W8A8 lm-head: one 256-column vocabulary tile of 16*MB rows per workgroup, the same
// column layout and epilogue as the bf16 head.  K runs in chunks of R = PF + 1 steps of
// 128; weight operands run PF steps ahead in a register ring of R slots.  The activation
// codes and row scales of chunk c+1 are loaded into registers during chunk c and written
// to the other half of a double LDS buffer at the start of chunk c+1, so the weight
// stream never waits for them.  Every load is unconditional (steps past the end re-read
// the last step) and the LDS copy is one chunk ahead, which keeps the compiler's vmcnt
// waits for the ring exact.  The MFMA operands are read from LDS by untracked inline asm
// with counted lgkmcnt waits (the wave's own stores precede the barrier that publishes
// them).  NT: the weights are streamed with the nontemporal policy (grids that read each
// weight once).  The weight block scales of the tile's two 128-column blocks sit in LDS
// for the whole kernel (K <= 128 * kF8MaxSteps).
// ---------------------------------------------------------------------------
constexpr int kF8MaxSteps = 256;

// The LDS stores below are read only by untracked inline asm, which the compiler does not
// see as a reader: without this fence it may drop them as dead.  An asm memory clobber
// counts as a read of every LDS array whose address escaped into asm (all of them here).
__device__ __forceinline__ void lds_publish() { asm volatile("" ::: "memory"); }


template <int MB, bool NT, bool ROWS_FAST, int PF = 1>
__global__ __launch_bounds__(256) void lm_head_fp8_kernel(const uint8_t *__restrict__ A8,
                                                          const int32_t *__restrict__ ea, int K,
                                                          const uint8_t *__restrict__ W8,
                                                          const int32_t *__restrict__ ew, int V,
                                                          const int32_t *__restrict__ target, int M,
                                                          float *__restrict__ part,
                                                          float *__restrict__ tgt_logit, int n_vt, int paired) {
  constexpr int R = PF + 1;                   // ring slots = K steps per chunk
  constexpr int ABLK = R * MB * 2;            // 1 KB activation blocks per chunk: (step, mb, half)
  constexpr int NE = R * MB * 16;             // row scales per chunk: (step, mb, row)
  constexpr int NEB = (NE + 63) / 64;         // ... in 64-entry copies
  constexpr int ACOPY = (ABLK + 3) / 4, ECOPY = (NEB + 3) / 4;  // copies per wave per chunk
  __shared__ float red[2][4][16 * MB];
  __shared__ u32x4 lds_a[2][ABLK * 64];
  __shared__ int32_t lds_e[2][NEB * 64];
  __shared__ int32_t lds_w[2][kF8MaxSteps];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, r16 = lane & 15;
  int tile = ROWS_FAST ? blockIdx.y : blockIdx.x;
  int rt = ROWS_FAST ? blockIdx.x : blockIdx.y;
  if (paired) {  // the bf16 head's paired 1-D grid: row tiles 0 and 1 of a vocabulary tile on one XCD
    tile = (blockIdx.x >> 4) * 8 + (blockIdx.x & 7);
    rt = (blockIdx.x >> 3) & 1;
    if (tile >= n_vt) return;
  }
  const int m0 = rt * 16 * MB;
  const int nk = K >> 7;
  const int rot = lm_rot(tile, nk);
  auto kidx = [&](int s) {  // the K block of step s (steps past the end re-read the last)
    const int t = (s < nk ? s : nk - 1) + rot;
    return t >= nk ? t - nk : t;
  };
  auto ldw = [&](const uint8_t *p) -> u32x4 {
    if (NT) return __builtin_nontemporal_load((const u32x4 __attribute__((address_space(1))) *)(p));
    return ld16(p);
  };
  const uint8_t *wp[4];  // block nb of this wave in step 0 of the tile; step s is s * 32 KB on
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) wp[nb] = W8 + (long)tile * nk * 32768 + (wave * 4 + nb) * 2048 + lane * 16;

  // Chunk c's activation blocks and row scales: loaded into registers (issue), then
  // stored to buffer buf (commit).  Every wave takes the same number of pieces: where the
  // blocks do not divide among the waves, the last block is copied again, with the same
  // bytes.  Row scale entries past NE (a step index >= R) are copied but never read.
  u32x4 sreg[ACOPY];
  int ereg[ECOPY];
  auto issue = [&](int c) {
#pragma unroll
    for (int i = 0; i < ACOPY; ++i) {
      const int q = min(i * 4 + wave, ABLK - 1);
      const int st = q / (2 * MB), mb = (q >> 1) % MB, h = q & 1;
      const int row = min(m0 + 16 * mb + r16, M - 1);
      sreg[i] = ld16(A8 + (long)row * K + kidx(c * R + st) * 128 + (lane >> 4) * 32 + h * 16);
    }
#pragma unroll
    for (int i = 0; i < ECOPY; ++i) {
      const int b = min(i * 4 + wave, NEB - 1), e = b * 64 + lane;
      const int st = e / (16 * MB), mb = (e >> 4) % MB, r = e & 15;
      ereg[i] = ea[(long)min(m0 + 16 * mb + r, M - 1) * nk + kidx(c * R + st)];
    }
  };
  auto commit = [&](int buf) {
#pragma unroll
    for (int i = 0; i < ACOPY; ++i) {
      const int q = min(i * 4 + wave, ABLK - 1);
      lds_a[buf][q * 64 + lane] = sreg[i];
    }
#pragma unroll
    for (int i = 0; i < ECOPY; ++i) {
      const int b = min(i * 4 + wave, NEB - 1);
      lds_e[buf][b * 64 + lane] = ereg[i];
    }
    lds_publish();
  };

  // Prologue: the loads of the weight block scales (the tile's two blocks), of chunk 0 and
  // of the ring's first PF steps all go out before any of them is waited for; then the
  // scales and chunk 0 go to LDS and chunk 1 is loaded.  The first barrier in the loop
  // publishes the LDS contents.
  int wsc[(2 * kF8MaxSteps + 255) / 256];
#pragma unroll
  for (int q = 0; q < (2 * kF8MaxSteps + 255) / 256; ++q) {
    const int i = q * 256 + threadIdx.x;
    wsc[q] = ew[(long)(tile * 2) * nk + min(i, 2 * nk - 1)];
  }
  issue(0);
  u32x4 rb[R][4][2];
#pragma unroll
  for (int s = 0; s < PF; ++s) {
    const long off = (long)kidx(s) * 32768;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      rb[s][nb][0] = ldw(wp[nb] + off);
      rb[s][nb][1] = ldw(wp[nb] + off + 1024);
    }
  }
#pragma unroll
  for (int q = 0; q < (2 * kF8MaxSteps + 255) / 256; ++q) {
    const int i = q * 256 + threadIdx.x;
    if (i < 2 * nk) lds_w[i / nk][i % nk] = wsc[q];
  }
  commit(0);
  issue(1);

  f32x4 acc[MB][4];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint32_t a_lane = lds_addr(&lds_a[0][0]) + lane * 16;
  const uint32_t e_lane = lds_addr(&lds_e[0][0]) + r16 * 4;
  const uint32_t w_base = lds_addr(&lds_w[wave >> 1][0]);
  const int nck = (nk + R - 1) / R;
  for (int c = 0; c < nck; ++c) {
    const int buf = c & 1;
    if (c > 0) {  // buffer buf was last read in chunk c-2, before the previous barrier
      commit(buf);
      issue(c + 1);
    }
    __syncthreads();  // chunk c (and, at c = 0, the weight scales) published
    const uint32_t a_base = a_lane + buf * (ABLK * 1024), e_base = e_lane + buf * (NEB * 256);
    static_for<R>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      const int ks = c * R + j;
      {
        const long off = (long)kidx(ks + PF) * 32768;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          rb[(j + PF) % R][nb][0] = ldw(wp[nb] + off);
          rb[(j + PF) % R][nb][1] = ldw(wp[nb] + off + 1024);
        }
      }
      if (ks < nk) {
        int sb;
        const uint32_t w_addr = w_base + kidx(ks) * 4;
        asm volatile("ds_read_b32 %0, %1" : "=v"(sb) : "v"(w_addr));
        u32x4 alo[MB], ahi[MB];
        int sa[MB];
        static_for<MB>([&](auto mc) {
          constexpr int mb = decltype(mc)::value;
          alo[mb] = lds_rd128<((j * MB + mb) * 2) * 1024>(a_base);
          ahi[mb] = lds_rd128<((j * MB + mb) * 2 + 1) * 1024>(a_base);
          sa[mb] = lds_rd32<(j * MB + mb) * 64>(e_base);
        });
        static_for<MB>([&](auto mc) {
          constexpr int mb = decltype(mc)::value;
          lds_wait<3 * (MB - 1 - mb)>();  // sb and the operands of blocks 0 .. mb are in
          settle(alo[mb]);
          settle(ahi[mb]);
          settle(sa[mb]);
          if (mb == 0) settle(sb);
          const i32x8 a = cat8(alo[mb], ahi[mb]);
#pragma unroll
          for (int nb = 0; nb < 4; ++nb)
            acc[mb][nb] = mfma_fp8(a, cat8(rb[j][nb][0], rb[j][nb][1]), acc[mb][nb], sa[mb], sb);
        });
      }
    });
  }
  lm_tile_epilogue<MB>(acc, red, wave, tile, m0, M, V, target, part, tgt_logit, n_vt);
}

// ---------------------------------------------------------------------------
// W8A8 projections (the same deployment rule for the model's GEMMs).  Weight [N, K]
// row-major bf16 -> codes [N, K] (one byte per weight, row-major) and biased exponents
// ew [ceil(N/128), K/128] of the 128 x 128 blocks (pack_fp8_exp_kernel over 128-row
// blocks).  16 codes per thread.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void quant_weight_fp8_codes_kernel(const bf16_t *__restrict__ src, int K,
                                                                     const int32_t *__restrict__ ew,
                                                                     uint8_t *__restrict__ dst, long n_pieces) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n_pieces) return;
  const int nk = K >> 7, per_row = K >> 4;
  const long row = i / per_row;
  const int k = (int)(i % per_row) * 16;
  const int be = ew[(row >> 7) * nk + (k >> 7)];
  const int sh = be == 255 ? 0 : 127 - be;
  const u32x4 v0 = ld16(src + row * K + k), v1 = ld16(src + row * K + k + 8);
  uint32_t hw[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    hw[j] = fp8_codes2(__builtin_ldexpf(bf2f((bf16_t)(v0[j] & 0xffffu)), sh),
                       __builtin_ldexpf(bf2f((bf16_t)(v0[j] >> 16)), sh));
    hw[4 + j] = fp8_codes2(__builtin_ldexpf(bf2f((bf16_t)(v1[j] & 0xffffu)), sh),
                           __builtin_ldexpf(bf2f((bf16_t)(v1[j] >> 16)), sh));
  }
  u32x4 out;
#pragma unroll
  for (int j = 0; j < 4; ++j) out[j] = hw[2 * j] | (hw[2 * j + 1] << 16);
  st16(dst + i * 16, out);
}

// C[M, N] = bf16(A W^T), or bf16(R + bf16(A W^T)), from the rows' codes A8 [M, K] and
// exponents ea [M, K/128] and the weight's codes W8 [N, K] and exponents ew
// [ceil(N/128), K/128].  Every output element is one chain of scaled FP8 MFMAs over K in
// 128-wide steps k = 0, 128, 256, ... in order, from zero: the M tile a workgroup owns,
// the grid and the number of rows never change it.
// Up to 256 rows: a workgroup of 4 waves covers 16*MB rows x 64 columns, wave w the 16
// columns n0 + 16w ..  The rows' codes and exponents of a chunk of kF8RowChunk steps are
// staged through LDS once per workgroup (double-buffered, wave w loading step w of the
// chunk); each wave streams its 16 weight rows' codes and their block exponent through a
// register ring S steps deep (every load unconditional: past the last step it re-reads it).
constexpr int kF8RowChunk = 4;

template <int MB, int S>
__global__ __launch_bounds__(256) void gemm_fp8_kernel(const uint8_t *__restrict__ A8, const int32_t *__restrict__ ea,
                                                       const uint8_t *__restrict__ W8, const int32_t *__restrict__ ew,
                                                       bf16_t *__restrict__ C, int ldc, const bf16_t *__restrict__ R,
                                                       int ldr, int M, int N, int K) {
  static_assert(S % kF8RowChunk == 0, "a chunk starts at a ring slot 0 .. S-1 boundary");
  __shared__ u32x4 lds_a[2][kF8RowChunk * MB * 2 * 64];
  __shared__ int32_t lds_e[2][kF8RowChunk * 16 * MB];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int grp = lane >> 4, r16 = lane & 15;
  const int m0 = blockIdx.y * 16 * MB;
  const int n0 = blockIdx.x * 64 + wave * 16;
  const int nk = K >> 7;
  const int col = min(n0 + r16, N - 1);  // columns past N are computed and dropped
  const uint8_t *wp = W8 + (long)col * K + grp * 32;
  const int32_t *swp = ew + (long)(col >> 7) * nk;
  const uint8_t *arow[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) arow[mb] = A8 + (long)min(m0 + 16 * mb + r16, M - 1) * K + grp * 32;
  const int32_t *erow = ea + (long)min(m0 + min(lane, 16 * MB - 1), M - 1) * nk;
  struct WOp {
    u32x4 lo, hi;
    int e;
  };
  auto load_w = [&](int s, WOp &o) {
    o.lo = ld16(wp + s * 128);
    o.hi = ld16(wp + s * 128 + 16);
    o.e = swp[s];
  };
  WOp ring[S];
#pragma unroll
  for (int j = 0; j < S - 1; ++j) load_w(min(j, nk - 1), ring[j]);
  f32x4 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < nk; k0 += S) {
#pragma unroll
    for (int j = 0; j < S; ++j) {
      const int ks = k0 + j;
      if (j % kF8RowChunk == 0 && ks < nk) {
        __syncthreads();  // every wave is done with the buffer about to be refilled
        const int buf = (ks / kF8RowChunk) & 1, st = ks + wave;
        if (st < nk) {
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            lds_a[buf][((wave * MB + mb) * 2 + 0) * 64 + lane] = ld16(arow[mb] + st * 128);
            lds_a[buf][((wave * MB + mb) * 2 + 1) * 64 + lane] = ld16(arow[mb] + st * 128 + 16);
          }
          if (lane < 16 * MB) lds_e[buf][wave * 16 * MB + lane] = erow[st];
        }
        __syncthreads();
      }
      load_w(min(ks + S - 1, nk - 1), ring[(j + S - 1) % S]);
      if (ks < nk) {
        const int buf = (ks / kF8RowChunk) & 1, st = ks % kF8RowChunk;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const u32x4 lo = lds_a[buf][((st * MB + mb) * 2 + 0) * 64 + lane];
          const u32x4 hi = lds_a[buf][((st * MB + mb) * 2 + 1) * 64 + lane];
          const int sa = lds_e[buf][st * 16 * MB + 16 * mb + r16];
          acc[mb] = mfma_fp8(cat8(lo, hi), cat8(ring[j].lo, ring[j].hi), acc[mb], sa, ring[j].e);
        }
      }
    }
  }
  const int c = n0 + r16;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = m0 + 16 * mb + 4 * grp + i;
      if (row < M && c < N) {
        float v = bf2f(f2bf(acc[mb][i]));
        if (R) v = bf2f(R[(long)row * ldr + c]) + v;
        C[(long)row * ldc + c] = f2bf(v);
      }
    }
  }
}

// W8A8 projections past 256 rows: 256-row x 256-column tiles on 8 waves (wave w: rows
// 128(w/4) .., columns 64(w%4) .., 8 x 4 blocks), on the persistent XCD-blocked grid of the
// bf16 wide kernel.  Each 128-wide K step's code operands (16 row blocks and 16 column
// blocks of 2 KB, each in MFMA lane order as two 1 KB halves) are copied once into LDS
// by direct-to-LDS loads, one step ahead in a 2-deep ring; the lanes' row and column
// exponents of the next step are plain loads issued with the copy.  The K order and the
// MFMA per step are those of gemm_fp8_kernel, so a row's bits are the same at any M.
constexpr int kF8WideRows = 256, kF8WideGrid = 256;

__global__ __launch_bounds__(512) void gemm_fp8_wide_kernel(const uint8_t *__restrict__ A8,
                                                            const int32_t *__restrict__ ea,
                                                            const uint8_t *__restrict__ W8,
                                                            const int32_t *__restrict__ ew, bf16_t *__restrict__ C,
                                                            int ldc, const bf16_t *__restrict__ R, int ldr, int M,
                                                            int N, int K, int br) {
  constexpr int kStepB = 64 * 1024;  // row blocks 0..15, then column blocks 0..15, 2 KB each
  __shared__ __attribute__((aligned(16))) uint8_t buf[2][kStepB];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int grp = lane >> 4, r16 = lane & 15;
  const int rg = wave >> 2, cg = wave & 3;
  const int nk = K >> 7;
  const int n_rt = (M + kF8WideRows - 1) / kF8WideRows, n_ct = (N + 255) / 256;
  const int bv = 32 / br;
  const int nbr = (n_rt + br - 1) / br, n_blocks = nbr * ((n_ct + bv - 1) / bv);
  const int xcd = blockIdx.x % 8, l = blockIdx.x / 8;
  const uint32_t lds0 = lds_addr(&buf[0][0]);
  const uint32_t abase = lds0 + rg * 16384 + lane * 16, bbase = lds0 + 32768 + cg * 8192 + lane * 16;
  for (int blk = xcd; blk < n_blocks; blk += 8) {
    const int rt = (blk % nbr) * br + l % br, tile = (blk / nbr) * bv + l / br;
    if (rt >= n_rt || tile >= n_ct) continue;  // the same for the whole workgroup
    const int m0 = rt * kF8WideRows, n0 = tile * 256;
    // this wave copies row blocks 2w, 2w+1 and column blocks 2w, 2w+1 (rows past M read
    // row M-1, columns past N column N-1; their results are dropped)
    const uint8_t *asrc[2], *wsrc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      asrc[j] = A8 + (long)min(m0 + 16 * (2 * wave + j) + r16, M - 1) * K + grp * 32;
      wsrc[j] = W8 + (long)min(n0 + 16 * (2 * wave + j) + r16, N - 1) * K + grp * 32;
    }
    // the lane's row exponent per row block, and the wave's column block exponent
    const int32_t *sap[8];
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) sap[mb] = ea + (long)min(m0 + rg * 128 + 16 * mb + r16, M - 1) * nk;
    const int32_t *swp = ew + (long)(min(n0 + cg * 64, N - 1) >> 7) * nk;
    auto copy_step = [&](int s) {
      uint8_t *b = &buf[s & 1][0];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          __builtin_amdgcn_global_load_lds(asrc[j] + s * 128 + 16 * h, b + (2 * wave + j) * 2048 + h * 1024, 16, 0, 0);
          __builtin_amdgcn_global_load_lds(wsrc[j] + s * 128 + 16 * h, b + 32768 + (2 * wave + j) * 2048 + h * 1024,
                                           16, 0, 0);
        }
      }
    };
    int sa[8], sb, sa_n[8], sb_n = 0;
    // every wave is done with the previous tile's buffers
    __syncthreads();
    copy_step(0);
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) sa_n[mb] = sap[mb][0];
    sb_n = swp[0];
    f32x4 acc[8][4];
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < nk; ++s) {
      // step s landed (this wave's copies and exponent loads), then the barrier: every
      // wave's blocks are visible and every wave is done with step s-1's buffer, which
      // the copy of step s+1 refills
      wait_vmem<0>();
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) sa[mb] = sa_n[mb];
      sb = sb_n;
      asm volatile("s_barrier" ::: "memory");
      if (s + 1 < nk) {
        copy_step(s + 1);
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) sa_n[mb] = sap[mb][s + 1];
        sb_n = swp[s + 1];
      }
      const uint32_t off = (uint32_t)(s & 1) * kStepB;
      u32x4 b[4][2];
      static_for<4>([&](auto nb_) {
        constexpr int nb = decltype(nb_)::value;
        b[nb][0] = lds_rd128<nb * 2048>(bbase + off);
        b[nb][1] = lds_rd128<nb * 2048 + 1024>(bbase + off);
      });
      u32x4 a[2][2];
      a[0][0] = lds_rd128<0>(abase + off);
      a[0][1] = lds_rd128<1024>(abase + off);
      static_for<8>([&](auto mb_) {
        constexpr int mb = decltype(mb_)::value;
        if constexpr (mb + 1 < 8) {  // the next row block's operand while this one's MFMAs run
          a[(mb + 1) & 1][0] = lds_rd128<(mb + 1) * 2048>(abase + off);
          a[(mb + 1) & 1][1] = lds_rd128<(mb + 1) * 2048 + 1024>(abase + off);
          lds_wait<2>();
        } else {
          lds_wait<0>();
        }
        if (mb == 0) {
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) {
            settle(b[nb][0]);
            settle(b[nb][1]);
          }
        }
        settle(a[mb & 1][0]);
        settle(a[mb & 1][1]);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          acc[mb][nb] = mfma_fp8(cat8(a[mb & 1][0], a[mb & 1][1]), cat8(b[nb][0], b[nb][1]), acc[mb][nb], sa[mb], sb);
      });
    }
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int col = n0 + cg * 64 + 16 * nb + r16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = m0 + rg * 128 + 16 * mb + 4 * grp + i;
          if (row < M && col < N) {
            float v = bf2f(f2bf(acc[mb][nb][i]));
            if (R) v = bf2f(R[(long)row * ldr + col]) + v;
            C[(long)row * ldc + col] = f2bf(v);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------

long proj_fp8_bytes(int N, int K) {
  if (N < 1 || K < 128 || K % 128) return 0;
  return (long)N * K + (long)((N + 127) / 128) * (K / 128) * 4;
}

hipError_t launch_quant_weight_fp8(const bf16_t *src, int N, int K, uint8_t *codes, int32_t *ew, hipStream_t st) {
  const long n_pieces = (long)N * K / 16;
  if (n_pieces == 0) return hipSuccess;
  const long blocks = (n_pieces + 255) / 256;
  if (blocks > 0x7fffffffL || K / 128 > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pack_fp8_exp_kernel, dim3((N + 127) / 128, K / 128), dim3(256), 0, st, src, N, K, ew);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(quant_weight_fp8_codes_kernel, dim3((unsigned)blocks), dim3(256), 0, st, src, K, ew, codes,
                     n_pieces);
  return hipGetLastError();
}

hipError_t launch_gemm_fp8(const GemmFp8Args &a, hipStream_t st) {
  if (a.M == 0) return hipSuccess;
  if (a.M > 256) {
    // many rows: 256 x 256 tiles with the code operands shared through LDS, on the
    // persistent XCD-blocked grid; the K order is unchanged
    const int n_rt = (a.M + kF8WideRows - 1) / kF8WideRows;
    const int br = n_rt >= 4 ? 4 : (n_rt >= 2 ? 2 : 1);
    hipLaunchKernelGGL(gemm_fp8_wide_kernel, dim3(kF8WideGrid), dim3(512), 0, st, a.A8, a.ea, a.W8, a.ew, a.C, a.ldc,
                       a.R, a.ldr, a.M, a.N, a.K, br);
    return hipGetLastError();
  }
#define RIL_G8(MB_, S_)                                                                                     \
  hipLaunchKernelGGL((gemm_fp8_kernel<MB_, S_>), dim3((a.N + 63) / 64, (a.M + 16 * MB_ - 1) / (16 * MB_)), dim3(256), \
                     0, st, a.A8, a.ea, a.W8, a.ew, a.C, a.ldc, a.R, a.ldr, a.M, a.N, a.K)
  if (a.M <= 16) RIL_G8(1, 8);
  else RIL_G8(4, 8);
#undef RIL_G8
  return hipGetLastError();
}

hipError_t launch_quant_rows_fp8(const QuantRowsArgs &a, hipStream_t st) {
  if (a.M == 0) return hipSuccess;
  const long threads = (long)a.M * (a.K / 128) * 16;
  const long blocks = (threads + 255) / 256;
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(quant_rows_fp8_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a.Z, a.ldz, a.M, a.K, a.A8,
                     a.ea);
  return hipGetLastError();
}

hipError_t launch_lm_head_fp8(const LmHeadArgs &a, hipStream_t st) {
  if (a.M == 0) return hipSuccess;
  const int n_vt = (a.V + kVocabTile - 1) / kVocabTile;
  const int mb = a.M <= 16 ? 1 : 4;
  const int n_rt = (a.M + 16 * mb - 1) / (16 * mb);
  // the grid choice of the bf16 head: one row tile streams the weights (NT), two share
  // each weight slice through an XCD's L2 (the paired grid, ordinary loads), more run
  // the row tiles of one vocabulary tile back to back; none changes a K order
  if (n_rt == 2) {
    const dim3 grid((unsigned)(16 * ((n_vt + 7) / 8)));
    hipLaunchKernelGGL((lm_head_fp8_kernel<4, false, false>), grid, dim3(256), 0, st, a.A8, a.ea, a.K, a.W8,
                       a.ew, a.V, a.target, a.M, a.part, a.tgt_logit, n_vt, 1);
  } else if (n_rt == 1) {
    dim3 grid(n_vt, 1);
    if (mb == 1)
      hipLaunchKernelGGL((lm_head_fp8_kernel<1, true, false>), grid, dim3(256), 0, st, a.A8, a.ea, a.K, a.W8,
                         a.ew, a.V, a.target, a.M, a.part, a.tgt_logit, n_vt, 0);
    else
      hipLaunchKernelGGL((lm_head_fp8_kernel<4, true, false>), grid, dim3(256), 0, st, a.A8, a.ea, a.K, a.W8,
                         a.ew, a.V, a.target, a.M, a.part, a.tgt_logit, n_vt, 0);
  } else {
    dim3 grid(n_rt, n_vt);
    hipLaunchKernelGGL((lm_head_fp8_kernel<4, false, true>), grid, dim3(256), 0, st, a.A8, a.ea, a.K, a.W8, a.ew,
                       a.V, a.target, a.M, a.part, a.tgt_logit, n_vt, 0);
  }
  return hipGetLastError();
}

long lm_head_fp8_code_bytes(int V, int K) {
  const long n_vt = (V + kVocabTile - 1) / kVocabTile;
  return n_vt * kVocabTile * (long)K;
}

long lm_head_fp8_exp_count(int V, int K) {
  const long n_vt = (V + kVocabTile - 1) / kVocabTile;
  return n_vt * 2 * (long)(K / 128);
}

hipError_t launch_pack_lm_head_fp8(const bf16_t *src, int V, int K, uint8_t *codes, int32_t *ew, hipStream_t st) {
  const int n_vt = (V + kVocabTile - 1) / kVocabTile;
  const long n_pieces = lm_head_fp8_code_bytes(V, K) / 16;
  if (n_pieces == 0) return hipSuccess;
  const long blocks = (n_pieces + 255) / 256;
  if (blocks > 0x7fffffffL || K / 128 > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pack_fp8_exp_kernel, dim3(2 * n_vt, K / 128), dim3(256), 0, st, src, V, K, ew);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(pack_fp8_codes_kernel, dim3((unsigned)blocks), dim3(256), 0, st, src, V, K, ew, codes,
                     n_pieces);
  return hipGetLastError();
}

}  // namespace ril
