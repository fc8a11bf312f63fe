// Dense parts of the path: embedding gather + RMSNorm (S2, S3), projection GEMMs with
// one MFMA K order and no split-K (S4), the lm-head with per-vocabulary-tile softmax
// partials and target-logit capture (S11), and the fixed-tree vocabulary merge that
// yields the logprob (S12).
//
// Batch invariance of the GEMMs (Bitwise-consistent RL post, section 4.1: one
// accumulation order for every M): each output element is one chain of
// v_mfma_f32_16x16x32_bf16 over K in 32-wide steps, k = 0, 32, 64, ... in order,
// starting from 0.  The M/N tile a workgroup owns, the grid and the number of rows
// never change that chain, and no K range is ever split across waves.
#include "common.h"
#include "kernels.h"
#include "lm_head.h"
#include "norm.h"

namespace ril {

// ---------------------------------------------------------------------------
// S2 + S3: y = bf16((x * rsqrt(mean(x^2) + eps)) * g), x = E[token] or a dense row.
// One wave per row, the arithmetic of rmsnorm_row (norm.h).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void rmsnorm_kernel(
    const bf16_t *__restrict__ x, int ldx, const int32_t *__restrict__ tok,
    const bf16_t *__restrict__ embed, int vocab, int d, const bf16_t *__restrict__ gain, float eps,
    bf16_t *__restrict__ y, int ldy, bf16_t *__restrict__ x_copy, int ldc) {
  const int row = blockIdx.x;
  const bf16_t *src;
  bool poison = false;
  if (tok) {
    int t = tok[row];
    if (t < 0 || t >= vocab) {
      poison = true;
      t = 0;
    }
    src = embed + (long)t * d;
  } else {
    src = x + (long)row * ldx;
  }
  bf16_t *yr = y + (long)row * ldy;
  bf16_t *xc = x_copy ? x_copy + (long)row * ldc : nullptr;
  rmsnorm_row([&](int e) { return ld16(src + e * 8); },
              [&](int e, u32x4 out, u32x4 v) {
                st16(yr + e * 8, out);
                if (xc) st16(xc + e * 8, v);
              },
              d, gain, eps, poison);
}

// ---------------------------------------------------------------------------
// SwiGLU activation between the two MLP GEMMs: silu(g) * u formed in fp32 and rounded to
// bf16 once (Bitwise-consistent RL post, section 4.4, condition 3: rounding silu before
// the multiply can move the result by an ulp).  silu(g) = g / (1 + 2^(-g log2 e)) with the
// hardware exp2 and an IEEE divide, the same instructions in every phase.  One thread per
// 8 columns of a row.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void silu_mul_kernel(const bf16_t *__restrict__ gu, int ldg,
                                                       bf16_t *__restrict__ act, int lda, int rows, int F) {
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const int per = F / 8;
  if (idx >= (long)rows * per) return;
  const int r = (int)(idx / per), j0 = (int)(idx % per) * 8;
  const u32x4 g8 = ld16(gu + (long)r * ldg + j0), u8 = ld16(gu + (long)r * ldg + F + j0);
  u32x4 out;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    float v[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float g = bf2f((bf16_t)(h ? (g8[w] >> 16) : (g8[w] & 0xffffu)));
      const float u = bf2f((bf16_t)(h ? (u8[w] >> 16) : (u8[w] & 0xffffu)));
      const float sg = __fdiv_rn(g, 1.0f + exp2f_hw(-g * kLog2e));
      v[h] = sg * u;
    }
    out[w] = pack2(v[0], v[1]);
  }
  st16(act + (long)r * lda + j0, out);
}

hipError_t launch_silu_mul(const SiluMulArgs &a, hipStream_t st) {
  const long n = (long)a.rows * (a.F / 8);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(silu_mul_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a.gu, a.ldg, a.act,
                     a.lda, a.rows, a.F);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// The K loop of every GEMM here: acc[mb][nb] += A_mb(k) B_nb(k)^T for k = 0, 32, 64, ...
// in order, one v_mfma_f32_16x16x32_bf16 per step and block.  Operand loads run PF steps
// ahead through a register ring (issue order only; the accumulation order is fixed).
// ---------------------------------------------------------------------------
template <int MB, int NB, int PF>
__device__ __forceinline__ void kloop(f32x4 (&acc)[MB][NB], const bf16_t *const (&ap)[MB],
                                      const bf16_t *const (&wp)[NB], int K) {
  constexpr int S = PF + 1;
  u32x4 ra[S][MB], rb[S][NB];
  const int nk = K / 32;
#pragma unroll
  for (int s = 0; s < PF; ++s) {
    if (s < nk) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) ra[s][mb] = ld16(ap[mb] + s * 32);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) rb[s][nb] = ld16(wp[nb] + s * 32);
    }
  }
  for (int k0 = 0; k0 < nk; k0 += S) {
#pragma unroll
    for (int j = 0; j < S; ++j) {
      const int ks = k0 + j;
      if (ks < nk) {
        const int kp = ks + PF;
        if (kp < nk) {
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) ra[(j + PF) % S][mb] = ld16(ap[mb] + kp * 32);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) rb[(j + PF) % S][nb] = ld16(wp[nb] + kp * 32);
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            acc[mb][nb] = mfma(as_bf16x8(ra[j][mb]), as_bf16x8(rb[j][nb]), acc[mb][nb]);
      }
    }
  }
}

// The K loop of the lm-head up to 128 rows, the activation operand staged through LDS.
// Every output column accumulates its 32-wide K steps in the order r, r+1, ..., nk-1, 0,
// ..., r-1 (rot = lm_rot(tile)).  The activation operand is staged through LDS in chunks
// of 8 K steps (each of the four waves loads two steps for the whole workgroup); weight
// operands run PF steps ahead in a register ring.  wp[nb] points at MFMA block nb's first
// operand; step s's operand is WSTEP elements further (512 in the packed layout).  NT: weight loads use the nontemporal (streaming) cache policy, for
// grids that read each weight once.  All four waves must call this (it synchronises the
// workgroup).
constexpr int kLdsSteps = 8;

template <int MB, int NB, int PF, int WSTEP, bool NT>
__device__ __forceinline__ void kloop_lds(f32x4 (&acc)[MB][NB], const bf16_t *const (&ap)[MB],
                                          const bf16_t *const (&wp)[NB], int K, int rot,
                                          u32x4 (*lds)[kLdsSteps * MB * 64]) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  constexpr int S = PF + 1;
  const int nk = K / 32;
  auto kidx = [&](int s) {
    const int t = s + rot;
    return t >= nk ? t - nk : t;
  };
  auto ldw = [&](const bf16_t *p) -> u32x4 {
    if (NT) return __builtin_nontemporal_load((const u32x4 __attribute__((address_space(1))) *)(p));
    return ld16(p);
  };
  u32x4 rb[S][NB];
#pragma unroll
  for (int s = 0; s < PF; ++s) {
    if (s < nk) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) rb[s][nb] = ldw(wp[nb] + (long)kidx(s) * WSTEP);
    }
  }
  for (int k0 = 0; k0 < nk; k0 += S) {
#pragma unroll
    for (int j = 0; j < S; ++j) {
      const int ks = k0 + j;
      if (ks < nk) {
        if (ks % kLdsSteps == 0) {
          __syncthreads();  // every wave is done with the buffer about to be refilled
          const int buf = (ks / kLdsSteps) & 1;
#pragma unroll
          for (int q = 0; q < kLdsSteps / 4; ++q) {
            const int st = wave * (kLdsSteps / 4) + q;
            if (ks + st < nk) {
#pragma unroll
              for (int mb = 0; mb < MB; ++mb) lds[buf][(st * MB + mb) * 64 + lane] = ld16(ap[mb] + kidx(ks + st) * 32);
            }
          }
          __syncthreads();
        }
        const int kp = ks + PF;
        if (kp < nk) {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) rb[(j + PF) % S][nb] = ldw(wp[nb] + (long)kidx(kp) * WSTEP);
        }
        const int buf = (ks / kLdsSteps) & 1, st = ks % kLdsSteps;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const bf16x8 a = as_bf16x8(lds[buf][(st * MB + mb) * 64 + lane]);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = mfma(a, as_bf16x8(rb[j][nb]), acc[mb][nb]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// S4: C[M,N] = bf16(A[M,K] W[N,K]^T) or bf16(R + bf16(A W^T)).
// Workgroup = 4 waves side by side along N; a wave owns MB x NB 16x16 blocks.
// ---------------------------------------------------------------------------
// The invariant path always runs with gridDim.z == 1 and part == nullptr: one sequential
// K loop per output element.  gridDim.z > 1 (K chunk kchunk, fp32 partials to `part`,
// reduced by gemm_reduce_kernel) is the shape-derived comparator's split-K only.
template <int MB, int NB>
__global__ __launch_bounds__(256) void gemm_kernel(const bf16_t *__restrict__ A, int lda,
                                                   const bf16_t *__restrict__ W, int ldw,
                                                   bf16_t *__restrict__ C, int ldc,
                                                   const bf16_t *__restrict__ R, int ldr, int M,
                                                   int N, int K, int kchunk, float *__restrict__ part) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int grp = lane >> 4, r16 = lane & 15;
  const int m0 = blockIdx.y * 16 * MB;
  const int n0 = (blockIdx.x * 4 + wave) * 16 * NB;
  if (n0 >= N) return;
  const int k0 = blockIdx.z * kchunk;
  const int klen = min(kchunk, K - k0);
  const bf16_t *ap[MB];
  const bf16_t *wp[NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) ap[mb] = A + (long)min(m0 + 16 * mb + r16, M - 1) * lda + k0 + grp * 8;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) wp[nb] = W + (long)min(n0 + 16 * nb + r16, N - 1) * ldw + k0 + grp * 8;
  f32x4 acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  kloop<MB, NB, 3>(acc, ap, wp, klen);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int col = n0 + 16 * nb + r16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = m0 + 16 * mb + 4 * grp + i;
        if (row < M && col < N) {
          if (part) {
            part[((long)blockIdx.z * M + row) * N + col] = acc[mb][nb][i];
          } else {
            float v = bf2f(f2bf(acc[mb][nb][i]));
            if (R) v = bf2f(R[(long)row * ldr + col]) + v;
            C[(long)row * ldc + col] = f2bf(v);
          }
        }
      }
    }
  }
}

// S4 for few rows and long K (M <= 256, K >= 1024): both operands streamed through LDS.
// A workgroup owns a tile of 16*RB rows x 16*CB columns.  Three producer waves copy the
// tile's operands into two LDS rings by direct-to-LDS loads -- one the rows' operand
// (L2-resident: every column tile reads it), two the weight's (streamed from HBM, so its
// ring is as deep as LDS allows) -- and four consumer waves read them back in the MFMA
// lane layout.  Each copy instruction moves eight rows x 128 bytes: two 32-wide K steps of
// each row, whole cache lines, which halves the L2 requests per byte against the one-step
// operand load (the L2 request rate, not HBM, bounds this shape; measured 2.4x at 128
// rows).  The 16-byte chunks of a row are rotated by the row index inside the copy, so
// the operand reads hit eight distinct bank groups per eight lanes.  One barrier per
// chunk of CH steps: each producer's copies of chunk c have landed, and every consumer is
// done with chunk c-1's buffers, which the producers then refill.  Tiles are sized so a
// 4096-column projection makes about 256 workgroups (one per CU), and the row tiles of
// one column tile land on one XCD, so a weight byte comes from HBM once.  Every element's
// K order is 0, 32, 64, ... with one v_mfma_f32_16x16x32_bf16 per step, the operands those
// of gemm_kernel: its bits are those of gemm_kernel and wide_kernel<false> at any M.
constexpr int kStreamProd = 3, kStreamCons = 4;
constexpr int kStreamThreads = 64 * (kStreamCons + kStreamProd);
constexpr int kStreamLds = 144 * 1024;
template <int RB, int CB, int CH>
struct StreamTile {
  // per chunk of CH steps (CH/2 K-step pairs): the row operand's and the weight's bytes,
  // and the copies of the row producer and of each of the two weight producers
  static constexpr int kABytes = (CH / 2) * 2 * RB * 1024;
  static constexpr int kWBytes = (CH / 2) * 2 * CB * 1024;
  static constexpr int kALoads = (CH / 2) * 2 * RB;
  static constexpr int kWLoads = (CH / 2) * CB;
  // ring depths in chunks: the rows (L2-resident, short latency) four chunks if the vmcnt
  // field allows, else three; the weight (from HBM) as deep as LDS and the field allow
  static constexpr int kARing = 2 * kALoads <= 63 ? 4 : 3;
  static_assert(kALoads <= 63, "the row producer's chunk fits the vmcnt field");
  static constexpr int kWByLds = (kStreamLds - kARing * kABytes) / kWBytes;
  static constexpr int kWByCnt = 63 / kWLoads + 2;
  static constexpr int kWRing0 = kWByLds < kWByCnt ? kWByLds : kWByCnt;
  static constexpr int kWRing = kWRing0 < 32 ? kWRing0 : 32;
  static_assert(kWRing >= 3 && (kARing - 2) * kALoads <= 63, "ring depths");
  // consumer wave w's blocks: RB >= 4: row blocks w, w+4, .. x every column block;
  // else CB >= 4: column blocks w, w+4, .. x every row block; else block (w / CB, w % CB)
  static constexpr int kWR = RB >= 4 ? RB / 4 : (CB >= 4 ? RB : 1);
  static constexpr int kWC = RB >= 4 ? CB : (CB >= 4 ? CB / 4 : 1);
};

template <int RB, int CB, int CH>
__global__ __launch_bounds__(kStreamThreads) void gemm_stream_kernel(const bf16_t *__restrict__ A, int lda,
                                                                     const bf16_t *__restrict__ W, int ldw,
                                                                     bf16_t *__restrict__ C, int ldc,
                                                                     const bf16_t *__restrict__ R, int ldr, int M,
                                                                     int N, int K) {
  using T = StreamTile<RB, CB, CH>;
  constexpr int NA = T::kARing, NW = T::kWRing;
  __shared__ __attribute__((aligned(16))) uint8_t aring[NA][T::kABytes];
  __shared__ __attribute__((aligned(16))) uint8_t wring[NW][T::kWBytes];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n0 = blockIdx.x * 16 * CB, m0 = blockIdx.y * 16 * RB;
  const int nk = K / 32, nc = (nk + CH - 1) / CH;
  if (wave >= kStreamCons) {
    // producers: wave 0 of them copies the rows' operand, waves 1 and 2 the weight's
    // (alternate eight-row pieces).  Per K-step pair an operand of 16*X rows is 2*X pieces
    // of eight rows x 128 bytes; lane l moves 16 bytes of row l/8 of its piece: chunk
    // c = (l - l/8) mod 8 of the row's 128 bytes, i.e. K values 8c .. 8c+7 of the pair,
    // into slot l (the rotation).  Past the last step a copy re-reads the last pair (and
    // K past the end is clamped into the row), so every chunk issues the same loads and
    // each producer's vmcnt waits (on its own copies only) are exact.
    const int p = wave - kStreamCons;
    const int rho = lane >> 3, cch = (lane - rho) & 7;
    const int npair = (nk + 1) / 2;
    const bool rows = p == 0;
    const bf16_t *base = rows ? A + (long)m0 * lda : W + (long)n0 * ldw;
    const int ld = rows ? lda : ldw, lim = rows ? M - 1 - m0 : N - 1 - n0;
    auto issue = [&](int c) {
      uint8_t *dst = rows ? &aring[c % NA][0] : &wring[c % NW][0];
      static_for<CH / 2>([&](auto q_) {
        constexpr int q = decltype(q_)::value;
        const int pair = min(c * (CH / 2) + q, npair - 1);
        const int k = min(pair * 64 + 8 * cch, K - 8);
        if (rows) {
          static_for<2 * RB>([&](auto i_) {
            constexpr int i = decltype(i_)::value;
            const bf16_t *src = base + (long)min(8 * i + rho, lim) * ld + k;
            __builtin_amdgcn_global_load_lds((void *)src, (void *)(dst + (q * 2 * RB + i) * 1024), 16, 0, 0);
          });
        } else {
          static_for<CB>([&](auto i_) {
            constexpr int i = 2 * decltype(i_)::value;
            const int piece = i + (p - 1);
            const bf16_t *src = base + (long)min(8 * piece + rho, lim) * ld + k;
            __builtin_amdgcn_global_load_lds((void *)src, (void *)(dst + (q * 2 * CB + piece) * 1024), 16, 0, 0);
          });
        }
      });
    };
    const int ahead = rows ? NA - 1 : NW - 1;
    for (int c = 0; c < ahead; ++c) issue(c);
    for (int c = 0; c < nc; ++c) {
      // chunk c landed (the later chunks this producer issued may be in flight)
      if (rows) wait_vmem<(NA - 2) * T::kALoads>();
      else wait_vmem<(NW - 2) * T::kWLoads>();
      asm volatile("s_barrier" ::: "memory");
      issue(c + ahead);  // into chunk c-1's buffer, which every consumer is done with
    }
    wait_vmem<0>();  // no copy may still write this workgroup's LDS when it ends
    return;
  }
  // consumer: blocks (rb0 + 4 i or rb0 + i, cb ...) as StreamTile describes
  constexpr int WR = T::kWR, WC = T::kWC;
  int rbs[WR], cbs[WC];
  if constexpr (RB >= 4) {
#pragma unroll
    for (int i = 0; i < WR; ++i) rbs[i] = wave + 4 * i;
#pragma unroll
    for (int i = 0; i < WC; ++i) cbs[i] = i;
  } else if constexpr (CB >= 4) {
#pragma unroll
    for (int i = 0; i < WR; ++i) rbs[i] = i;
#pragma unroll
    for (int i = 0; i < WC; ++i) cbs[i] = wave + 4 * i;
  } else {
    rbs[0] = wave / CB;
    cbs[0] = wave % CB;
  }
  // a wave with no block (fewer than four), or whose rows all lie past M, keeps the barriers
  const bool idle = (RB < 4 && CB < 4 && wave >= RB * CB) || m0 + 16 * rbs[0] >= M;
  if (idle) {
    for (int c = 0; c < nc; ++c) asm volatile("s_barrier" ::: "memory");
    return;
  }
  f32x4 acc[WR][WC];
#pragma unroll
  for (int i = 0; i < WR; ++i)
#pragma unroll
    for (int j = 0; j < WC; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // this lane's operand (row r16 of a 16-row block, K chunk grp of step u of a pair):
  // piece r16/8, row r16%8, 16-byte chunk 4u + grp, at its rotated slot
  const int grp = lane >> 4, r16 = lane & 15, rho = r16 & 7;
  uint32_t off[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) off[u] = (uint32_t)((r16 >> 3) * 1024 + (rho * 8 + ((4 * u + grp + rho) & 7)) * 16);
  const uint32_t abase = lds_addr(&aring[0][0]), wbase = lds_addr(&wring[0][0]);
  uint32_t a_off[WR], w_off[WC];
#pragma unroll
  for (int i = 0; i < WR; ++i) a_off[i] = (uint32_t)(rbs[i] * 2048);
#pragma unroll
  for (int j = 0; j < WC; ++j) w_off[j] = (uint32_t)(cbs[j] * 2048);
  // one K-step pair: read both steps' operands, then the MFMAs of step 0, then step 1
  auto pair_step = [&](uint32_t pa, uint32_t pw, int s0) {
    u32x4 a[2][WR], b[2][WC];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int i = 0; i < WR; ++i) a[u][i] = lds_rd128<0>(pa + a_off[i] + off[u]);
#pragma unroll
      for (int j = 0; j < WC; ++j) b[u][j] = lds_rd128<0>(pw + w_off[j] + off[u]);
    }
    lds_wait<0>();
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (u == 1 && s0 + 1 >= nk) break;  // an odd last step
#pragma unroll
      for (int i = 0; i < WR; ++i) settle(a[u][i]);
#pragma unroll
      for (int j = 0; j < WC; ++j) settle(b[u][j]);
#pragma unroll
      for (int i = 0; i < WR; ++i)
#pragma unroll
        for (int j = 0; j < WC; ++j) acc[i][j] = mfma(as_bf16x8(a[u][i]), as_bf16x8(b[u][j]), acc[i][j]);
    }
  };
  for (int c = 0; c < nc; ++c) {
    asm volatile("s_barrier" ::: "memory");  // chunk c's operands are in LDS
    const uint32_t ca = abase + (uint32_t)(c % NA) * T::kABytes, cw = wbase + (uint32_t)(c % NW) * T::kWBytes;
#pragma unroll
    for (int q = 0; q < CH / 2; ++q) {
      const int s0 = c * CH + 2 * q;
      if (s0 < nk) pair_step(ca + q * 2 * RB * 1024, cw + q * 2 * CB * 1024, s0);
    }
  }
#pragma unroll
  for (int i = 0; i < WR; ++i) {
#pragma unroll
    for (int j = 0; j < WC; ++j) {
      const int col = n0 + 16 * cbs[j] + r16;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = m0 + 16 * rbs[i] + 4 * grp + e;
        if (row < M && col < N) {
          float v = bf2f(f2bf(acc[i][j][e]));
          if (R) v = bf2f(R[(long)row * ldr + col]) + v;
          C[(long)row * ldc + col] = f2bf(v);
        }
      }
    }
  }
}

// Comparator split-K: C = bf16(sum_z part[z]) (+ residual as in gemm_kernel).
__global__ __launch_bounds__(256) void gemm_reduce_kernel(const float *__restrict__ part, int nz, int M, int N,
                                                          bf16_t *__restrict__ C, int ldc,
                                                          const bf16_t *__restrict__ R, int ldr) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long)M * N) return;
  const int row = (int)(i / N), col = (int)(i % N);
  float s = part[i];
  for (int z = 1; z < nz; ++z) s += part[(long)z * M * N + i];
  float v = bf2f(f2bf(s));
  if (R) v = bf2f(R[(long)row * ldr + col]) + v;
  C[(long)row * ldc + col] = f2bf(v);
}

// ---------------------------------------------------------------------------
// S11: logits of one 256-column vocabulary tile, never stored: the K loop here, the
// tile's softmax partials in lm_tile_epilogue (lm_head.h).
// ---------------------------------------------------------------------------
// The weight W is in the packed layout written by pack_lm_head_kernel: per vocabulary
// tile, per 16-column MFMA block, per 32-wide K step, the block's B operand in lane order
// (1 KB), so every weight load of a wave is one contiguous 1 KB read.
//   W(c, k) -> ((((c/256)*16 + (c%256)/16) * (K/32) + k/32) * 64 + ((k%32)/8)*16 + c%16) * 8 + k%8
// Columns past V in the last tile are zero.
__global__ __launch_bounds__(256) void pack_lm_head_kernel(const bf16_t *__restrict__ src, int V, int K,
                                                           bf16_t *__restrict__ dst, long n_chunks) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_chunks) return;
  const int nk = K / 32;
  const int lane = (int)(i % 64);
  const long blk_step = i / 64;  // (tile*16 + block) * nk + step
  const int step = (int)(blk_step % nk);
  const long blk = blk_step / nk;
  const long c = blk * 16 + lane % 16;
  const int k = step * 32 + (lane / 16) * 8;
  u32x4 v = u32x4{0u, 0u, 0u, 0u};
  if (c < V) v = ld16(src + c * K + k);
  st16(dst + i * 8, v);
}

template <int MB, bool NT>
__global__ __launch_bounds__(256) void lm_head_kernel(const bf16_t *__restrict__ Z, int ldz,
                                                      const bf16_t *__restrict__ W, int K, int V,
                                                      const int32_t *__restrict__ target, int M,
                                                      float *__restrict__ part,
                                                      float *__restrict__ tgt_logit, int n_vt, int paired) {
  __shared__ float red[2][4][16 * MB];
  __shared__ u32x4 lds_a[2][kLdsSteps * MB * 64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int grp = lane >> 4, r16 = lane & 15;
  int tile = blockIdx.x, rt = blockIdx.y;
  if (paired) {
    // two row tiles, one 1-D grid: workgroups 16k + x and 16k + 8 + x (x < 8) take row
    // tiles 0 and 1 of vocabulary tile 8k + x.  Workgroups are dispatched to the 8 XCDs
    // round-robin, so the pair shares an XCD and starts together: the second reads the
    // weight slice from that XCD's L2.
    tile = (blockIdx.x >> 4) * 8 + (blockIdx.x & 7);
    rt = (blockIdx.x >> 3) & 1;
    if (tile >= n_vt) return;  // the grid's last group of 16 may overhang
  }
  const int m0 = rt * 16 * MB;
  const bf16_t *ap[MB];
  const bf16_t *wp[4];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) ap[mb] = Z + (long)min(m0 + 16 * mb + r16, M - 1) * ldz + grp * 8;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) wp[nb] = W + (long)(tile * 16 + wave * 4 + nb) * (K / 32) * 512 + lane * 8;
  f32x4 acc[MB][4];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  kloop_lds<MB, 4, 7, 512, NT>(acc, ap, wp, K, lm_rot(tile, K / 32), lds_a);
  lm_tile_epilogue<MB>(acc, red, wave, tile, m0, M, V, target, part, tgt_logit, n_vt);
}

// S11 for many rows: a workgroup of 8 waves computes 256-row x 256-column tiles (kWideRows
// rows of one vocabulary tile).  Both operands of a 32-wide K step (the rows' 16 row blocks
// and the tile's 16 column blocks, 1 KB each in MFMA lane order) are copied once into LDS
// by direct-to-LDS loads, kWideBuf-1 steps ahead of the step being computed, and every
// block read from LDS feeds several MFMAs: wave w owns rows 128(w/4) .. +127 and columns
// 64(w%4) .. +63 (8 x 4 blocks).  Each column's K order (lm_rot) and its MFMA per step are
// those of lm_head_kernel, and the column group w%4 owns the same 64 columns in the
// epilogue, so a row's partials have the same bits from either kernel at any M.
//
// The grid is kWideGrid persistent workgroups.  Workgroup g runs on XCD g%8 (workgroups
// are dispatched to the 8 XCDs round-robin) and is its XCD's l = g/8; the 32 workgroups
// of an XCD work through blocks of br x (32/br) tiles (row tiles x vocabulary tiles, the
// vocabulary tiles an aligned run of lm_rot's groups of 8, so they share one K order),
// block b, b+8, ... for XCD b, one tile each per block.  Every workgroup starts its tiles
// at about the same time as the others of its block, so the block's row and weight
// slices are fetched once into the XCD's L2 and read there by all of them.  Which
// workgroup computes a tile never changes the tile's arithmetic.
constexpr int kWideRows = 256, kWideBuf = 5, kWideGrid = 256;

// s_waitcnt vmcnt(PER * min(ahead, MAXA)): this wave's copies of a step landed while at
// most `ahead` later steps of PER loads each may stay in flight
template <int PER, int MAXA>
__device__ __forceinline__ void wait_steps(int ahead) {
  if constexpr (MAXA == 0) {
    wait_vmem<0>();
  } else {
    if (ahead >= MAXA) wait_vmem<PER * MAXA>();
    else wait_steps<PER, MAXA - 1>(ahead);
  }
}

// LM = true: the lm-head (W packed, the K order of lm_rot, the softmax-partials epilogue),
// n_vt vocabulary tiles.  LM = false: a projection C[M, N] = bf16(Z W^T) [+ residual R]
// with W row-major [N, ldw] (each 16-column block's operand copied by per-lane addresses
// like the rows'), K order 0, 32, 64, ... (that of gemm_kernel and gemm_stream_kernel, so
// the bits are theirs at any M), n_vt = ceil(N / 256) column tiles.
template <bool LM>
__global__ __launch_bounds__(512) void wide_kernel(const bf16_t *__restrict__ Z, int ldz,
                                                   const bf16_t *__restrict__ W, int K, int V,
                                                   const int32_t *__restrict__ target, int M,
                                                   float *__restrict__ part, float *__restrict__ tgt_logit,
                                                   int n_vt, int br, int ldw, bf16_t *__restrict__ C, int ldc,
                                                   const bf16_t *__restrict__ R, int ldr) {
  constexpr int kStepB = 32 * 1024;  // one K step: row blocks 0..15, then column blocks 0..15
  // the K loop's step buffers; the epilogue's reduction scratch reuses the first 8 KB
  __shared__ __attribute__((aligned(16))) uint8_t buf[kWideBuf][kStepB];
  auto &red = *reinterpret_cast<float (*)[2][2][4][128]>(&buf[0][0]);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int grp = lane >> 4, r16 = lane & 15;
  const int rg = wave >> 2, cg = wave & 3;
  const int nk = K / 32;
  const int n_rt = (M + kWideRows - 1) / kWideRows;
  const int bv = 32 / br;
  const int nbr = (n_rt + br - 1) / br, n_blocks = nbr * ((n_vt + bv - 1) / bv);
  const int xcd = blockIdx.x % 8, l = blockIdx.x / 8;
  const uint32_t lds0 = lds_addr(&buf[0][0]);
  const uint32_t abase = lds0 + rg * 8192 + lane * 16, wbase = lds0 + 16384 + cg * 4096 + lane * 16;
  for (int blk = xcd; blk < n_blocks; blk += 8) {
    const int rt = (blk % nbr) * br + l % br, tile = (blk / nbr) * bv + l / br;
    if (rt >= n_rt || tile >= n_vt) continue;  // the same for the whole workgroup
    const int m0 = rt * kWideRows;
    const int rot = LM ? lm_rot(tile, nk) : 0;
    auto kidx = [&](int s) {
      const int t = s + rot;
      return t >= nk ? t - nk : t;
    };
    // this wave copies row blocks 2w, 2w+1 and column blocks 2w, 2w+1 of every step (rows
    // past M read row M-1; their results are dropped).  Sources: a wave-uniform base plus
    // a 32-bit lane offset in elements (the row tile's rows span less than 2^31 elements)
    const bf16_t *za = Z + (long)m0 * ldz;
    const bf16_t *wt = LM ? W + (long)tile * 16 * nk * 512 : W + (long)tile * 256 * ldw;
    uint32_t aoff[2], woffs[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      aoff[j] = (uint32_t)((min(m0 + 16 * (2 * wave + j) + r16, M - 1) - m0) * ldz + grp * 8);
      // projection: columns past N read column N-1; their results are dropped
      woffs[j] = LM ? 0u : (uint32_t)((min(tile * 256 + 16 * (2 * wave + j) + r16, V - 1) - tile * 256) * ldw + grp * 8);
    }
    const uint32_t woff = (uint32_t)((2 * wave) * nk * 512 + lane * 8);
    auto copy_step = [&](int s) {
      uint8_t *b = &buf[s % kWideBuf][0];
      const int k = kidx(s);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        __builtin_amdgcn_global_load_lds(za + (aoff[j] + k * 32), b + (2 * wave + j) * 1024, 16, 0, 0);
        const bf16_t *wsrc = LM ? wt + (woff + (uint32_t)(j * nk + k) * 512) : wt + (woffs[j] + (uint32_t)k * 32);
        __builtin_amdgcn_global_load_lds(wsrc, b + 16384 + (2 * wave + j) * 1024, 16, 0, 0);
      }
    };
    // every wave is done with the previous tile's epilogue (red lives in buf[0])
    __syncthreads();
    for (int s = 0; s < kWideBuf - 1 && s < nk; ++s) copy_step(s);
    f32x4 acc[8][4];
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // The operands of step s+1 are read from LDS while the MFMAs of step s run: the four
    // column blocks first (into the other of two register sets), then each row block
    // right after the MFMAs that used its register for step s.
    u32x4 bo[2][4], a[8];
    auto read_b = [&](int s, u32x4 (&b)[4]) {
      const uint32_t off = (uint32_t)(s % kWideBuf) * kStepB;
      static_for<4>([&](auto nb_) { b[decltype(nb_)::value] = lds_rd128<decltype(nb_)::value * 1024>(wbase + off); });
    };
    // Iteration s: step s+1 landed (this wave's copies, then the barrier for everyone's;
    // at most kWideBuf-3 later steps, 4 loads each, still in flight), the barrier also
    // tells that every wave is done with step s-1's buffer, which the copy of step
    // s + kWideBuf - 1 refills; then the MFMAs of step s with the reads of step s+1.
    // The barrier is a plain s_barrier: every copy and read it orders is waited for
    // explicitly (a fenced barrier would also drain the reads and copies in flight).
    auto iteration = [&](int s, u32x4 (&cur)[4], u32x4 (&nxt)[4]) {
      if (s + 1 < nk) wait_steps<4, kWideBuf - 3>(nk - 2 - s);
      asm volatile("s_barrier" ::: "memory");
      if (s + kWideBuf - 1 < nk) copy_step(s + kWideBuf - 1);
      // (after the last step these reads fetch a buffer's stale contents, never used)
      const uint32_t off = (uint32_t)((s + 1) % kWideBuf) * kStepB;
      read_b(s + 1, nxt);
      lds_wait<4>();  // step s's operands (read before these four) are in
#pragma unroll
      for (int i = 0; i < 4; ++i) settle(cur[i]);
      static_for<8>([&](auto mb_) {
        constexpr int mb = decltype(mb_)::value;
        settle(a[mb]);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = mfma(as_bf16x8(a[mb]), as_bf16x8(cur[nb]), acc[mb][nb]);
        a[mb] = lds_rd128<mb * 1024>(abase + off);
        __builtin_amdgcn_sched_barrier(0);  // keep this order: one register per row block
      });
    };
    wait_steps<4, kWideBuf - 2>(nk - 1);  // step 0 landed
    asm volatile("s_barrier" ::: "memory");
    read_b(0, bo[0]);
    static_for<8>([&](auto mb_) { a[decltype(mb_)::value] = lds_rd128<decltype(mb_)::value * 1024>(abase); });
    for (int s = 0; s < nk; s += 2) {
      iteration(s, bo[0], bo[1]);
      if (s + 1 < nk) iteration(s + 1, bo[1], bo[0]);
    }
    lds_wait<0>();
    // every wave's reads are done (each waited for its own) before red overwrites buf[0]
    asm volatile("s_barrier" ::: "memory");
    if constexpr (LM) {
      lm_tile_epilogue<8>(acc, red[rg], cg, tile, m0 + rg * 128, M, V, target, part, tgt_logit, n_vt);
    } else {
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const int col = tile * 256 + cg * 64 + 16 * nb + r16;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = m0 + rg * 128 + 16 * mb + 4 * grp + i;
            if (row < M && col < V) {
              float v = bf2f(f2bf(acc[mb][nb][i]));
              if (R) v = bf2f(R[(long)row * ldr + col]) + v;
              C[(long)row * ldc + col] = f2bf(v);
            }
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// S12: per row, merge the (max, sum) of every vocabulary tile with a fixed tree
// (lane j folds tiles j, j+64, ... left to right; then lanes combine by halving,
// the lower lane on the left) and return lp = (l_target - m) - ln(s).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void merge_vocab(float &m, float &s, float mb, float sb) {
  if (mb == neg_inf()) return;
  if (m == neg_inf()) {
    m = mb;
    s = sb;
    return;
  }
  const float mn = fmaxf(m, mb);
  s = __builtin_fmaf(s, exp2f_hw((m - mn) * kLog2e), sb * exp2f_hw((mb - mn) * kLog2e));
  m = mn;
}

__global__ __launch_bounds__(64) void vocab_merge_kernel(const float *__restrict__ part,
                                                         const float *__restrict__ tgt_logit,
                                                         const int32_t *__restrict__ target,
                                                         int n_vt, int V, float *__restrict__ out) {
  const int row = blockIdx.x, lane = threadIdx.x;
  float m = neg_inf(), s = 0.f;
  for (int t = lane; t < n_vt; t += 64)
    merge_vocab(m, s, part[((long)row * n_vt + t) * 2], part[((long)row * n_vt + t) * 2 + 1]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float mo = __shfl_down(m, off, 64);
    const float so = __shfl_down(s, off, 64);
    if (lane < off) merge_vocab(m, s, mo, so);
  }
  if (lane == 0) {
    const int tg = target[row];
    float lp;
    if (tg < 0 || tg >= V)
      lp = __builtin_nanf("");
    else
      lp = (tgt_logit[row] - m) - log2f_hw(s) * kLn2;
    out[row] = lp;
  }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------

hipError_t launch_rmsnorm(const RmsNormArgs &a, hipStream_t st) {
  if (a.rows == 0) return hipSuccess;
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(a.rows), dim3(64), 0, st, a.x, a.ldx, a.tok, a.embed,
                     a.vocab, a.d, a.gain, a.eps, a.y, a.ldy, a.x_copy, a.ldc);
  return hipGetLastError();
}

int gemm_tiles(int M, int N) {
  if (M <= 16) return ((N + 63) / 64) * ((M + 15) / 16);
  if (M <= 64) return ((N + 63) / 64) * ((M + 63) / 64);
  return ((N + 127) / 128) * ((M + 63) / 64);
}

hipError_t launch_gemm(const GemmArgs &a, hipStream_t st) {
  if (a.M == 0) return hipSuccess;
  int kchunk = a.K, nz = 1;
  float *part = nullptr;
  if (a.split_k > 1 && a.part) {
    kchunk = ((a.K + a.split_k - 1) / a.split_k + 31) / 32 * 32;
    nz = (a.K + kchunk - 1) / kchunk;
    if (nz > 1) part = a.part;
    else kchunk = a.K;
  }
  if (!part && a.M > 256) {
    // many rows: the 256 x 256 LDS-tiled kernel of the lm-head, on the same persistent
    // grid (blocks of 4 row tiles x 8 column tiles per XCD); the K order is unchanged
    const int n_rt = (a.M + kWideRows - 1) / kWideRows;
    const int br = n_rt >= 4 ? 4 : (n_rt >= 2 ? 2 : 1);
    hipLaunchKernelGGL(wide_kernel<false>, dim3(kWideGrid), dim3(512), 0, st, a.A, a.lda, a.W, a.K, a.N, nullptr,
                       a.M, nullptr, nullptr, (a.N + 255) / 256, br, a.ldw, a.C, a.ldc, a.R, a.ldr);
    return hipGetLastError();
  }
  if (!part && a.M <= 256 && a.K >= 1024) {
    // few rows, long K: both operands streamed through LDS in whole cache lines; tiles of
    // 16 x 16 .. 64 x 64 sized so that a 4096-column projection fills the CUs once
#define RIL_STREAM(RB_, CB_, CH_)                                                                                \
  hipLaunchKernelGGL((gemm_stream_kernel<RB_, CB_, CH_>), dim3((a.N + 16 * CB_ - 1) / (16 * CB_), (a.M + 16 * RB_ - 1) / (16 * RB_)), \
                     dim3(kStreamThreads), 0, st, a.A, a.lda, a.W, a.ldw, a.C, a.ldc, a.R, a.ldr, a.M, a.N, a.K)
    // (65536 -> 4096 at 16 / 32 / 64 / 128 / 256 rows: 101 / 125 / 157 / 206 / 286 us; larger
    // chunks mean fewer barriers, bounded by the LDS the rings need)
    if (a.M <= 16) RIL_STREAM(1, 1, 16);
    else if (a.M <= 32) RIL_STREAM(2, 1, 16);
    else if (a.M <= 64) RIL_STREAM(2, 2, 8);
    else if (a.M <= 128) RIL_STREAM(4, 2, 8);
    else RIL_STREAM(4, 4, 4);
#undef RIL_STREAM
    return hipGetLastError();
  }
  if (a.M <= 16) {
    dim3 grid((a.N + 63) / 64, (a.M + 15) / 16, nz);
    hipLaunchKernelGGL((gemm_kernel<1, 1>), grid, dim3(256), 0, st, a.A, a.lda, a.W, a.ldw, a.C,
                       a.ldc, a.R, a.ldr, a.M, a.N, a.K, kchunk, part);
  } else if (a.M <= 64) {
    dim3 grid((a.N + 63) / 64, (a.M + 63) / 64, nz);
    hipLaunchKernelGGL((gemm_kernel<4, 1>), grid, dim3(256), 0, st, a.A, a.lda, a.W, a.ldw, a.C,
                       a.ldc, a.R, a.ldr, a.M, a.N, a.K, kchunk, part);
  } else {
    dim3 grid((a.N + 127) / 128, (a.M + 63) / 64, nz);
    hipLaunchKernelGGL((gemm_kernel<4, 2>), grid, dim3(256), 0, st, a.A, a.lda, a.W, a.ldw, a.C,
                       a.ldc, a.R, a.ldr, a.M, a.N, a.K, kchunk, part);
  }
  if (part) {
    const long n = (long)a.M * a.N;
    hipLaunchKernelGGL(gemm_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, part, nz, a.M,
                       a.N, a.C, a.ldc, a.R, a.ldr);
  }
  return hipGetLastError();
}

hipError_t launch_lm_head(const LmHeadArgs &a, hipStream_t st) {
  if (a.M == 0) return hipSuccess;
  const int n_vt = (a.V + kVocabTile - 1) / kVocabTile;
  const int mb = a.M <= 16 ? 1 : 4;
  const int n_rt = (a.M + 16 * mb - 1) / (16 * mb);
  // One row tile: the weights are read once and streamed with the nontemporal policy
  // (192 -> 171 us at 64 rows on the 4096 x 129280 head).  Two row tiles: the paired
  // 1-D grid puts both tiles of a vocabulary tile on one XCD at the same time, and
  // ordinary loads let the second read the weight slice from L2 (128 rows: 329 us on
  // the 2-D grid with nontemporal loads, 274 paired with them, 252 paired without).
  // Past 128 rows the 256-row kernel shares both operands through LDS.  No choice
  // changes a column's K order or its MFMA per step.
  if (n_rt == 2) {
    const dim3 grid((unsigned)(16 * ((n_vt + 7) / 8)));
    hipLaunchKernelGGL((lm_head_kernel<4, false>), grid, dim3(256), 0, st, a.Z, a.ldz, a.W, a.K, a.V, a.target,
                       a.M, a.part, a.tgt_logit, n_vt, 1);
  } else if (n_rt == 1) {
    const dim3 grid(n_vt, 1);
    if (mb == 1)
      hipLaunchKernelGGL((lm_head_kernel<1, true>), grid, dim3(256), 0, st, a.Z, a.ldz, a.W, a.K, a.V,
                         a.target, a.M, a.part, a.tgt_logit, n_vt, 0);
    else
      hipLaunchKernelGGL((lm_head_kernel<4, true>), grid, dim3(256), 0, st, a.Z, a.ldz, a.W, a.K, a.V,
                         a.target, a.M, a.part, a.tgt_logit, n_vt, 0);
  } else {
    // many rows: 256-row tiles with both operands shared through LDS, on persistent
    // workgroups that take blocks of 4 x 8 tiles (fewer row tiles: 2 x 16 or 1 x 32)
    const int n_wrt = (a.M + kWideRows - 1) / kWideRows;
    const int br = n_wrt >= 4 ? 4 : (n_wrt >= 2 ? 2 : 1);
    hipLaunchKernelGGL(wide_kernel<true>, dim3(kWideGrid), dim3(512), 0, st, a.Z, a.ldz, a.W, a.K, a.V, a.target,
                       a.M, a.part, a.tgt_logit, n_vt, br, 0, nullptr, 0, nullptr, 0);
  }
  return hipGetLastError();
}

long lm_head_packed_elems(int V, int K) {
  const long n_vt = (V + kVocabTile - 1) / kVocabTile;
  return n_vt * kVocabTile * (long)K;
}

hipError_t launch_pack_lm_head(const bf16_t *src, int V, int K, bf16_t *dst, hipStream_t st) {
  const long n_chunks = lm_head_packed_elems(V, K) / 8;
  if (n_chunks == 0) return hipSuccess;
  const long blocks = (n_chunks + 255) / 256;
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pack_lm_head_kernel, dim3((unsigned)blocks), dim3(256), 0, st, src, V, K, dst, n_chunks);
  return hipGetLastError();
}

hipError_t launch_vocab_merge(const LmHeadArgs &a, hipStream_t st) {
  if (a.M == 0) return hipSuccess;
  const int n_vt = (a.V + kVocabTile - 1) / kVocabTile;
  hipLaunchKernelGGL(vocab_merge_kernel, dim3(a.M), dim3(64), 0, st, a.part, a.tgt_logit,
                     a.target, n_vt, a.V, a.out);
  return hipGetLastError();
}

}  // namespace ril
