// The lightweight indexer and the stable top-k selection of sparse attention (S6, S7).
//
// The indexer scores every history position of a query (Bitwise-consistent RL post,
// sections 3 and 4.3).  Its formula is a reading (the pages give none):
//   I[s] = sum_h relu(q_h . k_s),  64 heads x 128 dims, unit head weights,
// computed in fp32: each head's dot product a chain of fused multiply-adds (the exact
// q k + acc rounded once, v_fma_f32) over d = 0..127 from +0, the heads summed with one
// rounding per add over h = 0..63.  The selection is an integer decided by these floats,
// so the arithmetic is kept reproducible exactly: the same bits on every path, and in a
// float32 reference outside this library (C99 fmaf is the same operation).  One fused
// operation per term is half the instructions of a multiply and an add (the kernel is
// bound by them).
//
// The selection ranks positions by the unique key (score, position): higher score
// first, equal scores broken toward the lower position (post section 4.3 breaks ties
// toward the larger position; the workload spec asks for the lowest index), keeps the
// best k, and lists them by descending position with -1 padding, the order the
// attention then accumulates in.  Contexts of at most k positions select every
// position (the same list any longer path would produce: no shortcut changes it).
#include "attn_common.h"
#include "kernels.h"

namespace ril {

constexpr int kIdxHeads = 64, kIdxDim = 128;
constexpr int kTopkThreads = 1024;
constexpr int kTopkMax = 4096;

__device__ __forceinline__ void index_row(int mode, int r, int row0, const int32_t *ctx_len, const int32_t *cu,
                                          const int32_t *start_pos, int n_seqs, int &seq, int &ctx, long &qrow) {
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
// S6: grid (ceil(ctx_bound / 256), rows), one thread per history position.  The row's q
// (64 x 128 fp32, 32 KB) is staged in LDS once per workgroup and read back as 16-byte
// broadcast reads (every lane the same address) that the compiler can issue ahead of the
// multiplies; read as scalar loads it left every head waiting on a scalar-memory round
// trip (the scalar registers hold only part of a head).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void indexer_kernel(
    const float *__restrict__ q, int mode, int row0, const int32_t *__restrict__ ctx_len,
    const int32_t *__restrict__ cu, const int32_t *__restrict__ start_pos, int n_seqs,
    const int32_t *__restrict__ page_table, int page_stride, const bf16_t *__restrict__ pool, int page_elems,
    int n_pages, int ctx_bound, int key_off, float *__restrict__ scores, int score_stride) {
  __shared__ __attribute__((aligned(16))) float qs[kIdxHeads * kIdxDim];
  const int r = blockIdx.y;
  int seq, ctx;
  long qrow;
  index_row(mode, r, row0, ctx_len, cu, start_pos, n_seqs, seq, ctx, qrow);
  if (ctx < 1 || ctx > ctx_bound || blockIdx.x * blockDim.x >= ctx) return;  // the same for the whole workgroup
  const float *qr = q + qrow * (kIdxHeads * kIdxDim);
  for (int i = threadIdx.x; i < kIdxHeads * kIdxDim / 4; i += blockDim.x)
    reinterpret_cast<u32x4 *>(qs)[i] = ld16(qr + 4 * i);
  __syncthreads();
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= ctx) return;
  float *out = scores + (long)r * score_stride + s;
  const int pid = page_table[(long)seq * page_stride + s / kPage];
  if ((unsigned)pid >= (unsigned)n_pages) {
    *out = __builtin_nanf("");
    return;
  }
  const float *kp = reinterpret_cast<const float *>(pool + (long)pid * page_elems + key_off) + (s % kPage) * kIdxDim;
  float k[kIdxDim];
#pragma unroll
  for (int i = 0; i < kIdxDim / 4; ++i) {
    const u32x4 v = ld16(kp + 4 * i);
#pragma unroll
    for (int j = 0; j < 4; ++j) k[4 * i + j] = __uint_as_float(v[j]);
  }
  float total = 0.f;
  for (int h = 0; h < kIdxHeads; ++h) {
    const u32x4 *qh = reinterpret_cast<const u32x4 *>(qs + h * kIdxDim);
    float acc = 0.f;
#pragma unroll
    for (int d4 = 0; d4 < kIdxDim / 4; ++d4) {
      const u32x4 qv = qh[d4];
#pragma unroll
      for (int j = 0; j < 4; ++j) acc = __fmaf_rn(__uint_as_float(qv[j]), k[4 * d4 + j], acc);
    }
    total = __fadd_rn(total, acc > 0.f ? acc : 0.f);
  }
  *out = total;
}

// Order-preserving map of fp32 to uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t ord32(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kTopkRow = 257;  // one lane's histogram row, padded against bank aliasing

// A row of at most K positions (or an invalid row: n = 0) selects every position,
// listed in descending order, -1 after them.
__device__ __forceinline__ void topk_every_position(int32_t *out, int32_t *cpy, int K, int n) {
  for (int i = threadIdx.x; i < K; i += kTopkThreads) {
    const int v = i < n ? n - 1 - i : -1;
    out[i] = v;
    if (cpy) cpy[i] = v;
  }
}

// One radix pass after the per-lane histogram rows are filled: sum the 64 rows per bin,
// then wave 0 finds the digit (bits shift .. shift+7) where the count of keys with a
// larger digit first reaches `need`, and narrows (prefix, need) to that digit; `ties` is
// the digit's count.  The caller synchronises before reading the results.
__device__ __forceinline__ void topk_pick_digit(const int *hist, int (&part)[4][256], int shift, uint32_t prefix,
                                                uint32_t &s_prefix, int &s_need, int &s_ties) {
  const int tid = threadIdx.x, lane = tid & 63;
  {
    const int b = tid & 255, q4 = tid >> 8;  // bin, quarter of the 64 rows
    int c = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) c += hist[(16 * q4 + i) * kTopkRow + b];
    part[q4][b] = c;
  }
  __syncthreads();
  if (tid < 64) {
    // lane l holds bins 255 - 4l .. 252 - 4l
    int cnt[4], loc = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int b = 255 - 4 * lane - j;
      cnt[j] = part[0][b] + part[1][b] + part[2][b] + part[3][b];
      loc += cnt[j];
    }
    int incl = loc;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(incl, off, 64);
      if (lane >= off) incl += t;
    }
    const int need = s_need;
    int cum = incl - loc;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (cum < need && cum + cnt[j] >= need) {
        s_prefix = prefix | ((uint32_t)(255 - 4 * lane - j) << shift);
        s_need = need - cum;
        s_ties = cnt[j];
      }
      cum += cnt[j];
    }
  }
}

// ---------------------------------------------------------------------------
// S7: grid (rows), 1024 threads.  Radix select of the k-th largest score over four
// 8-bit digits (histograms in LDS: their counts do not depend on thread order), then
// the lowest-position ties at the threshold by a wave-ordered prefix count, then a
// bitonic sort of the k positions into descending order.
// Histograms: lane i of every wave counts into its own row of 257 counters, so the lanes
// of one atomic instruction never share an address and lanes that hit the same bin sit
// in different LDS banks (bin b of row i is in bank (i + b) mod 64); scores cluster in a
// few digits, and one shared 256-bin histogram serialised most of its atomics.  The rows
// are summed per bin, and one wave finds the threshold digit with a scan across lanes.
// Selected positions are appended with one atomic per wave (a ballot gives each lane its
// place); the sort fixes their order.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(
    const float *__restrict__ scores, int score_stride, int mode, int row0, const int32_t *__restrict__ ctx_len,
    const int32_t *__restrict__ cu, const int32_t *__restrict__ start_pos, int n_seqs, int ctx_bound, int K,
    int32_t *__restrict__ sel, int32_t *__restrict__ sel_copy) {
  constexpr int kUnroll = 8;  // score loads issued together per scan step
  __shared__ int hist[64 * kTopkRow];
  __shared__ int part[4][256];
  __shared__ int buf[kTopkMax];
  __shared__ int wave_cnt[kTopkThreads / 64];
  __shared__ uint32_t s_prefix;
  __shared__ int s_need, s_ties, s_count, s_taken;
  const int r = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  int seq, ctx;
  long qrow;
  index_row(mode, r, row0, ctx_len, cu, start_pos, n_seqs, seq, ctx, qrow);
  int32_t *out = sel + (long)r * K;
  int32_t *cpy = sel_copy ? sel_copy + (row0 + (long)r) * K : nullptr;
  if (ctx < 1 || ctx > ctx_bound || ctx <= K) {
    // every position, descending (an invalid row selects nothing; its attention is NaN)
    topk_every_position(out, cpy, K, (ctx < 1 || ctx > ctx_bound) ? 0 : ctx);
    return;
  }
  const int n = ctx;
  const float *sc = scores + (long)r * score_stride;
  if (tid == 0) {
    s_prefix = 0u;
    s_need = K;
  }
  const unsigned long long below_me = (1ull << lane) - 1ull;
  uint32_t mask = 0u;
  int *my_row = hist + lane * kTopkRow;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < 64 * kTopkRow; i += kTopkThreads) hist[i] = 0;
    __syncthreads();
    const uint32_t prefix = s_prefix;
    for (int c0 = 0; c0 < n; c0 += kUnroll * kTopkThreads) {
      uint32_t u[kUnroll];  // all loads of the batch in flight before the first count
#pragma unroll
      for (int j = 0; j < kUnroll; ++j) {
        const int s = c0 + j * kTopkThreads + tid;
        u[j] = s < n ? ord32(sc[s]) : 0u;
      }
#pragma unroll
      for (int j = 0; j < kUnroll; ++j)
        if (c0 + j * kTopkThreads + tid < n && (u[j] & mask) == prefix) atomicAdd(&my_row[(u[j] >> shift) & 255u], 1);
    }
    __syncthreads();
    topk_pick_digit(hist, part, shift, prefix, s_prefix, s_need, s_ties);
    mask |= 0xFFu << shift;
    __syncthreads();
  }
  const uint32_t thr = s_prefix;
  const int need = s_need, ties = s_ties;
  if (tid == 0) {
    s_count = 0;
    s_taken = 0;
  }
  __syncthreads();
  // everything above the threshold, in any order (the sort below fixes the order)
  for (int c0 = 0; c0 < n; c0 += kUnroll * kTopkThreads) {
    uint32_t u[kUnroll];
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      const int s = c0 + j * kTopkThreads + tid;
      u[j] = s < n ? ord32(sc[s]) : 0u;
    }
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      const int s = c0 + j * kTopkThreads + tid;
      const bool take = s < n && (u[j] > thr || (u[j] == thr && need == ties));
      const unsigned long long bal = __ballot(take);
      int base = 0;
      if (lane == 0 && bal) base = atomicAdd(&s_count, __popcll(bal));
      base = __shfl(base, 0, 64);
      if (take) buf[base + __popcll(bal & below_me)] = s;
    }
  }
  if (need < ties) {
    // the `need` lowest positions among the scores equal to the threshold
    for (int c0 = 0; c0 < n; c0 += kTopkThreads) {
      __syncthreads();
      const int s = c0 + tid;
      const bool flag = s < n && ord32(sc[s]) == thr;
      const unsigned long long bal = __ballot(flag);
      const int below = __popcll(bal & below_me);
      if (lane == 0) wave_cnt[wave] = __popcll(bal);
      __syncthreads();
      int before = s_taken;
      for (int w = 0; w < wave; ++w) before += wave_cnt[w];
      const bool take = flag && before + below < need;
      const unsigned long long tb = __ballot(take);
      int base = 0;
      if (lane == 0 && tb) base = atomicAdd(&s_count, __popcll(tb));
      base = __shfl(base, 0, 64);
      if (take) buf[base + __popcll(tb & below_me)] = s;
      __syncthreads();
      if (tid == 0) {
        int t = 0;
        for (int w = 0; w < kTopkThreads / 64; ++w) t += wave_cnt[w];
        s_taken += t;
      }
      __syncthreads();
      if (s_taken >= need) break;
    }
  }
  __syncthreads();
  // bitonic sort, descending
  for (int size = 2; size <= K; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < K / 2; i += kTopkThreads) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool desc = (lo & size) == 0;
        const int a = buf[lo], b = buf[hi];
        if ((a < b) == desc) {
          buf[lo] = b;
          buf[hi] = a;
        }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < K; i += kTopkThreads) {
    out[i] = buf[i];
    if (cpy) cpy[i] = buf[i];
  }
}

// ---------------------------------------------------------------------------
// S7 for rows of at most kTopkThreads * kTopkPer positions: the same selection (the same
// histograms, threshold digit by digit, and lowest-position ties), with the row's keys
// read once into registers (thread t holds positions j * 1024 + t, j = 0 .. 63) and the
// selected positions written straight to their places in descending order, with no sort.
// Blocks of 64 consecutive positions (block b = 16 j + wave) count their keys above and
// equal to the threshold; one pass over the 1024 blocks gives each block the ties at
// lower positions (ascending: the ties taken are the `need` lowest) and the selected
// positions above it (descending: its first output slot); each lane then adds the
// selected lanes above it in its block.
// ---------------------------------------------------------------------------
constexpr int kTopkPer = 64;
constexpr int kTopkBlocks = kTopkPer * (kTopkThreads / 64);  // 1024 blocks of 64 positions

__global__ __launch_bounds__(kTopkThreads) void topk_regs_kernel(
    const float *__restrict__ scores, int score_stride, int mode, int row0, const int32_t *__restrict__ ctx_len,
    const int32_t *__restrict__ cu, const int32_t *__restrict__ start_pos, int n_seqs, int ctx_bound, int K,
    int32_t *__restrict__ sel, int32_t *__restrict__ sel_copy) {
  static_assert(kTopkBlocks == kTopkThreads, "one thread per block of 64 positions in the block pass");
  __shared__ int hist[64 * kTopkRow];
  __shared__ int part[4][256];
  __shared__ int n_gt[kTopkBlocks], n_eq[kTopkBlocks];  // per block: keys above / at the threshold
  __shared__ int tie0[kTopkBlocks], out0[kTopkBlocks];   // ties below the block; its first output slot
  __shared__ int wsum[kTopkThreads / 64];
  __shared__ uint32_t s_prefix;
  __shared__ int s_need, s_ties;
  const int r = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  int seq, ctx;
  long qrow;
  index_row(mode, r, row0, ctx_len, cu, start_pos, n_seqs, seq, ctx, qrow);
  int32_t *out = sel + (long)r * K;
  int32_t *cpy = sel_copy ? sel_copy + (row0 + (long)r) * K : nullptr;
  if (ctx < 1 || ctx > ctx_bound || ctx <= K) {
    topk_every_position(out, cpy, K, (ctx < 1 || ctx > ctx_bound) ? 0 : ctx);
    return;
  }
  const int n = ctx;  // <= ctx_bound <= kTopkThreads * kTopkPer (the launcher's choice)
  const float *sc = scores + (long)r * score_stride;
  // Entries past the row (positions n ..) hold key 0, the smallest key.  A pass counts
  // them in bin 0 whenever its prefix is 0, and one atomic subtracts them again, so the
  // bin totals are those of the row's positions alone.  They are never selected: never
  // above a threshold, and as ties they sit above every position of the row, while the
  // ties taken are the lowest `need` of the row's own (need <= their count).  So no
  // later step tests the bound.  Every load is issued at once (past the end a lane
  // rereads the last position).
  const int n_past = kTopkThreads * kTopkPer - n;
  // this thread's entries j < nv are positions of the row (n > K >= 64 > tid - 1024)
  const int nv = min(kTopkPer, (n - tid + kTopkThreads - 1) / kTopkThreads);
  uint32_t u[kTopkPer];
#pragma unroll
  for (int j = 0; j < kTopkPer; ++j) {
    const uint32_t v = ord32(sc[min(j * kTopkThreads + tid, n - 1)]);
    u[j] = v & (uint32_t)((j - nv) >> 31);  // all ones for j < nv, else 0
  }
  if (tid == 0) {
    s_prefix = 0u;
    s_need = K;
  }
  uint32_t mask = 0u;
  int *my_row = hist + lane * kTopkRow;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < 64 * kTopkRow; i += kTopkThreads) hist[i] = 0;
    __syncthreads();
    const uint32_t prefix = s_prefix;
#pragma unroll
    for (int j = 0; j < kTopkPer; ++j)
      if ((u[j] & mask) == prefix) atomicAdd(&my_row[(u[j] >> shift) & 255u], 1);
    if (tid == 0 && prefix == 0u && n_past > 0) atomicSub(&hist[0], n_past);
    __syncthreads();
    topk_pick_digit(hist, part, shift, prefix, s_prefix, s_need, s_ties);
    mask |= 0xFFu << shift;
    __syncthreads();
  }
  const uint32_t thr = s_prefix;
  const int need = s_need;
  const unsigned long long below_me = (1ull << lane) - 1ull;
  const unsigned long long above_me = lane == 63 ? 0ull : ~0ull << (lane + 1);
#pragma unroll
  for (int j = 0; j < kTopkPer; ++j) {
    const unsigned long long bg = __ballot(u[j] > thr), be = __ballot(u[j] == thr);
    if (lane == 0) {
      n_gt[j * 16 + wave] = __popcll(bg);
      n_eq[j * 16 + wave] = __popcll(be);
    }
  }
  __syncthreads();
  {
    // thread b = block b (positions 64 b ..): ties at lower positions (exclusive prefix
    // of n_eq), then the selected count at higher positions (exclusive suffix)
    const int b = tid, e = n_eq[b];
    int inc = e;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(inc, off, 64);
      if (lane >= off) inc += t;
    }
    if (lane == 63) wsum[wave] = inc;
    __syncthreads();
    int below = inc - e;
    for (int w = 0; w < wave; ++w) below += wsum[w];
    tie0[b] = below;
    const int taken = n_gt[b] + min(max(need - below, 0), e);
    __syncthreads();  // every wave has read wsum
    int suf = taken;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_down(suf, off, 64);
      if (lane + off < 64) suf += t;
    }
    if (lane == 0) wsum[wave] = suf;
    __syncthreads();
    int above = suf - taken;
    for (int w = wave + 1; w < kTopkThreads / 64; ++w) above += wsum[w];
    out0[b] = above;
  }
  __syncthreads();
  // the threshold read again after the barrier: the compiler then recomputes each
  // comparison here instead of keeping all 128 masks of the counting loop alive (and
  // spilling them)
  const uint32_t thr_w = s_prefix;
  int tid_w;  // likewise the thread index (else the loads' positions stay alive, in scratch)
  asm volatile("v_mov_b32 %0, %1" : "=v"(tid_w) : "v"(tid));
#pragma unroll
  for (int j = 0; j < kTopkPer; ++j) {
    const int s = j * kTopkThreads + tid_w, b = j * 16 + wave;
    const bool eq = u[j] == thr_w;
    const unsigned long long be = __ballot(eq);
    const bool take = u[j] > thr_w || (eq && tie0[b] + __popcll(be & below_me) < need);
    const unsigned long long bt = __ballot(take);
    if (take) {
      const int i = out0[b] + __popcll(bt & above_me);
      out[i] = s;
      if (cpy) cpy[i] = s;
    }
  }
}

hipError_t launch_indexer(const IndexerArgs &a, hipStream_t st) {
  if (a.n_rows == 0) return hipSuccess;
  dim3 grid((a.ctx_bound + 255) / 256, a.n_rows);
  hipLaunchKernelGGL(indexer_kernel, grid, dim3(256), 0, st, a.q, a.mode, a.row0, a.ctx_len, a.cu, a.start_pos,
                     a.n_seqs, a.page_table, a.page_stride, a.pool, a.page_elems, a.n_pages, a.ctx_bound, a.key_off, a.scores,
                     a.score_stride);
  return hipGetLastError();
}

hipError_t launch_topk(const IndexerArgs &a, hipStream_t st) {
  if (a.n_rows == 0) return hipSuccess;
  // rows up to 65536 positions keep their keys in registers; longer bounds stream them
  if (a.ctx_bound <= kTopkThreads * kTopkPer)
    hipLaunchKernelGGL(topk_regs_kernel, dim3(a.n_rows), dim3(kTopkThreads), 0, st, a.scores, a.score_stride,
                       a.mode, a.row0, a.ctx_len, a.cu, a.start_pos, a.n_seqs, a.ctx_bound, a.topk, a.sel,
                       a.sel_copy);
  else
    hipLaunchKernelGGL(topk_kernel, dim3(a.n_rows), dim3(kTopkThreads), 0, st, a.scores, a.score_stride, a.mode,
                       a.row0, a.ctx_len, a.cu, a.start_pos, a.n_seqs, a.ctx_bound, a.topk, a.sel, a.sel_copy);
  return hipGetLastError();
}

}  // namespace ril
