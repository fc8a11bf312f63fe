// Mamba-2 selective state-space mixer (SSD) whose decode replays the prefill's chunked
// arithmetic (Bitwise-consistent RL post, section 6: Nemotron's Mamba-2 layers; the
// zero-mismatch-rl README's key-features table: decode replays the prefill chunk math).
//
// The layer, per head h (P = 64 channels) reading state group g = h / (H / G), per
// position t (dt_t > 0 given, A_h < 0 and D_h model constants):
//   S_t = exp(dt_t A_h) S_{t-1} + dt_t B_t x_t^T   (N = 128 state rows)
//   y_t = S_t^T C_t + D_h x_t                       (stored as bf16)
//
// It is evaluated in chunks of Q = 128 positions fixed from position 0 (the SSD chunked
// form, an exact rewriting of the recurrence).  With L_s = sum of dt_r A over the chunk's
// positions r <= s (a fixed-order scan), S_in the state entering the chunk and every
// product below one v_mfma_f32_16x16x32_bf16 chain over its K range in a fixed order:
//   G[s][t]  = B_s . C_t                                   (K = n)
//   W[s][t]  = bf16(G[s][t] * exp(L_t - L_s) * dt_s) for s <= t, else 0
//   Y2[p][t] = sum_s x_s[p] W[s][t]                        (K = s, all 128 in every call)
//   Y1[p][t] = sum_n bf16(S_in)[p][n] C_t[n]               (K = n)
//   y_t[p]   = bf16((Y1 * exp(L_t) + Y2) + D_h x_t[p])
// and when a chunk is complete its exit state is
//   S_out = exp(L_end) S_in + sum_s x_s bf16(B_s exp(L_end - L_s) dt_s)^T   (K = s).
// The bf16 operand points (W, the state operand, the scaled B) are those of the common
// Mamba-2 chunk kernels.  Every output element's MFMA chain depends only on its own row
// (channel p) and column (position t), so a position's bits do not depend on which other
// positions share its call: a decode step is this computation for one column, a prefill
// for many, and any split of a sequence into calls gives the same bits.  (Columns past a
// call's last position see zero inputs in the W product; in a longer call the same
// entries see real inputs times W = 0: both give +-0 products, as for attention's masked
// tail.)
//
// Per sequence a cache slot holds the state entering the current chunk (fp32 [H][P][N])
// and the current chunk's earlier inputs (x [Q][H][P], B [Q][G][N] bf16, dt [Q][H] fp32).
// A call runs: plan (its chunks), state (the exit-state sums of the chunks it completes),
// scan (states through those chunks, in order), out (every position's y), commit (the
// new entry state into the slot), write (the inputs of an unfinished last chunk into the
// slot).  Decode completes a chunk exactly as prefill does: the same kernels.
#include "attn_common.h"
#include "kernels.h"

namespace ril {

constexpr int kSsdPad = kSsdQ + 8;  // LDS row length (elements) of a 128-wide operand tile
constexpr int kSsdThreads = 256;

__host__ __device__ inline long ssd_state_bytes(int H) { return (long)H * kSsdP * kSsdN * 4; }
long ssd_slot_bytes(int H, int G) {
  const long b = ssd_state_bytes(H) + (long)kSsdQ * H * kSsdP * 2 + (long)kSsdQ * G * kSsdN * 2 + (long)kSsdQ * H * 4;
  return (b + 255) / 256 * 256;
}

// exp(x) as every SSD kernel computes it: one fp32 multiply by log2(e), then v_exp_f32
__device__ __forceinline__ float ssd_exp(float x) { return exp2f_hw(x * kLog2e); }

// Per sequence of a call: its positions [p0, p1), first token tok0, slot, and its
// chunks: n_ch touched (chunk indices off ..), of which the first n_done are completed by
// the call (completed-chunk indices done ..; completed chunk i's exit-state sums, decay
// and exit state -- the state entering chunk cf + i + 1 -- sit at index done + i).
struct SsdSeq {
  int p0, p1, tok0, slot, off, n_ch, done, n_done;
};
// plan layout (int32, n = n_seqs): off[0..n], done[0..n], p0[n], p1[n], tok0[n], slot[n]
__device__ __forceinline__ SsdSeq ssd_seq(const int32_t *plan, int n, int s) {
  SsdSeq q;
  q.off = plan[s];
  q.n_ch = plan[s + 1] - q.off;
  q.done = plan[n + 1 + s];
  q.n_done = plan[n + 2 + s] - q.done;
  q.p0 = plan[2 * n + 2 + s];
  q.p1 = plan[3 * n + 2 + s];
  q.tok0 = plan[4 * n + 2 + s];
  q.slot = plan[5 * n + 2 + s];
  return q;
}
// the sequence s with pre[s] <= b < pre[s + 1] for a prefix array pre[0..n]; -1 past the end
__device__ __forceinline__ int ssd_owner(const int32_t *pre, int n, int b) {
  if (b >= pre[n]) return -1;
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pre[mid] <= b) lo = mid; else hi = mid - 1;
  }
  return lo;
}

struct SsdSlot {
  float *state;
  bf16_t *x, *B;
  float *dt;
};
__device__ __forceinline__ SsdSlot ssd_slot(uint8_t *pool, long slot_bytes, int slot, int H, int G) {
  uint8_t *b = pool + (long)slot * slot_bytes;
  SsdSlot s;
  s.state = reinterpret_cast<float *>(b);
  s.x = reinterpret_cast<bf16_t *>(b + ssd_state_bytes(H));
  s.B = s.x + (long)kSsdQ * H * kSsdP;
  s.dt = reinterpret_cast<float *>(s.B + (long)kSsdQ * G * kSsdN);
  return s;
}

// The inputs of position pos (chunk offset j = pos % Q) for head h / group g: from the
// call if pos >= p0, else (earlier positions of the call's first chunk) from the slot.
struct SsdTok {
  const bf16_t *x, *B;
  float dt;
};
__device__ __forceinline__ SsdTok ssd_tok(const SsdArgs &a, const SsdSeq &q, const SsdSlot &sl, int pos, int h,
                                          int g) {
  SsdTok t;
  if (pos >= q.p0) {
    const long j = q.tok0 + (pos - q.p0);
    t.x = a.x + (j * a.H + h) * kSsdP;
    t.B = a.B + (j * a.G + g) * kSsdN;
    t.dt = a.dt[j * a.H + h];
  } else {
    const int j = pos % kSsdQ;
    t.x = sl.x + ((long)j * a.H + h) * kSsdP;
    t.B = sl.B + ((long)j * a.G + g) * kSsdN;
    t.dt = sl.dt[(long)j * a.H + h];
  }
  return t;
}

// L_s = sum over the chunk's positions r <= s of dt_r * A (fp32), for s < n_valid; one
// wave.  Lane i holds positions 2i and 2i + 1; pair sums, then a doubling scan across
// lanes.  Every lane's result depends only on positions at or before its own, so a
// partial chunk (n_valid < Q) gives the same L_s as the complete one for every s it has.
__device__ __forceinline__ void ssd_cumsum(const float *dts, float A, int n_valid, float *Ls) {
  const int i = threadIdx.x & 63;
  const float l0 = 2 * i < n_valid ? dts[2 * i] * A : 0.f;
  const float l1 = 2 * i + 1 < n_valid ? dts[2 * i + 1] * A : 0.f;
  float v = l0 + l1;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const float u = __shfl_up(v, d, 64);
    if (i >= d) v = v + u;
  }
  float prev = __shfl_up(v, 1, 64);
  if (i == 0) prev = 0.f;
  Ls[2 * i] = prev + l0;
  Ls[2 * i + 1] = v;
}

// ---------------------------------------------------------------------------
// plan: one thread walks the sequences in order
// ---------------------------------------------------------------------------
__global__ void ssd_plan_kernel(SsdArgs a) {
  if (threadIdx.x != 0) return;
  const int n = a.n_seqs;
  int32_t *plan = a.plan;
  int off = 0, done = 0;
  plan[0] = 0;
  plan[n + 1] = 0;
  for (int s = 0; s < n; ++s) {
    int tok0, len, p0;
    if (a.mode == 0) {
      tok0 = a.cu[s];
      len = a.cu[s + 1] - tok0;
      p0 = a.start_pos[s];
    } else {
      tok0 = s;
      len = 1;
      p0 = a.ctx_len[s] - 1;
    }
    bool ok = len >= 1 && p0 >= 0 && tok0 >= 0 && (long)tok0 + len <= a.n_tok && (long)p0 + len <= 0x7fffffffL;
    int slot = ok ? a.page_table[(long)s * a.page_stride] : -1;
    const int p1 = ok ? p0 + len : p0;
    const int n_ch = ok ? (p1 - 1) / kSsdQ - p0 / kSsdQ + 1 : 0;
    const int n_done = ok ? p1 / kSsdQ - p0 / kSsdQ : 0;
    // a sequence the grids cannot hold (only with inconsistent batch arrays) is dropped
    ok = ok && off + n_ch <= a.max_chunks && done + n_done <= a.max_done;
    if (!ok || (unsigned)slot >= (unsigned)a.n_slots) slot = -1;
    if (ok) {
      off += n_ch;
      done += n_done;
    }
    plan[s + 1] = off;
    plan[n + 2 + s] = done;
    plan[2 * n + 2 + s] = ok ? p0 : 0;
    plan[3 * n + 2 + s] = ok ? p1 : 0;
    plan[4 * n + 2 + s] = ok ? tok0 : 0;
    plan[5 * n + 2 + s] = slot;
  }
}

// ---------------------------------------------------------------------------
// state: for each chunk the call completes, dS^T[p][n] = sum_s x_s[p] bf16(B_s[n] w_s)
// (w_s = exp(L_end - L_s) dt_s) and its decay exp(L_end).  Grid (completed chunks, H),
// 4 waves: wave w owns channels 16w .. 16w + 15 and all 128 state rows.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kSsdThreads) void ssd_state_kernel(SsdArgs a) {
  __shared__ __attribute__((aligned(16))) bf16_t Xt[kSsdP][kSsdPad];  // x^T [p][s]
  __shared__ __attribute__((aligned(16))) bf16_t Bt[kSsdN][kSsdPad];  // B^T [n][s]
  __shared__ float dts[kSsdQ], Ls[kSsdQ], ws[kSsdQ];
  const int e_ = blockIdx.x, h = blockIdx.y, n = a.n_seqs;
  const int s_ = ssd_owner(a.plan + n + 1, n, e_);
  if (s_ < 0) return;
  const SsdSeq q = ssd_seq(a.plan, n, s_);
  const int c = q.p0 / kSsdQ + (e_ - q.done), c0 = c * kSsdQ;
  if (q.slot < 0) return;
  const int g = h / (a.H / a.G);
  const SsdSlot sl = ssd_slot(a.pool, a.slot_bytes, q.slot, a.H, a.G);
  const int tid = threadIdx.x;
  // x rows: 8 pieces of 8 channels per position; B rows: 16 pieces of 8 state rows
  for (int it = tid; it < kSsdQ * 8; it += kSsdThreads) {
    const int j = it >> 3, pc = it & 7;
    const SsdTok tk = ssd_tok(a, q, sl, c0 + j, h, g);
    const u32x4 v = ld16(tk.x + 8 * pc);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      Xt[8 * pc + 2 * e][j] = (bf16_t)(v[e] & 0xffffu);
      Xt[8 * pc + 2 * e + 1][j] = (bf16_t)(v[e] >> 16);
    }
    if (pc == 0) dts[j] = tk.dt;
  }
  for (int it = tid; it < kSsdQ * 16; it += kSsdThreads) {
    const int j = it >> 4, nc = it & 15;
    const SsdTok tk = ssd_tok(a, q, sl, c0 + j, h, g);
    const u32x4 v = ld16(tk.B + 8 * nc);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      Bt[8 * nc + 2 * e][j] = (bf16_t)(v[e] & 0xffffu);
      Bt[8 * nc + 2 * e + 1][j] = (bf16_t)(v[e] >> 16);
    }
  }
  __syncthreads();
  const float A = a.A[h];
  if (tid < 64) ssd_cumsum(dts, A, kSsdQ, Ls);
  __syncthreads();
  if (tid < kSsdQ) ws[tid] = ssd_exp(Ls[kSsdQ - 1] - Ls[tid]) * dts[tid];
  if (tid == 0) a.dec[(long)e_ * a.H + h] = ssd_exp(Ls[kSsdQ - 1]);
  __syncthreads();
  const int wave = tid >> 6, lane = tid & 63, grp = lane >> 4, r16 = lane & 15;
  bf16x8 xop[kSsdQ / 32];
#pragma unroll
  for (int kk = 0; kk < kSsdQ / 32; ++kk)
    xop[kk] = as_bf16x8(*reinterpret_cast<const u32x4 *>(&Xt[16 * wave + r16][32 * kk + 8 * grp]));
  float *out = a.dS + ((long)e_ * a.H + h) * (kSsdP * kSsdN);
  for (int nb = 0; nb < kSsdN / 16; ++nb) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < kSsdQ / 32; ++kk) {
      const u32x4 raw = *reinterpret_cast<const u32x4 *>(&Bt[16 * nb + r16][32 * kk + 8 * grp]);
      u32x4 op;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int s0 = 32 * kk + 8 * grp + 2 * e;
        op[e] = pack2(bf2f((bf16_t)(raw[e] & 0xffffu)) * ws[s0], bf2f((bf16_t)(raw[e] >> 16)) * ws[s0 + 1]);
      }
      acc = mfma(xop[kk], as_bf16x8(op), acc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) out[(16 * wave + 4 * grp + i) * kSsdN + 16 * nb + r16] = acc[i];
  }
}

// ---------------------------------------------------------------------------
// scan: per (sequence, head), the state through the call's completed chunks, in order:
// S <- exp(L_end) S + dS (one fp32 multiply, then one add, per element); completed chunk
// i's exit state (the state entering the next chunk) goes to entry[done + i].
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kSsdThreads) void ssd_scan_kernel(SsdArgs a) {
  const int s_ = blockIdx.x, h = blockIdx.y, n = a.n_seqs;
  const SsdSeq q = ssd_seq(a.plan, n, s_);
  if (q.slot < 0 || q.n_done <= 0) return;
  const int cf = q.p0 / kSsdQ;
  constexpr int kPer = kSsdP * kSsdN / (4 * kSsdThreads);  // float4s per thread (8)
  const SsdSlot sl = ssd_slot(a.pool, a.slot_bytes, q.slot, a.H, a.G);
  const float *s_in = sl.state + (long)h * kSsdP * kSsdN;
  f32x4 S[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k)
    S[k] = cf == 0 ? f32x4{0.f, 0.f, 0.f, 0.f}
                   : *reinterpret_cast<const f32x4 *>(s_in + 4 * (threadIdx.x + kSsdThreads * k));
  for (int i = 0; i < q.n_done; ++i) {
    const long e = q.done + i;
    const float dec = a.dec[e * a.H + h];
    const float *ds = a.dS + (e * a.H + h) * (long)(kSsdP * kSsdN);
    float *ent = a.entry + (e * a.H + h) * (long)(kSsdP * kSsdN);
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int at = 4 * (threadIdx.x + kSsdThreads * k);
      S[k] = S[k] * dec + *reinterpret_cast<const f32x4 *>(ds + at);
      *reinterpret_cast<f32x4 *>(ent + at) = S[k];
    }
  }
}

// ---------------------------------------------------------------------------
// out: every position of the call in one chunk, one head.  Grid (chunks, H), 4 waves;
// the chunk's inputs up to the call's last position are staged in LDS (x^T [p][s],
// B [s][n], dt) with the entry state as bf16 [p][n]; 16-position column blocks go to
// the waves in turn.  Per block: G^T (rows s, columns t), W^T from G^T's output layout
// (so the W product runs its 32-wide steps in the order s = 4g + i, 16 + 4g + i of each
// step, lane group g), then Y2^T and Y1^T (rows p, columns t) and the epilogue.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kSsdThreads) void ssd_out_kernel(SsdArgs a) {
  __shared__ __attribute__((aligned(16))) bf16_t Xt[kSsdP][kSsdPad];  // x^T [p][s]
  __shared__ __attribute__((aligned(16))) bf16_t Sb[kSsdP][kSsdPad];  // bf16(S_in) [p][n]
  __shared__ __attribute__((aligned(16))) bf16_t Bc[kSsdQ][kSsdPad];  // B [s][n]
  __shared__ float dts[kSsdQ], Ls[kSsdQ];
  const int b = blockIdx.x, h = blockIdx.y, n = a.n_seqs;
  const int s_ = ssd_owner(a.plan, n, b);
  if (s_ < 0) return;
  const SsdSeq q = ssd_seq(a.plan, n, s_);
  const int cf = q.p0 / kSsdQ, c = cf + (b - q.off), c0 = c * kSsdQ;
  const int ta = max(q.p0, c0) - c0, tb = min(q.p1, c0 + kSsdQ) - c0;  // the call's offsets
  const int g = h / (a.H / a.G), tid = threadIdx.x;
  if (q.slot < 0) {  // a sequence without a valid slot: its outputs are NaN
    for (int it = tid; it < (tb - ta) * kSsdP; it += kSsdThreads) {
      const long j = q.tok0 + (c0 + ta + it / kSsdP - q.p0);
      a.y[(j * a.H + h) * kSsdP + it % kSsdP] = (bf16_t)0x7fc0u;
    }
    return;
  }
  const SsdSlot sl = ssd_slot(a.pool, a.slot_bytes, q.slot, a.H, a.G);
  for (int it = tid; it < kSsdQ * 8; it += kSsdThreads) {
    const int j = it >> 3, pc = it & 7;
    u32x4 v = {0u, 0u, 0u, 0u};
    float d = 0.f;
    if (j < tb) {
      const SsdTok tk = ssd_tok(a, q, sl, c0 + j, h, g);
      v = ld16(tk.x + 8 * pc);
      d = tk.dt;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      Xt[8 * pc + 2 * e][j] = (bf16_t)(v[e] & 0xffffu);
      Xt[8 * pc + 2 * e + 1][j] = (bf16_t)(v[e] >> 16);
    }
    if (pc == 0) dts[j] = d;
  }
  for (int it = tid; it < kSsdQ * 16; it += kSsdThreads) {
    const int j = it >> 4, nc = it & 15;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (j < tb) v = ld16(ssd_tok(a, q, sl, c0 + j, h, g).B + 8 * nc);
    *reinterpret_cast<u32x4 *>(&Bc[j][8 * nc]) = v;
  }
  {
    const float *src = c == 0 ? nullptr
                       : c == cf ? sl.state + (long)h * kSsdP * kSsdN
                                 : a.entry + ((long)(q.done + (c - cf - 1)) * a.H + h) * (kSsdP * kSsdN);
    for (int it = tid; it < kSsdP * kSsdN / 8; it += kSsdThreads) {
      const int p = it >> 4, nc = it & 15;
      u32x4 w = {0u, 0u, 0u, 0u};
      if (src) {
        const f32x4 lo = *reinterpret_cast<const f32x4 *>(src + p * kSsdN + 8 * nc);
        const f32x4 hi = *reinterpret_cast<const f32x4 *>(src + p * kSsdN + 8 * nc + 4);
        w = u32x4{pack2(lo[0], lo[1]), pack2(lo[2], lo[3]), pack2(hi[0], hi[1]), pack2(hi[2], hi[3])};
      }
      *reinterpret_cast<u32x4 *>(&Sb[p][8 * nc]) = w;
    }
  }
  __syncthreads();
  const float A = a.A[h], Dh = a.D[h];
  if (tid < 64) ssd_cumsum(dts, A, tb, Ls);
  __syncthreads();
  const int wave = tid >> 6, lane = tid & 63, grp = lane >> 4, r16 = lane & 15;
  const int cb0 = ta / 16, cb1 = (tb - 1) / 16;
  for (int cb = cb0 + wave; cb <= cb1; cb += 4) {
    const int t = 16 * cb + r16;  // this lane's column
    const bool live = t >= ta && t < tb;
    const long jt = q.tok0 + (c0 + t - q.p0);
    // C^T operand (k = n, column t), zero for columns outside the call
    bf16x8 cop[kSsdN / 32];
#pragma unroll
    for (int kk = 0; kk < kSsdN / 32; ++kk) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (live) v = ld16(a.C + (jt * a.G + g) * kSsdN + 32 * kk + 8 * grp);
      cop[kk] = as_bf16x8(v);
    }
    const float Lt = live ? Ls[t] : 0.f;
    // W^T for s-blocks 0..7 (rows s = 16 sb + 4 grp + i), packed per 32-wide step
    u32x4 wop[kSsdQ / 32];
#pragma unroll
    for (int sb = 0; sb < kSsdQ / 16; ++sb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < kSsdN / 32; ++kk)
        acc = mfma(as_bf16x8(*reinterpret_cast<const u32x4 *>(&Bc[16 * sb + r16][32 * kk + 8 * grp])), cop[kk], acc);
      float w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int s = 16 * sb + 4 * grp + i;
        w[i] = (live && s <= t) ? acc[i] * ssd_exp(Lt - Ls[s]) * dts[s] : 0.f;
      }
      wop[sb >> 1][2 * (sb & 1)] = pack2(w[0], w[1]);
      wop[sb >> 1][2 * (sb & 1) + 1] = pack2(w[2], w[3]);
    }
    const float et = ssd_exp(Lt);
#pragma unroll
    for (int pb = 0; pb < kSsdP / 16; ++pb) {
      const int p = 16 * pb + r16;
      f32x4 y2 = {0.f, 0.f, 0.f, 0.f}, y1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < kSsdQ / 32; ++kk) {
        const u32x2 lo = *reinterpret_cast<const u32x2 *>(&Xt[p][32 * kk + 4 * grp]);
        const u32x2 hi = *reinterpret_cast<const u32x2 *>(&Xt[p][32 * kk + 16 + 4 * grp]);
        y2 = mfma(as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]}), as_bf16x8(wop[kk]), y2);
      }
#pragma unroll
      for (int kk = 0; kk < kSsdN / 32; ++kk)
        y1 = mfma(as_bf16x8(*reinterpret_cast<const u32x4 *>(&Sb[p][32 * kk + 8 * grp])), cop[kk], y1);
      if (live) {
        uint32_t o[2];
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          const int pp = 16 * pb + 4 * grp + i;
          const float v0 = (y1[i] * et + y2[i]) + Dh * bf2f(Xt[pp][t]);
          const float v1 = (y1[i + 1] * et + y2[i + 1]) + Dh * bf2f(Xt[pp + 1][t]);
          o[i / 2] = pack2(v0, v1);
        }
        *reinterpret_cast<u32x2 *>(a.y + (jt * a.H + h) * kSsdP + 16 * pb + 4 * grp) = u32x2{o[0], o[1]};
      }
    }
  }
}

// ---------------------------------------------------------------------------
// commit: the state entering the sequence's new current chunk into its slot
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kSsdThreads) void ssd_commit_kernel(SsdArgs a) {
  const int s_ = blockIdx.x, h = blockIdx.y;
  const SsdSeq q = ssd_seq(a.plan, a.n_seqs, s_);
  if (q.slot < 0 || q.n_done <= 0) return;
  const SsdSlot sl = ssd_slot(a.pool, a.slot_bytes, q.slot, a.H, a.G);
  const float *fin = a.entry + ((long)(q.done + q.n_done - 1) * a.H + h) * (kSsdP * kSsdN);
  float *dst = sl.state + (long)h * kSsdP * kSsdN;
  for (int e = 4 * threadIdx.x; e < kSsdP * kSsdN; e += 4 * kSsdThreads)
    *reinterpret_cast<f32x4 *>(dst + e) = *reinterpret_cast<const f32x4 *>(fin + e);
}

// ---------------------------------------------------------------------------
// write: the inputs of an unfinished last chunk into the slot (offset pos % Q).  One
// thread per (token, 16-byte unit): H * 8 units of x, G * 16 of B, H / 4 of dt.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kSsdThreads) void ssd_write_kernel(SsdArgs a) {
  const int per = a.H * 8 + a.G * 16 + a.H / 4;
  const long idx = (long)blockIdx.x * kSsdThreads + threadIdx.x;
  if (idx >= (long)a.n_tok * per) return;
  const int j = (int)(idx / per), u = (int)(idx % per);
  const int s_ = a.mode == 0 ? locate_seq(a.cu, a.n_seqs, j) : j;
  if (s_ >= a.n_seqs) return;
  const SsdSeq q = ssd_seq(a.plan, a.n_seqs, s_);
  if (q.slot < 0 || q.n_ch <= 0 || j < q.tok0 || j >= q.tok0 + (q.p1 - q.p0)) return;
  const int pos = q.p0 + (j - q.tok0), last0 = (q.p1 - 1) / kSsdQ * kSsdQ;
  if (q.p1 % kSsdQ == 0 || pos < last0) return;  // the last chunk is complete, or pos is before it
  const SsdSlot sl = ssd_slot(a.pool, a.slot_bytes, q.slot, a.H, a.G);
  const int k = pos % kSsdQ;
  if (u < a.H * 8) {
    st16(sl.x + ((long)k * a.H) * kSsdP + 8 * u, ld16(a.x + (long)j * a.H * kSsdP + 8 * u));
  } else if (u < a.H * 8 + a.G * 16) {
    const int v = u - a.H * 8;
    st16(sl.B + ((long)k * a.G) * kSsdN + 8 * v, ld16(a.B + (long)j * a.G * kSsdN + 8 * v));
  } else {
    const int v = u - a.H * 8 - a.G * 16;
    st16(sl.dt + (long)k * a.H + 4 * v, ld16(a.dt + (long)j * a.H + 4 * v));
  }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
hipError_t launch_ssd_plan(const SsdArgs &a, hipStream_t st) {
  if (a.n_seqs == 0) return hipSuccess;
  hipLaunchKernelGGL(ssd_plan_kernel, dim3(1), dim3(64), 0, st, a);
  return hipGetLastError();
}
hipError_t launch_ssd_state(const SsdArgs &a, hipStream_t st) {
  if (a.n_seqs == 0 || a.max_done == 0) return hipSuccess;
  hipLaunchKernelGGL(ssd_state_kernel, dim3(a.max_done, a.H), dim3(kSsdThreads), 0, st, a);
  return hipGetLastError();
}
hipError_t launch_ssd_scan(const SsdArgs &a, hipStream_t st) {
  if (a.n_seqs == 0) return hipSuccess;
  hipLaunchKernelGGL(ssd_scan_kernel, dim3(a.n_seqs, a.H), dim3(kSsdThreads), 0, st, a);
  return hipGetLastError();
}
hipError_t launch_ssd_out(const SsdArgs &a, hipStream_t st) {
  if (a.n_seqs == 0) return hipSuccess;
  hipLaunchKernelGGL(ssd_out_kernel, dim3(a.max_chunks, a.H), dim3(kSsdThreads), 0, st, a);
  return hipGetLastError();
}
hipError_t launch_ssd_commit(const SsdArgs &a, hipStream_t st) {
  if (a.n_seqs == 0) return hipSuccess;
  hipLaunchKernelGGL(ssd_commit_kernel, dim3(a.n_seqs, a.H), dim3(kSsdThreads), 0, st, a);
  return hipGetLastError();
}
hipError_t launch_ssd_write(const SsdArgs &a, hipStream_t st) {
  const long total = (long)a.n_tok * (a.H * 8 + a.G * 16 + a.H / 4);
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(ssd_write_kernel, dim3((unsigned)((total + kSsdThreads - 1) / kSsdThreads)), dim3(kSsdThreads),
                     0, st, a);
  return hipGetLastError();
}

}  // namespace ril
