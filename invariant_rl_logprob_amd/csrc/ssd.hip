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
// The state of chunk c sits in one of two buffers by the parity of c, so the step that
// completes a chunk writes the next chunk's state beside the one it read: repeating a
// decode step (a replay, a retry) reads and writes the same bytes again.
// A call runs: plan (its chunks), state (the exit-state sums of the chunks it completes),
// scan (states through those chunks, in order), out (every position's y), commit (the
// new entry state into the slot), write (the inputs of an unfinished last chunk into the
// slot).  Decode completes a chunk exactly as prefill does: the same kernels.
#include "attn_common.h"
#include "kernels.h"

namespace ril {

// LDS row lengths (elements): 128-wide operand tiles (B, the entry state) and the x tile
// [s][p].  The state kernel also groups rows in blocks of 8 with 64 elements (128 bytes)
// after each block.  Measured with the LDS bank-conflict counter, per access: the
// 16-byte reads of rows 16 sb + i take rows of 288 bytes (272 conflicted two-way); the
// transposing reads take rows of 160 bytes, and the state kernel's, whose 16-lane groups
// start 8 rows apart, also the block gap, which puts rows 8 apart half a bank row apart
// (288- and 160-byte rows alone leave them two-way conflicted).
constexpr int kSsdPad = kSsdQ + 16;
constexpr int kSsdXRow = kSsdP + 16;
constexpr int kSsdXBlk = 8 * kSsdXRow + 64, kSsdBBlk = 8 * kSsdPad + 64;  // elements per 8-row block

// Transposing LDS reads of a tile stored position-major ([s][c], row length RL elements):
// lane L = 4e + m of each 16-lane group addresses the 4 columns c0 + 4m .. of row s0 + e,
// and ds_read_b64_tr_b16 hands lane i the column c0 + i of rows s0 .. s0 + 3 (4 values,
// rows ascending): one MFMA operand half with K along the positions.  This returns the
// lane's base address for row 0, column 0 of the tile; callers add s0 and c0 as an
// immediate offset.
template <int RL>
__device__ __forceinline__ uint32_t ssd_tr_base(const bf16_t *tile) {
  const int l = threadIdx.x & 15;
  return lds_addr(tile) + 2 * ((l >> 2) * RL + 4 * (l & 3));
}
constexpr int kSsdThreads = 256;

__host__ __device__ inline long ssd_state_bytes(int H) { return (long)H * kSsdP * kSsdN * 4; }
long ssd_slot_bytes(int H, int G) {
  const long b = 2 * ssd_state_bytes(H) + (long)kSsdQ * H * kSsdP * 2 + (long)kSsdQ * G * kSsdN * 2 + (long)kSsdQ * H * 4;
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
  float *state;  // two [H][P][N] buffers: the state entering chunk c at state + (c & 1) * H P N
  bf16_t *x, *B;
  float *dt;
};
__device__ __forceinline__ SsdSlot ssd_slot(uint8_t *pool, long slot_bytes, int slot, int H, int G) {
  uint8_t *b = pool + (long)slot * slot_bytes;
  SsdSlot s;
  s.state = reinterpret_cast<float *>(b);
  s.x = reinterpret_cast<bf16_t *>(b + 2 * ssd_state_bytes(H));
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
// plan: one wave.  Sequence s's positions, tokens and chunk counts; off / done are the
// running sums of the chunk counts in sequence order.  Lanes take 64 sequences at a time
// and wave prefix sums give the running sums.  A sequence the grids cannot hold (only
// with batch arrays inconsistent with the host's bounds) is dropped and adds nothing;
// should one appear, lane 0 redoes the whole plan in order, so the plan is always that
// of the in-order walk.
// ---------------------------------------------------------------------------
struct SsdPlanRow {
  bool ok;
  int tok0, p0, p1, slot, n_ch, n_done;
};
__device__ __forceinline__ SsdPlanRow ssd_plan_row(const SsdArgs &a, int s) {
  SsdPlanRow r;
  int len;
  if (a.mode == 0) {
    r.tok0 = a.cu[s];
    len = a.cu[s + 1] - r.tok0;
    r.p0 = a.start_pos[s];
  } else {
    r.tok0 = s;
    len = 1;
    r.p0 = a.ctx_len[s] - 1;
  }
  r.ok = len >= 1 && r.p0 >= 0 && r.tok0 >= 0 && (long)r.tok0 + len <= a.n_tok && (long)r.p0 + len <= 0x7fffffffL;
  r.slot = r.ok ? a.page_table[(long)s * a.page_stride] : -1;
  r.p1 = r.ok ? r.p0 + len : r.p0;
  r.n_ch = r.ok ? (r.p1 - 1) / kSsdQ - r.p0 / kSsdQ + 1 : 0;
  r.n_done = r.ok ? r.p1 / kSsdQ - r.p0 / kSsdQ : 0;
  return r;
}
__device__ __forceinline__ void ssd_plan_store(const SsdArgs &a, int s, const SsdPlanRow &r, bool ok, int off,
                                               int done) {
  const int n = a.n_seqs;
  int32_t *plan = a.plan;
  plan[s + 1] = off;
  plan[n + 2 + s] = done;
  plan[2 * n + 2 + s] = ok ? r.p0 : 0;
  plan[3 * n + 2 + s] = ok ? r.p1 : 0;
  plan[4 * n + 2 + s] = ok ? r.tok0 : 0;
  plan[5 * n + 2 + s] = (ok && (unsigned)r.slot < (unsigned)a.n_slots) ? r.slot : -1;
}
__global__ __launch_bounds__(64) void ssd_plan_kernel(SsdArgs a) {
  const int n = a.n_seqs, lane = threadIdx.x;
  if (lane == 0) {
    a.plan[0] = 0;
    a.plan[n + 1] = 0;
  }
  int off0 = 0, done0 = 0;  // running sums before this group of 64
  bool fits = true;
  for (int base = 0; base < n && fits; base += 64) {
    const int s = base + lane;
    SsdPlanRow r = {false, 0, 0, 0, -1, 0, 0};
    if (s < n) r = ssd_plan_row(a, s);
    int ch = r.n_ch, dn = r.n_done;  // inclusive prefix sums over the group
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int uc = __shfl_up(ch, d, 64), ud = __shfl_up(dn, d, 64);
      if (lane >= d) {
        ch += uc;
        dn += ud;
      }
    }
    const int off = off0 + ch, done = done0 + dn;
    fits = !__any(s < n && r.ok && (off > a.max_chunks || done > a.max_done));
    if (fits && s < n) ssd_plan_store(a, s, r, r.ok, off, done);
    off0 = __shfl(off, 63, 64);
    done0 = __shfl(done, 63, 64);
  }
  if (fits) return;  // uniform over the wave
  __threadfence();   // the stores above land before the in-order walk's
  if (lane != 0) return;
  int off = 0, done = 0;
  for (int s = 0; s < n; ++s) {
    const SsdPlanRow r = ssd_plan_row(a, s);
    const bool ok = r.ok && off + r.n_ch <= a.max_chunks && done + r.n_done <= a.max_done;
    if (ok) {
      off += r.n_ch;
      done += r.n_done;
    }
    ssd_plan_store(a, s, r, ok, off, done);
  }
}

// ---------------------------------------------------------------------------
// state: for each chunk the call completes, dS^T[p][n] = sum_s x_s[p] bf16(B_s[n] w_s)
// (w_s = exp(L_end - L_s) dt_s) and its decay exp(L_end).  Grid (completed chunks, H),
// 4 waves: wave w owns channels 16w .. 16w + 15 and all 128 state rows.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kSsdThreads) void ssd_state_kernel(SsdArgs a) {
  __shared__ __attribute__((aligned(16))) bf16_t Xn[kSsdQ / 8][kSsdXBlk];  // x [s][p], 8-row blocks
  __shared__ __attribute__((aligned(16))) bf16_t Bn[kSsdQ / 8][kSsdBBlk];  // B [s][n], 8-row blocks
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
  // x rows: 8 pieces of 8 channels per position; B rows: 16 pieces of 8 state rows; every
  // load of a thread issued before its first store
  constexpr int kXPer = kSsdQ * 8 / kSsdThreads, kBPer = kSsdQ * 16 / kSsdThreads;
  u32x4 xv[kXPer], bv[kBPer];
  float dv[kXPer];
#pragma unroll
  for (int k = 0; k < kXPer; ++k) {
    const int it = tid + kSsdThreads * k;
    const SsdTok tk = ssd_tok(a, q, sl, c0 + (it >> 3), h, g);
    xv[k] = ld16(tk.x + 8 * (it & 7));
    dv[k] = tk.dt;
  }
#pragma unroll
  for (int k = 0; k < kBPer; ++k) {
    const int it = tid + kSsdThreads * k;
    bv[k] = ld16(ssd_tok(a, q, sl, c0 + (it >> 4), h, g).B + 8 * (it & 15));
  }
#pragma unroll
  for (int k = 0; k < kXPer; ++k) {
    const int it = tid + kSsdThreads * k, j = it >> 3, pc = it & 7;
    *reinterpret_cast<u32x4 *>(&Xn[j >> 3][(j & 7) * kSsdXRow + 8 * pc]) = xv[k];
    if (pc == 0) dts[j] = dv[k];
  }
#pragma unroll
  for (int k = 0; k < kBPer; ++k) {
    const int it = tid + kSsdThreads * k;
    const int j = it >> 4;
    *reinterpret_cast<u32x4 *>(&Bn[j >> 3][(j & 7) * kSsdPad + 8 * (it & 15)]) = bv[k];
  }
  __syncthreads();
  const float A = a.A[h];
  if (tid < 64) ssd_cumsum(dts, A, kSsdQ, Ls);
  __syncthreads();
  if (tid < kSsdQ) ws[tid] = ssd_exp(Ls[kSsdQ - 1] - Ls[tid]) * dts[tid];
  if (tid == 0) a.dec[(long)e_ * a.H + h] = ssd_exp(Ls[kSsdQ - 1]);
  __syncthreads();
  const int wave = tid >> 6, lane = tid & 63, grp = lane >> 4, r16 = lane & 15;
  // x^T operand (rows p = 16 wave + i, K = s = 32 kk + 8 grp + 0..7) by transposing reads
  const uint32_t xa = ssd_tr_base<kSsdXRow>(&Xn[grp][16 * wave]);  // row 8 grp
  u32x2 xr[2 * (kSsdQ / 32)];
  static_for<kSsdQ / 32>([&](auto kk_) {
    constexpr int kk = decltype(kk_)::value;
    xr[2 * kk] = lds_rdtr<2 * 4 * kk * kSsdXBlk>(xa);  // rows 32 kk .., then 32 kk + 4 ..
    xr[2 * kk + 1] = lds_rdtr<2 * (4 * kk * kSsdXBlk + 4 * kSsdXRow)>(xa);
  });
  lds_wait<0>();
  bf16x8 xop[kSsdQ / 32];
#pragma unroll
  for (int kk = 0; kk < kSsdQ / 32; ++kk) {
    settle(xr[2 * kk]);
    settle(xr[2 * kk + 1]);
    xop[kk] = as_bf16x8(u32x4{xr[2 * kk][0], xr[2 * kk][1], xr[2 * kk + 1][0], xr[2 * kk + 1][1]});
  }
  const uint32_t ba = ssd_tr_base<kSsdPad>(&Bn[grp][0]);  // row 8 grp
  float *out = a.dS + ((long)e_ * a.H + h) * (kSsdP * kSsdN);
  static_for<kSsdN / 16>([&](auto nb_) {
    constexpr int nb = decltype(nb_)::value;
    // B operand (K = s, column n = 16 nb + i), each value times w_s, rounded to bf16
    u32x2 br[2 * (kSsdQ / 32)];
    static_for<kSsdQ / 32>([&](auto kk_) {
      constexpr int kk = decltype(kk_)::value;
      br[2 * kk] = lds_rdtr<2 * (4 * kk * kSsdBBlk + 16 * nb)>(ba);
      br[2 * kk + 1] = lds_rdtr<2 * (4 * kk * kSsdBBlk + 4 * kSsdPad + 16 * nb)>(ba);
    });
    lds_wait<0>();
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < kSsdQ / 32; ++kk) {
      u32x4 op;
#pragma unroll
      for (int hlf = 0; hlf < 2; ++hlf) {
        u32x2 raw = br[2 * kk + hlf];
        settle(raw);
        const int s0 = 32 * kk + 8 * grp + 4 * hlf;
        op[2 * hlf] = pack2(bf2f((bf16_t)(raw[0] & 0xffffu)) * ws[s0], bf2f((bf16_t)(raw[0] >> 16)) * ws[s0 + 1]);
        op[2 * hlf + 1] = pack2(bf2f((bf16_t)(raw[1] & 0xffffu)) * ws[s0 + 2], bf2f((bf16_t)(raw[1] >> 16)) * ws[s0 + 3]);
      }
      acc = mfma(xop[kk], as_bf16x8(op), acc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) out[(16 * wave + 4 * grp + i) * kSsdN + 16 * nb + r16] = acc[i];
  });
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
  const float *s_in = sl.state + ((long)(cf & 1) * a.H + h) * kSsdP * kSsdN;
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
// the chunk's inputs up to the call's last position (x [s][p], read transposed, B [s][n],
// dt) and the entry state as bf16 [p][n] are staged in LDS; 16-position column blocks go
// to the waves in turn.  Per block: G^T (rows s, columns t), W^T from G^T's output layout
// (so the W product runs its 32-wide steps in the order s = 4g + i, 16 + 4g + i of each
// step, lane group g), then Y2^T and Y1^T (rows p, columns t) and the epilogue.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kSsdThreads) void ssd_out_kernel(SsdArgs a) {
  __shared__ __attribute__((aligned(16))) bf16_t Xn[kSsdQ][kSsdXRow];  // x [s][p]
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
  // Stage the chunk's inputs up to the call's last position and the entry state in LDS.
  // Every load of a thread is issued before its first store, and a position past the
  // call loads a valid one and stores zeros, so the loads carry no branches: a few memory
  // round trips per workgroup instead of one per piece.
  constexpr int kXPer = kSsdQ * 8 / kSsdThreads, kBPer = kSsdQ * 16 / kSsdThreads;
  constexpr int kSPer = kSsdP * kSsdN / 8 / kSsdThreads;
  const float *src = c == 0 ? nullptr
                     : c == cf ? sl.state + ((long)(c & 1) * a.H + h) * kSsdP * kSsdN
                               : a.entry + ((long)(q.done + (c - cf - 1)) * a.H + h) * (kSsdP * kSsdN);
  u32x4 xv[kXPer], bv[kBPer];
  float dv[kXPer];
  f32x4 sv[2 * kSPer];
#pragma unroll
  for (int k = 0; k < kXPer; ++k) {
    const int it = tid + kSsdThreads * k, j = it >> 3;
    const SsdTok tk = ssd_tok(a, q, sl, c0 + min(j, tb - 1), h, g);
    xv[k] = ld16(tk.x + 8 * (it & 7));
    dv[k] = tk.dt;
  }
#pragma unroll
  for (int k = 0; k < kBPer; ++k) {
    const int it = tid + kSsdThreads * k, j = it >> 4;
    bv[k] = ld16(ssd_tok(a, q, sl, c0 + min(j, tb - 1), h, g).B + 8 * (it & 15));
  }
  const float *sp = src ? src : a.dec;  // any readable address when the state is zero
#pragma unroll
  for (int k = 0; k < kSPer; ++k) {
    const int it = tid + kSsdThreads * k, off = src ? (it >> 4) * kSsdN + 8 * (it & 15) : 0;
    sv[2 * k] = *reinterpret_cast<const f32x4 *>(sp + off);
    sv[2 * k + 1] = *reinterpret_cast<const f32x4 *>(sp + off + 4);
  }
#pragma unroll
  for (int k = 0; k < kXPer; ++k) {
    const int it = tid + kSsdThreads * k, j = it >> 3, pc = it & 7;
    *reinterpret_cast<u32x4 *>(&Xn[j][8 * pc]) = j < tb ? xv[k] : u32x4{0u, 0u, 0u, 0u};
    if (pc == 0) dts[j] = j < tb ? dv[k] : 0.f;
  }
#pragma unroll
  for (int k = 0; k < kBPer; ++k) {
    const int it = tid + kSsdThreads * k, j = it >> 4;
    *reinterpret_cast<u32x4 *>(&Bc[j][8 * (it & 15)]) = j < tb ? bv[k] : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int k = 0; k < kSPer; ++k) {
    const int it = tid + kSsdThreads * k;
    const f32x4 lo = sv[2 * k], hi = sv[2 * k + 1];
    const u32x4 w = src ? u32x4{pack2(lo[0], lo[1]), pack2(lo[2], lo[3]), pack2(hi[0], hi[1]), pack2(hi[2], hi[3])}
                        : u32x4{0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4 *>(&Sb[it >> 4][8 * (it & 15)]) = w;
  }
  __syncthreads();
  const float A = a.A[h], Dh = a.D[h];
  if (tid < 64) ssd_cumsum(dts, A, tb, Ls);
  __syncthreads();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, grp = lane >> 4, r16 = lane & 15;
  const int cb0 = ta / 16, cb1 = (tb - 1) / 16;
  // Column block cb: this lane's column t, the C^T operand (K = n, column t; zero for
  // columns outside the call), L_t.
  struct Col {
    int t;
    bool live;
    long jt;
    float Lt;
    bf16x8 cop[kSsdN / 32];
  };
  auto column = [&](int cb) {
    Col c;
    c.t = 16 * cb + r16;
    c.live = c.t >= ta && c.t < tb;
    c.jt = q.tok0 + (c0 + c.t - q.p0);
#pragma unroll
    for (int kk = 0; kk < kSsdN / 32; ++kk) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (c.live) v = ld16(a.C + (c.jt * a.G + g) * kSsdN + 32 * kk + 8 * grp);
      c.cop[kk] = as_bf16x8(v);
    }
    c.Lt = c.live ? Ls[c.t] : 0.f;
    return c;
  };
  // W^T of s-block sb (rows s = 16 sb + 4 grp + i): G^T's MFMA chain over n, then the
  // decayed, dt-weighted value rounded to bf16 (0 past the column), as two packed words
  auto wblock = [&](const Col &c, int sb) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < kSsdN / 32; ++kk)
      acc = mfma(as_bf16x8(*reinterpret_cast<const u32x4 *>(&Bc[16 * sb + r16][32 * kk + 8 * grp])), c.cop[kk], acc);
    float w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = 16 * sb + 4 * grp + i;
      w[i] = (c.live && s <= c.t) ? acc[i] * ssd_exp(c.Lt - Ls[s]) * dts[s] : 0.f;
    }
    return u32x2{pack2(w[0], w[1]), pack2(w[2], w[3])};
  };
  // p-block pb: Y2^T (the W product, x^T read transposed in W's K order: s = 32 kk +
  // 4 grp + 0..3, then 32 kk + 16 + 4 grp + 0..3), Y1^T (the state product) and the
  // epilogue for channels 16 pb ..
  const uint32_t xa = ssd_tr_base<kSsdXRow>(&Xn[4 * grp][0]);
  auto outblock = [&](const Col &c, int pb, const u32x4 (&wop)[kSsdQ / 32]) {
    const uint32_t xb = xa + 32 * pb;
    u32x2 xr[2 * (kSsdQ / 32)];
    static_for<kSsdQ / 32>([&](auto kk_) {
      constexpr int kk = decltype(kk_)::value;
      xr[2 * kk] = lds_rdtr<2 * 32 * kk * kSsdXRow>(xb);
      xr[2 * kk + 1] = lds_rdtr<2 * (32 * kk + 16) * kSsdXRow>(xb);
    });
    lds_wait<0>();
    f32x4 y2 = {0.f, 0.f, 0.f, 0.f}, y1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < kSsdQ / 32; ++kk) {
      settle(xr[2 * kk]);
      settle(xr[2 * kk + 1]);
      const u32x2 lo = xr[2 * kk], hi = xr[2 * kk + 1];
      y2 = mfma(as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]}), as_bf16x8(wop[kk]), y2);
    }
#pragma unroll
    for (int kk = 0; kk < kSsdN / 32; ++kk)
      y1 = mfma(as_bf16x8(*reinterpret_cast<const u32x4 *>(&Sb[16 * pb + r16][32 * kk + 8 * grp])), c.cop[kk], y1);
    if (c.live) {
      const float et = ssd_exp(c.Lt);
      uint32_t o[2];
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        const int pp = 16 * pb + 4 * grp + i;
        const float v0 = (y1[i] * et + y2[i]) + Dh * bf2f(Xn[c.t][pp]);
        const float v1 = (y1[i + 1] * et + y2[i + 1]) + Dh * bf2f(Xn[c.t][pp + 1]);
        o[i / 2] = pack2(v0, v1);
      }
      *reinterpret_cast<u32x2 *>(a.y + (c.jt * a.H + h) * kSsdP + 16 * pb + 4 * grp) = u32x2{o[0], o[1]};
    }
  };
  if (cb1 - cb0 + 1 >= 4) {
    // many columns (prefill): each wave takes whole column blocks in turn
    for (int cb = cb0 + wave; cb <= cb1; cb += 4) {
      const Col c = column(cb);
      u32x4 wop[kSsdQ / 32];
#pragma unroll
      for (int kk = 0; kk < kSsdQ / 32; ++kk) {
        const u32x2 lo = wblock(c, 2 * kk), hi = wblock(c, 2 * kk + 1);
        wop[kk] = u32x4{lo[0], lo[1], hi[0], hi[1]};
      }
#pragma unroll
      for (int pb = 0; pb < kSsdP / 16; ++pb) outblock(c, pb, wop);
    }
  } else {
    // few columns (decode): the four waves share each column block.  Wave w computes the
    // W^T of s-blocks 2w and 2w + 1 -- step w of the W product's K -- and hands it over in
    // LDS; then wave w runs p-block w.  The same MFMA chains as above, split over waves.
    __shared__ u32x4 wx[4][64];
    for (int cb = cb0; cb <= cb1; ++cb) {
      const Col c = column(cb);
      const u32x2 lo = wblock(c, 2 * wave), hi = wblock(c, 2 * wave + 1);
      wx[wave][lane] = u32x4{lo[0], lo[1], hi[0], hi[1]};
      __syncthreads();
      u32x4 wop[kSsdQ / 32];
#pragma unroll
      for (int kk = 0; kk < kSsdQ / 32; ++kk) wop[kk] = wx[kk][lane];
      outblock(c, wave, wop);
      __syncthreads();  // every wave has read wx before the next block overwrites it
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
  const int c_next = q.p0 / kSsdQ + q.n_done;  // the chunk this state enters
  float *dst = sl.state + ((long)(c_next & 1) * a.H + h) * kSsdP * kSsdN;
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
