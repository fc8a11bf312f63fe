// C ABI of the invariant logprob forward: validation, the host page allocator (S1),
// workspace layout from static limits, and the launch sequence on the caller's stream.
// The host never reads device memory and never synchronises (Bitwise-consistent RL
// post, section 4.6: no host sync or batch-dependent shapes on the hot path).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <climits>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.h"
#include "ril.h"
#include "ril_bench.h"

using namespace ril;

struct ril_model {
  ril_model_desc d;
  int G;            // q heads per kv head
  int n_vt;         // vocabulary tiles of 256 columns
  int max_splits;   // splits of the longest context
  float cscale;     // softmax_scale * log2(e), rounded once to fp32
  size_t page_bytes;
  bool kv_fp8;      // GQA pages hold FP8 E4M3 codes
  float k_scale, v_scale;  // 2^k_scale_exp, 2^v_scale_exp
  bool mla, sparse;
  // workspace segment offsets (bytes) and total
  size_t off_x, off_h, off_qkv, off_attn, off_y, off_z, off_vpart, off_tgt, off_po, off_pml;
  size_t off_scores, off_sel;  // sparse: indexer scores [max_rows, max_ctx], selections [max_rows, topk]
  size_t off_gu = 0, off_act = 0, off_y2 = 0;  // SwiGLU MLP: [R, 2F], [R, F], [R, d_model] bf16
  bool lm_fp8 = false;                        // W8A8 block-FP8 lm-head
  bool proj_fp8 = false;                      // W8A8 block-FP8 projections
  size_t off_p8 = 0, off_pe = 0;              // projection rows' codes and exponents
  size_t off_a8 = 0, off_ea = 0;              // its activation codes [R, d_head], exponents [R, d_head/128]
  size_t ws_base;   // end of the invariant path's segments
  size_t ws_total;  // ws_base + the comparator's split-K partials when that policy is on
  // comparator (benchmarking only): RIL_POLICY_SHAPE_DERIVED picks splits from the batch
  int policy = RIL_POLICY_INVARIANT;
  int attn_split_override = 0;
  int n_cu = 0;
  size_t off_gpart = 0;
  // SSD mixer: plan, completed chunks' state sums and exit states, their decays
  bool ssd = false;
  int ssd_max_done = 0;
  size_t off_ssd_plan = 0, off_ssd_ds = 0, off_ssd_ent = 0, off_ssd_dec = 0;
};

struct ril_kv {
  size_t page_bytes;
  void *pool;
  int32_t n_pages;
  std::vector<int32_t> free_list;  // popped from the back
  std::vector<uint8_t> assigned;
};

static thread_local std::string g_err;

static ril_status fail(ril_status s, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

static bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
static bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
static size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

extern "C" const char *ril_last_error(void) { return g_err.c_str(); }

extern "C" ril_status ril_model_create(const ril_model_desc *desc, ril_model **out) {
  if (!desc || !out) return fail(RIL_EINVAL, "model_create: null argument");
  const ril_model_desc &d = *desc;
  if (d.attn_kind != RIL_ATTN_GQA && d.attn_kind != RIL_ATTN_MLA && d.attn_kind != RIL_ATTN_MLA_SPARSE &&
      d.attn_kind != RIL_ATTN_SSD)
    return fail(RIL_EUNSUPPORTED, "model_create: attn_kind %d", d.attn_kind);
  const bool sparse = d.attn_kind == RIL_ATTN_MLA_SPARSE;
  const bool mla = d.attn_kind == RIL_ATTN_MLA || sparse;
  const bool ssd = d.attn_kind == RIL_ATTN_SSD;
  if (ssd) {
    if (d.head_dim != kSsdP || d.ssm_state != kSsdN || d.ssm_chunk != kSsdQ)
      return fail(RIL_EUNSUPPORTED, "model_create: SSD needs head_dim %d, ssm_state %d, ssm_chunk %d", kSsdP, kSsdN,
                  kSsdQ);
    if (d.n_q_heads < 4 || d.n_q_heads % 4 || d.n_kv_heads < 1 || d.n_q_heads % d.n_kv_heads)
      return fail(RIL_EINVAL, "model_create: SSD heads %d / groups %d (heads a multiple of 4 and of groups)",
                  d.n_q_heads, d.n_kv_heads);
    if (d.input_mode != RIL_INPUT_QKV || d.rope_dim || d.kv_dtype != RIL_KV_BF16)
      return fail(RIL_EUNSUPPORTED, "model_create: SSD takes given inputs, no rope, a bf16 cache");
    if (!d.ssm_A || !d.ssm_D || !aligned4(d.ssm_A) || !aligned4(d.ssm_D))
      return fail(RIL_EINVAL, "model_create: SSD needs ssm_A and ssm_D (fp32 [H])");
  } else if (d.ssm_state || d.ssm_chunk || d.ssm_A || d.ssm_D) {
    return fail(RIL_EINVAL, "model_create: ssm_* fields are for SSD");
  }
  if (sparse) {
    if (d.index_heads != 64 || d.index_dim != 128)
      return fail(RIL_EUNSUPPORTED, "model_create: indexer must be 64 heads x 128 dims");
    if (d.topk < 64 || d.topk > 4096 || (d.topk & (d.topk - 1)))
      return fail(RIL_EINVAL, "model_create: topk %d (a power of two in [64, 4096])", d.topk);
  } else if (d.index_heads || d.index_dim || d.topk) {
    return fail(RIL_EINVAL, "model_create: index_heads/index_dim/topk are for MLA_SPARSE");
  }
  if (d.input_mode != RIL_INPUT_TOKENS && d.input_mode != RIL_INPUT_QKV)
    return fail(RIL_EINVAL, "model_create: input_mode %d", d.input_mode);
  int G = 1;
  if (ssd) {
    G = d.n_q_heads / d.n_kv_heads;
  } else if (mla) {
    if (d.head_dim != 512 || d.rope_dim != 64 || d.n_kv_heads != 1)
      return fail(RIL_EUNSUPPORTED, "model_create: MLA needs head_dim 512, rope_dim 64, n_kv_heads 1");
    if (d.n_q_heads < 64 || d.n_q_heads % 64)
      return fail(RIL_EUNSUPPORTED, "model_create: MLA n_q_heads %d (a multiple of 64)", d.n_q_heads);
    if (d.input_mode != RIL_INPUT_QKV) return fail(RIL_EUNSUPPORTED, "model_create: MLA takes q/latent input");
    if (d.split_tokens <= 0 || d.split_tokens % 64 || d.split_tokens > 2048)
      return fail(RIL_EINVAL, "model_create: split_tokens %d (a multiple of 64, at most 2048)", d.split_tokens);
  } else {
    if (d.head_dim != 64 && d.head_dim != 128)
      return fail(RIL_EUNSUPPORTED, "model_create: head_dim %d (64 or 128)", d.head_dim);
    if (d.rope_dim != 0) return fail(RIL_EINVAL, "model_create: rope_dim is for MLA");
    if (d.n_q_heads < 1 || d.n_kv_heads < 1 || d.n_q_heads % d.n_kv_heads)
      return fail(RIL_EINVAL, "model_create: heads %d/%d", d.n_q_heads, d.n_kv_heads);
    G = d.n_q_heads / d.n_kv_heads;
    if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16)
      return fail(RIL_EUNSUPPORTED, "model_create: group size %d (1, 2, 4, 8 or 16)", G);
    if (d.split_tokens <= 0 || d.split_tokens % 64 || d.split_tokens > 1024)
      return fail(RIL_EINVAL, "model_create: split_tokens %d (a multiple of 64, at most 1024)", d.split_tokens);
  }
  if (d.page_tokens != 16) return fail(RIL_EUNSUPPORTED, "model_create: page_tokens %d (16)", d.page_tokens);
  if (d.d_ff < 0 || d.d_ff % 32)
    return fail(RIL_EINVAL, "model_create: d_ff %d (0 or a multiple of 32)", d.d_ff);
  if (d.d_ff && (d.input_mode != RIL_INPUT_TOKENS || !d.w_gate_up || !d.w_down ||
                 ((uintptr_t)d.w_gate_up & 15) || ((uintptr_t)d.w_down & 15) || ((uintptr_t)d.norm_mlp & 15)))
    return fail(RIL_EINVAL, "model_create: the MLP block needs TOKENS input and 16-byte aligned w_gate_up/w_down");
  if (!d.d_ff && (d.w_gate_up || d.w_down || d.norm_mlp))
    return fail(RIL_EINVAL, "model_create: MLP weights given with d_ff = 0");
  if (d.lm_dtype != RIL_LM_BF16 && d.lm_dtype != RIL_LM_W8A8_FP8)
    return fail(RIL_EINVAL, "model_create: lm_dtype %d", d.lm_dtype);
  if (d.proj_dtype != RIL_PROJ_BF16 && d.proj_dtype != RIL_PROJ_W8A8_FP8)
    return fail(RIL_EINVAL, "model_create: proj_dtype %d", d.proj_dtype);
  if (d.proj_dtype == RIL_PROJ_W8A8_FP8) {
    const bool tk = d.input_mode == RIL_INPUT_TOKENS;
    const int qk = d.n_q_heads * d.head_dim;
    if ((tk && d.d_model % 128) || (d.w_o && qk % 128) || (d.d_ff && d.d_ff % 128))
      return fail(RIL_EINVAL, "model_create: W8A8 projections need every K (d_model %d, Hq*D %d, d_ff %d) a "
                  "multiple of 128", d.d_model, qk, d.d_ff);
  }
  if (d.lm_dtype == RIL_LM_W8A8_FP8 && (d.d_head <= 0 || d.d_head % 128))
    return fail(RIL_EINVAL, "model_create: the W8A8 lm-head needs d_head a multiple of 128 (%d)", d.d_head);
  if (d.kv_dtype != RIL_KV_BF16 && d.kv_dtype != RIL_KV_FP8_E4M3)
    return fail(RIL_EINVAL, "model_create: kv_dtype %d", d.kv_dtype);
  if (d.kv_dtype == RIL_KV_FP8_E4M3 && mla && d.k_scale_exp != d.v_scale_exp)
    return fail(RIL_EINVAL, "model_create: an FP8 MLA latent has one scale (k_scale_exp %d != v_scale_exp %d)",
                d.k_scale_exp, d.v_scale_exp);
  if (d.k_scale_exp < -32 || d.k_scale_exp > 32 || d.v_scale_exp < -32 || d.v_scale_exp > 32)
    return fail(RIL_EINVAL, "model_create: k/v_scale_exp %d/%d (in [-32, 32])", d.k_scale_exp, d.v_scale_exp);
  if (d.kv_dtype == RIL_KV_BF16 && (d.k_scale_exp || d.v_scale_exp))
    return fail(RIL_EINVAL, "model_create: k/v_scale_exp are for the FP8 KV cache");
  if (d.vocab < 1) return fail(RIL_EINVAL, "model_create: vocab %d", d.vocab);
  if (d.max_rows < 1 || d.max_tokens < 1 || d.max_ctx < 1)
    return fail(RIL_EINVAL, "model_create: limits %d/%d/%d", d.max_rows, d.max_tokens, d.max_ctx);
  if (!(d.softmax_scale > 0.f) || !std::isfinite(d.softmax_scale))
    return fail(RIL_EINVAL, "model_create: softmax_scale");
  if (!(d.rms_eps >= 0.f) || !std::isfinite(d.rms_eps)) return fail(RIL_EINVAL, "model_create: rms_eps");
  const int qw = d.n_q_heads * d.head_dim;
  if (d.input_mode == RIL_INPUT_TOKENS) {
    if (d.d_model <= 0 || d.d_model % 32) return fail(RIL_EINVAL, "model_create: d_model %d", d.d_model);
    if (!d.embed || !d.w_qkv || !d.w_o) return fail(RIL_EINVAL, "model_create: TOKENS needs embed, w_qkv, w_o");
    if (d.d_head != d.d_model) return fail(RIL_EINVAL, "model_create: TOKENS needs d_head == d_model");
    if (qw % 32) return fail(RIL_EINVAL, "model_create: Hq*D %d not a multiple of 32", qw);
  } else {
    if (d.w_o ? (d.d_head <= 0 || d.d_head % 32) : (d.d_head != qw))
      return fail(RIL_EINVAL, "model_create: d_head %d", d.d_head);
  }
  if (!d.w_lm) return fail(RIL_EINVAL, "model_create: w_lm is required");
  const void *ptrs[] = {d.embed, d.w_qkv, d.w_o, d.norm_attn, d.norm_final, d.w_lm};
  for (const void *p : ptrs)
    if (p && !aligned16(p)) return fail(RIL_EINVAL, "model_create: weight pointer not 16-byte aligned");

  ril_model *m = new ril_model();
  m->d = d;
  m->G = G;
  m->n_vt = (d.vocab + 255) / 256;
  m->max_splits = ssd ? 1 : (d.max_ctx + d.split_tokens - 1) / d.split_tokens;
  m->cscale = (float)((double)d.softmax_scale * 1.4426950408889634);
  m->kv_fp8 = d.kv_dtype == RIL_KV_FP8_E4M3;
  m->k_scale = std::ldexp(1.0f, d.k_scale_exp);
  m->v_scale = std::ldexp(1.0f, d.v_scale_exp);
  m->mla = mla;
  m->sparse = sparse;
  if (sparse)  // split count of the selection, not of the context
    m->max_splits = (std::min(d.max_ctx, d.topk) + d.split_tokens - 1) / d.split_tokens;
  const size_t kv_elem = d.kv_dtype == RIL_KV_FP8_E4M3 ? 1 : 2;  // bytes per cached value
  m->page_bytes = mla ? (size_t)16 * (d.head_dim + d.rope_dim) * kv_elem + (sparse ? (size_t)16 * d.index_dim * 4 : 0)
                      : (size_t)d.n_kv_heads * 2 * 16 * d.head_dim * kv_elem;
  m->ssd = ssd;
  if (ssd) m->page_bytes = (size_t)ril::ssd_slot_bytes(d.n_q_heads, d.n_kv_heads);
  const size_t R = (size_t)std::max(d.max_rows, d.max_tokens);
  const bool tok = d.input_mode == RIL_INPUT_TOKENS;
  size_t o = 0;
  auto seg = [&](size_t bytes) { size_t at = o; o += round256(bytes); return at; };
  m->off_x = seg(tok ? R * d.d_model * 2 : 0);
  m->off_h = seg(tok ? R * d.d_model * 2 : 0);
  m->off_qkv = seg(tok ? R * (size_t)(d.n_q_heads + 2 * d.n_kv_heads) * d.head_dim * 2 : 0);
  m->off_attn = seg(R * qw * 2);
  m->off_y = seg(d.w_o ? R * d.d_head * 2 : 0);
  m->off_z = seg(R * d.d_head * 2);
  if (d.d_ff) {
    m->off_gu = seg(R * 2 * (size_t)d.d_ff * 2);
    m->off_act = seg(R * (size_t)d.d_ff * 2);
    m->off_y2 = seg(R * (size_t)d.d_model * 2);
  }
  m->lm_fp8 = d.lm_dtype == RIL_LM_W8A8_FP8;
  if (m->lm_fp8) {
    m->off_a8 = seg(R * d.d_head);
    m->off_ea = seg(R * (size_t)(d.d_head / 128) * sizeof(int32_t));
  }
  m->proj_fp8 = d.proj_dtype == RIL_PROJ_W8A8_FP8;
  if (m->proj_fp8) {
    size_t kmax = d.w_o ? (size_t)qw : 0;
    if (tok) kmax = std::max(kmax, (size_t)d.d_model);
    if (d.d_ff) kmax = std::max(kmax, (size_t)d.d_ff);
    m->off_p8 = seg(R * kmax);
    m->off_pe = seg(R * (kmax / 128) * sizeof(int32_t));
  }
  m->off_vpart = seg(R * m->n_vt * 2 * sizeof(float));
  m->off_tgt = seg(R * sizeof(float));
  m->off_po = seg((size_t)d.max_rows * d.n_q_heads * m->max_splits * d.head_dim * sizeof(float));
  m->off_pml = seg((size_t)d.max_rows * d.n_q_heads * m->max_splits * 2 * sizeof(float));
  m->off_scores = seg(sparse ? (size_t)d.max_rows * d.max_ctx * sizeof(float) : 0);
  m->off_sel = seg(sparse ? (size_t)d.max_rows * d.topk * sizeof(int32_t) : 0);
  if (ssd) {
    // a call completes at most one chunk per sequence beyond its whole chunks of tokens
    m->ssd_max_done = d.max_rows + R / kSsdQ;
    const size_t st = (size_t)d.n_q_heads * kSsdP * kSsdN * sizeof(float);
    m->off_ssd_plan = seg((6 * (size_t)d.max_rows + 2) * sizeof(int32_t));
    m->off_ssd_ds = seg((size_t)m->ssd_max_done * st);
    m->off_ssd_ent = seg((size_t)m->ssd_max_done * st);
    m->off_ssd_dec = seg((size_t)m->ssd_max_done * d.n_q_heads * sizeof(float));
  }
  m->ws_base = m->ws_total = o;
  *out = m;
  return RIL_OK;
}

extern "C" void ril_model_destroy(ril_model *m) { delete m; }

static bf16_t *wsb(void *ws, size_t off) { return reinterpret_cast<bf16_t *>(static_cast<char *>(ws) + off); }
static float *wsf(void *ws, size_t off) { return reinterpret_cast<float *>(static_cast<char *>(ws) + off); }

// Comparator: the widest projection output, for the split-K partial buffer.
static int widest_gemm_n(const ril_model_desc &d) {
  int n = d.w_o ? d.d_head : 0;
  if (d.input_mode == RIL_INPUT_TOKENS) n = std::max(n, (d.n_q_heads + 2 * d.n_kv_heads) * d.head_dim);
  return n;
}
static constexpr int kMaxSplitK = 16;

extern "C" ril_status ril_set_policy(ril_model *m, int32_t policy, int32_t attn_split_tokens) {
  if (!m) return fail(RIL_EINVAL, "set_policy: null model");
  if (policy != RIL_POLICY_INVARIANT && policy != RIL_POLICY_SHAPE_DERIVED)
    return fail(RIL_EINVAL, "set_policy: policy %d", policy);
  const int max_split = m->mla ? 2048 : 1024;
  if (attn_split_tokens != 0 && (attn_split_tokens % 64 || attn_split_tokens < 64 || attn_split_tokens > max_split))
    return fail(RIL_EINVAL, "set_policy: attn_split_tokens %d (0, or a multiple of 64 in [64, %d])",
                attn_split_tokens, max_split);
  if (policy == RIL_POLICY_SHAPE_DERIVED && m->n_cu == 0) {
    int dev = 0, cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu < 1)
      return fail(RIL_EHIP, "set_policy: cannot read the device's compute-unit count");
    m->n_cu = cu;
  }
  m->policy = policy;
  m->attn_split_override = attn_split_tokens;
  m->ws_total = m->ws_base;
  m->off_gpart = 0;
  if (policy == RIL_POLICY_SHAPE_DERIVED) {
    const size_t R = (size_t)std::max(m->d.max_rows, m->d.max_tokens);
    m->off_gpart = m->ws_base;
    m->ws_total = m->ws_base + round256((size_t)kMaxSplitK * R * widest_gemm_n(m->d) * sizeof(float));
  }
  return RIL_OK;
}

// Comparator: the KV split a throughput-first engine would choose for this batch (two
// waves per SIMD of work items), or the caller's override; widened until the partials
// fit the invariant path's buffer.  `bound` is the longest context (or selection).
static int shape_split(const ril_model *m, int rows, int bound) {
  const ril_model_desc &d = m->d;
  const int max_split = m->mla ? 2048 : 1024;
  int split = m->attn_split_override;
  if (split == 0) {
    const long want = 2L * 4 * m->n_cu;
    const long items = (long)rows * (m->mla ? d.n_q_heads / 64 : d.n_kv_heads);
    const long per = std::max(1L, (want + items - 1) / items);
    split = (int)(((bound + per - 1) / per + 63) / 64 * 64);
  }
  split = std::min(std::max(split, 64), max_split);
  const long cap = (long)d.max_rows * m->max_splits;
  while ((long)rows * ((bound + split - 1) / split) > cap && split < max_split) split = std::min(2 * split, max_split);
  return split;
}

// Comparator split-K for a projection of M x N: chunks when the tile grid is smaller
// than the machine, at least 256 K per chunk.
static void shape_split_k(const ril_model *m, GemmArgs &g, void *ws) {
  if (m->policy != RIL_POLICY_SHAPE_DERIVED) return;
  const int tiles = gemm_tiles(g.M, g.N);
  if (tiles >= m->n_cu) return;
  int sk = std::min(kMaxSplitK, (2 * m->n_cu + tiles - 1) / tiles);
  sk = std::min(sk, g.K / 256);
  if (sk < 2) return;
  g.split_k = sk;
  g.part = wsf(ws, m->off_gpart);
}
extern "C" size_t ril_workspace_bytes(const ril_model *m) { return m ? m->ws_total : 0; }
extern "C" size_t ril_kv_page_bytes(const ril_model *m) { return m ? m->page_bytes : 0; }

extern "C" size_t ril_lm_head_packed_bytes(int32_t vocab, int32_t d_head) {
  if (vocab < 1 || d_head < 32 || d_head % 32 != 0) return 0;
  return (size_t)ril::lm_head_packed_elems(vocab, d_head) * sizeof(uint16_t);
}

extern "C" ril_status ril_pack_lm_head(const void *src, int32_t vocab, int32_t d_head, void *dst,
                                       size_t packed_bytes, void *stream) {
  const size_t need = ril_lm_head_packed_bytes(vocab, d_head);
  if (need == 0) return fail(RIL_EINVAL, "pack_lm_head: vocab must be >= 1 and d_head a positive multiple of 32");
  if (!src || !dst) return fail(RIL_EINVAL, "pack_lm_head: src and dst are required");
  if (((uintptr_t)src | (uintptr_t)dst) % 16) return fail(RIL_EINVAL, "pack_lm_head: pointers must be 16-byte aligned");
  if (packed_bytes < need) return fail(RIL_EINVAL, "pack_lm_head: dst is smaller than ril_lm_head_packed_bytes");
  const uintptr_t s0 = (uintptr_t)src, s1 = s0 + (size_t)vocab * d_head * 2, d0 = (uintptr_t)dst, d1 = d0 + need;
  if (s0 < d1 && d0 < s1) return fail(RIL_EINVAL, "pack_lm_head: src and dst overlap");
  const hipError_t e = ril::launch_pack_lm_head((const bf16_t *)src, vocab, d_head, (bf16_t *)dst,
                                                (hipStream_t)stream);
  if (e != hipSuccess) return fail(RIL_EHIP, "pack_lm_head: %s", hipGetErrorString(e));
  return RIL_OK;
}
extern "C" size_t ril_lm_head_fp8_packed_bytes(int32_t vocab, int32_t d_head) {
  if (vocab < 1 || d_head < 128 || d_head % 128 != 0) return 0;
  return (size_t)ril::lm_head_fp8_code_bytes(vocab, d_head) +
         (size_t)ril::lm_head_fp8_exp_count(vocab, d_head) * sizeof(int32_t);
}

extern "C" ril_status ril_pack_lm_head_fp8(const void *src, int32_t vocab, int32_t d_head, void *dst,
                                           size_t packed_bytes, void *stream) {
  const size_t need = ril_lm_head_fp8_packed_bytes(vocab, d_head);
  if (need == 0) return fail(RIL_EINVAL, "pack_lm_head_fp8: vocab must be >= 1 and d_head a positive multiple of 128");
  if (!src || !dst) return fail(RIL_EINVAL, "pack_lm_head_fp8: src and dst are required");
  if (((uintptr_t)src | (uintptr_t)dst) % 16) return fail(RIL_EINVAL, "pack_lm_head_fp8: pointers must be 16-byte aligned");
  if (packed_bytes < need) return fail(RIL_EINVAL, "pack_lm_head_fp8: dst is smaller than ril_lm_head_fp8_packed_bytes");
  const uintptr_t s0 = (uintptr_t)src, s1 = s0 + (size_t)vocab * d_head * 2, d0 = (uintptr_t)dst, d1 = d0 + need;
  if (s0 < d1 && d0 < s1) return fail(RIL_EINVAL, "pack_lm_head_fp8: src and dst overlap");
  uint8_t *codes = static_cast<uint8_t *>(dst);
  int32_t *ew = reinterpret_cast<int32_t *>(codes + ril::lm_head_fp8_code_bytes(vocab, d_head));
  const hipError_t e = ril::launch_pack_lm_head_fp8((const bf16_t *)src, vocab, d_head, codes, ew, (hipStream_t)stream);
  if (e != hipSuccess) return fail(RIL_EHIP, "pack_lm_head_fp8: %s", hipGetErrorString(e));
  return RIL_OK;
}
extern "C" ril_status ril_quantize_rows_fp8(const void *src, int32_t rows, int32_t K, int32_t ld, void *codes,
                                            void *exps, void *stream) {
  if (rows < 0 || K < 128 || K % 128 || ld < K || ld % 8)
    return fail(RIL_EINVAL, "quantize_rows_fp8: rows %d, K %d, ld %d", rows, K, ld);
  if (rows == 0) return RIL_OK;
  if (!src || !codes || !exps || !aligned16(src) || !aligned16(codes) || !aligned4(exps))
    return fail(RIL_EINVAL, "quantize_rows_fp8: null or misaligned pointer");
  QuantRowsArgs q{(const bf16_t *)src, ld, rows, K, static_cast<uint8_t *>(codes), static_cast<int32_t *>(exps)};
  const hipError_t e = launch_quant_rows_fp8(q, (hipStream_t)stream);
  if (e != hipSuccess) return fail(RIL_EHIP, "quantize_rows_fp8: %s", hipGetErrorString(e));
  return RIL_OK;
}
extern "C" size_t ril_proj_fp8_bytes(int32_t N, int32_t K) { return (size_t)ril::proj_fp8_bytes(N, K); }

extern "C" ril_status ril_quantize_weight_fp8(const void *src, int32_t N, int32_t K, void *dst, size_t dst_bytes,
                                              void *stream) {
  const size_t need = (size_t)ril::proj_fp8_bytes(N, K);
  if (need == 0) return fail(RIL_EINVAL, "quantize_weight_fp8: N %d, K %d (K a positive multiple of 128)", N, K);
  if (!src || !dst || !aligned16(src) || !aligned16(dst))
    return fail(RIL_EINVAL, "quantize_weight_fp8: null or misaligned pointer");
  if (dst_bytes < need) return fail(RIL_EINVAL, "quantize_weight_fp8: dst %zu bytes, %zu needed", dst_bytes, need);
  const uintptr_t s0 = (uintptr_t)src, s1 = s0 + (size_t)N * K * 2, d0 = (uintptr_t)dst, d1 = d0 + need;
  if (s0 < d1 && d0 < s1) return fail(RIL_EINVAL, "quantize_weight_fp8: src and dst overlap");
  uint8_t *codes = static_cast<uint8_t *>(dst);
  int32_t *ew = reinterpret_cast<int32_t *>(codes + (size_t)N * K);
  const hipError_t e = ril::launch_quant_weight_fp8((const bf16_t *)src, N, K, codes, ew, (hipStream_t)stream);
  if (e != hipSuccess) return fail(RIL_EHIP, "quantize_weight_fp8: %s", hipGetErrorString(e));
  return RIL_OK;
}

extern "C" ril_status ril_proj_w8a8(const void *codes, const void *exps, int32_t rows, int32_t K, const void *w,
                                    size_t w_bytes, int32_t N, void *out, int32_t ldo, void *stream) {
  if (rows < 0 || N < 1 || K < 128 || K % 128 || ldo < N)
    return fail(RIL_EINVAL, "proj_w8a8: rows %d, K %d, N %d, ldo %d", rows, K, N, ldo);
  const size_t need = (size_t)ril::proj_fp8_bytes(N, K);
  if (w_bytes < need) return fail(RIL_EINVAL, "proj_w8a8: weight %zu bytes, %zu needed for N %d, K %d", w_bytes,
                                  need, N, K);
  if (rows == 0) return RIL_OK;
  if (!codes || !exps || !w || !out || !aligned16(codes) || !aligned4(exps) || !aligned16(w) ||
      ((uintptr_t)out & 1))
    return fail(RIL_EINVAL, "proj_w8a8: null or misaligned pointer");
  const uint8_t *w8 = static_cast<const uint8_t *>(w);
  GemmFp8Args f{static_cast<const uint8_t *>(codes), static_cast<const int32_t *>(exps), w8,
                reinterpret_cast<const int32_t *>(w8 + (size_t)N * K), static_cast<bf16_t *>(out), ldo, nullptr, 0,
                rows, N, K};
  const hipError_t e = ril::launch_gemm_fp8(f, (hipStream_t)stream);
  if (e != hipSuccess) return fail(RIL_EHIP, "proj_w8a8: %s", hipGetErrorString(e));
  return RIL_OK;
}

extern "C" ril_status ril_proj_bf16(const void *A, int32_t rows, int32_t K, int32_t lda, const void *W, int32_t N,
                                    int32_t ldw, const void *residual, int32_t ldr, void *out, int32_t ldo,
                                    void *stream) {
  if (rows < 0 || N < 1 || K < 32 || K % 32 || lda < K || lda % 8 || ldw < K || ldw % 8 || ldo < N ||
      (residual && ldr < N))
    return fail(RIL_EINVAL, "proj_bf16: rows %d, K %d, N %d, lda %d, ldw %d, ldr %d, ldo %d", rows, K, N, lda, ldw,
                ldr, ldo);
  // the kernels form 32-bit element offsets inside a 256-row (256-column) tile
  if ((long)lda * 256 + K >= (1L << 31) || (long)ldw * 256 + K >= (1L << 31))
    return fail(RIL_EINVAL, "proj_bf16: row strides %d / %d too large", lda, ldw);
  if (rows == 0) return RIL_OK;
  if (!A || !W || !out || !aligned16(A) || !aligned16(W) || ((uintptr_t)out & 1) || ((uintptr_t)residual & 1))
    return fail(RIL_EINVAL, "proj_bf16: null or misaligned pointer");
  GemmArgs g{(const bf16_t *)A, lda, (const bf16_t *)W, ldw, (bf16_t *)out, ldo, (const bf16_t *)residual, ldr,
             rows, N, K};
  const hipError_t e = ril::launch_gemm(g, (hipStream_t)stream);
  if (e != hipSuccess) return fail(RIL_EHIP, "proj_bf16: %s", hipGetErrorString(e));
  return RIL_OK;
}

extern "C" int32_t ril_hbm_read_probe_words(void) { return ril::hbm_read_probe_blocks(); }

extern "C" ril_status ril_hbm_read_probe(const void *src, size_t bytes, uint32_t *out, void *stream) {
  if (!src || !out || !aligned16(src) || !aligned4(out)) return fail(RIL_EINVAL, "hbm_read_probe: null or misaligned pointer");
  const hipError_t e = ril::launch_hbm_read_probe(src, bytes, out, (hipStream_t)stream);
  if (e != hipSuccess) return fail(RIL_EHIP, "hbm_read_probe: %s", hipGetErrorString(e));
  return RIL_OK;
}
extern "C" size_t ril_ws_attn_offset(const ril_model *m) { return m ? m->off_attn : 0; }

// ---------------------------------------------------------------------------
// S1: page allocator
// ---------------------------------------------------------------------------

static uint64_t splitmix64(uint64_t &s) {
  uint64_t z = (s += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

extern "C" ril_status ril_kv_alloc(const ril_model *m, void *pool_dev, size_t pool_bytes,
                                   uint64_t shuffle_seed, ril_kv **out) {
  if (!m || !pool_dev || !out) return fail(RIL_EINVAL, "kv_alloc: null argument");
  if (!aligned16(pool_dev)) return fail(RIL_EINVAL, "kv_alloc: pool not 16-byte aligned");
  const size_t n = pool_bytes / m->page_bytes;
  if (n < 1) return fail(RIL_ENOSPC, "kv_alloc: pool smaller than one page (%zu bytes)", m->page_bytes);
  if (n > (size_t)INT32_MAX) return fail(RIL_ERANGE, "kv_alloc: too many pages");
  ril_kv *kv = new ril_kv();
  kv->page_bytes = m->page_bytes;
  kv->pool = pool_dev;
  kv->n_pages = (int32_t)n;
  kv->free_list.resize(n);
  // pop_back hands out ids in free_list order reversed; store so that 0 comes first
  for (size_t i = 0; i < n; ++i) kv->free_list[i] = (int32_t)(n - 1 - i);
  if (shuffle_seed) {
    uint64_t s = shuffle_seed;
    for (size_t i = n - 1; i > 0; --i) {
      const size_t j = (size_t)(splitmix64(s) % (uint64_t)(i + 1));
      std::swap(kv->free_list[i], kv->free_list[j]);
    }
  }
  kv->assigned.assign(n, 0);
  *out = kv;
  return RIL_OK;
}

extern "C" ril_status ril_kv_assign(ril_kv *kv, int32_t n_pages, int32_t *page_ids_out) {
  if (!kv || n_pages < 0 || (n_pages > 0 && !page_ids_out)) return fail(RIL_EINVAL, "kv_assign: bad argument");
  if ((size_t)n_pages > kv->free_list.size())
    return fail(RIL_ENOSPC, "kv_assign: %d pages asked, %zu free", n_pages, kv->free_list.size());
  for (int32_t i = 0; i < n_pages; ++i) {
    const int32_t id = kv->free_list.back();
    kv->free_list.pop_back();
    kv->assigned[id] = 1;
    page_ids_out[i] = id;
  }
  return RIL_OK;
}

extern "C" ril_status ril_kv_release(ril_kv *kv, int32_t n_pages, const int32_t *ids) {
  if (!kv || n_pages < 0 || (n_pages > 0 && !ids)) return fail(RIL_EINVAL, "kv_release: bad argument");
  std::vector<uint8_t> seen;
  for (int32_t i = 0; i < n_pages; ++i) {
    const int32_t id = ids[i];
    if (id < 0 || id >= kv->n_pages || !kv->assigned[id])
      return fail(RIL_EINVAL, "kv_release: page %d is not assigned", id);
    if (seen.empty()) seen.assign(kv->n_pages, 0);
    if (seen[id]) return fail(RIL_EINVAL, "kv_release: page %d listed twice", id);
    seen[id] = 1;
  }
  for (int32_t i = 0; i < n_pages; ++i) {
    kv->assigned[ids[i]] = 0;
    kv->free_list.push_back(ids[i]);
  }
  return RIL_OK;
}

extern "C" int32_t ril_kv_free_pages(const ril_kv *kv) { return kv ? (int32_t)kv->free_list.size() : 0; }
extern "C" int32_t ril_kv_total_pages(const ril_kv *kv) { return kv ? kv->n_pages : 0; }
extern "C" void ril_kv_free(ril_kv *kv) { delete kv; }

// ---------------------------------------------------------------------------
// forward passes
// ---------------------------------------------------------------------------


// ---------------------------------------------------------------------------
// kernel trace: hipEvent pairs recorded around launches while enabled
// ---------------------------------------------------------------------------

namespace {
struct TraceRec {
  int k;
  hipEvent_t a, b;
};
std::mutex g_tr_mu;
bool g_tr_on = false;
std::vector<TraceRec> g_tr_pending;
std::vector<hipEvent_t> g_tr_pool;
double g_tr_ms[RIL_K_COUNT];
int64_t g_tr_n[RIL_K_COUNT];

hipEvent_t trace_event() {
  if (!g_tr_pool.empty()) {
    hipEvent_t e = g_tr_pool.back();
    g_tr_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

void trace_drain() {  // caller holds g_tr_mu
  for (const TraceRec &r : g_tr_pending) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) == hipSuccess && hipEventElapsedTime(&ms, r.a, r.b) == hipSuccess) {
      g_tr_ms[r.k] += ms;
      g_tr_n[r.k] += 1;
    }
    g_tr_pool.push_back(r.a);
    g_tr_pool.push_back(r.b);
  }
  g_tr_pending.clear();
}

// Launch `fn` and, while tracing, bracket it with events on `st`.
// Set while this thread records a graph: launches are captured, never bracketed.
thread_local bool g_capturing = false;

template <typename F>
hipError_t traced(int k, hipStream_t st, F fn) {
  if (!g_tr_on || g_capturing) return fn();
  std::lock_guard<std::mutex> lk(g_tr_mu);
  hipEvent_t a = trace_event(), b = trace_event();
  const bool ra = a && hipEventRecord(a, st) == hipSuccess;
  hipError_t e = fn();
  const bool rb = b && hipEventRecord(b, st) == hipSuccess;
  if (ra && rb) {
    g_tr_pending.push_back({k, a, b});
  } else {
    if (a) g_tr_pool.push_back(a);
    if (b) g_tr_pool.push_back(b);
  }
  return e;
}
}  // namespace

extern "C" ril_status ril_trace_enable(int on) {
  std::lock_guard<std::mutex> lk(g_tr_mu);
  trace_drain();
  for (int k = 0; k < RIL_K_COUNT; ++k) {
    g_tr_ms[k] = 0.0;
    g_tr_n[k] = 0;
  }
  g_tr_on = on != 0;
  return RIL_OK;
}

extern "C" ril_status ril_trace_read(int kernel, double *total_ms, int64_t *launches) {
  if (kernel < 0 || kernel >= RIL_K_COUNT || !total_ms || !launches)
    return fail(RIL_EINVAL, "trace_read: bad argument");
  std::lock_guard<std::mutex> lk(g_tr_mu);
  trace_drain();
  *total_ms = g_tr_ms[kernel];
  *launches = g_tr_n[kernel];
  return RIL_OK;
}

#define RIL_LAUNCH(kid, expr)                                                                 \
  do {                                                                                        \
    hipError_t e_ = traced((kid), st, [&]() { return (expr); });                              \
    if (e_ != hipSuccess) return fail(RIL_EHIP, "%s: %s", #expr, hipGetErrorString(e_));      \
  } while (0)

static ril_status check_common(const ril_model *m, ril_kv *kv, void *ws, size_t ws_bytes,
                               int ctx_bound, const void *page_table, int page_stride, const char *who) {
  if (!m || !kv) return fail(RIL_EINVAL, "%s: null model or kv", who);
  if (kv->page_bytes != m->page_bytes) return fail(RIL_EINVAL, "%s: kv pool made for another page size", who);
  if (!ws || !aligned16(ws)) return fail(RIL_EINVAL, "%s: workspace null or misaligned", who);
  if (ws_bytes < m->ws_total)
    return fail(RIL_ERANGE, "%s: workspace %zu bytes, %zu needed", who, ws_bytes, m->ws_total);
  if (ctx_bound < 1 || ctx_bound > m->d.max_ctx)
    return fail(RIL_ERANGE, "%s: max_ctx_bound %d outside [1, %d]", who, ctx_bound, m->d.max_ctx);
  if (!page_table || !aligned4(page_table)) return fail(RIL_EINVAL, "%s: page_table", who);
  if (m->ssd) {  // one cache slot per sequence, in column 0
    if (page_stride < 1) return fail(RIL_EINVAL, "%s: page_stride %d < 1", who, page_stride);
    return RIL_OK;
  }
  if (page_stride < (ctx_bound + 15) / 16)
    return fail(RIL_EINVAL, "%s: page_stride %d < %d pages", who, page_stride, (ctx_bound + 15) / 16);
  return RIL_OK;
}

static ril_status run_lm_head(const ril_model *m, int rows, const bf16_t *z, int ldz, const int32_t *targets,
                              float *out, void *ws, hipStream_t st);

// One projection C = bf16(A W^T) [+ residual]: the bf16 GEMM (with the comparator's
// shape-derived split-K under that policy), or with W8A8 projections the rows' block-FP8
// quantization and the W8A8 GEMM (no comparator form: its K order is always 0, 128, ...).
static ril_status run_proj(const ril_model *m, GemmArgs g, void *ws, hipStream_t st) {
  if (m->proj_fp8) {
    uint8_t *a8 = reinterpret_cast<uint8_t *>(ws) + m->off_p8;
    int32_t *ea = reinterpret_cast<int32_t *>(static_cast<char *>(ws) + m->off_pe);
    QuantRowsArgs q{g.A, g.lda, g.M, g.K, a8, ea};
    RIL_LAUNCH(RIL_K_QUANT_ROWS, launch_quant_rows_fp8(q, st));
    const uint8_t *w8 = reinterpret_cast<const uint8_t *>(g.W);
    GemmFp8Args f{a8, ea, w8, reinterpret_cast<const int32_t *>(w8 + (size_t)g.N * g.K), g.C, g.ldc, g.R, g.ldr,
                  g.M, g.N, g.K};
    RIL_LAUNCH(RIL_K_GEMM_FP8, launch_gemm_fp8(f, st));
    return RIL_OK;
  }
  shape_split_k(m, g, ws);
  RIL_LAUNCH(RIL_K_GEMM, launch_gemm(g, st));
  return RIL_OK;
}

// Attention output (in the workspace) -> [O GEMM (+ residual)] -> RMSNorm -> lm-head.
static ril_status run_head(const ril_model *m, int rows, const int32_t *targets, float *out, void *ws,
                           hipStream_t st) {
  const ril_model_desc &d = *&m->d;
  const int qw = d.n_q_heads * d.head_dim;
  const bf16_t *src = wsb(ws, m->off_attn);
  int ld = qw;
  if (d.w_o) {
    const bool tok = d.input_mode == RIL_INPUT_TOKENS;
    GemmArgs g{src, qw, (const bf16_t *)d.w_o, qw, wsb(ws, m->off_y), d.d_head,
               tok ? wsb(ws, m->off_x) : nullptr, d.d_model, rows, d.d_head, qw};
    const ril_status s = run_proj(m, g, ws, st);
    if (s != RIL_OK) return s;
    src = wsb(ws, m->off_y);
    ld = d.d_head;
  }
  if (d.d_ff) {  // the SwiGLU block (TOKENS only: d_head = d_model)
    const int F = d.d_ff;
    RmsNormArgs rn{src, ld, nullptr, nullptr, d.vocab, d.d_model, (const bf16_t *)d.norm_mlp, d.rms_eps,
                   wsb(ws, m->off_h), d.d_model, nullptr, 0, rows};
    RIL_LAUNCH(RIL_K_RMSNORM, launch_rmsnorm(rn, st));
    GemmArgs g1{wsb(ws, m->off_h), d.d_model, (const bf16_t *)d.w_gate_up, d.d_model, wsb(ws, m->off_gu), 2 * F,
                nullptr, 0, rows, 2 * F, d.d_model};
    ril_status s = run_proj(m, g1, ws, st);
    if (s != RIL_OK) return s;
    SiluMulArgs sm{wsb(ws, m->off_gu), 2 * F, wsb(ws, m->off_act), F, rows, F};
    RIL_LAUNCH(RIL_K_SILU_MUL, launch_silu_mul(sm, st));
    GemmArgs g2{wsb(ws, m->off_act), F, (const bf16_t *)d.w_down, F, wsb(ws, m->off_y2), d.d_model,
                src, ld, rows, d.d_model, F};
    s = run_proj(m, g2, ws, st);
    if (s != RIL_OK) return s;
    src = wsb(ws, m->off_y2);
    ld = d.d_model;
  }
  RmsNormArgs r{src, ld, nullptr, nullptr, d.vocab, d.d_head, (const bf16_t *)d.norm_final, d.rms_eps,
                wsb(ws, m->off_z), d.d_head, nullptr, 0, rows};
  RIL_LAUNCH(RIL_K_RMSNORM, launch_rmsnorm(r, st));
  return run_lm_head(m, rows, wsb(ws, m->off_z), d.d_head, targets, out, ws, st);
}

// Normalised rows z -> lm-head (bf16 or W8A8) -> vocabulary merge -> logprobs.
static ril_status run_lm_head(const ril_model *m, int rows, const bf16_t *z, int ldz, const int32_t *targets,
                              float *out, void *ws, hipStream_t st) {
  const ril_model_desc &d = m->d;
  LmHeadArgs lh{z, ldz, (const bf16_t *)d.w_lm, d.d_head, d.vocab, targets, rows,
                wsf(ws, m->off_vpart), wsf(ws, m->off_tgt), out};
  if (m->lm_fp8) {
    uint8_t *a8 = reinterpret_cast<uint8_t *>(ws) + m->off_a8;
    int32_t *ea = reinterpret_cast<int32_t *>(static_cast<char *>(ws) + m->off_ea);
    QuantRowsArgs q{z, ldz, rows, d.d_head, a8, ea};
    RIL_LAUNCH(RIL_K_QUANT_ROWS, launch_quant_rows_fp8(q, st));
    lh.A8 = a8;
    lh.ea = ea;
    lh.W8 = static_cast<const uint8_t *>(d.w_lm);
    lh.ew = reinterpret_cast<const int32_t *>(lh.W8 + ril::lm_head_fp8_code_bytes(d.vocab, d.d_head));
    RIL_LAUNCH(RIL_K_LM_HEAD_FP8, launch_lm_head_fp8(lh, st));
  } else {
    RIL_LAUNCH(RIL_K_LM_HEAD, launch_lm_head(lh, st));
  }
  RIL_LAUNCH(RIL_K_VOCAB_MERGE, launch_vocab_merge(lh, st));
  return RIL_OK;
}

// TOKENS mode front: embedding + RMSNorm + QKV projection into the workspace.
static ril_status run_token_front(const ril_model *m, int rows, const int32_t *tok, void *ws, hipStream_t st) {
  const ril_model_desc &d = m->d;
  const int wqkv = (d.n_q_heads + 2 * d.n_kv_heads) * d.head_dim;
  RmsNormArgs r{nullptr, 0, tok, (const bf16_t *)d.embed, d.vocab, d.d_model, (const bf16_t *)d.norm_attn,
                d.rms_eps, wsb(ws, m->off_h), d.d_model, wsb(ws, m->off_x), d.d_model, rows};
  RIL_LAUNCH(RIL_K_RMSNORM, launch_rmsnorm(r, st));
  GemmArgs g{wsb(ws, m->off_h), d.d_model, (const bf16_t *)d.w_qkv, d.d_model, wsb(ws, m->off_qkv), wqkv,
             nullptr, 0, rows, wqkv, d.d_model};
  return run_proj(m, g, ws, st);
}

static ril_status check_prefill(const ril_model *m, ril_kv *kv, const ril_prefill_batch *b, void *ws,
                                size_t ws_bytes, bool need_logprob, const char *who) {
  if (!b) return fail(RIL_EINVAL, "%s: null batch", who);
  ril_status s = check_common(m, kv, ws, need_logprob ? ws_bytes : m->ws_total, b->max_ctx_bound,
                              b->page_table, b->page_stride, who);
  if (s != RIL_OK) return s;
  // The history writer uses no workspace, so only the logprob calls are held to max_tokens.
  const int lim = need_logprob ? m->d.max_tokens : INT32_MAX;
  if (b->n_seqs < 1 || b->n_seqs > lim)
    return fail(RIL_ERANGE, "%s: n_seqs %d outside [1, %d]", who, b->n_seqs, lim);
  if (b->total_tokens < 1 || b->total_tokens > lim)
    return fail(RIL_ERANGE, "%s: total_tokens %d outside [1, %d]", who, b->total_tokens, lim);
  if (!b->cu_tokens || !b->start_pos || !aligned4(b->cu_tokens) || !aligned4(b->start_pos))
    return fail(RIL_EINVAL, "%s: cu_tokens/start_pos", who);
  const bool tok = m->d.input_mode == RIL_INPUT_TOKENS;
  if (need_logprob) {
    if (!b->target_ids || !aligned4(b->target_ids)) return fail(RIL_EINVAL, "%s: target_ids", who);
    if (tok && (!b->token_ids || !aligned4(b->token_ids))) return fail(RIL_EINVAL, "%s: token_ids", who);
    if (!tok && (!b->q || !aligned16(b->q))) return fail(RIL_EINVAL, "%s: q", who);
  }
  const bool need_v = !m->mla;
  if ((!tok || !need_logprob) && (!b->k || !aligned16(b->k) || (need_v && (!b->v || !aligned16(b->v)))))
    return fail(RIL_EINVAL, "%s: k/v", who);
  if (m->ssd) {
    if (b->n_seqs > m->d.max_rows)
      return fail(RIL_ERANGE, "%s: n_seqs %d > max_rows %d (one cache slot per sequence)", who, b->n_seqs,
                  m->d.max_rows);
    if (!b->dt || !aligned16(b->dt)) return fail(RIL_EINVAL, "%s: dt", who);
  }
  if (m->sparse) {
    if (!b->k_index || !aligned16(b->k_index)) return fail(RIL_EINVAL, "%s: k_index", who);
    if (need_logprob && (!b->q_index || !aligned16(b->q_index))) return fail(RIL_EINVAL, "%s: q_index", who);
    if (b->selected_out && !aligned4(b->selected_out)) return fail(RIL_EINVAL, "%s: selected_out", who);
  }
  return RIL_OK;
}

// The shared latent (and indexer key) write of both MLA kinds.
static ril_status run_mla_write(const ril_model *m, ril_kv *kv, const bf16_t *c, const float *kidx, int n_tok,
                                int mode, const int32_t *cu, const int32_t *start_pos, int n_seqs,
                                const int32_t *ctx_len, const int32_t *page_table, int page_stride, hipStream_t st) {
  const ril_model_desc &d = m->d;
  MlaKvWriteArgs a{c, d.head_dim + d.rope_dim, m->sparse ? kidx : nullptr, n_tok, mode, cu, start_pos, n_seqs,
                   ctx_len, page_table, page_stride, (bf16_t *)kv->pool, (int)(m->page_bytes / 2), kv->n_pages,
                   m->kv_fp8, 1.0f / m->k_scale, m->sparse};
  RIL_LAUNCH(RIL_K_KV_WRITE, launch_mla_kv_write(a, st));
  return RIL_OK;
}

// MLA attention for `rows` rows (mode 0: decode rows; mode 1: packed prefill tokens),
// enqueued in groups of max_rows rows that reuse the workspace in stream order.  The
// sparse kind first scores every history position (S6) and selects the top-k (S7).
static ril_status run_mla(const ril_model *m, ril_kv *kv, const bf16_t *q, const float *q_index,
                          int32_t *sel_out, int mode, int rows, const int32_t *ctx_len, const int32_t *cu,
                          const int32_t *start_pos, int n_seqs, const int32_t *page_table, int page_stride,
                          int ctx_bound, void *ws, hipStream_t st) {
  const ril_model_desc &d = m->d;
  const int page_elems = (int)(m->page_bytes / 2);
  for (int r0 = 0; r0 < rows; r0 += d.max_rows) {
    const int n = std::min(d.max_rows, rows - r0);
    int32_t *sel = nullptr;
    if (m->sparse) {
      sel = reinterpret_cast<int32_t *>(static_cast<char *>(ws) + m->off_sel);
      IndexerArgs ia{q_index, mode, r0, n, ctx_len, cu, start_pos, n_seqs, page_table, page_stride,
                     (const bf16_t *)kv->pool, page_elems, kv->n_pages, ctx_bound,
                     16 * (d.head_dim + d.rope_dim) * (m->kv_fp8 ? 1 : 2) / 2, wsf(ws, m->off_scores),
                     d.max_ctx, d.topk, sel, sel_out};
      RIL_LAUNCH(RIL_K_INDEXER, launch_indexer(ia, st));
      RIL_LAUNCH(RIL_K_TOPK, launch_topk(ia, st));
    }
    int split = d.split_tokens, max_splits = m->max_splits;
    if (m->policy == RIL_POLICY_SHAPE_DERIVED && mode == 0) {
      const int bound = m->sparse ? std::min(ctx_bound, d.topk) : ctx_bound;
      split = shape_split(m, n, bound);
      max_splits = (bound + split - 1) / split;
    }
    MlaAttnArgs a{q, mode, r0, n, ctx_len, cu, start_pos, n_seqs, page_table, page_stride,
                  (const bf16_t *)kv->pool, page_elems, kv->n_pages, d.n_q_heads, split, ctx_bound,
                  max_splits, sel, d.topk, m->cscale, wsf(ws, m->off_po), wsf(ws, m->off_pml),
                  wsb(ws, m->off_attn), m->kv_fp8, m->k_scale};
    RIL_LAUNCH(RIL_K_ATTN_SPLIT, launch_mla_split(a, st));
    RIL_LAUNCH(RIL_K_ATTN_MERGE, launch_mla_merge(a, st));
  }
  return RIL_OK;
}

// The SSD mixer for one call (mode 0: packed prefill sequences; 1: decode rows): plan,
// the completed chunks' state sums, the state scan, the outputs (if asked), the slot
// commit and the unfinished chunk's inputs, in that order on the stream.
static ril_status run_ssd(const ril_model *m, ril_kv *kv, int mode, int n_seqs, int n_tok, const int32_t *cu,
                          const int32_t *start_pos, const int32_t *ctx_len, const int32_t *page_table,
                          int page_stride, const void *C, const void *B, const void *x, const float *dt, bool out,
                          void *ws, hipStream_t st) {
  const ril_model_desc &d = m->d;
  SsdArgs a{};
  a.mode = mode;
  a.n_seqs = n_seqs;
  a.n_tok = n_tok;
  a.cu = cu;
  a.start_pos = start_pos;
  a.ctx_len = ctx_len;
  a.page_table = page_table;
  a.page_stride = page_stride;
  a.pool = static_cast<uint8_t *>(kv->pool);
  a.slot_bytes = (long)m->page_bytes;
  a.n_slots = kv->n_pages;
  a.H = d.n_q_heads;
  a.G = d.n_kv_heads;
  a.x = (const bf16_t *)x;
  a.B = (const bf16_t *)B;
  a.C = (const bf16_t *)C;
  a.dt = dt;
  a.A = (const float *)d.ssm_A;
  a.D = (const float *)d.ssm_D;
  // a sequence touches at most ceil(len / Q) + 1 chunks and completes at most len / Q + 1
  a.max_chunks = std::min(n_tok, n_tok / kSsdQ + 2 * n_seqs);
  a.max_done = std::min(m->ssd_max_done, n_tok / kSsdQ + n_seqs);
  a.plan = reinterpret_cast<int32_t *>(static_cast<char *>(ws) + m->off_ssd_plan);
  a.dS = wsf(ws, m->off_ssd_ds);
  a.entry = wsf(ws, m->off_ssd_ent);
  a.dec = wsf(ws, m->off_ssd_dec);
  a.y = wsb(ws, m->off_attn);
  RIL_LAUNCH(RIL_K_SSD_CHUNK, launch_ssd_plan(a, st));
  RIL_LAUNCH(RIL_K_SSD_CHUNK, launch_ssd_state(a, st));
  RIL_LAUNCH(RIL_K_SSD_CHUNK, launch_ssd_scan(a, st));
  if (out) RIL_LAUNCH(RIL_K_SSD_OUT, launch_ssd_out(a, st));
  RIL_LAUNCH(RIL_K_SSD_CHUNK, launch_ssd_commit(a, st));
  RIL_LAUNCH(RIL_K_SSD_CHUNK, launch_ssd_write(a, st));
  return RIL_OK;
}

extern "C" ril_status ril_kv_write(const ril_model *m, ril_kv *kv, const ril_prefill_batch *b, void *stream) {
  if (!m) return fail(RIL_EINVAL, "kv_write: null model");
  // the history writer needs no workspace; pass a dummy aligned pointer through the checks
  static char dummy alignas(16)[16];
  if (m->ssd)
    return fail(RIL_EUNSUPPORTED, "kv_write: an SSD state depends on every position; lay history down with "
                "prefill calls");
  ril_status s = check_prefill(m, kv, b, dummy, 0, false, "kv_write");
  if (s != RIL_OK) return s;
  const ril_model_desc &d = m->d;
  hipStream_t st = (hipStream_t)stream;
  if (m->mla)
    return run_mla_write(m, kv, (const bf16_t *)b->k, b->k_index, b->total_tokens, 0, b->cu_tokens, b->start_pos,
                         b->n_seqs, nullptr, b->page_table, b->page_stride, st);
  KvWriteArgs a{(const bf16_t *)b->k, (const bf16_t *)b->v, d.n_kv_heads * d.head_dim, b->total_tokens, 0,
                b->cu_tokens, b->start_pos, b->n_seqs, nullptr, b->page_table, b->page_stride,
                (bf16_t *)kv->pool, kv->n_pages, d.n_kv_heads, d.head_dim, m->kv_fp8, m->k_scale, m->v_scale};
  RIL_LAUNCH(RIL_K_KV_WRITE, launch_kv_write(a, st));
  return RIL_OK;
}

extern "C" ril_status ril_prefill_logprobs(const ril_model *m, ril_kv *kv, const ril_prefill_batch *b,
                                           float *logprob_out, void *ws, size_t ws_bytes, void *stream) {
  ril_status s = check_prefill(m, kv, b, ws, ws_bytes, true, "prefill_logprobs");
  if (s != RIL_OK) return s;
  if (!logprob_out || !aligned4(logprob_out)) return fail(RIL_EINVAL, "prefill_logprobs: logprob_out");
  const ril_model_desc &d = m->d;
  hipStream_t st = (hipStream_t)stream;
  const int T = b->total_tokens;
  if (m->ssd) {
    s = run_ssd(m, kv, 0, b->n_seqs, T, b->cu_tokens, b->start_pos, nullptr, b->page_table, b->page_stride, b->q,
                b->k, b->v, b->dt, true, ws, st);
    if (s != RIL_OK) return s;
    return run_head(m, T, b->target_ids, logprob_out, ws, st);
  }
  if (m->mla) {
    s = run_mla_write(m, kv, (const bf16_t *)b->k, b->k_index, T, 0, b->cu_tokens, b->start_pos, b->n_seqs,
                      nullptr, b->page_table, b->page_stride, st);
    if (s != RIL_OK) return s;
    s = run_mla(m, kv, (const bf16_t *)b->q, b->q_index, b->selected_out, 1, T, nullptr, b->cu_tokens,
                b->start_pos, b->n_seqs, b->page_table, b->page_stride, b->max_ctx_bound, ws, st);
    if (s != RIL_OK) return s;
    return run_head(m, T, b->target_ids, logprob_out, ws, st);
  }
  const bool tok = d.input_mode == RIL_INPUT_TOKENS;
  const int wqkv = (d.n_q_heads + 2 * d.n_kv_heads) * d.head_dim;
  const bf16_t *q, *k, *v;
  int q_stride, kv_stride;
  if (tok) {
    s = run_token_front(m, T, b->token_ids, ws, st);
    if (s != RIL_OK) return s;
    q = wsb(ws, m->off_qkv);
    k = q + d.n_q_heads * d.head_dim;
    v = k + d.n_kv_heads * d.head_dim;
    q_stride = kv_stride = wqkv;
  } else {
    q = (const bf16_t *)b->q;
    k = (const bf16_t *)b->k;
    v = (const bf16_t *)b->v;
    q_stride = d.n_q_heads * d.head_dim;
    kv_stride = d.n_kv_heads * d.head_dim;
  }
  KvWriteArgs kw{k, v, kv_stride, T, 0, b->cu_tokens, b->start_pos, b->n_seqs, nullptr, b->page_table,
                 b->page_stride, (bf16_t *)kv->pool, kv->n_pages, d.n_kv_heads, d.head_dim,
                 m->kv_fp8, m->k_scale, m->v_scale};
  RIL_LAUNCH(RIL_K_KV_WRITE, launch_kv_write(kw, st));
  AttnPrefillArgs ap{q, q_stride, b->cu_tokens, b->start_pos, b->n_seqs, T, b->page_table, b->page_stride,
                     (const bf16_t *)kv->pool, kv->n_pages, d.n_kv_heads, m->G, d.head_dim, d.split_tokens,
                     b->max_ctx_bound, m->cscale, wsb(ws, m->off_attn), m->kv_fp8, m->k_scale, m->v_scale};
  RIL_LAUNCH(RIL_K_ATTN_PREFILL, launch_attn_prefill(ap, st));
  return run_head(m, T, b->target_ids, logprob_out, ws, st);
}

static ril_status decode_enqueue(const ril_model *m, ril_kv *kv, const ril_decode_batch *b,
                                 float *logprob_out, void *ws, size_t ws_bytes, void *stream) {
  if (!b) return fail(RIL_EINVAL, "decode_step_logprobs: null batch");
  ril_status s = check_common(m, kv, ws, ws_bytes, b->max_ctx_bound, b->page_table, b->page_stride,
                              "decode_step_logprobs");
  if (s != RIL_OK) return s;
  const ril_model_desc &d = m->d;
  if (b->n_rows < 1 || b->n_rows > d.max_rows)
    return fail(RIL_ERANGE, "decode_step_logprobs: n_rows %d outside [1, %d]", b->n_rows, d.max_rows);
  if (!b->ctx_len || !aligned4(b->ctx_len) || !b->target_ids || !aligned4(b->target_ids))
    return fail(RIL_EINVAL, "decode_step_logprobs: ctx_len/target_ids");
  if (!logprob_out || !aligned4(logprob_out)) return fail(RIL_EINVAL, "decode_step_logprobs: logprob_out");
  const bool tok = d.input_mode == RIL_INPUT_TOKENS;
  if (tok && (!b->token_ids || !aligned4(b->token_ids))) return fail(RIL_EINVAL, "decode_step_logprobs: token_ids");
  const bool need_v = !m->mla;
  if (!tok && (!b->q || !b->k || !aligned16(b->q) || !aligned16(b->k) || (need_v && (!b->v || !aligned16(b->v)))))
    return fail(RIL_EINVAL, "decode_step_logprobs: q/k/v");
  if (m->sparse && (!b->q_index || !b->k_index || !aligned16(b->q_index) || !aligned16(b->k_index) ||
                    (b->selected_out && !aligned4(b->selected_out))))
    return fail(RIL_EINVAL, "decode_step_logprobs: q_index/k_index/selected_out");
  if (m->ssd && (!b->dt || !aligned16(b->dt))) return fail(RIL_EINVAL, "decode_step_logprobs: dt");
  hipStream_t st = (hipStream_t)stream;
  const int R = b->n_rows;
  if (m->ssd) {
    s = run_ssd(m, kv, 1, R, R, nullptr, nullptr, b->ctx_len, b->page_table, b->page_stride, b->q, b->k, b->v,
                b->dt, true, ws, st);
    if (s != RIL_OK) return s;
    return run_head(m, R, b->target_ids, logprob_out, ws, st);
  }
  if (m->mla) {
    s = run_mla_write(m, kv, (const bf16_t *)b->k, b->k_index, R, 1, nullptr, nullptr, 0, b->ctx_len, b->page_table,
                      b->page_stride, st);
    if (s != RIL_OK) return s;
    s = run_mla(m, kv, (const bf16_t *)b->q, b->q_index, b->selected_out, 0, R, b->ctx_len, nullptr, nullptr, 0,
                b->page_table, b->page_stride, b->max_ctx_bound, ws, st);
    if (s != RIL_OK) return s;
    return run_head(m, R, b->target_ids, logprob_out, ws, st);
  }
  const int wqkv = (d.n_q_heads + 2 * d.n_kv_heads) * d.head_dim;
  const bf16_t *q, *k, *v;
  int q_stride, kv_stride;
  if (tok) {
    s = run_token_front(m, R, b->token_ids, ws, st);
    if (s != RIL_OK) return s;
    q = wsb(ws, m->off_qkv);
    k = q + d.n_q_heads * d.head_dim;
    v = k + d.n_kv_heads * d.head_dim;
    q_stride = kv_stride = wqkv;
  } else {
    q = (const bf16_t *)b->q;
    k = (const bf16_t *)b->k;
    v = (const bf16_t *)b->v;
    q_stride = d.n_q_heads * d.head_dim;
    kv_stride = d.n_kv_heads * d.head_dim;
  }
  KvWriteArgs kw{k, v, kv_stride, R, 1, nullptr, nullptr, 0, b->ctx_len, b->page_table, b->page_stride,
                 (bf16_t *)kv->pool, kv->n_pages, d.n_kv_heads, d.head_dim, m->kv_fp8, m->k_scale, m->v_scale};
  RIL_LAUNCH(RIL_K_KV_WRITE, launch_kv_write(kw, st));
  int split = d.split_tokens, max_splits = m->max_splits;
  if (m->policy == RIL_POLICY_SHAPE_DERIVED) {
    split = shape_split(m, R, b->max_ctx_bound);
    max_splits = (b->max_ctx_bound + split - 1) / split;
  }
  AttnDecodeArgs ad{q, q_stride, b->ctx_len, b->page_table, b->page_stride, (const bf16_t *)kv->pool,
                    kv->n_pages, d.n_kv_heads, m->G, d.head_dim, split, b->max_ctx_bound, R,
                    max_splits, m->cscale, wsf(ws, m->off_po), wsf(ws, m->off_pml), wsb(ws, m->off_attn),
                    m->kv_fp8, m->k_scale, m->v_scale};
  RIL_LAUNCH(RIL_K_ATTN_SPLIT, launch_attn_split(ad, st));
  if (!d.w_o && !d.d_ff && d.n_q_heads * d.head_dim <= ril::kMergeNormMaxD) {
    // the attention output goes straight into the final RMSNorm: merge and normalise in
    // one launch (the same arithmetic as the merge kernel followed by the RMSNorm kernel)
    RIL_LAUNCH(RIL_K_ATTN_MERGE, launch_attn_merge_norm(ad, (const bf16_t *)d.norm_final, d.rms_eps,
                                                        wsb(ws, m->off_z), d.d_head, st));
    return run_lm_head(m, R, wsb(ws, m->off_z), d.d_head, b->target_ids, logprob_out, ws, st);
  }
  RIL_LAUNCH(RIL_K_ATTN_MERGE, launch_attn_merge(ad, st));
  return run_head(m, R, b->target_ids, logprob_out, ws, st);
}

extern "C" ril_status ril_lm_head_logprobs(const ril_model *m, int32_t rows, const void *z, int32_t ldz,
                                           const int32_t *target_ids, float *logprob_out, void *ws,
                                           size_t ws_bytes, void *stream) {
  if (!m) return fail(RIL_EINVAL, "lm_head_logprobs: null model");
  const int R = std::max(m->d.max_rows, m->d.max_tokens);
  if (rows < 0 || rows > R) return fail(RIL_ERANGE, "lm_head_logprobs: rows %d outside [0, %d]", rows, R);
  if (ldz < m->d.d_head || ldz % 8) return fail(RIL_EINVAL, "lm_head_logprobs: ldz %d", ldz);
  if (!z || !aligned16(z) || !target_ids || !aligned4(target_ids) || !logprob_out || !aligned4(logprob_out))
    return fail(RIL_EINVAL, "lm_head_logprobs: null or misaligned pointer");
  if (!ws || !aligned16(ws)) return fail(RIL_EINVAL, "lm_head_logprobs: workspace null or misaligned");
  if (ws_bytes < m->ws_total)
    return fail(RIL_ERANGE, "lm_head_logprobs: workspace %zu bytes, %zu needed", ws_bytes, m->ws_total);
  if (rows == 0) return RIL_OK;
  hipStream_t st = (hipStream_t)stream;
  return run_lm_head(m, rows, (const bf16_t *)z, ldz, target_ids, logprob_out, ws, st);
}

extern "C" ril_status ril_decode_step_logprobs(const ril_model *m, ril_kv *kv, const ril_decode_batch *b,
                                               float *logprob_out, void *ws, size_t ws_bytes, void *stream) {
  return decode_enqueue(m, kv, b, logprob_out, ws, ws_bytes, stream);
}

// ---------------------------------------------------------------------------
// Decode step on the library's own device scratch, for callers that cannot allocate
// ---------------------------------------------------------------------------

// The workspace of ril_decode_step_logprobs_noalloc: one static array per device, held
// until the process ends.  Host code never passes `scratch` itself to a kernel (in host
// code the name is a host-side stand-in, not a device address): it looks the device
// address up once per device with hipGetSymbolAddress and uses that pointer.
static __device__ __align__(256) unsigned char scratch[RIL_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // per device, set on the first call with that device current
}  // namespace

// The device address of the current device's scratch array, looked up on the first call
// made with that device current.
static ril_status scratch_for_current_device(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(RIL_EHIP, "decode_step_logprobs_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(RIL_EUNSUPPORTED, "decode_step_logprobs_noalloc: device %d (at most %d devices)", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(RIL_EHIP, "decode_step_logprobs_noalloc: hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return RIL_OK;
}

extern "C" ril_status ril_decode_step_logprobs_noalloc(const ril_model *m, ril_kv *kv, const ril_decode_batch *b,
                                                       float *logprob_out, void *stream) {
  if (!m) return fail(RIL_EINVAL, "decode_step_logprobs_noalloc: null model");
  if (m->ws_total > (size_t)RIL_NOALLOC_SCRATCH_BYTES)
    return fail(RIL_ERANGE,
                "decode_step_logprobs_noalloc: the model needs a %zu-byte workspace, above the library's %zu-byte "
                "scratch (create the model with smaller max_rows / max_tokens / max_ctx)",
                m->ws_total, (size_t)RIL_NOALLOC_SCRATCH_BYTES);
  void *ws = nullptr;
  const ril_status s = scratch_for_current_device(&ws);
  if (s != RIL_OK) return s;
  // every segment is written before it is read within a call, so nothing is cleared
  return decode_enqueue(m, kv, b, logprob_out, ws, (size_t)RIL_NOALLOC_SCRATCH_BYTES, stream);
}

// ---------------------------------------------------------------------------
// HIP-graph capture of a decode step
// ---------------------------------------------------------------------------

struct ril_graph {
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
};

extern "C" ril_status ril_decode_graph_create(const ril_model *m, ril_kv *kv, const ril_decode_batch *b,
                                              float *logprob_out, void *ws, size_t ws_bytes, ril_graph **out) {
  if (!out) return fail(RIL_EINVAL, "decode_graph_create: null out");
  *out = nullptr;
  hipStream_t cs = nullptr;
  hipError_t e = hipStreamCreateWithFlags(&cs, hipStreamNonBlocking);
  if (e != hipSuccess) return fail(RIL_EHIP, "decode_graph_create: stream: %s", hipGetErrorString(e));
  e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) {
    (void)hipStreamDestroy(cs);
    return fail(RIL_EHIP, "decode_graph_create: begin capture: %s", hipGetErrorString(e));
  }
  g_capturing = true;
  const ril_status s = decode_enqueue(m, kv, b, logprob_out, ws, ws_bytes, cs);
  g_capturing = false;
  hipGraph_t graph = nullptr;
  e = hipStreamEndCapture(cs, &graph);
  (void)hipStreamDestroy(cs);
  if (s != RIL_OK) {  // the argument check's message stands
    if (graph) (void)hipGraphDestroy(graph);
    return s;
  }
  if (e != hipSuccess || !graph) {
    if (graph) (void)hipGraphDestroy(graph);
    return fail(RIL_EHIP, "decode_graph_create: end capture: %s", hipGetErrorString(e));
  }
  hipGraphExec_t exec = nullptr;
  e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    (void)hipGraphDestroy(graph);
    return fail(RIL_EHIP, "decode_graph_create: instantiate: %s", hipGetErrorString(e));
  }
  ril_graph *g = new ril_graph;
  g->graph = graph;
  g->exec = exec;
  *out = g;
  return RIL_OK;
}

extern "C" ril_status ril_graph_launch(ril_graph *g, void *stream) {
  if (!g || !g->exec) return fail(RIL_EINVAL, "graph_launch: null graph");
  const hipError_t e = hipGraphLaunch(g->exec, (hipStream_t)stream);
  if (e != hipSuccess) return fail(RIL_EHIP, "graph_launch: %s", hipGetErrorString(e));
  return RIL_OK;
}

extern "C" void ril_graph_destroy(ril_graph *g) {
  if (!g) return;
  if (g->exec) (void)hipGraphExecDestroy(g->exec);
  if (g->graph) (void)hipGraphDestroy(g->graph);
  delete g;
}
