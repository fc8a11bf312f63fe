// Host-side checks of the C ABI's validation and page allocator, built with AddressSanitizer
// and UndefinedBehaviorSanitizer on the host code only (tests/test_abi_sanitize.py builds
// and runs it on the CPU; no kernel is launched: every call either fails validation
// before anything is enqueued or is host-only).  Device pointers are fake, aligned
// addresses: validation checks them and never dereferences them.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "ril.h"
#include "ril_bench.h"

static int g_fail = 0;
#define EXPECT(cond)                                                       \
  do {                                                                     \
    if (!(cond)) {                                                         \
      std::fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #cond); \
      ++g_fail;                                                            \
    }                                                                      \
  } while (0)
#define EXPECT_ERR(expr)                                                   \
  do {                                                                     \
    const ril_status s_ = (expr);                                          \
    EXPECT(s_ != RIL_OK);                                                  \
    EXPECT(ril_last_error() != nullptr && ril_last_error()[0] != 0);       \
  } while (0)

static const void *fake(uintptr_t a) { return reinterpret_cast<const void *>(a); }

static ril_model_desc gqa() {
  ril_model_desc d;
  std::memset(&d, 0, sizeof d);
  d.attn_kind = RIL_ATTN_GQA;
  d.input_mode = RIL_INPUT_QKV;
  d.n_q_heads = 32;
  d.n_kv_heads = 8;
  d.head_dim = 128;
  d.d_head = 4096;
  d.vocab = 129280;
  d.page_tokens = 16;
  d.split_tokens = 512;
  d.max_rows = 64;
  d.max_tokens = 1024;
  d.max_ctx = 8192;
  d.softmax_scale = 0.088388f;
  d.rms_eps = 1e-6f;
  d.w_lm = fake(0x10000);
  return d;
}

static void model_descriptions() {
  ril_model *m = nullptr;
  EXPECT(ril_model_create(nullptr, &m) != RIL_OK);
  ril_model_desc d = gqa();
  EXPECT_ERR(ril_model_create(&d, nullptr));
  // one broken field at a time
  auto bad = [&](void (*edit)(ril_model_desc &)) {
    ril_model_desc e = gqa();
    edit(e);
    ril_model *mm = nullptr;
    EXPECT_ERR(ril_model_create(&e, &mm));
    EXPECT(mm == nullptr);
  };
  bad([](ril_model_desc &e) { e.attn_kind = 9; });
  bad([](ril_model_desc &e) { e.head_dim = 96; });
  bad([](ril_model_desc &e) { e.n_kv_heads = 5; });
  bad([](ril_model_desc &e) { e.page_tokens = 32; });
  bad([](ril_model_desc &e) { e.split_tokens = 100; });
  bad([](ril_model_desc &e) { e.vocab = 0; });
  bad([](ril_model_desc &e) { e.w_lm = nullptr; });
  bad([](ril_model_desc &e) { e.w_lm = fake(0x10008); });
  bad([](ril_model_desc &e) { e.max_ctx = 0; });
  bad([](ril_model_desc &e) { e.softmax_scale = 0.f; });
  bad([](ril_model_desc &e) { e.kv_dtype = 7; });
  bad([](ril_model_desc &e) { e.k_scale_exp = 40; });
  bad([](ril_model_desc &e) { e.lm_dtype = 3; });
  bad([](ril_model_desc &e) { e.d_ff = 500; });
  bad([](ril_model_desc &e) { e.ssm_state = 128; });
  bad([](ril_model_desc &e) {  // SSD without its constants
    e.attn_kind = RIL_ATTN_SSD;
    e.n_q_heads = 8;
    e.n_kv_heads = 2;
    e.head_dim = 64;
    e.ssm_state = 128;
    e.ssm_chunk = 128;
    e.d_head = 512;
  });
  // every kind that is valid creates and destroys cleanly
  EXPECT(ril_model_create(&d, &m) == RIL_OK);
  EXPECT(ril_workspace_bytes(m) > 0 && ril_kv_page_bytes(m) == 8 * 2 * 16 * 128 * 2);
  ril_model_destroy(m);
  ril_model_desc s = gqa();
  s.attn_kind = RIL_ATTN_SSD;
  s.n_q_heads = 8;
  s.n_kv_heads = 2;
  s.head_dim = 64;
  s.d_head = 512;
  s.ssm_state = 128;
  s.ssm_chunk = 128;
  s.ssm_A = fake(0x20000);
  s.ssm_D = fake(0x30000);
  EXPECT(ril_model_create(&s, &m) == RIL_OK);
  EXPECT(ril_kv_page_bytes(m) > 0);
  ril_model_destroy(m);
  ril_model_desc ml = gqa();
  ml.attn_kind = RIL_ATTN_MLA_SPARSE;
  ml.n_q_heads = 128;
  ml.n_kv_heads = 1;
  ml.head_dim = 512;
  ml.rope_dim = 64;
  ml.index_heads = 64;
  ml.index_dim = 128;
  ml.topk = 2048;
  ml.split_tokens = 256;
  ml.d_head = 65536;
  ml.kv_dtype = RIL_KV_FP8_E4M3;
  EXPECT(ril_model_create(&ml, &m) == RIL_OK);
  EXPECT(ril_kv_page_bytes(m) == 16 * 576 + 16 * 128 * 4);
  ril_model_destroy(m);
}

static void page_allocator() {
  ril_model_desc d = gqa();
  ril_model *m = nullptr;
  EXPECT(ril_model_create(&d, &m) == RIL_OK);
  const size_t pb = ril_kv_page_bytes(m);
  ril_kv *kv = nullptr;
  EXPECT_ERR(ril_kv_alloc(m, nullptr, pb * 10, 1, &kv));
  EXPECT_ERR(ril_kv_alloc(m, const_cast<void *>(fake(0x100008)), pb * 10, 1, &kv));
  EXPECT(ril_kv_alloc(m, const_cast<void *>(fake(0x100000)), pb * 10 + 5, 77, &kv) == RIL_OK);
  EXPECT(ril_kv_total_pages(kv) == 10 && ril_kv_free_pages(kv) == 10);
  std::vector<int32_t> ids(10, -1);
  EXPECT(ril_kv_assign(kv, 4, ids.data()) == RIL_OK);
  EXPECT_ERR(ril_kv_assign(kv, 7, ids.data() + 4));  // only 6 left: nothing taken
  EXPECT(ril_kv_free_pages(kv) == 6);
  EXPECT(ril_kv_assign(kv, 6, ids.data() + 4) == RIL_OK);
  std::vector<int32_t> seen(10, 0);
  for (int32_t id : ids) {
    EXPECT(id >= 0 && id < 10);
    if (id >= 0 && id < 10) ++seen[id];
  }
  for (int c : seen) EXPECT(c == 1);
  EXPECT(ril_kv_release(kv, 3, ids.data()) == RIL_OK);
  EXPECT_ERR(ril_kv_release(kv, 1, ids.data()));  // released twice
  const int32_t out_of_range = 10;
  EXPECT_ERR(ril_kv_release(kv, 1, &out_of_range));
  EXPECT(ril_kv_free_pages(kv) == 3);
  ril_kv_free(kv);
  ril_model_destroy(m);
}

static void batch_validation() {
  ril_model_desc d = gqa();
  ril_model *m = nullptr;
  EXPECT(ril_model_create(&d, &m) == RIL_OK);
  const size_t pb = ril_kv_page_bytes(m), wsb = ril_workspace_bytes(m);
  ril_kv *kv = nullptr;
  EXPECT(ril_kv_alloc(m, const_cast<void *>(fake(0x1000000)), pb * 100, 3, &kv) == RIL_OK);
  void *ws = const_cast<void *>(fake(0x40000000));
  float *out = reinterpret_cast<float *>(0x50000000);
  ril_decode_batch b;
  std::memset(&b, 0, sizeof b);
  b.n_rows = 4;
  b.max_ctx_bound = 100;
  b.ctx_len = reinterpret_cast<const int32_t *>(0x60000000);
  b.page_table = reinterpret_cast<const int32_t *>(0x60010000);
  b.page_stride = 7;
  b.target_ids = reinterpret_cast<const int32_t *>(0x60020000);
  b.q = fake(0x60030000);
  b.k = fake(0x60040000);
  b.v = fake(0x60050000);
  EXPECT_ERR(ril_decode_step_logprobs(m, kv, nullptr, out, ws, wsb, nullptr));
  EXPECT_ERR(ril_decode_step_logprobs(m, kv, &b, out, ws, wsb - 1, nullptr));     // workspace too small
  EXPECT_ERR(ril_decode_step_logprobs(m, kv, &b, out, const_cast<void *>(fake(0x40000008)), wsb, nullptr));
  ril_decode_batch e = b;
  e.n_rows = 65;
  EXPECT_ERR(ril_decode_step_logprobs(m, kv, &e, out, ws, wsb, nullptr));
  e = b;
  e.max_ctx_bound = 9000;
  EXPECT_ERR(ril_decode_step_logprobs(m, kv, &e, out, ws, wsb, nullptr));
  e = b;
  e.page_stride = 6;  // 100 positions need 7 pages
  EXPECT_ERR(ril_decode_step_logprobs(m, kv, &e, out, ws, wsb, nullptr));
  e = b;
  e.q = fake(0x60030008);
  EXPECT_ERR(ril_decode_step_logprobs(m, kv, &e, out, ws, wsb, nullptr));
  EXPECT_ERR(ril_decode_step_logprobs(m, kv, &b, nullptr, ws, wsb, nullptr));
  ril_prefill_batch p;
  std::memset(&p, 0, sizeof p);
  p.n_seqs = 2;
  p.total_tokens = 10;
  p.max_ctx_bound = 100;
  p.cu_tokens = reinterpret_cast<const int32_t *>(0x61000000);
  p.start_pos = reinterpret_cast<const int32_t *>(0x61010000);
  p.page_table = reinterpret_cast<const int32_t *>(0x61020000);
  p.page_stride = 7;
  p.target_ids = reinterpret_cast<const int32_t *>(0x61030000);
  p.q = fake(0x61040000);
  p.k = fake(0x61050000);
  p.v = fake(0x61060000);
  ril_prefill_batch f = p;
  f.total_tokens = 1025;
  EXPECT_ERR(ril_prefill_logprobs(m, kv, &f, out, ws, wsb, nullptr));
  f = p;
  f.cu_tokens = nullptr;
  EXPECT_ERR(ril_prefill_logprobs(m, kv, &f, out, ws, wsb, nullptr));
  f = p;
  f.v = nullptr;
  EXPECT_ERR(ril_prefill_logprobs(m, kv, &f, out, ws, wsb, nullptr));
  EXPECT_ERR(ril_kv_write(m, kv, nullptr, nullptr));
  EXPECT_ERR(ril_lm_head_logprobs(m, 2000, fake(0x62000000), 4096, reinterpret_cast<const int32_t *>(0x62100000),
                                  out, ws, wsb, nullptr));
  EXPECT_ERR(ril_proj_bf16(fake(0x63000000), 4, 100, 128, fake(0x63100000), 64, 128, nullptr, 0,
                           const_cast<void *>(fake(0x63200000)), 64, nullptr));  // K not a multiple of 32
  EXPECT_ERR(ril_set_policy(m, 5, 0));
  EXPECT_ERR(ril_set_policy(m, RIL_POLICY_SHAPE_DERIVED, 100));
  EXPECT_ERR(ril_hbm_read_probe(nullptr, 1024, reinterpret_cast<uint32_t *>(0x64000000), nullptr));
  double ms = 0;
  int64_t n = 0;
  EXPECT_ERR(ril_trace_read(-1, &ms, &n));
  EXPECT_ERR(ril_trace_read(0, nullptr, &n));
  ril_kv_free(kv);
  ril_model_destroy(m);
}

int main() {
  model_descriptions();
  page_allocator();
  batch_validation();
  if (g_fail) {
    std::fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  std::printf("sanitized ABI checks passed\n");
  return 0;
}
