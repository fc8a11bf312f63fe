// Host-side launch interface of the HIP kernels (argument bundles + launchers).
// Every launcher enqueues exactly one kernel on the given stream and returns
// hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ril {

typedef uint16_t bf16_t;

struct KvWriteArgs {
  const bf16_t *k, *v;  // [n_tok, row_stride] rows, kv head g at g*D
  int row_stride, n_tok, mode;  // mode 0: packed prefill tokens; 1: decode rows
  const int32_t *cu, *start_pos;
  int n_seqs;
  const int32_t *ctx_len, *page_table;
  int page_stride;
  bf16_t *pool;
  int n_pages, Hkv, D;
  int kv_fp8 = 0;                        // pool pages hold FP8 E4M3 codes
  float k_scale = 1.f, v_scale = 1.f;    // stored code = e4m3(x / scale), scale a power of two
};

struct AttnDecodeArgs {
  const bf16_t *q;  // row r at q + r*q_row_stride, head h at +h*D
  int q_row_stride;
  const int32_t *ctx_len, *page_table;
  int page_stride;
  const bf16_t *pool;
  int n_pages, Hkv, G, D, split_tokens, ctx_bound, n_rows, max_splits;
  float cscale;
  float *part_o, *part_ml;
  bf16_t *out;  // [rows, Hq, D]
  int kv_fp8 = 0;
  float k_scale = 1.f, v_scale = 1.f;
};

struct AttnPrefillArgs {
  const bf16_t *q;
  int q_row_stride;
  const int32_t *cu, *start_pos;
  int n_seqs, n_tok;
  const int32_t *page_table;
  int page_stride;
  const bf16_t *pool;
  int n_pages, Hkv, G, D, split_tokens, ctx_bound;
  float cscale;
  bf16_t *out;  // [n_tok, Hq, D]
  int kv_fp8 = 0;
  float k_scale = 1.f, v_scale = 1.f;
};

// SwiGLU activation: act[r, j] = bf16(silu(gu[r, j]) * gu[r, F + j]), formed in fp32.
struct SiluMulArgs {
  const bf16_t *gu;  // [rows, 2F] at row stride ldg
  int ldg;
  bf16_t *act;       // [rows, F] at row stride lda
  int lda, rows, F;
};
hipError_t launch_silu_mul(const SiluMulArgs &a, hipStream_t st);

struct RmsNormArgs {
  const bf16_t *x;
  int ldx;
  const int32_t *tok;
  const bf16_t *embed;
  int vocab, d;
  const bf16_t *gain;
  float eps;
  bf16_t *y;
  int ldy;
  bf16_t *x_copy;
  int ldc, rows;
};

struct GemmArgs {
  const bf16_t *A;
  int lda;
  const bf16_t *W;
  int ldw;
  bf16_t *C;
  int ldc;
  const bf16_t *R;
  int ldr, M, N, K;
  // comparator only: K split into split_k chunks with fp32 partials in `part`
  // ([split_k, M, N]); 1 / nullptr on the invariant path
  int split_k = 1;
  float *part = nullptr;
};

struct LmHeadArgs {
  const bf16_t *Z;
  int ldz;
  const bf16_t *W;
  int K, V;
  const int32_t *target;
  int M;
  float *part, *tgt_logit, *out;
  // W8A8 head: activation codes [M, K] and biased E8M0 exponents [M, K/128]; the packed
  // weight codes and their block exponents [2 * n_vt, K/128] (Z and W unused)
  const uint8_t *A8 = nullptr;
  const int32_t *ea = nullptr;
  const uint8_t *W8 = nullptr;
  const int32_t *ew = nullptr;
};

// Block-FP8 activation quantization: A8 = E4M3 codes of Z, ea = biased E8M0 exponents
// of its 1 x 128 groups.
// W8A8 projection: C = bf16(A W^T) (+ residual as GemmArgs) from block-FP8 codes and
// biased E8M0 exponents (rows: [M, K] + [M, K/128]; weight: [N, K] + [ceil(N/128), K/128]).
struct GemmFp8Args {
  const uint8_t *A8;
  const int32_t *ea;
  const uint8_t *W8;
  const int32_t *ew;
  bf16_t *C;
  int ldc;
  const bf16_t *R;
  int ldr, M, N, K;
};

struct QuantRowsArgs {
  const bf16_t *Z;
  int ldz, M, K;
  uint8_t *A8;
  int32_t *ea;
};

struct MlaKvWriteArgs {
  const bf16_t *c;  // latent rows [n_tok, row_stride], 576 dims used
  int row_stride;
  const float *kidx;  // sparse only: fp32 indexer keys [n_tok, 128], else null
  int n_tok, mode;
  const int32_t *cu, *start_pos;
  int n_seqs;
  const int32_t *ctx_len, *page_table;
  int page_stride;
  bf16_t *pool;
  int page_elems, n_pages;
  bool fp8;         // the latent is stored as E4M3 codes of c * inv_scale (token-major)
  float inv_scale;  // 2^-scale_exp
  bool token_major;  // bf16 latent token-major (the sparse kind), else in the K-operand layout
};

struct MlaAttnArgs {
  const bf16_t *q;  // [rows or tokens, H, 576]
  int mode, row0, n_rows;  // mode 0: decode rows; 1: prefill tokens row0 .. row0+n_rows-1
  const int32_t *ctx_len, *cu, *start_pos;
  int n_seqs;
  const int32_t *page_table;
  int page_stride;
  const bf16_t *pool;
  int page_elems, n_pages, H, split_tokens, ctx_bound, max_splits;
  const int32_t *sel;  // sparse: selection lists [n_rows, topk] (rows of this launch), else null
  int topk;
  float cscale;
  float *part_o, *part_ml;
  bf16_t *out;  // [rows or tokens, H, 512]
  bool fp8;     // FP8 latent pages, read back as code * scale
  float scale;  // 2^scale_exp
};

struct IndexerArgs {
  const float *q;  // [rows or tokens, 64, 128] fp32
  int mode, row0, n_rows;
  const int32_t *ctx_len, *cu, *start_pos;
  int n_seqs;
  const int32_t *page_table;
  int page_stride;
  const bf16_t *pool;
  int page_elems, n_pages, ctx_bound;
  int key_off;    // bf16 elements from a page's start to its fp32 indexer keys
  float *scores;  // [n_rows, score_stride] (rows of this launch)
  int score_stride;
  int topk;
  int32_t *sel;  // [n_rows, topk]
  int32_t *sel_copy;  // optional caller copy [all rows, topk] at row0, or null
};

// Mamba-2 SSD mixer (csrc/ssd.hip).  One call's sequences (prefill) or rows (decode),
// their cache slots (state + the current chunk's inputs) and the workspace it plans in.
constexpr int kSsdP = 64, kSsdN = 128, kSsdQ = 128;  // head channels, state size, chunk
struct SsdArgs {
  int mode;                  // 0: packed prefill tokens (cu, start_pos); 1: decode rows (ctx_len)
  int n_seqs, n_tok;
  const int32_t *cu, *start_pos, *ctx_len;
  const int32_t *page_table;  // slot id of sequence s at [s * page_stride]
  int page_stride;
  uint8_t *pool;
  long slot_bytes;
  int n_slots, H, G;
  const bf16_t *x, *B, *C;    // [n_tok, H, 64], [n_tok, G, 128], [n_tok, G, 128]
  const float *dt;            // [n_tok, H], positive
  const float *A, *D;         // [H]
  int max_chunks, max_done;   // host bounds on the chunks the call touches / completes
  int32_t *plan;              // [6 * n_seqs + 2]
  float *dS, *entry, *dec;    // per completed chunk: [max_done][H][64][128] x 2, [max_done][H]
  bf16_t *y;                  // [n_tok, H, 64]
};
long ssd_slot_bytes(int H, int G);
hipError_t launch_ssd_plan(const SsdArgs &a, hipStream_t st);
hipError_t launch_ssd_state(const SsdArgs &a, hipStream_t st);
hipError_t launch_ssd_scan(const SsdArgs &a, hipStream_t st);
hipError_t launch_ssd_out(const SsdArgs &a, hipStream_t st);
hipError_t launch_ssd_commit(const SsdArgs &a, hipStream_t st);
hipError_t launch_ssd_write(const SsdArgs &a, hipStream_t st);

hipError_t launch_indexer(const IndexerArgs &a, hipStream_t st);
hipError_t launch_topk(const IndexerArgs &a, hipStream_t st);

hipError_t launch_kv_write(const KvWriteArgs &a, hipStream_t st);
hipError_t launch_mla_kv_write(const MlaKvWriteArgs &a, hipStream_t st);
hipError_t launch_mla_split(const MlaAttnArgs &a, hipStream_t st);
hipError_t launch_mla_merge(const MlaAttnArgs &a, hipStream_t st);
hipError_t launch_attn_split(const AttnDecodeArgs &a, hipStream_t st);
hipError_t launch_attn_merge(const AttnDecodeArgs &a, hipStream_t st);
hipError_t launch_attn_prefill(const AttnPrefillArgs &a, hipStream_t st);
hipError_t launch_rmsnorm(const RmsNormArgs &a, hipStream_t st);
// Decode merge + final RMSNorm in one launch (rows with no output projection or MLP block);
// the row (Hq * D values) is staged in LDS.
constexpr int kMergeNormMaxD = 16384;
hipError_t launch_attn_merge_norm(const AttnDecodeArgs &a, const bf16_t *gain, float eps, bf16_t *z, int ldz,
                                  hipStream_t st);
hipError_t launch_gemm(const GemmArgs &a, hipStream_t st);
int gemm_tiles(int M, int N);
hipError_t launch_lm_head(const LmHeadArgs &a, hipStream_t st);
hipError_t launch_vocab_merge(const LmHeadArgs &a, hipStream_t st);
long lm_head_packed_elems(int V, int K);
hipError_t launch_pack_lm_head(const bf16_t *src, int V, int K, bf16_t *dst, hipStream_t st);
hipError_t launch_quant_rows_fp8(const QuantRowsArgs &a, hipStream_t st);
hipError_t launch_lm_head_fp8(const LmHeadArgs &a, hipStream_t st);
long lm_head_fp8_code_bytes(int V, int K);
long lm_head_fp8_exp_count(int V, int K);
int hbm_read_probe_blocks();
hipError_t launch_hbm_read_probe(const void *src, size_t bytes, uint32_t *out, hipStream_t st);
hipError_t launch_pack_lm_head_fp8(const bf16_t *src, int V, int K, uint8_t *codes, int32_t *ew, hipStream_t st);
long proj_fp8_bytes(int N, int K);
hipError_t launch_quant_weight_fp8(const bf16_t *src, int N, int K, uint8_t *codes, int32_t *ew, hipStream_t st);
hipError_t launch_gemm_fp8(const GemmFp8Args &a, hipStream_t st);

}  // namespace ril
