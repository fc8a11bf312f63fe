/*
 * ril.h -- C ABI of the invariant sampled-token logprob forward on MI355X (gfx950).
 *
 * What it computes.  For every token it is given, the library returns the fp32
 * logprob of that token's target id under one attention layer followed by an
 * RMSNorm and an lm-head with a log-softmax over the vocabulary.  The value is
 * bitwise identical whether the token comes through prefill_logprobs (a
 * whole-prefix or chunked pass: the trainer's recompute) or through
 * decode_step_logprobs (one token per row: the rollout), and whatever batch,
 * row order, page placement or prefill chunk size it is computed with.  This
 * is the "diff = 0" contract of "vLLM Achieves Bitwise-Consistent RL
 * Training" (section 2: kernel determinism, batch independence and phase
 * consistency; section 3.1: the same kernels define the values on both
 * sides).
 *
 * How: one numerical path shared by both entry points -- a paged KV cache with
 * one write path (section 4.2), attention whose KV split is a fixed number of
 * tokens (the zero-mismatch-rl README, key-features table: fixed-split
 * attention), split states merged left to right in split order, GEMMs with one
 * MFMA instruction and one K order for every M and no split-K (section 4.1),
 * and a vocabulary log-softmax reduced over fixed 256-column tiles in a fixed
 * tree, gathering the target's logit.
 *
 * Conventions for every entry point.
 *   Ownership: the caller owns every device buffer (weights, KV pool, page
 *     tables, inputs, outputs, workspace) and the stream.  The library never
 *     allocates or frees device memory, never synchronises the stream or the
 *     device, and never reads device memory from the host.  Device pointers
 *     must stay valid until the enqueued work has completed.
 *   Streams: `stream` is a hipStream_t passed as void* (NULL = the default
 *     stream).  All work of a call is enqueued on it in order.
 *   Errors: every argument is validated on the host before anything is
 *     enqueued; on any status other than RIL_OK nothing has been enqueued,
 *     except RIL_EHIP (a launch failed: earlier kernels of the call may have
 *     been enqueued).  ril_last_error() returns a thread-local message for the
 *     last failing call.  Device-side values the host cannot check (a page id
 *     outside the pool, a context beyond the call's bound) never cause an
 *     out-of-bounds access: the affected row's logprob is written as NaN.
 *   Threading: handles are not thread-safe; distinct handles may be used from
 *     different threads.
 *   Alignment: every device pointer must be 16-byte aligned.
 *   Layouts are row-major; bf16 is IEEE bfloat16 stored as uint16.
 */
#ifndef RIL_H
#define RIL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ril_status {
  RIL_OK = 0,
  RIL_EINVAL = -1,        /* a pointer, size or layout argument is invalid */
  RIL_ERANGE = -2,        /* a size exceeds a limit fixed at model_create */
  RIL_ENOSPC = -3,        /* the KV pool has too few free pages */
  RIL_EUNSUPPORTED = -4,  /* a valid configuration this build does not implement */
  RIL_EHIP = -5           /* the HIP runtime reported an error */
} ril_status;

/* Attention kinds.
 *   GQA: per-kv-head K and V of head_dim each; q head h reads kv head h*Hkv/Hq.
 *   MLA: absorbed multi-head latent attention; every q head reads one shared cached
 *        latent row per token of head_dim + rope_dim values (512 + 64); scores use
 *        all of it, values its first head_dim (Bitwise-consistent RL post, section 3:
 *        MLA compresses KV before caching).
 *   MLA_SPARSE: MLA over the top-k history positions a lightweight indexer selects
 *        (post sections 3 and 4.3).  Per position an fp32 indexer key is cached beside
 *        the latent; per query an fp32 indexer query of index_heads x index_dim.
 *        Scores I[s] = sum_h relu(q_h . k_s) in fp32, one rounding per multiply and
 *        add, d then h in order; the k best (score, position) keys win, equal scores
 *        going to the lower position; the list is ordered by descending position
 *        (-1 padding last) and the attention accumulates in that order, splitting it
 *        into runs of split_tokens entries.  Contexts of at most k positions select
 *        every position. */
/* RIL_ATTN_SSD: a Mamba-2 selective state-space mixer in place of attention
 *   (Bitwise-consistent RL post, section 6: Nemotron's Mamba-2 layers, whose decode
 *   replays the prefill's chunked arithmetic; the zero-mismatch-rl README's key
 *   features).  H = n_q_heads heads of head_dim = 64 channels, G = n_kv_heads groups of
 *   ssm_state = 128 state rows (head h reads group h / (H / G)); per position t, with
 *   dt_t > 0 given per head and A (< 0), D model constants per head:
 *     S_t = exp(dt_t A) S_{t-1} + dt_t B_t x_t^T,   y_t = S_t^T C_t + D x_t   (bf16)
 *   y replaces the attention output of the QKV input mode (then [O GEMM], RMSNorm,
 *   lm-head).  The batch's q holds C [tokens, G, 128], k holds B [tokens, G, 128], v holds
 *   x [tokens, H, 64] (bf16), dt the fp32 [tokens, H] steps.  It is evaluated in chunks of
 *   ssm_chunk = 128 positions counted from position 0, every phase through the same
 *   kernels (csrc/ssd.hip), so a position's bits do not depend on how its sequence is cut
 *   into calls.  The "KV pool" holds one cache slot per sequence (ril_kv_page_bytes: the
 *   state entering the current chunk, fp32, kept in one of two buffers by the chunk's
 *   parity so that a repeated decode step reads what it read before, and that chunk's
 *   earlier inputs): page_table
 *   column 0 of a sequence is its slot, page_stride >= 1.  A slot's state is read only
 *   when a sequence continues past its first chunk; a sequence restarted at position 0
 *   starts from zero state.  Prefill calls carry at most max_rows sequences; history is
 *   laid down by prefill calls (ril_kv_write does not apply: the state depends on every
 *   position).  H a multiple of 4 and of G; bf16 cache only. */
enum { RIL_ATTN_GQA = 0, RIL_ATTN_MLA = 1, RIL_ATTN_MLA_SPARSE = 2, RIL_ATTN_SSD = 3 };

/* KV cache storage (GQA, and the MLA latent).  FP8_E4M3 follows the Bitwise-consistent RL post, section
 * 4.2 (FP8 KV cache: FP8 storage, one write path, one dequantizing read shared by
 * prefill, decode and the trainer's recompute): each K (V) value x is stored as the OCP
 * E4M3 code of x * 2^-k_scale_exp (2^-v_scale_exp), rounded to nearest even, magnitudes
 * beyond 448 saturating to 448, NaN kept as NaN with its sign; every attention reads
 * code * 2^scale_exp, a bf16 value exactly, and runs the bf16 arithmetic unchanged.  A
 * page then takes n_kv_heads * 16 * 2 * head_dim bytes (half of BF16's).  The in-page
 * byte layout is documented in csrc/attn_common.h (and, for the bf16 MLA latent, in
 * csrc/mla.hip: the dense kind's pages in the K-operand layout, the sparse kind's
 * token-major).  MLA (dense and sparse): the latent
 * row (head_dim + rope_dim values) is one tensor with one scale, so k_scale_exp must equal
 * v_scale_exp; a page holds 16 x 576 codes, token-major (code of (t, d) at byte 576 t + d),
 * then, for the sparse kind, the fp32 indexer keys as with BF16 (csrc/mla.hip). */
enum { RIL_KV_BF16 = 0, RIL_KV_FP8_E4M3 = 1 };

/* lm-head arithmetic.  W8A8_FP8 follows the Bitwise-consistent RL post, section 4.1
 * (the deployment GEMM is W8A8 with block-FP8 weights; the trainer quantizes its bf16
 * weights to block FP8 by the same rule and calls the same GEMM, one accumulation order
 * for every M): the normalised rows are quantized per group of 128 K values and the
 * weight per block of 128 vocabulary columns x 128 K values, each group or block to OCP
 * E4M3 codes e4m3(x * 2^-e) (nearest even) with one E8M0 scale 2^e, e the smallest
 * integer >= -127 with max|x| <= 448 * 2^e (0 for an all-zero group, the E8M0 NaN code
 * for a group holding an infinity or NaN, which makes every logit it enters NaN).  The
 * logits are the fp32 sums over K of code products times both scales, accumulated one
 * 128-wide K block at a time in the column's fixed order; the softmax partials and the
 * logprob are then formed exactly as in the bf16 head. */
enum { RIL_LM_BF16 = 0, RIL_LM_W8A8_FP8 = 1 };
/* Projection precision (same post, section 4.1: the deployment's GEMMs are W8A8 with
 * block-FP8 weights, and the trainer runs the same GEMMs).  RIL_PROJ_W8A8_FP8: every
 * projection of the model (w_qkv, w_o, w_gate_up, w_down) multiplies the rows' block-FP8
 * codes (1 x 128 groups by the rule above, quantized at each call) by the weight's
 * block-FP8 codes (128 x 128 blocks, written by ril_quantize_weight_fp8): fp32 sums over
 * K of code products times both scales, one 128-wide K block at a time in the order
 * k = 0, 128, 256, ... for every M; the output is rounded to bf16 and the residual added
 * as in the bf16 path.  Each projection's K (d_model, Hq*D, d_ff) is a multiple of 128. */
enum { RIL_PROJ_BF16 = 0, RIL_PROJ_W8A8_FP8 = 1 };
enum { RIL_INPUT_TOKENS = 0, RIL_INPUT_QKV = 1 };

/* Model description.  All sizes are fixed for the life of the handle; the
 * split and page sizes are model constants, never derived from a batch, a
 * context length or the GPU (Bitwise-consistent RL post, section 2: no
 * kernel choice by batch size, no dynamic split count).                     */
typedef struct ril_model_desc {
  int32_t attn_kind;     /* RIL_ATTN_GQA | RIL_ATTN_MLA | RIL_ATTN_MLA_SPARSE */
  int32_t input_mode;    /* RIL_INPUT_TOKENS: token ids -> embedding -> RMSNorm -> QKV GEMM
                            -> attention -> O GEMM + residual -> RMSNorm -> lm-head;
                            RIL_INPUT_QKV: q/k/v given -> attention -> [O GEMM] -> RMSNorm
                            -> lm-head */
  int32_t d_model;       /* TOKENS: residual width (multiple of 32); QKV: ignored */
  int32_t n_q_heads;     /* Hq (MLA: a multiple of 64) */
  int32_t n_kv_heads;    /* GQA: Hkv, Hq/Hkv in {1, 2, 4, 8, 16}; MLA: 1 */
  int32_t head_dim;      /* D = value width per head: GQA 64 or 128; MLA 512 (latent rank) */
  int32_t rope_dim;      /* MLA: extra score-only dims of the latent row (64); GQA: 0 */
  int32_t index_heads;   /* MLA_SPARSE: indexer heads (64); else 0 */
  int32_t index_dim;     /* MLA_SPARSE: indexer dim (128); else 0 */
  int32_t topk;          /* MLA_SPARSE: positions kept, a power of two in [64, 4096]; else 0 */
  int32_t d_head;        /* width the final RMSNorm and lm-head consume (multiple of 32):
                            TOKENS: = d_model; QKV: = o-proj out width if w_o, else Hq*D */
  int32_t vocab;         /* V >= 1 */
  int32_t page_tokens;   /* tokens per KV page: 16 */
  int32_t split_tokens;  /* attention KV split in tokens: a multiple of 64; GQA <= 1024,
                            MLA <= 2048 (512 for GQA and 2048 for MLA here) */
  int32_t max_rows;      /* most rows one decode call may carry */
  int32_t max_tokens;    /* most tokens one prefill call may carry */
  int32_t max_ctx;       /* longest context (tokens, including the current one) */
  float softmax_scale;   /* multiplies q.k (1/sqrt(D) for the workloads here) */
  float rms_eps;         /* RMSNorm epsilon */
  /* device weights, bf16, nn.Linear layout [out, in]; caller-owned */
  const void *embed;      /* [V, d_model]                   TOKENS only            */
  const void *w_qkv;      /* [(Hq + 2 Hkv) D, d_model]      TOKENS only: q|k|v rows */
  const void *w_o;        /* [d_head, Hq D]                 TOKENS: required; QKV: optional */
  const void *norm_attn;  /* [d_model] RMSNorm gain          TOKENS only; NULL = 1   */
  const void *norm_final; /* [d_head]  RMSNorm gain          NULL = 1                */
  const void *w_lm;       /* [V, d_head] in the packed lm-head layout written by
                             ril_pack_lm_head (ril_lm_head_packed_bytes)      required */
  int32_t kv_dtype;       /* RIL_KV_BF16 (0) | RIL_KV_FP8_E4M3                            */
  int32_t k_scale_exp;    /* FP8: K stored as e4m3(k * 2^-k_scale_exp), in [-32, 32]; BF16: 0 */
  int32_t v_scale_exp;    /* FP8: V likewise                                               */
  /* TOKENS only: an optional SwiGLU MLP block after the attention block (d_ff = 0: none):
   *   h = bf16(rms(y) norm_mlp);  [g|u] = bf16(h w_gate_up^T);  a = bf16(silu(g) * u)
   *   y' = bf16(y + bf16(a w_down^T))
   * where silu(g) * u is formed in fp32 and rounded once (Bitwise-consistent RL post,
   * section 4.4, condition 3: SwiGLU's activation rounded once). */
  int32_t d_ff;           /* F, a multiple of 32, or 0                                      */
  const void *w_gate_up;  /* [2F, d_model]: gate rows 0..F-1, then up rows                  */
  const void *w_down;     /* [d_model, F]                                                    */
  const void *norm_mlp;   /* [d_model] RMSNorm gain; NULL = 1                                */
  int32_t lm_dtype;       /* RIL_LM_BF16 (0): w_lm as written by ril_pack_lm_head;
                             RIL_LM_W8A8_FP8 (1): w_lm as written by ril_pack_lm_head_fp8,
                             d_head a multiple of 128                                       */
  int32_t proj_dtype;     /* RIL_PROJ_BF16 (0): w_qkv, w_o, w_gate_up, w_down bf16 as above;
                             RIL_PROJ_W8A8_FP8 (1): each written by ril_quantize_weight_fp8
                             from that bf16 matrix (16-byte aligned)                        */
  int32_t ssm_state;      /* SSD: state rows N (128); else 0                                 */
  int32_t ssm_chunk;      /* SSD: chunk Q (128); else 0                                      */
  const void *ssm_A;      /* SSD: device fp32 [H], negative; else NULL                       */
  const void *ssm_D;      /* SSD: device fp32 [H]; else NULL                                 */
} ril_model_desc;

typedef struct ril_model ril_model;  /* opaque: copy of the description + derived sizes */
typedef struct ril_kv ril_kv;        /* opaque: KV pool pointer + host free list */

/* Create a model handle.  Validates the description (sizes, required weight
 * pointers, alignment).  The weights are referenced, not copied. */
ril_status ril_model_create(const ril_model_desc *desc, ril_model **out);
void ril_model_destroy(ril_model *m);

/* Bytes of device workspace every prefill/decode call on `m` needs.  Depends
 * only on the model's static limits (section 4.6 of the post: workspaces are
 * sized by model limits so they can be allocated once, before capture). */
size_t ril_workspace_bytes(const ril_model *m);

/* Bytes of one KV page: Hkv x 2 (K, V) x page_tokens x D x 2 bytes. */
size_t ril_kv_page_bytes(const ril_model *m);

/* S11 weight layout.  The lm-head reads its weight in a packed form: per vocabulary
 * tile of 256 columns, per 16-column MFMA block, per 32-wide K step, that block's
 * MFMA operand in lane order, so each weight load of a wavefront is one contiguous
 * 1 KB read (the row-major [V, K] matrix would be read 64 bytes per row per step).
 * Element (column c, k) of W sits at
 *   ((((c/256)*16 + (c%256)/16) * (K/32) + k/32) * 64 + ((k%32)/8)*16 + c%16) * 8 + k%8
 * and the columns past V in the last tile are zero.  Only the addresses change: the
 * lm-head's arithmetic (its K order included) is the same for any layout.
 *
 * ril_lm_head_packed_bytes: size of the packed weight, ceil(V/256)*256*K*2 bytes
 * (0 for V < 1 or K not a positive multiple of 32).
 * ril_pack_lm_head: enqueue, on `stream`, the packing of the row-major bf16 device
 * matrix src[V, K] (row stride K) into dst (device, packed_bytes >= the size above,
 * 16-byte aligned, not overlapping src).  Call it again after every weight update.
 * Returns RIL_EINVAL on bad sizes, alignment or a short dst, RIL_EHIP on a launch
 * error; nothing is enqueued on error. */
size_t ril_lm_head_packed_bytes(int32_t vocab, int32_t d_head);
ril_status ril_pack_lm_head(const void *src, int32_t vocab, int32_t d_head, void *dst, size_t packed_bytes,
                            void *stream);

/* W8A8 weight layout (RIL_LM_W8A8_FP8).  One buffer: the E4M3 codes, then the biased
 * E8M0 exponents (int32, 127 + e, 255 = NaN) of the 128 x 128 blocks,
 * [2 * ceil(V/256), K/128], block b covering columns 128b .. 128b+127 (columns past V
 * count as zero).  Codes: per vocabulary tile of 256 columns, per 128-wide K step, a
 * contiguous 32 KB piece holding the 2 KB FP8 MFMA operands of the tile's sixteen
 * 16-column blocks in lane order:
 *   code(c, k) at ((c/256) * (K/128) + k/128) * 32768 + ((c%256)/16) * 2048
 *                 + ((k%32)/16) * 1024 + (((k%128)/32) * 16 + c%16) * 16 + k%16
 * ril_lm_head_fp8_packed_bytes: ceil(V/256)*256*K + 2*ceil(V/256)*(K/128)*4 bytes (0 for
 * V < 1 or K not a positive multiple of 128).
 * ril_pack_lm_head_fp8: enqueue, on `stream`, the quantization and packing of the
 * row-major bf16 device matrix src[V, K] into dst (device, packed_bytes >= the size
 * above, 16-byte aligned, not overlapping src); two kernels (block scales, then codes).
 * Call it again after every weight update.  Returns RIL_EINVAL on bad sizes, alignment
 * or a short dst, RIL_EHIP on a launch error. */
size_t ril_lm_head_fp8_packed_bytes(int32_t vocab, int32_t d_head);

/* The W8A8 head's activation quantization, for callers that quantize rows themselves
 * (a trainer applying the deployment rule): enqueue, on `stream`, the block-FP8
 * quantization of rows x rows of the bf16 device matrix src (row stride ld elements,
 * K a positive multiple of 128, ld >= K and a multiple of 8) into the E4M3 codes
 * codes[rows, K] (row-major, device) and the biased E8M0 exponents exps[rows, K/128]
 * (int32 device, 127 + e, 255 = NaN), by the rule of RIL_LM_W8A8_FP8.  Pointers 16-byte
 * (exps: 4-byte) aligned.  Returns RIL_EINVAL on bad sizes or pointers, RIL_EHIP on a
 * launch error; rows = 0 enqueues nothing. */
ril_status ril_quantize_rows_fp8(const void *src, int32_t rows, int32_t K, int32_t ld, void *codes, void *exps,
                                 void *stream);
ril_status ril_pack_lm_head_fp8(const void *src, int32_t vocab, int32_t d_head, void *dst, size_t packed_bytes,
                                void *stream);

/* Block-FP8 projection weight (RIL_PROJ_W8A8_FP8).  One buffer: the E4M3 codes [N, K]
 * (row-major, one byte per weight), then the biased E8M0 exponents (int32, 127 + e,
 * 255 = NaN) of the 128 x 128 blocks, [ceil(N/128), K/128]: block (b, kb) covers rows
 * 128b .. 128b+127 and K values 128kb .. 128kb+127, rows past N counting as zero.
 * ril_proj_fp8_bytes: N*K + ceil(N/128)*(K/128)*4 (0 for N < 1 or K not a positive
 * multiple of 128).
 * ril_quantize_weight_fp8: enqueue, on `stream`, the quantization of the row-major bf16
 * device matrix src[N, K] into dst (device, dst_bytes >= the size above, 16-byte
 * aligned, not overlapping src); two kernels (block scales, then codes).  Call it again
 * after every weight update.  Returns RIL_EINVAL on bad sizes, alignment or a short dst,
 * RIL_EHIP on a launch error. */
size_t ril_proj_fp8_bytes(int32_t N, int32_t K);
ril_status ril_quantize_weight_fp8(const void *src, int32_t N, int32_t K, void *dst, size_t dst_bytes, void *stream);

/* The W8A8 projection GEMM alone, for callers that run a projection outside a model (a
 * trainer's recompute, tests): enqueue out[rows, N] = bf16(A W^T) with A given as codes
 * [rows, K] (row-major, row stride K) and exps [rows, K/128] (ril_quantize_rows_fp8) and W
 * as written by ril_quantize_weight_fp8 (N rows, the same K) in a buffer of w_bytes bytes.
 * out is bf16 device memory, row stride ldo >= N elements.  Each element's K order is
 * k = 0, 128, ... for every rows.  Pointers 16-byte (exps: 4-byte; out: 2-byte) aligned.
 * Returns RIL_EINVAL on bad sizes or pointers or w_bytes < ril_proj_fp8_bytes(N, K),
 * RIL_EHIP on a launch error; rows = 0 enqueues nothing. */
ril_status ril_proj_w8a8(const void *codes, const void *exps, int32_t rows, int32_t K, const void *w,
                         size_t w_bytes, int32_t N, void *out, int32_t ldo, void *stream);

/* S4 alone: the bf16 projection GEMM the model runs for its QKV, O and MLP projections,
 * for callers that run a projection outside a model (a trainer's recompute, tests of the
 * GEMM at its own boundary).  Enqueue, on `stream`,
 *   out[r, n] = bf16(sum_k A[r, k] W[n, k])                      (residual == NULL)
 *   out[r, n] = bf16(residual[r, n] + bf16(sum_k A[r, k] W[n, k]))
 * with fp32 accumulation of bf16 x bf16 products in the order k = 0, 32, 64, ..., one
 * 16x16x32 MFMA step at a time, never split: the Bitwise-consistent RL post, section 4.1
 * (one accumulation order for every M, no split-K).  The kernel and tile shape follow
 * `rows` (and K), the bits of a row never do: the same row gives the same output at any
 * rows.  A is bf16 [rows, K] at row stride lda, W bf16 [N, K] (nn.Linear layout) at row
 * stride ldw, residual and out bf16 [rows, N] at row strides ldr and ldo; all device
 * memory.  K is a positive multiple of 32; lda, ldw >= K and multiples of 8; ldo (ldr)
 * >= N.  A and W 16-byte aligned, out and residual 2-byte aligned; out must not overlap
 * the inputs except that residual may equal out with ldr == ldo.  Returns RIL_EINVAL on
 * bad sizes or pointers, RIL_EHIP on a launch error; rows = 0 enqueues nothing. */
ril_status ril_proj_bf16(const void *A, int32_t rows, int32_t K, int32_t lda, const void *W, int32_t N,
                         int32_t ldw, const void *residual, int32_t ldr, void *out, int32_t ldo, void *stream);

/* S1: page assignment.  Decode reads a paged cache whose page placement
 * must not change a single bit of the result (Bitwise-consistent RL post,
 * section 4.3: prefill's contiguous and decode's paged reads are bitwise
 * identical; section 4.2: the cache's storage sets concurrency).  The pages
 * are position-independent blocks, so a sequence's bits are the same for any
 * page ids, and a pool copied elsewhere (a restored checkpoint) serves the
 * same results.  Wrap a caller-owned device pool of `pool_bytes`
 * bytes (16-byte aligned) as floor(pool_bytes / page_bytes) pages and build a
 * host free list over them.  shuffle_seed != 0 permutes the free list with a
 * seeded Fisher-Yates shuffle (random page tables); 0 hands pages out in
 * order.  Launches nothing. */
ril_status ril_kv_alloc(const ril_model *m, void *pool_dev, size_t pool_bytes,
                        uint64_t shuffle_seed, ril_kv **out);
/* Take `n_pages` pages off the free list; their ids are written to the host
 * array `page_ids_out`.  RIL_ENOSPC (and nothing taken) if fewer are free. */
ril_status ril_kv_assign(ril_kv *kv, int32_t n_pages, int32_t *page_ids_out);
/* Return pages to the free list.  RIL_EINVAL (and nothing returned) if an id
 * is out of range or not currently assigned. */
ril_status ril_kv_release(ril_kv *kv, int32_t n_pages, const int32_t *page_ids);
int32_t ril_kv_free_pages(const ril_kv *kv);
int32_t ril_kv_total_pages(const ril_kv *kv);
void ril_kv_free(ril_kv *kv);

/* A prefill batch: n_seqs sequences, each contributing a contiguous run of
 * tokens at consecutive positions start_pos[s], start_pos[s]+1, ...
 * Tokens are packed: sequence s owns tokens cu_tokens[s] .. cu_tokens[s+1]-1.
 * A one-token sequence is exactly a decode row, so a mixed continuous batch
 * (prefill chunks + decode rows) is one prefill call.
 * Every position before start_pos[s] must already be in the KV cache (written
 * by an earlier prefill/decode call or by ril_kv_write). */
typedef struct ril_prefill_batch {
  int32_t n_seqs;           /* 1 .. max_rows */
  int32_t total_tokens;     /* host copy of cu_tokens[n_seqs]: 1 .. max_tokens */
  int32_t max_ctx_bound;    /* host upper bound on start_pos[s] + len_s over the batch
                               (<= model max_ctx); grids are sized from it */
  const int32_t *cu_tokens; /* device [n_seqs + 1], cu_tokens[0] = 0, non-decreasing */
  const int32_t *start_pos; /* device [n_seqs] */
  const int32_t *page_table;/* device [n_seqs, page_stride]: page ids of positions
                               16j .. 16j+15 of sequence s at [s * page_stride + j] */
  int32_t page_stride;      /* >= ceil(max_ctx_bound / page_tokens) */
  const int32_t *target_ids;/* device [total_tokens]: id whose logprob is returned */
  const int32_t *token_ids; /* TOKENS: device [total_tokens] */
  const void *q;            /* QKV: device bf16 [total_tokens, Hq, D]  (MLA: [.., Hq, D + rope]) */
  const void *k;            /* QKV: device bf16 [total_tokens, Hkv, D] (MLA: latent [.., D + rope]) */
  const void *v;            /* QKV: device bf16 [total_tokens, Hkv, D] (MLA: unused, may be NULL) */
  const float *q_index;     /* MLA_SPARSE: device fp32 [total_tokens, index_heads, index_dim] */
  const float *k_index;     /* MLA_SPARSE: device fp32 [total_tokens, index_dim] (cached per position) */
  int32_t *selected_out;    /* MLA_SPARSE, optional: device int32 [total_tokens, topk] receives each
                               token's selection list; NULL = not returned */
  const float *dt;          /* SSD: device fp32 [total_tokens, H], 16-byte aligned; else unused */
} ril_prefill_batch;

/* A decode batch: n_rows rows, one new token each, at position ctx_len[r]-1. */
typedef struct ril_decode_batch {
  int32_t n_rows;           /* 1 .. max_rows */
  int32_t max_ctx_bound;    /* host upper bound on ctx_len[r] (<= model max_ctx) */
  const int32_t *ctx_len;   /* device [n_rows]: context including the new token, >= 1 */
  const int32_t *page_table;/* device [n_rows, page_stride] */
  int32_t page_stride;      /* >= ceil(max_ctx_bound / page_tokens) */
  const int32_t *target_ids;/* device [n_rows] */
  const int32_t *token_ids; /* TOKENS: device [n_rows] */
  const void *q;            /* QKV: device bf16 [n_rows, Hq, D]  (MLA: [n_rows, Hq, D + rope]) */
  const void *k;            /* QKV: device bf16 [n_rows, Hkv, D] (the new token's; MLA: latent
                               [n_rows, D + rope]) */
  const void *v;            /* QKV: device bf16 [n_rows, Hkv, D] (MLA: unused, may be NULL) */
  const float *q_index;     /* MLA_SPARSE: device fp32 [n_rows, index_heads, index_dim] */
  const float *k_index;     /* MLA_SPARSE: device fp32 [n_rows, index_dim] (the new token's) */
  int32_t *selected_out;    /* MLA_SPARSE, optional: device int32 [n_rows, topk] */
  const float *dt;          /* SSD: device fp32 [n_rows, H], 16-byte aligned; else unused */
} ril_decode_batch;

/* Trainer-side recompute: the trainer's forward calls the rollout's kernels
 * (Bitwise-consistent RL post, section 3.1), and a prefill chunk, a whole
 * sequence or a decode row give one position the same bits (section 2, phase
 * consistency).  Writes every batch token's K/V into its page
 * (S5), attends causally over the cache (S10), then the head (S4, S3, S11,
 * S12).  logprob_out: device fp32 [total_tokens].  ws: device workspace of at
 * least ril_workspace_bytes(m) bytes. */
ril_status ril_prefill_logprobs(const ril_model *m, ril_kv *kv, const ril_prefill_batch *b,
                                float *logprob_out, void *ws, size_t ws_bytes, void *stream);

/* Rollout-side step: decode runs the same read path and arithmetic as
 * prefill, with a work partition that never depends on the batch
 * (Bitwise-consistent RL post, section 4.2; the zero-mismatch-rl README's
 * fixed-split attention).  Writes each row's new K/V into its page (S5), attends
 * over the row's ctx_len[r] positions with fixed-size splits (S8) merged in
 * split order (S9), then the head.  logprob_out: device fp32 [n_rows]. */
ril_status ril_decode_step_logprobs(const ril_model *m, ril_kv *kv, const ril_decode_batch *b,
                                    float *logprob_out, void *ws, size_t ws_bytes, void *stream);

/* The head alone (S11, S12): logprobs of target_ids[r] for normalised rows z (the final
 * RMSNorm's output), through the model's lm-head (bf16 or W8A8 by lm_dtype), the same
 * kernels and launch shapes the prefill and decode calls use for the same row count.  For
 * callers that run the model body themselves and want the head's logprobs (and for
 * checking the head at its own boundary).  z: device bf16 [rows, d_head], row stride ldz
 * elements (>= d_head, a multiple of 8, 16-byte aligned); target_ids: device int32 [rows];
 * logprob_out: device fp32 [rows] (NaN for a target outside [0, V)); rows in
 * [0, max(max_rows, max_tokens)].  Returns RIL_EINVAL / RIL_ERANGE on bad arguments
 * (nothing enqueued), RIL_EHIP on a launch error. */
ril_status ril_lm_head_logprobs(const ril_model *m, int32_t rows, const void *z, int32_t ldz,
                                const int32_t *target_ids, float *logprob_out, void *ws, size_t ws_bytes,
                                void *stream);

/* The rollout step without a caller workspace, for callers that cannot allocate device
 * memory (code under HIP-graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same as ril_decode_step_logprobs(m, kv, b, logprob_out, ws, ws_bytes,
 * stream) -- the same kernels, the same bits -- with the workspace taken from a static
 * device array of RIL_NOALLOC_SCRATCH_BYTES bytes inside the library: one per device,
 * allocated when the library's code is loaded on that device and held until the process
 * ends.  The call itself allocates and frees nothing.  The array's device address is
 * looked up on the first call made with a device current.
 * Limits: ril_workspace_bytes(m) must not exceed RIL_NOALLOC_SCRATCH_BYTES (create a
 * decode model with small max_tokens; 64 decode rows of 32 x 128-dim heads at contexts up
 * to 8192 with a 129280-word head need about 18 MiB); else RIL_ERANGE.
 * Sharing: every call on a device uses that device's one array, which keeps the last
 * call's contents.  Calls on one device whose work can overlap in time (different
 * streams, or threads, without ordering between them) race on it: order them on one
 * stream.  Nothing in the array needs clearing between calls (each call writes every
 * part it reads).  Errors as ril_decode_step_logprobs, plus RIL_EHIP if the array's
 * address cannot be looked up and RIL_EUNSUPPORTED for a device index of 64 or more. */
#define RIL_NOALLOC_SCRATCH_BYTES (64u << 20)
ril_status ril_decode_step_logprobs_noalloc(const ril_model *m, ril_kv *kv, const ril_decode_batch *b,
                                            float *logprob_out, void *stream);

/* HIP-graph capture of one decode step, for steps whose launch overhead matters
 * (small batches, short contexts).
 *
 * ril_decode_graph_create records the kernels ril_decode_step_logprobs(m, kv,
 * b, logprob_out, ws, ws_bytes, stream) would enqueue into a graph, on a
 * private stream, and instantiates it; nothing runs at creation.  The graph
 * holds the batch's device pointers and its host values (n_rows,
 * max_ctx_bound, page_stride), which size the grids.  Each replay
 * (ril_graph_launch) reads the device buffers as they are at replay time, so
 * the caller may rewrite in place, between replays, ctx_len (each <= the
 * captured max_ctx_bound), page_table, target_ids, token_ids / q / k / v, the
 * weights and the KV pool; n_rows and the addresses stay as captured.  A
 * replay gives bitwise the logprobs of the uncaptured call on the same inputs
 * (the same kernels with the same arguments).  Replays on one stream run in
 * order; the workspace is shared with every other call that uses `ws`, so a
 * replay and another call on the same workspace must be ordered (same stream).
 * Errors: the arguments are checked as ril_decode_step_logprobs checks them
 * (RIL_EINVAL / RIL_ERANGE, nothing captured); a capture or instantiation
 * failure returns RIL_EHIP.  *out receives the graph, to be released with
 * ril_graph_destroy (which must not run while a replay is pending). */
typedef struct ril_graph ril_graph;
ril_status ril_decode_graph_create(const ril_model *m, ril_kv *kv, const ril_decode_batch *b,
                                   float *logprob_out, void *ws, size_t ws_bytes, ril_graph **out);
ril_status ril_graph_launch(ril_graph *g, void *stream);
void ril_graph_destroy(ril_graph *g);

/* The shared KV write path alone (S5): writes the batch's k/v (QKV layout
 * of ril_prefill_batch; target_ids, token_ids and q are ignored) into the
 * pages, nothing else.  Used to lay down history that no logprob is asked
 * for.  Needs no workspace, so n_seqs and total_tokens are not bounded by
 * max_tokens. */
ril_status ril_kv_write(const ril_model *m, ril_kv *kv, const ril_prefill_batch *b, void *stream);

/* Thread-local message describing the last non-OK status. */
const char *ril_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* RIL_H */
