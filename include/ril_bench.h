/* Benchmarking, profiling and test hooks of the invariant logprob library.
 *
 * These entry points are not part of the method's path: a comparator policy that
 * deliberately gives up invariance (to price it), an HBM read-rate probe, a per-kernel
 * event trace and a workspace view for tests.  They are exported by the same library
 * (libril.so) and declared apart so that a caller of the path (include/ril.h) never
 * needs them.  Same conventions as ril.h: plain pointers, ril_status returns, validation
 * on the host before anything is enqueued. */
#ifndef RIL_BENCH_H
#define RIL_BENCH_H

#include "ril.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Comparator, for benchmarking only.  RIL_POLICY_INVARIANT (the default) is the
 * method: every reduction order is fixed by the model alone.  RIL_POLICY_SHAPE_DERIVED
 * makes the same kernels choose their work split from the call's shape, as a
 * throughput-first engine would, so that the price of invariance can be measured:
 *   - decode attention's KV split (tokens): attn_split_tokens if non-zero (a multiple
 *     of 64, at most 1024 for GQA and 2048 for MLA), else enough splits for two waves
 *     per SIMD of the device, ceil(max_ctx_bound / splits) rounded up to 64, widened
 *     until the partials fit the invariant workspace;
 *   - projection GEMMs whose tile grid is smaller than the device's compute-unit count
 *     split their K loop (at most 16 chunks of at least 256) and add the fp32 chunk
 *     results in a second kernel.
 * Under it, results depend on the batch and decode no longer equals prefill.  Setting
 * it queries the current device's compute-unit count and enlarges
 * ril_workspace_bytes(m) by the split-K partial buffer.  Returns RIL_EINVAL for an
 * unknown policy or a bad override, RIL_EHIP if the device cannot be queried. */
enum { RIL_POLICY_INVARIANT = 0, RIL_POLICY_SHAPE_DERIVED = 1 };
ril_status ril_set_policy(ril_model *m, int32_t policy, int32_t attn_split_tokens);

/* HBM read ceiling probe, for benchmarking only (like ril_set_policy): enqueue, on
 * `stream`, one grid-stride read of the first floor(bytes / 16) * 16 bytes of the device
 * buffer src (16-byte aligned) with the nontemporal policy, as the path's streaming
 * kernels read, folding the data into out[ril_hbm_read_probe_words()] (device uint32)
 * so the reads cannot be elided.  Time it with events to get the practical read rate.
 * Returns RIL_EINVAL on a null or misaligned pointer, RIL_EHIP on a launch error. */
int32_t ril_hbm_read_probe_words(void);
ril_status ril_hbm_read_probe(const void *src, size_t bytes, uint32_t *out, void *stream);

/* Kernel trace, a profiling hook.  While enabled, every launch of the kernels
 * below is bracketed by two hipEvents recorded on the launch stream (the
 * kernels themselves are unchanged).  ril_trace_read waits for the events
 * recorded so far -- a host wait, so call it outside a timed loop -- and
 * returns the summed elapsed milliseconds and the launch count of one kernel
 * since the last ril_trace_enable.  Process-wide; not for concurrent use. */
enum {
  RIL_K_KV_WRITE = 0,     /* S5 */
  RIL_K_ATTN_SPLIT = 1,   /* S8  decode split-KV attention */
  RIL_K_ATTN_MERGE = 2,   /* S9  decode split merge */
  RIL_K_ATTN_PREFILL = 3, /* S10 */
  RIL_K_RMSNORM = 4,      /* S2/S3 */
  RIL_K_GEMM = 5,         /* S4 */
  RIL_K_LM_HEAD = 6,      /* S11 */
  RIL_K_VOCAB_MERGE = 7,  /* S12 */
  RIL_K_INDEXER = 8,      /* S6 */
  RIL_K_TOPK = 9,         /* S7 */
  RIL_K_SILU_MUL = 10,    /* the SwiGLU activation */
  RIL_K_QUANT_ROWS = 11,  /* W8A8 head: block-FP8 activation quantization */
  RIL_K_LM_HEAD_FP8 = 12, /* S11 in W8A8 block FP8 */
  RIL_K_GEMM_FP8 = 13,    /* S4 in W8A8 block FP8 */
  RIL_K_SSD_CHUNK = 14,   /* SSD: plan, chunk state sums, state scan, commit, input write */
  RIL_K_SSD_OUT = 15,     /* SSD: the positions' outputs */
  RIL_K_COUNT = 16
};
ril_status ril_trace_enable(int on);
ril_status ril_trace_read(int kernel, double *total_ms, int64_t *launches);

/* Debug/test view: the attention output of the last call on this thread's
 * workspace is bf16 [rows, Hq, D] at byte offset ril_ws_attn_offset(m) of
 * `ws`.  Lets tests compare attention outputs, not just logprobs. */
size_t ril_ws_attn_offset(const ril_model *m);

#ifdef __cplusplus
}
#endif
#endif /* RIL_BENCH_H */
