/* The indexer's scores in the precision the top-k selection is decided in.
 *
 * TEST INFRASTRUCTURE ONLY: part of the CPU oracle (see oracle/__init__.py).  It shares
 * no code with the HIP library; only the oracle's Python side loads it.
 *
 * The pages say only that an indexer scores every history position before the top-k
 * selection (Bitwise-consistent RL post, sections 3 and 4.3).
 * The reading taken: I[s] = sum over heads h of relu(q_h . k_s), with unit head weights,
 * in float32, each dot product a chain of fused multiply-adds over d = 0, 1, ..., D-1
 * starting from +0 (one rounding per term: fmaf, the C99 fused multiply-add, which
 * rounds the exact a*b + c once to the nearest float, ties to even), and the heads
 * summed h = 0, 1, ..., H-1 with one float32 rounding per add, relu(x) = x if x > 0
 * else +0.  A selection is an integer decided by these floats, so the checker must
 * take the same roundings as the kernel, not merely come close.
 *
 * q [heads][dim], kt = K transposed [dim][n] (so the loop over positions runs over
 * contiguous memory), out [n], acc [n] scratch.  Every position is computed on its own;
 * the loops over positions only evaluate many of them side by side.
 */
#include <math.h>

void oracle_indexer_fma(const float *q, int heads, int dim, const float *kt, long n, float *out,
                        float *acc) {
  for (long s = 0; s < n; ++s) out[s] = 0.0f;
  for (int h = 0; h < heads; ++h) {
    for (long s = 0; s < n; ++s) acc[s] = 0.0f;
    for (int d = 0; d < dim; ++d) {
      const float qv = q[(long)h * dim + d];
      const float *kd = kt + (long)d * n;
      for (long s = 0; s < n; ++s) acc[s] = fmaf(qv, kd[s], acc[s]);
    }
    for (long s = 0; s < n; ++s) out[s] = out[s] + (acc[s] > 0.0f ? acc[s] : 0.0f);
  }
}
