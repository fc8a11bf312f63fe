// RMSNorm of one row by one wave (S3), shared by the stand-alone RMSNorm kernel and the
// decode merge kernel that normalises the merged attention row it has just formed, so
// both produce the same bits by construction.
//   y = bf16((x * r) * g),  r = 1 / sqrt(mean(x^2) + eps)  (IEEE divides and square root)
// Lane l owns the 8-element chunks l, l+64, ...; its sum of squares is one fma chain over
// its chunks in order (elements in order within a chunk), then the whole-wave xor
// butterfly sum64.  `load(e)` returns chunk e (8 bf16 as 4 words), `store(e, w)` writes
// chunk e of y.
#pragma once

#include "common.h"

namespace ril {

template <typename Load, typename Store>
__device__ __forceinline__ void rmsnorm_row(Load load, Store store, int d, const bf16_t *__restrict__ gain,
                                            float eps, bool poison) {
  const int lane = threadIdx.x & 63, n8 = d / 8;
  float acc = 0.f;
  for (int e = lane; e < n8; e += 64) {
    const u32x4 v = load(e);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float a = bf2f((bf16_t)(v[w] & 0xffffu)), b = bf2f((bf16_t)(v[w] >> 16));
      acc = __builtin_fmaf(a, a, acc);
      acc = __builtin_fmaf(b, b, acc);
    }
  }
  acc = sum64(acc);
  const float mean = __fdiv_rn(acc, (float)d);
  float r = __fdiv_rn(1.0f, __fsqrt_rn(mean + eps));
  if (poison) r = __builtin_nanf("");
  for (int e = lane; e < n8; e += 64) {
    const u32x4 v = load(e);
    u32x4 g = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};  // bf16 1.0 pairs
    if (gain) g = ld16(gain + e * 8);
    u32x4 out;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float a = bf2f((bf16_t)(v[w] & 0xffffu)), b = bf2f((bf16_t)(v[w] >> 16));
      const float ga = bf2f((bf16_t)(g[w] & 0xffffu)), gb = bf2f((bf16_t)(g[w] >> 16));
      out[w] = pack2((a * r) * ga, (b * r) * gb);
    }
    store(e, out, v);
  }
}

}  // namespace ril
