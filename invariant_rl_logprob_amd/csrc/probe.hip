// HBM read ceiling probe (benchmarking only): a grid-stride read of a device buffer with
// the nontemporal policy, 16 bytes per lane per load, folded into one word per
// workgroup so the reads cannot be dropped.  The rate it reaches is the practical
// ceiling for the read-streaming kernels of the path (the published 8 TB/s is the other
// reference).
#include "common.h"
#include "kernels.h"

namespace ril {

constexpr int kProbeBlocks = 2048;

__global__ __launch_bounds__(256) void hbm_read_probe_kernel(const uint8_t *__restrict__ src, long n16,
                                                             uint32_t *__restrict__ out) {
  __shared__ uint32_t red[4];
  const long tid = (long)blockIdx.x * 256 + threadIdx.x, nt = (long)gridDim.x * 256;
  u32x4 x = u32x4{0u, 0u, 0u, 0u};
  for (long i = tid; i < n16; i += nt)
    x ^= __builtin_nontemporal_load((const u32x4 __attribute__((address_space(1))) *)(src + i * 16));
  uint32_t v = x[0] ^ x[1] ^ x[2] ^ x[3];
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) v ^= (uint32_t)__shfl_xor((int)v, off, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

int hbm_read_probe_blocks() { return kProbeBlocks; }

hipError_t launch_hbm_read_probe(const void *src, size_t bytes, uint32_t *out, hipStream_t st) {
  const long n16 = (long)(bytes / 16);
  if (n16 == 0) return hipSuccess;
  hipLaunchKernelGGL(hbm_read_probe_kernel, dim3(kProbeBlocks), dim3(256), 0, st, (const uint8_t *)src, n16, out);
  return hipGetLastError();
}

}  // namespace ril
