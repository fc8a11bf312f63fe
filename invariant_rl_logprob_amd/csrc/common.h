// Device helpers shared by every kernel of the invariant path (gfx950 / CDNA4).
//
// Invariance rules these helpers encode (Bitwise-consistent RL post, section 2):
//  * one MFMA instruction for every contraction (v_mfma_f32_16x16x32_bf16), so an
//    output element's rounding never depends on which kernel or tile size computed it;
//  * bf16 rounding is round-to-nearest-even everywhere (section 4.4, condition 1: one
//    elementwise round-to-nearest rule);
//  * every reduction is a fixed tree over a fixed element->lane map: lane-local
//    sequential sums, then xor-butterflies whose adds are commutative, so all lanes
//    of a butterfly end with the same bits;
//  * exp2/log2 are the hardware v_exp_f32 / v_log_f32, used identically everywhere;
//  * the library is compiled with -ffp-contract=off: an FMA appears only where
//    written as __builtin_fmaf.
#pragma once

#include <hip/hip_runtime.h>
#include <utility>
#include <stdint.h>

namespace ril {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_t;  // storage type of bf16 values

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kPage = 16;        // tokens per KV page
constexpr int kTile = 64;        // tokens per attention KV tile
constexpr int kVocabTile = 256;  // lm-head columns per vocabulary tile

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float exp2f_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2f_hw(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float bf2f(bf16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// fp32 -> bf16, round to nearest even (the IEEE conversion, one v_cvt_pk_bf16_f32 per
// pair on gfx950); NaN stays NaN.  The instruction's results equal the written-out rule
// (add 0x7fff plus the lowest kept bit, truncate) for every non-NaN input, denormals
// included.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// 16-byte loads and stores of global (device) memory; p must point into global memory,
// never into LDS.  The explicit address space makes these global_load/global_store
// instructions: a flat access would also count against the LDS/scalar counter, so every
// wait for an LDS or scalar result would drain all loads in flight.
typedef const u32x4 __attribute__((address_space(1))) *gptr_c16;
typedef u32x4 __attribute__((address_space(1))) *gptr_16;
__device__ __forceinline__ u32x4 ld16(const void *p) { return *(gptr_c16)(p); }
__device__ __forceinline__ void st16(void *p, u32x4 v) { *(gptr_16)(p) = v; }

__device__ __forceinline__ float shfl_xor_f(float v, int mask) { return __shfl_xor(v, mask, 64); }

// Sum over the 16 lanes that share (lane >> 4): xor 1, 2, 4, 8.  Each add is
// commutative, so every lane of the group ends with identical bits.
__device__ __forceinline__ float sum16(float v) {
  v = v + shfl_xor_f(v, 1);
  v = v + shfl_xor_f(v, 2);
  v = v + shfl_xor_f(v, 4);
  v = v + shfl_xor_f(v, 8);
  return v;
}
__device__ __forceinline__ float max16(float v) {
  v = fmaxf(v, shfl_xor_f(v, 1));
  v = fmaxf(v, shfl_xor_f(v, 2));
  v = fmaxf(v, shfl_xor_f(v, 4));
  v = fmaxf(v, shfl_xor_f(v, 8));
  return v;
}
// The value of lane l and of lane l^16 (xchg16) or l^32 (xchg32), as a pair whose order
// depends on the lane: the row swaps of gfx950 (v_permlane16/32_swap, plain VALU work with
// no LDS round trip) applied to two copies of v.  Callers combine the pair with a
// commutative operation, so both lanes of a pair end with identical bits.  The whole wave
// must be active.
struct f32pair {
  float a, b;
};
__device__ __forceinline__ f32pair xchg16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ f32pair xchg32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
// Across the 4 lane groups (lanes l, l^16, l^32, l^48): xor 16 then xor 32.
__device__ __forceinline__ float sum_groups(float v) {
  f32pair p = xchg16(v);
  v = p.a + p.b;
  p = xchg32(v);
  return p.a + p.b;
}
__device__ __forceinline__ float max_groups(float v) {
  f32pair p = xchg16(v);
  v = fmaxf(p.a, p.b);
  p = xchg32(v);
  return fmaxf(p.a, p.b);
}
// Whole-wave sum: xor 32, 16, 8, 4, 2, 1.
__device__ __forceinline__ float sum64(float v) {
  f32pair p = xchg32(v);
  v = p.a + p.b;
  p = xchg16(v);
  v = p.a + p.b;
  v = v + shfl_xor_f(v, 8);
  v = v + shfl_xor_f(v, 4);
  v = v + shfl_xor_f(v, 2);
  v = v + shfl_xor_f(v, 1);
  return v;
}

// LDS reads the compiler's wait pass does not track (inline asm, no memory clobber): the
// data arrives by direct-to-LDS loads, and a tracked LDS read would make the pass wait
// for every such load in flight.  Callers order them after the copies they read (vmcnt
// wait + barrier), wait for them with lds_wait<N> (LDS reads complete in order, so at
// most the N newest are then pending) and pass each value through settle() before use.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}
// base: this lane's LDS byte address; OFF: a byte offset common to all lanes, folded into
// the instruction (< 65536)
template <int OFF>
__device__ __forceinline__ u32x4 lds_rd128(uint32_t base) {
  static_assert(OFF >= 0 && OFF < 65536, "LDS offset field");
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(base), "i"(OFF));
  return r;
}
template <int OFF>
__device__ __forceinline__ int lds_rd32(uint32_t base) {
  static_assert(OFF >= 0 && OFF < 65536, "LDS offset field");
  int r;
  asm volatile("ds_read_b32 %0, %1 offset:%2" : "=v"(r) : "v"(base), "i"(OFF));
  return r;
}
// transposing read: lane i of each 16-lane group gets element i%4 of the 8-byte chunks
// addressed by lanes 4e + i/4 of its group, e = 0..3
template <int OFF>
__device__ __forceinline__ u32x2 lds_rdtr(uint32_t base) {
  static_assert(OFF >= 0 && OFF < 65536, "LDS offset field");
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(base), "i"(OFF));
  return r;
}
// f(integral_constant<int, 0>), ..., f(integral_constant<int, N-1>), in order
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F &f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}
template <int N>
__device__ __forceinline__ void lds_wait() {
  static_assert(N >= 0 && N <= 15, "lgkmcnt field");
  asm volatile("s_waitcnt lgkmcnt(%0)" ::"i"(N) : "memory");
}
template <typename T>
__device__ __forceinline__ void settle(T &v) { asm volatile("" : "+v"(v)); }
// s_waitcnt vmcnt(N): wait until at most N vector-memory operations of this wave are
// outstanding (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N <= 63, "vmcnt field");
  asm volatile("s_waitcnt vmcnt(%0)" ::"i"(N) : "memory");
}

// Two OCP E4M3 codes (low 16 bits: a, then b) of values already multiplied by their
// scale's inverse.  The hardware conversion rounds to nearest even but turns magnitudes
// past 464 into NaN, so the clamp to +-448 (satfinite) comes first; NaN is encoded here
// with its sign.
__device__ __forceinline__ uint32_t fp8_codes2(float a, float b) {
  const float ca = fminf(fmaxf(a, -448.f), 448.f), cb = fminf(fmaxf(b, -448.f), 448.f);
  uint32_t r = __builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, 0, false) & 0xffffu;
  if (a != a) r = (r & 0xff00u) | (0x7fu | ((__float_as_uint(a) >> 24) & 0x80u));
  if (b != b) r = (r & 0x00ffu) | ((0x7fu | ((__float_as_uint(b) >> 24) & 0x80u)) << 8);
  return r;
}

// Sequence lookup for packed token j: the s with cu[s] <= j < cu[s+1].
__device__ __forceinline__ int locate_seq(const int32_t *__restrict__ cu, int n_seqs, int j) {
  int lo = 0, hi = n_seqs - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= j) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace ril
