// Device helpers shared by the gfx950 kernels of libdsa.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define DSA_WAVE 64

typedef uint16_t bf16_bits;

__device__ __forceinline__ float bf16_to_f32(bf16_bits b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// Element loads widened to float.
__device__ __forceinline__ float ld_f(const float* p, size_t i) { return p[i]; }
__device__ __forceinline__ float ld_f(const bf16_bits* p, size_t i) { return bf16_to_f32(p[i]); }

// Eight consecutive elements (16-byte aligned for bf16, 32-byte for fp32).
__device__ __forceinline__ void ld8(const bf16_bits* p, float* o) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  o[0] = __uint_as_float(u.x << 16); o[1] = __uint_as_float(u.x & 0xffff0000u);
  o[2] = __uint_as_float(u.y << 16); o[3] = __uint_as_float(u.y & 0xffff0000u);
  o[4] = __uint_as_float(u.z << 16); o[5] = __uint_as_float(u.z & 0xffff0000u);
  o[6] = __uint_as_float(u.w << 16); o[7] = __uint_as_float(u.w & 0xffff0000u);
}
__device__ __forceinline__ void ld8(const float* p, float* o) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
  o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}

// Order-preserving map of a float32 score to an unsigned key: a larger score
// gives a larger key; -0.0 is mapped like +0.0 so that the two compare equal.
__device__ __forceinline__ uint32_t radix_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (DSA_WAVE - 1); }

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = lane_id();
  return (l == 0) ? 0ull : ((~0ull) >> (64 - l));
}

// Inclusive prefix sum across the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  const int l = lane_id();
#pragma unroll
  for (int o = 1; o < DSA_WAVE; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, DSA_WAVE);
    if (l >= o) x += y;
  }
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = DSA_WAVE / 2; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, DSA_WAVE));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = DSA_WAVE / 2; o > 0; o >>= 1) x += __shfl_xor(x, o, DSA_WAVE);
  return x;
}

// Exclusive prefix sum over the threads of a block (thread-index order).
// `scratch` holds one uint32 per wave plus one for the total.  Returns the
// exclusive prefix; `total` receives the block sum.  Contains barriers: every
// thread of the block must call it.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t x, uint32_t* scratch, uint32_t& total) {
  constexpr int NW = NT / DSA_WAVE;
  const int w = threadIdx.x / DSA_WAVE;
  const uint32_t inc = wave_incl_scan(x);
  if (lane_id() == DSA_WAVE - 1) scratch[w] = inc;
  __syncthreads();
  uint32_t off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const uint32_t s = scratch[i];
    off += (i < w) ? s : 0u;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return off + inc - x;
}

// Ordered compaction helper: for a predicate evaluated by every thread of a
// block, the rank of this thread among the set predicates of lower thread
// index, and the block count.  Uses one ballot per wave.  Contains barriers.
template <int NT>
__device__ __forceinline__ uint32_t block_rank(bool pred, uint32_t* scratch, uint32_t& total) {
  constexpr int NW = NT / DSA_WAVE;
  const int w = threadIdx.x / DSA_WAVE;
  const uint64_t m = __ballot(pred);
  const uint32_t in_wave = (uint32_t)__popcll(m & lanemask_lt());
  if (lane_id() == 0) scratch[w] = (uint32_t)__popcll(m);
  __syncthreads();
  uint32_t off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const uint32_t s = scratch[i];
    off += (i < w) ? s : 0u;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return off + in_wave;
}
