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

// One step of a DPP prefix pattern: op(x, x of the lane the control selects),
// `ident` where that lane is outside the row or the row is masked off.
#define DSA_DPP_STEP(x, ident, op, ctrl, rmask) \
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)(ident), (int)(x), ctrl, rmask, 0xf, false))

// Inclusive prefix of a wave's 64 lanes under op on the DPP network: shifts
// by 1, 2, 4 and 8 lanes within each row of 16, then lane 15 of each row
// broadcast into rows 1 and 3 and lane 31 into rows 2 and 3.  No LDS traffic.
template <class Op>
__device__ __forceinline__ uint32_t wave_incl_dpp(uint32_t x, uint32_t ident, Op op) {
  DSA_DPP_STEP(x, ident, op, 0x111, 0xf);   // row_shr:1
  DSA_DPP_STEP(x, ident, op, 0x112, 0xf);   // row_shr:2
  DSA_DPP_STEP(x, ident, op, 0x114, 0xf);   // row_shr:4
  DSA_DPP_STEP(x, ident, op, 0x118, 0xf);   // row_shr:8
  DSA_DPP_STEP(x, ident, op, 0x142, 0xa);   // row_bcast:15
  DSA_DPP_STEP(x, ident, op, 0x143, 0xc);   // row_bcast:31
  return x;
}

// Sum over each aligned group of G lanes (G = 2, 4, 8 or 16) on the DPP
// network, every lane of the group getting the sum: swaps of neighbours and
// of lane pairs within each quad, then the mirror of each half row (quad 0
// with quad 1) and of each row (its halves).  The pairs combined at each step
// hold equal partial sums in both lanes, so every lane of a group ends with
// the same bits.
template <int G>
__device__ __forceinline__ float group_sum_dpp(float x) {
  static_assert(G == 2 || G == 4 || G == 8 || G == 16, "lane groups of 2 to 16");
#define DSA_DPP_ADD(v, ctrl) \
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), ctrl, 0xf, 0xf, false))
  DSA_DPP_ADD(x, 0xb1);                           // quad_perm [1,0,3,2]
  if constexpr (G >= 4) DSA_DPP_ADD(x, 0x4e);     // quad_perm [2,3,0,1]
  if constexpr (G >= 8) DSA_DPP_ADD(x, 0x141);    // row_half_mirror
  if constexpr (G >= 16) DSA_DPP_ADD(x, 0x140);   // row_mirror
#undef DSA_DPP_ADD
  return x;
}

// Inclusive prefix sum across the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  return wave_incl_dpp(x, 0u, [](uint32_t p, uint32_t q) { return p + q; });
}

// Wave-wide sum, minimum, and 64-bit maximum (every lane gets the result).
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(x), 63);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
  const uint32_t r = wave_incl_dpp(x, 0xffffffffu, [](uint32_t p, uint32_t q) { return min(p, q); });
  return (uint32_t)__builtin_amdgcn_readlane((int)r, 63);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  const uint32_t r = wave_incl_dpp(x, 0u, [](uint32_t p, uint32_t q) { return max(p, q); });
  return (uint32_t)__builtin_amdgcn_readlane((int)r, 63);
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#define DSA_DPP_MAX64(ctrl, rmask)                                                              \
  {                                                                                             \
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, ctrl, rmask, 0xf, false); \
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), ctrl, rmask, 0xf, false); \
    v = max(v, ((uint64_t)hi << 32) | lo);                                                      \
  }
  DSA_DPP_MAX64(0x111, 0xf)
  DSA_DPP_MAX64(0x112, 0xf)
  DSA_DPP_MAX64(0x114, 0xf)
  DSA_DPP_MAX64(0x118, 0xf)
  DSA_DPP_MAX64(0x142, 0xa)
  DSA_DPP_MAX64(0x143, 0xc)
#undef DSA_DPP_MAX64
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
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
