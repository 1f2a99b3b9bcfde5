// bf16 MFMA helpers for gfx950 (16x16x32, fp32 accumulation).
//
// Operand layout of v_mfma_f32_16x16x32_bf16 for lane l = 16 q + i:
//   A (16 x 32): lane supplies row i, k = 8 q .. 8 q + 7
//   B (32 x 16): lane supplies column i, k = 8 q .. 8 q + 7
//   D (16 x 16): lane holds rows 4 q .. 4 q + 3 of column i
// The transposing LDS read (ds_read_b64_tr_b16) hands lane i of each 16-lane
// group element i % 4 of the 8-byte pieces addressed by lanes 4 k + i / 4,
// k = 0..3, which turns a row-major [key][dim] tile into the A operand of
// V^T without a register shuffle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
// 16 raw bytes as a native vector (HIP's uint4 is a struct whose copies can
// keep arrays of it out of registers)
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) {
  bf16x8 r;
  __builtin_memcpy(&r, &u, 16);
  return r;
}

// Eight floats -> bf16, round to nearest even (gfx950 converts two per
// v_cvt_pk_bf16_f32; finite inputs).
__device__ __forceinline__ bf16x8 pack8(const float* p) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)p[i];
  return r;
}

// 2^x with the hardware instruction alone (v_exp_f32): softmax arguments are
// <= 0, where results below the normal range flushing to zero is harmless.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Reductions over lane pairs l, l ^ 16 and l, l ^ 32 with the gfx950 lane
// swaps (VALU, no LDS round trip).  With x in both operands each lane gets
// the values of the pair's lower and upper lane, in that order, so both lanes
// of a pair compute the same result bit for bit.
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Transposing 8-byte LDS read at lds_base + byte_off (see above).
__device__ __forceinline__ uint2 lds_tr(const char* lds_base, int byte_off) {
  const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4i16*)((__attribute__((address_space(3))) char*)lds_base + byte_off));
  uint2 r;
  __builtin_memcpy(&r, &v, 8);
  return r;
}

}  // namespace dsa
