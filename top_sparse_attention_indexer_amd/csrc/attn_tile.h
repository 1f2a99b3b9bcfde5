// Per-step core of the bf16 MFMA attention kernels (gfx950), shared by the
// prefill kernels: one wave, 32 keys per step, the 16 MFMA columns being
// query heads or query rows.
//
//   S^T [16 keys x 16 cols] = K_tile [16 x d] . Q^T [d x 16]   (two halves)
//   online softmax per column, in registers (a lane owns one column; the
//     four lane quads hold 4 keys each of every 16-key half);
//   O^T [16 dims x 16 cols] += V^T [16 dims x 32 keys] . P^T [32 keys x 16]
//     with P^T the MFMA B operand straight from registers and V^T read from a
//     row-major LDS tile with the transposing LDS load.
// Scores are kept in the log2 domain (scale * log2(e) folded in), so the
// exponentials are single v_exp_f32 instructions.
#pragma once

#include "common.h"
#include "mfma.h"

namespace dsa {

constexpr int VSTR = 288;        // LDS row stride of a 32 x d value tile (bytes)
constexpr int KSTR = 272;        // LDS row stride of a key tile (bytes)
constexpr float kLog2e = 1.4426950408889634f;

// Shared per-step core: given this wave's two 16-key halves (A operands for
// S^T already loaded), the 32 x d value tile in LDS, update the running
// state of the lane's column.
template <int HD>
struct ColState {
  float m, l;
  f32x4 o[HD / 16];
};

template <int HD>
__device__ __forceinline__ void step_core(const uint4 (&ka)[2][HD / 32], const bf16x8 (&qb)[HD / 32],
                                          const bool (&kvalid)[2][4], const char* vtile,
                                          float scale_log2, ColState<HD>& st) {
  constexpr int T = HD / 32;
  const int lane = threadIdx.x & 63;
  const int q = lane >> 4, i = lane & 15;
  float s[8];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < T; ++t) acc = mfma16(as_bf16x8(ka[u][t]), qb[t], acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) s[u * 4 + r] = kvalid[u][r] ? acc[r] * scale_log2 : -INFINITY;
  }
  float mt = s[0];
#pragma unroll
  for (int x = 1; x < 8; ++x) mt = fmaxf(mt, s[x]);
  mt = max_xor16(mt);
  mt = max_xor32(mt);
  const float mnew = fmaxf(st.m, mt);
  float alpha = 1.f;
  float p[8];
  if (mnew == -INFINITY) {
#pragma unroll
    for (int x = 0; x < 8; ++x) p[x] = 0.f;
  } else {
    alpha = exp2_fast(st.m - mnew);
#pragma unroll
    for (int x = 0; x < 8; ++x) p[x] = exp2_fast(s[x] - mnew);
  }
  float ps = 0.f;
#pragma unroll
  for (int x = 0; x < 8; ++x) ps += p[x];
  st.l = st.l * alpha + ps;  // this lane's keys only; summed over quads at the end
  st.m = mnew;
  const bf16x8 pb = pack8(p);
  // value tile rows: first half keys 4q+k, second half 16+4q+k; this lane
  // (4k + c within its 16-lane group) points at row 4q + i/4, dims 4*(i%4)
  const int row0 = 4 * q + (i >> 2);
  const int colb = (i & 3) * 8;  // bytes
#pragma unroll
  for (int dt = 0; dt < HD / 16; ++dt) {
    const uint2 lo = lds_tr(vtile, row0 * VSTR + dt * 32 + colb);
    const uint2 hi = lds_tr(vtile, (16 + row0) * VSTR + dt * 32 + colb);
    uint4 u;
    u.x = lo.x; u.y = lo.y; u.z = hi.x; u.w = hi.y;
    f32x4 o = st.o[dt];
#pragma unroll
    for (int r = 0; r < 4; ++r) o[r] *= alpha;
    st.o[dt] = mfma16(as_bf16x8(u), pb, o);
  }
}

// Byte offset of bytes [cb, cb + 8) of row R in a value tile of HD-wide bf16
// rows stored back to back (row stride HD * 2 bytes, as the direct
// global-to-LDS load writes them) with the 16-byte chunks of row R permuted
// by chunk ^ 2 * (R mod CPR/2): the transposing read of four consecutive rows
// (one 16-lane group) then touches four different bank ranges.
template <int HD>
__device__ __forceinline__ int vt_swz(int R, int cb) {
  constexpr int CPR = HD / 8;
  const int c16 = cb >> 4;
  return R * (HD * 2) + ((c16 ^ ((R & (CPR / 2 - 1)) << 1)) << 4) + (cb & 15);
}

// Byte offset of 16-byte chunk c16 of row R in a key tile of HD-wide bf16
// rows stored back to back, chunks permuted by c16 ^ (R mod CPR): sixteen
// lanes reading the same chunk of sixteen consecutive rows hit sixteen
// different bank ranges.
template <int HD>
__device__ __forceinline__ int kt_swz(int R, int c16) {
  constexpr int CPR = HD / 8;
  return R * (HD * 2) + ((c16 ^ (R & (CPR - 1))) << 4);
}

// Running maximum with a lazy update: the reference maximum m of a column
// moves only when a new score exceeds it by more than kLazyLog2 (log2
// units), so most steps skip the rescale of the accumulators.  Exact: every
// weight is exp2(s - m) with the same m for numerator and denominator, and
// bounded by 2^kLazyLog2 (fine for the fp32 sums and the bf16 P operand).
constexpr float kLazyLog2 = 8.f;

// Chunk permutation of the sparse path's key and value tiles: 16-byte chunk
// c16 of tile row R sits at chunk c16 ^ sp_f(R) of the row (rows back to
// back, HD * 2 bytes each).  sp_f is a permutation of bits of R, hence
// linear under xor: sp_f(a ^ b) = sp_f(a) ^ sp_f(b).  It keeps both reads of
// a tile free of bank conflicts: the key read (sixteen lanes, one chunk of
// sixteen consecutive rows) meets sixteen different 16-byte bank ranges, and
// the transposing value read (each 16-lane group, 32 bytes of four
// consecutive rows) keeps the two chunks of a 32-byte piece together (bit 0
// of sp_f only swaps them) while the rows' pieces land on different ranges.
// Because one permutation serves both tiles, the staging lane that loads
// row R of either tile fetches global chunk ch ^ sp_f(R) and stores it at
// chunk ch of the tile row: its store addresses differ by whole rows, which
// the LDS store takes as an immediate offset.
template <int HD>
__device__ __forceinline__ int sp_f(int R) {
  static_assert(HD == 64 || HD == 128, "sparse tiles hold 64- or 128-wide rows");
  if constexpr (HD == 128) return ((R & 7) << 1) | ((R >> 3) & 1);
  else return (((R >> 1) & 3) << 1) | ((R >> 3) & 1);
}

// 32-key step with both tiles in LDS (rows back to back, chunks permuted by
// sp_f): the key rows are read as the A operand (lane quad q takes logical
// bytes 64 t + 16 q of its key row, the order the query operand uses), the
// value rows with the transposing read.  All value reads of the step are
// issued right after the score MFMAs, so their latency runs under the
// softmax instead of once per output MFMA.  Raw scores s; the scale c
// (softmax scale * log2 e) enters through p = exp2(s * c - m).
template <int HD>
__device__ __forceinline__ void step32_lds(const char* ktile, const char* vtile,
                                           const bf16x8 (&qb)[HD / 32], const bool (&kvalid)[2][4],
                                           float c, ColState<HD>& st) {
  constexpr int T = HD / 32;
  constexpr int RB = HD * 2;            // tile row bytes
  const int lane = threadIdx.x & 63;
  const int q = lane >> 4, i = lane & 15;
  float s[8];
  uint4 ka[2][T];
  const int fi = sp_f<HD>(i);           // rows i and 16 + i permute alike
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int t = 0; t < T; ++t)
      ka[u][t] = *reinterpret_cast<const uint4*>(ktile + (u * 16 + i) * RB +
                                                 (((4 * t + q) ^ fi) << 4));
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < T; ++t) acc = mfma16(as_bf16x8(ka[u][t]), qb[t], acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) s[u * 4 + r] = kvalid[u][r] ? acc[r] : -INFINITY;
  }
  // value tile rows: first half keys 4q+k, second half 16+4q+k; this lane
  // (4k + c within its 16-lane group) reads row 4q + i/4, bytes 8 * (i % 4)
  // of each 32-byte piece
  const int row0 = 4 * q + (i >> 2);
  const int vb = row0 * RB + ((((i & 3) >> 1) ^ sp_f<HD>(row0)) << 4) + (i & 1) * 8;
  uint4 vv[HD / 16];
#pragma unroll
  for (int dt = 0; dt < HD / 16; ++dt) {
    const uint2 lo = lds_tr(vtile, vb ^ (dt << 5));
    const uint2 hi = lds_tr(vtile, (vb ^ (dt << 5)) + 16 * RB);
    vv[dt].x = lo.x; vv[dt].y = lo.y; vv[dt].z = hi.x; vv[dt].w = hi.y;
  }
  float mt = s[0];
#pragma unroll
  for (int x = 1; x < 8; ++x) mt = fmaxf(mt, s[x]);
  mt = max_xor32(max_xor16(mt)) * c;
  // lazy maximum: move only on a jump of more than kLazyLog2 (or the first
  // finite score); the rescale runs only if some column of the wave moved
  const bool bump = mt > st.m + kLazyLog2;
  if (__builtin_amdgcn_ballot_w64(bump)) {
    const float mnew = bump ? mt : st.m;
    const float alpha = exp2_fast(st.m - mnew);   // 1 where unchanged, 0 from -inf
#pragma unroll
    for (int dt = 0; dt < HD / 16; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) st.o[dt][r] *= alpha;
    st.l *= alpha;
    st.m = mnew;
  }
  // a column whose maximum is still -inf has only masked scores, which give
  // exp2(-inf) = 0 against any finite subtrahend
  const float msub = st.m == -INFINITY ? 0.f : st.m;
  float p[8];
#pragma unroll
  for (int x = 0; x < 8; ++x) p[x] = exp2_fast(fmaf(s[x], c, -msub));
  float ps = 0.f;
#pragma unroll
  for (int x = 0; x < 8; ++x) ps += p[x];
  st.l += ps;
  const bf16x8 pb = pack8(p);
#pragma unroll
  for (int dt = 0; dt < HD / 16; ++dt) st.o[dt] = mfma16(as_bf16x8(vv[dt]), pb, st.o[dt]);
}

}  // namespace dsa
