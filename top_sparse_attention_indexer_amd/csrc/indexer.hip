// Indexer scores: s[b,n,j] = q_idx[b,n,:] . k_idx[b,j,:] for visible j.
//
// The plain product of the page "超大规模MoE架构中稀疏注意力机制的演进与实践"
// (§二.1 coarse relevance of the query to every past position, §二.2 no
// rotary term) and of "混合注意力架构演进：从线性注意力到稀疏门控的技术权衡"
// (§三, the indexer_score stage).  float32 accumulation in a fixed order.
#include "common.h"
#include "launch.h"
#include "mfma.h"

namespace dsa {
namespace {

__device__ __forceinline__ bool seq_has_sparse(const uint8_t* route, int b, int Hq) {
  if (!route) return true;
  for (int h = 0; h < Hq; ++h)
    if (route[(size_t)b * Hq + h]) return true;
  return false;
}

// 64 query rows x 64 keys per workgroup, 4x4 outputs per thread.
template <typename TI>
__global__ __launch_bounds__(256) void k_indexer_tiles(
    const TI* __restrict__ q_idx, const TI* __restrict__ k_idx, int N, int L, int D,
    int n0, int R, int ncols, float* __restrict__ out, size_t ld, int write_masked,
    const uint8_t* __restrict__ route, int Hq, int rpt) {
  const int b = blockIdx.z;
  const int r0 = blockIdx.y * 64;
  const int j0 = blockIdx.x * 64;
  if (!seq_has_sparse(route, b, Hq)) return;
  const int rows_here = min(64, R - r0);
  const int p_last = L - N + (n0 + r0 + rows_here - 1) / rpt;
  const bool tile_masked = j0 > p_last;
  if (tile_masked && !write_masked) return;

  __shared__ float qs[64][33];
  __shared__ float ks[64][33];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) acc[i][jj] = 0.f;

  if (!tile_masked) {
    for (int c0 = 0; c0 < D; c0 += 32) {
      for (int e = threadIdx.x; e < 64 * 32; e += 256) {
        const int rr = e >> 5, cc = e & 31;
        const int rq = r0 + rr, jk = j0 + rr;
        float qv = 0.f, kv = 0.f;
        if (rq < R && c0 + cc < D) qv = ld_f(q_idx, ((size_t)b * N * rpt + n0 + rq) * D + c0 + cc);
        if (jk < L && c0 + cc < D) kv = ld_f(k_idx, ((size_t)b * L + jk) * D + c0 + cc);
        qs[rr][cc] = qv;
        ks[rr][cc] = kv;
      }
      __syncthreads();
#pragma unroll 8
      for (int cc = 0; cc < 32; ++cc) {
        float a[4], bb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = qs[ty * 4 + i][cc];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) bb[jj] = ks[tx + 16 * jj][cc];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) acc[i][jj] = fmaf(a[i], bb[jj], acc[i][jj]);
      }
      __syncthreads();
    }
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = r0 + ty * 4 + i;
    if (r >= R) continue;
    const int p = L - N + (n0 + r) / rpt;
    float* orow = out + ((size_t)b * R + r) * ld;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int j = j0 + tx + 16 * jj;
      if (j >= ncols) continue;
      if (j <= p) orow[j] = acc[i][jj];
      else if (write_masked) orow[j] = -INFINITY;
    }
  }
}

// bf16 indexer inputs on MFMA: 64 query rows x 128 keys per workgroup.  Wave
// w takes query rows 16 w .. 16 w + 15 as the MFMA columns against eight
// blocks of 16 keys as the MFMA rows (S^T = K Q^T, fp32 accumulation over
// d_idx in 32-wide chunks), so each lane ends with 4 consecutive keys of one
// query row and writes them with one 16-byte store.  The key rows of a block
// are read as 64 contiguous bytes per key by the four lane quads.
template <int DIDX>
__global__ __launch_bounds__(256) void k_indexer_mfma(
    const bf16_bits* __restrict__ q_idx, const bf16_bits* __restrict__ k_idx, int N, int L,
    int n0, int R, int ncols, float* __restrict__ out, size_t ld, int write_masked,
    const uint8_t* __restrict__ route, int Hq, int rpt) {
  constexpr int T = DIDX / 32;
  constexpr int UB = T <= 2 ? 8 : 4;   // key blocks whose loads are in flight together
  const int b = blockIdx.z;
  const int r0 = blockIdx.y * 64;
  const int j0 = blockIdx.x * 128;
  if (!seq_has_sparse(route, b, Hq)) return;
  const int rows_here = min(64, R - r0);
  const int p_last = L - N + (n0 + r0 + rows_here - 1) / rpt;
  if (j0 > p_last && !write_masked) return;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int q = lane >> 4, i = lane & 15;
  const int r = r0 + w * 16 + i;      // this lane's query row
  const bool rv = r < R;
  const int p = L - N + (n0 + r) / rpt;
  bf16x8 qb[T];
  {
    const bf16_bits* qr = q_idx + ((size_t)b * N * rpt + n0 + (rv ? r : 0)) * DIDX;
#pragma unroll
    for (int t = 0; t < T; ++t)
      qb[t] = as_bf16x8(rv ? *reinterpret_cast<const uint4*>(qr + t * 32 + q * 8)
                           : make_uint4(0, 0, 0, 0));
  }
  float* orow = out + ((size_t)b * R + (rv ? r : 0)) * ld;
  const bool vec = (ld & 3) == 0;
  const bf16_bits* kseq = k_idx + (size_t)b * L * DIDX;
  for (int u0 = 0; u0 < 8; u0 += UB) {
    if (j0 + 16 * u0 > p_last && !write_masked) break;
    uint4 kb[UB][T];
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const int jk = j0 + 16 * (u0 + u) + i;
      const bool kv = jk < L && jk <= p_last;
#pragma unroll
      for (int t = 0; t < T; ++t)
        kb[u][t] = kv ? *reinterpret_cast<const uint4*>(kseq + (size_t)jk * DIDX + t * 32 + q * 8)
                      : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < T; ++t) acc = mfma16(as_bf16x8(kb[u][t]), qb[t], acc);
      const int jj = j0 + 16 * (u0 + u) + 4 * q;   // keys jj .. jj + 3 of row r
      if (!rv) continue;
      if (vec && jj + 3 < ncols && (jj + 3 <= p || write_masked)) {
        float4 v;
        v.x = (jj <= p) ? acc[0] : -INFINITY;
        v.y = (jj + 1 <= p) ? acc[1] : -INFINITY;
        v.z = (jj + 2 <= p) ? acc[2] : -INFINITY;
        v.w = (jj + 3 <= p) ? acc[3] : -INFINITY;
        *reinterpret_cast<float4*>(orow + jj) = v;
      } else {
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int j = jj + x;
          if (j >= ncols) continue;
          if (j <= p) orow[j] = acc[x];
          else if (write_masked) orow[j] = -INFINITY;
        }
      }
    }
  }
}

// One thread per key; the key row is read once for all RM query rows.
template <typename TI, int RM>
__global__ __launch_bounds__(256) void k_indexer_scan(
    const TI* __restrict__ q_idx, const TI* __restrict__ k_idx, int N, int L, int D,
    int n0, int R, int ncols, float* __restrict__ out, size_t ld, int write_masked,
    const uint8_t* __restrict__ route, int Hq, int rpt) {
  const int b = blockIdx.y;
  if (!seq_has_sparse(route, b, Hq)) return;
  __shared__ float qs[RM][128];
  for (int e = threadIdx.x; e < R * D; e += 256) {
    const int r = e / D, c = e - r * D;
    qs[r][c] = ld_f(q_idx, ((size_t)b * N * rpt + n0 + r) * D + c);
  }
  __syncthreads();
  const int p_max = L - N + (n0 + R - 1) / rpt;
  for (int j = blockIdx.x * 256 + threadIdx.x; j < ncols; j += gridDim.x * 256) {
    float acc[RM];
#pragma unroll
    for (int r = 0; r < RM; ++r) acc[r] = 0.f;
    if (j <= p_max) {
      const TI* kr = k_idx + ((size_t)b * L + j) * D;
      for (int c = 0; c < D; c += 8) {
        float kv[8];
        ld8(kr + c, kv);
#pragma unroll
        for (int r = 0; r < RM; ++r)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[r] = fmaf(qs[r][c + e], kv[e], acc[r]);
      }
    }
#pragma unroll
    for (int r = 0; r < RM; ++r) {
      if (r >= R) break;
      const int p = L - N + (n0 + r) / rpt;
      float* orow = out + ((size_t)b * R + r) * ld;
      if (j <= p) orow[j] = acc[r];
      else if (write_masked) orow[j] = -INFINITY;
    }
  }
}

template <typename TI>
hipError_t scan_dispatch(const Dims& D, const TI* qi, const TI* ki, int n0, int R, int ncols,
                         float* out, size_t ld, bool wm, const uint8_t* route, hipStream_t s) {
  const int blocks = max(1, min((ncols + 255) / 256, 8192));
  dim3 grid(blocks, D.B);
#define DSA_SCAN(RM)                                                                          \
  hipLaunchKernelGGL((k_indexer_scan<TI, RM>), grid, dim3(256), 0, s, qi, ki, D.N, D.L, D.didx, \
                     n0, R, ncols, out, ld, (int)wm, route, D.Hq, D.IH)
  if (R <= 1) DSA_SCAN(1);
  else if (R <= 2) DSA_SCAN(2);
  else if (R <= 4) DSA_SCAN(4);
  else DSA_SCAN(8);
#undef DSA_SCAN
  return hipGetLastError();
}

}  // namespace

hipError_t launch_indexer_tiles(const Dims& D, const void* q_idx, const void* k_idx, int n0, int R,
                                int ncols, float* out, size_t ld, bool write_masked,
                                const uint8_t* route, hipStream_t s) {
  if (D.B == 0 || R == 0 || ncols == 0) return hipSuccess;
  ProfScope ps(s, kStageIndexer);
  if (D.idx_bf16 && (D.didx == 32 || D.didx == 64 || D.didx == 128)) {
    const dim3 g((ncols + 127) / 128, (R + 63) / 64, D.B);
#define DSA_IDX_MFMA(DI)                                                                       \
  hipLaunchKernelGGL(k_indexer_mfma<DI>, g, dim3(256), 0, s, (const bf16_bits*)q_idx,           \
                     (const bf16_bits*)k_idx, D.N, D.L, n0, R, ncols, out, ld, (int)write_masked, \
                     route, D.Hq, D.IH)
    if (D.didx == 32) DSA_IDX_MFMA(32);
    else if (D.didx == 64) DSA_IDX_MFMA(64);
    else DSA_IDX_MFMA(128);
#undef DSA_IDX_MFMA
    return hipGetLastError();
  }
  dim3 grid((ncols + 63) / 64, (R + 63) / 64, D.B);
  if (D.idx_bf16)
    hipLaunchKernelGGL(k_indexer_tiles<bf16_bits>, grid, dim3(256), 0, s, (const bf16_bits*)q_idx,
                       (const bf16_bits*)k_idx, D.N, D.L, D.didx, n0, R, ncols, out, ld,
                       (int)write_masked, route, D.Hq, D.IH);
  else
    hipLaunchKernelGGL(k_indexer_tiles<float>, grid, dim3(256), 0, s, (const float*)q_idx,
                       (const float*)k_idx, D.N, D.L, D.didx, n0, R, ncols, out, ld,
                       (int)write_masked, route, D.Hq, D.IH);
  return hipGetLastError();
}

hipError_t launch_indexer_scan(const Dims& D, const void* q_idx, const void* k_idx, int n0, int R,
                               int ncols, float* out, size_t ld, bool write_masked,
                               const uint8_t* route, hipStream_t s) {
  if (D.B == 0 || R == 0 || ncols == 0) return hipSuccess;
  if (R > 8) return hipErrorInvalidValue;
  ProfScope ps(s, kStageIndexer);
  if (D.idx_bf16)
    return scan_dispatch(D, (const bf16_bits*)q_idx, (const bf16_bits*)k_idx, n0, R, ncols, out, ld,
                         write_masked, route, s);
  return scan_dispatch(D, (const float*)q_idx, (const float*)k_idx, n0, R, ncols, out, ld,
                       write_masked, route, s);
}

}  // namespace dsa
