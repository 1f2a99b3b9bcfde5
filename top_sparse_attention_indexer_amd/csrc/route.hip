// Route producer: the per-head full/sparse decision of a light two-layer
// router on the keys of the call's tokens ("Elastic Attention" page, §2.2:
// the router reads the current key hidden states, is a two-layer MLP and
// decides per attention head; trained with Gumbel-Softmax and a
// straight-through estimator, it takes the hard decision at inference).
//
//   x      = mean over the call's tokens (positions L - N .. L - 1) of their
//            key rows, one vector of C = Hkv * d
//   hidden = max(0, x W1 + b1)                        W1 [C, Hr], b1 [Hr]
//   z      = hidden W2 + b2                           W2 [Hr, Hq, 2], b2 [Hq, 2]
//   route[h] = z[h][1] > z[h][0]  (column 1 sparse, column 0 full; a tie
//              keeps full attention)
//
// The pooling reads every current key once (HBM-bound: N * C * element
// bytes per sequence); the MLP is a few MB of fp32 weights read per
// sequence.  Four launches, all in a fixed summation order, so the same
// input always gives the same decision:
//   k_route_pool    chunk partial sums of the key rows   grid (C / 128, chunks, B)
//   k_route_reduce  mean over the chunks                 grid (C / 64, B)
//   k_route_hidden  first layer + ReLU                   grid (Hr / 64, B), 16 waves
//   k_route_out     second layer, logits and decision    grid (2 Hq / 64, B), 16 waves
#include <hip/hip_runtime.h>

#include <algorithm>

#include "common.h"
#include "launch.h"

namespace dsa {
namespace {

constexpr int RT = 256;
constexpr int MT = 1024;             // threads of the two layer kernels
constexpr int kMinRows = 64;         // key rows per pooling workgroup at least
constexpr int kPoolGroups = 2048;    // pooling workgroups aimed for (all sequences)

// Pooling workgroup: 16 column groups of 8 values x 16 row lanes.
constexpr int kPoolCols = 16, kPoolLanes = RT / kPoolCols;

struct RoutePlan {
  int ncol, nch, rows;    // column blocks, chunks per sequence, rows per chunk
  size_t part_off, x_off, h_off, total;
};

RoutePlan route_plan(const Dims& D, int hidden) {
  RoutePlan P;
  const long long n = std::max(1, D.N);
  const int C = D.Hkv * D.d;
  P.ncol = (C / 8 + kPoolCols - 1) / kPoolCols;
  long long nch = std::max<long long>(1, kPoolGroups / ((long long)P.ncol * std::max(1, D.B)));
  nch = std::min(nch, (n + kMinRows - 1) / kMinRows);
  P.rows = (int)((n + nch - 1) / nch);
  P.nch = (int)((n + P.rows - 1) / P.rows);
  auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
  P.part_off = 0;
  P.x_off = al((size_t)D.B * P.nch * C * 4);
  P.h_off = P.x_off + al((size_t)D.B * C * 4);
  P.total = P.h_off + al((size_t)D.B * hidden * 4);
  return P;
}

__device__ __forceinline__ void load8(const bf16_bits* p, float* v) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ void load8(const float* p, float* v) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// Partial sums of the key rows of one chunk and one block of 128 columns:
// part[b][ch][c].  Thread (row lane ro, group g) adds 8 columns of rows
// ro, ro + 16, ... of the chunk (four loads in flight, added in row order);
// the 16 row lanes of a group are then added in lane order.
template <typename T>
__global__ __launch_bounds__(RT) void k_route_pool(const T* __restrict__ k, int L, int N, int C,
                                                   int rows, int nch, float* __restrict__ part) {
  __shared__ float red[kPoolLanes][kPoolCols * 8 + 4];
  const int cb = blockIdx.x, ch = blockIdx.y, b = blockIdx.z;
  const int t = threadIdx.x;
  const int gl = t % kPoolCols, ro = t / kPoolCols;
  const int g = cb * kPoolCols + gl;
  const bool gv = g < C / 8;
  const long long j0 = (long long)L - N + (long long)ch * rows;
  const long long j1 = std::min<long long>(L, j0 + rows);
  const T* kb = k + (size_t)b * L * C + (gv ? g * 8 : 0);
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  if (gv) {
    long long j = j0 + ro;
    for (; j + 3LL * kPoolLanes < j1; j += 4LL * kPoolLanes) {
      float v[4][8];
#pragma unroll
      for (int u = 0; u < 4; ++u) load8(kb + (size_t)(j + (long long)u * kPoolLanes) * C, v[u]);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += v[u][e];
    }
    for (; j < j1; j += kPoolLanes) {
      float v[8];
      load8(kb + (size_t)j * C, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += v[e];
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[ro][gl * 8 + e] = acc[e];
  __syncthreads();
  // one thread per column of the block adds the 16 row lanes
  if (t < kPoolCols * 8) {
    const int c = cb * kPoolCols * 8 + t;
    float s = red[0][t];
    for (int r = 1; r < kPoolLanes; ++r) s += red[r][t];
    if (c < C) part[((size_t)b * nch + ch) * C + c] = s;
  }
}

// x[b][c] = (sum over chunks of part[b][ch][c]) / N; wave w adds chunks
// w, w + 4, ... (eight loads in flight, added in chunk order); the four wave
// sums are added in wave order.
__global__ __launch_bounds__(RT) void k_route_reduce(const float* __restrict__ part, int nch, int C,
                                                     int N, float* __restrict__ x) {
  __shared__ float s[4][64];
  const int b = blockIdx.y, w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = blockIdx.x * 64 + lane;
  float acc = 0.f;
  if (c < C) {
    const float* pb = part + (size_t)b * nch * C + c;
    int ch = w;
    for (; ch + 28 < nch; ch += 32) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = pb[(size_t)(ch + 4 * u) * C];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc += v[u];
    }
    for (; ch < nch; ch += 4) acc += pb[(size_t)ch * C];
  }
  s[w][lane] = acc;
  __syncthreads();
  if (w == 0 && c < C) x[(size_t)b * C + c] = (((s[0][lane] + s[1][lane]) + s[2][lane]) + s[3][lane]) / (float)N;
}

// Dot products of one vector with 64 columns of a row-major [R, ncols]
// matrix, R split over the 16 waves (eight rows in flight per lane); the
// wave sums are added in wave order into red[0][lane].
__device__ __forceinline__ void gemv64(const float* __restrict__ vec, const float* __restrict__ m,
                                       int R, int ncols, int col, float (*red)[64]) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int q = (R + 15) / 16;
  const int r0 = w * q, r1 = std::min(R, r0 + q);
  float acc = 0.f;
  if (col < ncols) {
    int r = r0;
    for (; r + 7 < r1; r += 8) {
      float a[8], v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        a[u] = vec[r + u];
        v[u] = m[(size_t)(r + u) * ncols + col];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) acc = fmaf(a[u], v[u], acc);
    }
    for (; r < r1; ++r) acc = fmaf(vec[r], m[(size_t)r * ncols + col], acc);
  }
  red[w][lane] = acc;
  __syncthreads();
  if (w == 0) {
    float t = red[0][lane];
    for (int i = 1; i < 16; ++i) t += red[i][lane];
    red[0][lane] = t;
  }
}

// hidden[b][u] = max(0, sum_c x[b][c] W1[c][u] + b1[u]) for 64 units u.
__global__ __launch_bounds__(MT) void k_route_hidden(const float* __restrict__ x,
                                                     const float* __restrict__ w1,
                                                     const float* __restrict__ b1, int C, int Hr,
                                                     float* __restrict__ hid) {
  __shared__ float red[16][64];
  const int b = blockIdx.y, lane = threadIdx.x & 63;
  const int u = blockIdx.x * 64 + lane;
  gemv64(x + (size_t)b * C, w1, C, Hr, u, red);
  if (threadIdx.x < 64 && u < Hr) {
    const float a = red[0][lane] + b1[u];
    hid[(size_t)b * Hr + u] = a > 0.f ? a : 0.f;
  }
}

// z[b][o] = sum_u hidden[b][u] W2[u][o] + b2[o] for 64 outputs o < 2 Hq;
// the pair (2h, 2h + 1) of head h sits in neighbouring lanes of wave 0.
__global__ __launch_bounds__(MT) void k_route_out(const float* __restrict__ hid,
                                                  const float* __restrict__ w2,
                                                  const float* __restrict__ b2, int Hr, int Hq,
                                                  float* __restrict__ logits,
                                                  uint8_t* __restrict__ route) {
  __shared__ float red[16][64];
  const int b = blockIdx.y, lane = threadIdx.x & 63;
  const int O = 2 * Hq;
  const int o = blockIdx.x * 64 + lane;
  gemv64(hid + (size_t)b * Hr, w2, Hr, O, o, red);
  if (threadIdx.x < 64) {
    const float z = o < O ? red[0][lane] + b2[o] : 0.f;
    const float other = __shfl_xor(z, 1);
    if (o < O) {
      if (logits) logits[(size_t)b * O + o] = z;
      if ((o & 1) == 0) route[(size_t)b * Hq + (o >> 1)] = other > z ? 1 : 0;
    }
  }
}

}  // namespace

size_t route_ws_bytes(const Dims& D, int hidden) { return route_plan(D, hidden).total; }

hipError_t launch_route(const Dims& D, const RouterArgs& r, const void* k, uint8_t* route,
                        float* logits, void* ws, hipStream_t s) {
  if (D.B == 0 || D.N == 0) return hipSuccess;
  const RoutePlan P = route_plan(D, r.hidden);
  const int C = D.Hkv * D.d;
  char* w = (char*)ws;
  float* part = (float*)(w + P.part_off);
  float* x = (float*)(w + P.x_off);
  float* hid = (float*)(w + P.h_off);
  ProfScope ps(s, kStageRoute);
  const dim3 gp(P.ncol, P.nch, D.B);
  if (D.qkv_bf16)
    hipLaunchKernelGGL(k_route_pool<bf16_bits>, gp, dim3(RT), 0, s, (const bf16_bits*)k, D.L, D.N,
                       C, P.rows, P.nch, part);
  else
    hipLaunchKernelGGL(k_route_pool<float>, gp, dim3(RT), 0, s, (const float*)k, D.L, D.N, C,
                       P.rows, P.nch, part);
  hipLaunchKernelGGL(k_route_reduce, dim3((C + 63) / 64, D.B), dim3(RT), 0, s, part, P.nch, C,
                     D.N, x);
  hipLaunchKernelGGL(k_route_hidden, dim3((r.hidden + 63) / 64, D.B), dim3(MT), 0, s, x, r.w1,
                     r.b1, C, r.hidden, hid);
  hipLaunchKernelGGL(k_route_out, dim3((2 * D.Hq + 63) / 64, D.B), dim3(MT), 0, s, hid, r.w2, r.b2,
                     r.hidden, D.Hq, logits, route);
  return hipGetLastError();
}

}  // namespace dsa
