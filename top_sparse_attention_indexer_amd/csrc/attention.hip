// Attention over the selected key/value rows (sparse heads) or over every
// visible key (dense heads), with online softmax and the gate blend.
//
// Sparse heads: gather of the selected rows and softmax(q k^T * scale) v over
// them, as in "混合注意力架构演进：从线性注意力到稀疏门控的技术权衡" §三 and the
// gated forward of "超大规模MoE架构中稀疏注意力机制的演进与实践" §四.1 (steps
// 3-5).  Dense heads: the full causal attention of the "Advanced Attention
// Mechanisms" article §2.1, which the page "Elastic Attention：动态路由优化大模型
// 长文本处理" §2.2/§3.1 mixes per head with the sparse kind.  The running
// maximum / running sum normalisation follows that article's §3.2 (tiles kept
// on chip, max and sum updated as tiles arrive).  Gate: g*a + (1-g)*y2.
//
// Work item = (query token, KV head, key split).  All query heads of one KV
// head share the item, so each gathered key/value row is read once per token
// and KV head.  With more than one split, partial (max, sum, accumulator)
// triples go to the workspace and a merge kernel combines them.
#include "common.h"
#include "launch.h"

namespace dsa {
namespace {

constexpr int AT = 256;   // threads
constexpr int TK = 32;    // keys per tile
constexpr int HB = 16;    // heads per pass
constexpr float kLog2e = 1.4426950408889634f;

template <typename T, int HD>
__global__ __launch_bounds__(AT) void k_attn(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const int32_t* __restrict__ topk, int idx_rows_per_b, int idx_n_base,
    const float* __restrict__ gate, const float* __restrict__ y2, const uint8_t* __restrict__ route,
    float* __restrict__ out, float* __restrict__ part, int N, int L, int Hq, int Hkv, int K,
    int n0, int R, int splits, int split_stride, int dense_mode, float scale_log2, int IH) {
  // blockIdx.x = ((b * R + r) * Hkv + g) * splits + s
  const int s = blockIdx.x % splits;
  const int item = blockIdx.x / splits;
  const int g = item % Hkv;
  const int row = item / Hkv;  // b * R + r
  const int b = row / R, r = row - b * R;
  const int n = n0 + r;
  const int p = L - N + n;
  const int G = Hq / Hkv;

  __shared__ int act[256];
  __shared__ int nact_s;
  __shared__ float qs[HB][HD];
  __shared__ float ks[TK][HD + 1];
  __shared__ float vs[TK][HD + 1];
  __shared__ float sc[HB][TK];
  __shared__ float m_s[HB], l_s[HB], al_s[HB];
  __shared__ int kidx[TK];

  if (threadIdx.x == 0) {
    int c = 0;
    for (int i = 0; i < G; ++i) {
      const int h = g * G + i;
      const bool sparse = route ? (route[(size_t)b * Hq + h] != 0) : true;
      if (sparse != (dense_mode != 0)) act[c++] = h;
    }
    nact_s = c;
  }
  __syncthreads();
  const int nact = nact_s;
  if (nact == 0) return;

  // key range of this split
  int e0, e1;
  if (dense_mode) {
    const int per = ((L + splits - 1) / splits + TK - 1) / TK * TK;
    e0 = s * per;
    e1 = min(p + 1, e0 + per);
  } else {
    const int per = ((K + splits - 1) / splits + TK - 1) / TK * TK;
    e0 = s * per;
    e1 = min(K, e0 + per);
  }
  // index rows of this token: one per indexer head (IH), query head h using
  // row h / (Hq / IH); a pass over heads stays within one row
  const int32_t* trow = topk ? topk + ((size_t)b * idx_rows_per_b + (n - idx_n_base)) * IH * K : nullptr;
  const int HPS = Hq / IH;

  constexpr int CPT = HB * HD / AT;        // accumulators per thread
  constexpr int HSTEP = AT / HD;           // head stride between a thread's accumulators
  const int c_own = threadIdx.x % HD;
  const int h_own = threadIdx.x / HD;

  for (int hc = 0, nh = 0; hc < nact; hc += nh) {
    nh = 1;
    while (nh < HB && hc + nh < nact && act[hc + nh] / HPS == act[hc] / HPS) ++nh;
    const int32_t* irow = trow ? trow + (size_t)(act[hc] / HPS) * K : nullptr;
    for (int e = threadIdx.x; e < HB * HD; e += AT) {
      const int hh = e / HD, c = e - hh * HD;
      float x = 0.f;
      if (hh < nh) x = ld_f(q, (((size_t)b * N + n) * Hq + act[hc + hh]) * HD + c) * scale_log2;
      qs[hh][c] = x;
    }
    if (threadIdx.x < HB) {
      m_s[threadIdx.x] = -INFINITY;
      l_s[threadIdx.x] = 0.f;
    }
    float acc[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) acc[i] = 0.f;
    __syncthreads();

    for (int t0 = e0; t0 < e1; t0 += TK) {
      if (threadIdx.x < TK) {
        const int e = t0 + threadIdx.x;
        int j = -1;
        if (e < e1) {
          if (dense_mode) j = e;
          else {
            j = irow[e];
            if (j < 0 || j > p) j = -1;
          }
        }
        kidx[threadIdx.x] = j;
      }
      __syncthreads();
      // gather the key and value rows of this tile (8 elements per load)
      for (int e = threadIdx.x; e < TK * (HD / 8); e += AT) {
        const int t = e / (HD / 8), c8 = (e - t * (HD / 8)) * 8;
        const int j = kidx[t];
        float kv[8], vv[8];
        if (j >= 0) {
          const size_t off = (((size_t)b * L + j) * Hkv + g) * HD + c8;
          ld8(k + off, kv);
          ld8(v + off, vv);
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) kv[i] = vv[i] = 0.f;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          ks[t][c8 + i] = kv[i];
          vs[t][c8 + i] = vv[i];
        }
      }
      __syncthreads();
      // scores: thread -> key t, heads hh and hh + 8
      {
        const int t = threadIdx.x % TK;
        const int hh = threadIdx.x / TK;  // 0..7
        float s0 = 0.f, s1 = 0.f;
#pragma unroll 8
        for (int c = 0; c < HD; ++c) {
          const float kc = ks[t][c];
          s0 = fmaf(qs[hh][c], kc, s0);
          s1 = fmaf(qs[hh + 8][c], kc, s1);
        }
        const bool ok = kidx[t] >= 0;
        sc[hh][t] = (ok && hh < nh) ? s0 : -INFINITY;
        sc[hh + 8][t] = (ok && hh + 8 < nh) ? s1 : -INFINITY;
      }
      __syncthreads();
      // online softmax update, one thread per head
      if (threadIdx.x < HB) {
        const int hh = threadIdx.x;
        const float mold = m_s[hh];
        float mt = -INFINITY;
        for (int t = 0; t < TK; ++t) mt = fmaxf(mt, sc[hh][t]);
        const float mnew = fmaxf(mold, mt);
        float alpha = 1.f, sum = 0.f;
        if (mnew == -INFINITY) {
          for (int t = 0; t < TK; ++t) sc[hh][t] = 0.f;
        } else {
          alpha = exp2f(mold - mnew);
          for (int t = 0; t < TK; ++t) {
            const float pv = exp2f(sc[hh][t] - mnew);
            sc[hh][t] = pv;
            sum += pv;
          }
        }
        l_s[hh] = l_s[hh] * alpha + sum;
        m_s[hh] = mnew;
        al_s[hh] = alpha;
      }
      __syncthreads();
      // PV
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int hh = h_own + HSTEP * i;
        float a = acc[i] * al_s[hh];
#pragma unroll 8
        for (int t = 0; t < TK; ++t) a = fmaf(sc[hh][t], vs[t][c_own], a);
        acc[i] = a;
      }
      __syncthreads();
    }

    // finalize this head chunk
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int hh = h_own + HSTEP * i;
      if (hh >= nh) continue;
      const int h = act[hc + hh];
      const size_t orow = (((size_t)b * N + n) * Hq + h);
      if (split_stride == 1) {
        const float l = l_s[hh];
        float a = (l > 0.f) ? acc[i] / l : 0.f;
        if (gate) {
          const float gg = gate[orow];
          a = fmaf(gg, a, (1.f - gg) * y2[orow * HD + c_own]);
        }
        out[orow * HD + c_own] = a;
      } else {
        const size_t pi = (((size_t)row * Hq + h) * split_stride + s);
        part[pi * (HD + 2) + 2 + c_own] = acc[i];
        if (c_own == 0) {
          part[pi * (HD + 2) + 0] = m_s[hh];
          part[pi * (HD + 2) + 1] = l_s[hh];
        }
      }
    }
    __syncthreads();
  }
}

// Combines the split partials of one (token, head) and applies the gate.
template <int HD>
__global__ __launch_bounds__(HD) void k_attn_merge(const float* __restrict__ part,
                                                   const float* __restrict__ gate,
                                                   const float* __restrict__ y2,
                                                   const uint8_t* __restrict__ route,
                                                   float* __restrict__ out, int N, int Hq, int n0,
                                                   int R, int splits_sparse, int splits_dense,
                                                   int split_stride) {
  const int h = blockIdx.x % Hq;
  const int row = blockIdx.x / Hq;
  const int b = row / R, r = row - b * R;
  const int n = n0 + r;
  const bool sparse = route ? (route[(size_t)b * Hq + h] != 0) : true;
  const int S = sparse ? splits_sparse : splits_dense;
  const int c = threadIdx.x;
  const float* pp = part + ((size_t)row * Hq + h) * split_stride * (HD + 2);
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, pp[s * (HD + 2)]);
  float a = 0.f;
  if (M != -INFINITY) {
    float l = 0.f, acc = 0.f;
    for (int s = 0; s < S; ++s) {
      const float ms = pp[s * (HD + 2)];
      const float w = (ms == -INFINITY) ? 0.f : exp2f(ms - M);
      l = fmaf(w, pp[s * (HD + 2) + 1], l);
      acc = fmaf(w, pp[s * (HD + 2) + 2 + c], acc);
    }
    a = (l > 0.f) ? acc / l : 0.f;
  }
  const size_t orow = ((size_t)b * N + n) * Hq + h;
  if (gate) {
    const float gg = gate[orow];
    a = fmaf(gg, a, (1.f - gg) * y2[orow * HD + c]);
  }
  out[orow * HD + c] = a;
}

template <typename T, int HD>
hipError_t attn_launch(const Dims& D, const AttnArgs& a, hipStream_t s) {
  const float sl2 = D.scale * kLog2e;
  // with more than one split anywhere, every head goes through the merge
  const int stride = a.route ? std::max(a.splits_sparse, a.splits_dense) : a.splits_sparse;
  const size_t items = (size_t)D.B * a.R * D.Hkv;
  for (int mode = 0; mode < 2; ++mode) {
    if (mode == 1 && !a.route) break;
    const int splits = mode ? a.splits_dense : a.splits_sparse;
    const size_t blocks = items * splits;
    ProfScope ps(s, kStageAttention);
    hipLaunchKernelGGL((k_attn<T, HD>), dim3((unsigned)blocks), dim3(AT), 0, s, (const T*)a.q,
                       (const T*)a.k, (const T*)a.v, a.topk, a.idx_rows_per_b, a.idx_n_base,
                       a.gate, a.y2, a.route, a.out, a.part, D.N, D.L, D.Hq, D.Hkv, D.K, a.n0, a.R,
                       splits, stride, mode, sl2, D.IH);
  }
  if (stride > 1) {
    const size_t blocks = (size_t)D.B * a.R * D.Hq;
    ProfScope ps(s, kStageMerge);
    hipLaunchKernelGGL((k_attn_merge<HD>), dim3((unsigned)blocks), dim3(HD), 0, s, a.part, a.gate,
                       a.y2, a.route, a.out, D.N, D.Hq, a.n0, a.R, a.splits_sparse,
                       a.route ? a.splits_dense : 1, stride);
  }
  return hipGetLastError();
}

}  // namespace

void attn_pick_splits(const Dims& D, int R, int& splits_sparse, int& splits_dense) {
  const long long items = (long long)D.B * R * D.Hkv;
  const long long want = items >= 1024 ? 1 : (1024 + items - 1) / items;
  const long long max_sparse = (D.K + TK - 1) / TK;
  const long long max_dense = std::min<long long>(256, (D.L + TK - 1) / TK);
  splits_sparse = (int)std::max<long long>(1, std::min(want, max_sparse));
  splits_dense = (int)std::max<long long>(1, std::min(want, max_dense));
  // make every split non-empty for the sparse list
  const int per = ((D.K + splits_sparse - 1) / splits_sparse + TK - 1) / TK * TK;
  splits_sparse = (D.K + per - 1) / per;
  const int perd = ((D.L + splits_dense - 1) / splits_dense + TK - 1) / TK * TK;
  splits_dense = (D.L + perd - 1) / perd;
}

size_t attn_part_bytes(const Dims& D, int R, int splits) {
  if (splits <= 1) return 0;
  return (size_t)D.B * R * D.Hq * splits * (D.d + 2) * sizeof(float);
}

hipError_t launch_attention(const Dims& D, const AttnArgs& a, hipStream_t s) {
  if (D.B == 0 || a.R == 0) return hipSuccess;
  if (D.qkv_bf16) {
    if (D.d == 128) return attn_launch<bf16_bits, 128>(D, a, s);
    return attn_launch<bf16_bits, 64>(D, a, s);
  }
  if (D.d == 128) return attn_launch<float, 128>(D, a, s);
  return attn_launch<float, 64>(D, a, s);
}

}  // namespace dsa
