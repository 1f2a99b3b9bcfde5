// Attention with bf16 MFMA for prefill-shaped calls: both routes of the
// per-head route in one launch.
//
// Sparse heads: softmax(q k^T * scale) v over the selected rows of each query
// token ("混合注意力架构演进：从线性注意力到稀疏门控的技术权衡" §三; steps 3-4 of
// the gated forward on "超大规模MoE架构中稀疏注意力机制的演进与实践" §四.1).
// Dense heads: full causal attention ("Advanced Attention Mechanisms" article
// §2.1) with the running max / running sum over key tiles of its §3.2.  The
// page "Elastic Attention：动态路由优化大模型长文本处理" §3.1 puts both kinds of
// head in one fused op with load balancing; here the grid is one list of
// work items, dense query tiles first (longest first), then sparse tokens.
//
// Per 32-key step and wave (all math in fp32 accumulators):
//   S^T [16 keys x 16 cols] = K_tile [16 x d] . Q^T [d x 16]   (two halves)
//     K rows go straight from memory into the MFMA A operand; the 16 columns
//     are 16 query rows of one head (dense) or the heads of one KV head
//     (sparse).  Dense tiles read K from LDS with the d axis permuted (lane
//     quad q takes dims 32 q ..), sparse tokens read K rows from memory in
//     plain order (the four quads of a key cover 64 contiguous bytes per
//     load); Q^T follows the same order in each case.
//   online softmax per column, in registers (a lane owns one column);
//   O^T [16 dims x 16 cols] += V^T [16 dims x 32 keys] . P^T [32 keys x 16]
//     P^T is the MFMA B operand directly from registers (keys 4q..4q+3 of
//     the first half and 16+4q.. of the second half for lane quad q); V^T is
//     read from a row-major LDS tile with the transposing LDS load, which
//     hands lane i of a 16-lane group element i%4 of the 8-byte chunks read
//     by lanes 4k + i/4.
#include "common.h"
#include "launch.h"
#include "mfma.h"
#include "attn_tile.h"

namespace dsa {
namespace {

constexpr int MT = 256;          // threads (4 waves)

struct MfmaArgs {
  const bf16_bits* q; const bf16_bits* k; const bf16_bits* v;
  const int32_t* topk; int idx_rows_per_b, idx_n_base;
  const float* gate; const float* y2; const uint8_t* route;
  float* out;
  int B, N, L, Hq, Hkv, K;
  int n0, R;          // query rows [n0, n0 + R) of each sequence
  int qtiles;         // dense query tiles of DROWS rows per (b, h); 0 = no dense work
  int do_sparse;      // sparse tokens carried by this launch
  int sgpl;           // sparse tokens: KV heads per item (a divisor of Hkv)
  float scale_log2;
};

// Final normalisation, gate and store of one column (lane owns column i; the
// four quads hold dims 16*dt + 4q + r).
template <int HD>
__device__ __forceinline__ void finish_col(ColState<HD>& st, const MfmaArgs& a, size_t orow,
                                           bool write) {
  const int lane = threadIdx.x & 63;
  const int q = lane >> 4;
  float l = st.l;
  l = sum_xor16(l);
  l = sum_xor32(l);
  if (!write) return;
  const float inv = (l > 0.f) ? 1.f / l : 0.f;
  const float g = a.gate ? a.gate[orow] : 1.f;
#pragma unroll
  for (int dt = 0; dt < HD / 16; ++dt) {
    const int d0 = dt * 16 + 4 * q;
    float4 r;
    float* rv = &r.x;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      float val = (l > 0.f) ? st.o[dt][x] * inv : 0.f;
      if (a.gate) val = fmaf(g, val, (1.f - g) * a.y2[orow * HD + d0 + x]);
      rv[x] = val;
    }
    *reinterpret_cast<float4*>(a.out + orow * HD + d0) = r;
  }
}


// Dense query tile: 128 query rows of one (sequence, head), 32 per wave as two
// 16-column tiles, against 64-key steps of the causal prefix.  The key and
// value tiles of a step are double-buffered in LDS: the global loads of step
// s + 1 are issued before the MFMAs of step s and written to the other buffer
// afterwards, so one barrier per step suffices.  Both column tiles share
// every K operand read and every transposed V^T read.
constexpr int DROWS = 128;       // query rows per dense tile
constexpr int DKEYS = 64;        // keys per dense step
constexpr int kDenseLds = 2 * DKEYS * KSTR + 2 * DKEYS * VSTR;

template <int HD>
__device__ void dense_tile(const MfmaArgs& a, int b, int h, int tile, char* smem) {
  constexpr int T = HD / 32;
  constexpr int CPR = HD / 8;                    // 16-byte chunks per row
  constexpr int NLD = DKEYS * CPR / MT;          // chunks per thread per tile
  char* kbuf0 = smem;
  char* vbuf0 = smem + 2 * DKEYS * KSTR;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int q = lane >> 4, i = lane & 15;
  const int g = h / (a.Hq / a.Hkv);
  const int rbase = tile * DROWS;
  const int off = a.L - a.N + a.n0;              // position of local row 0
  const int rlast = min(a.R - 1, rbase + DROWS - 1);
  const int pmax = off + rlast;                  // last key any row of the tile sees
  const int wlast = min(a.R - 1, rbase + w * 32 + 31);
  const int pmax_wave = off + wlast;
  bf16x8 qb[2][T];
  int prow[2];
  bool rvalid[2];
  size_t orow[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int r = rbase + w * 32 + c * 16 + i;
    rvalid[c] = r < a.R;
    const int n = a.n0 + (rvalid[c] ? r : 0);
    prow[c] = rvalid[c] ? off + r : -1;
    orow[c] = ((size_t)b * a.N + n) * a.Hq + h;
    const bf16_bits* qr = a.q + orow[c] * HD;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      uint4 u = rvalid[c] ? *reinterpret_cast<const uint4*>(qr + q * (HD / 4) + t * 8)
                          : make_uint4(0, 0, 0, 0);
      qb[c][t] = as_bf16x8(u);
    }
  }
  ColState<HD> st[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    st[c].m = -INFINITY;
    st[c].l = 0.f;
#pragma unroll
    for (int dt = 0; dt < HD / 16; ++dt) st[c].o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const bf16_bits* kbase = a.k + ((size_t)b * a.L * a.Hkv + g) * HD;
  const bf16_bits* vbase = a.v + ((size_t)b * a.L * a.Hkv + g) * HD;
  const size_t rstride = (size_t)a.Hkv * HD;
  uint4 kreg[NLD], vreg[NLD];
  auto fetch = [&](int j0) {
#pragma unroll
    for (int x = 0; x < NLD; ++x) {
      const int cidx = x * MT + threadIdx.x;
      const int r = cidx / CPR, cc = cidx - r * CPR;
      const int j = j0 + r;
      kreg[x] = make_uint4(0, 0, 0, 0);
      vreg[x] = make_uint4(0, 0, 0, 0);
      if (j <= pmax) {
        kreg[x] = *reinterpret_cast<const uint4*>(kbase + (size_t)j * rstride + cc * 8);
        vreg[x] = *reinterpret_cast<const uint4*>(vbase + (size_t)j * rstride + cc * 8);
      }
    }
  };
  auto stash = [&](int buf) {
    char* kt = kbuf0 + buf * DKEYS * KSTR;
    char* vt = vbuf0 + buf * DKEYS * VSTR;
#pragma unroll
    for (int x = 0; x < NLD; ++x) {
      const int cidx = x * MT + threadIdx.x;
      const int r = cidx / CPR, cc = cidx - r * CPR;
      *reinterpret_cast<uint4*>(kt + r * KSTR + cc * 16) = kreg[x];
      *reinterpret_cast<uint4*>(vt + r * VSTR + cc * 16) = vreg[x];
    }
  };
  const int nsteps = pmax / DKEYS + 1;
  fetch(0);
  stash(0);
  __syncthreads();
  const int row0 = 4 * q + (i >> 2);   // value row this lane points at (transposing read)
  const int colb = (i & 3) * 8;
  for (int sidx = 0; sidx < nsteps; ++sidx) {
    const int j0 = sidx * DKEYS;
    const bool more = sidx + 1 < nsteps;
    if (more) fetch(j0 + DKEYS);
    if (j0 <= pmax_wave) {
      const char* kt = kbuf0 + (sidx & 1) * DKEYS * KSTR;
      const char* vt = vbuf0 + (sidx & 1) * DKEYS * VSTR;
      // S^T: 4 blocks of 16 keys x 16 columns, for both column tiles
      f32x4 sacc[2][4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        bf16x8 ka[T];
#pragma unroll
        for (int t = 0; t < T; ++t)
          ka[t] = as_bf16x8(*reinterpret_cast<const uint4*>(kt + (u * 16 + i) * KSTR +
                                                             (q * (HD / 4) + t * 8) * 2));
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int t = 0; t < T; ++t) acc = mfma16(ka[t], qb[c][t], acc);
          sacc[c][u] = acc;
        }
      }
      // online softmax per column; P^T packed per 32-key half
      bf16x8 pb[2][2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        float sv[16];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int j = j0 + u * 16 + 4 * q + r;
            sv[u * 4 + r] = (j <= prow[c]) ? sacc[c][u][r] * a.scale_log2 : -INFINITY;
          }
        float mt = sv[0];
#pragma unroll
        for (int x = 1; x < 16; ++x) mt = fmaxf(mt, sv[x]);
        mt = max_xor16(mt);
        mt = max_xor32(mt);
        const float mnew = fmaxf(st[c].m, mt);
        float alpha = 1.f;
        float pv[16];
        if (mnew == -INFINITY) {
#pragma unroll
          for (int x = 0; x < 16; ++x) pv[x] = 0.f;
        } else {
          alpha = exp2_fast(st[c].m - mnew);
#pragma unroll
          for (int x = 0; x < 16; ++x) pv[x] = exp2_fast(sv[x] - mnew);
        }
        float ps = 0.f;
#pragma unroll
        for (int x = 0; x < 16; ++x) ps += pv[x];
        st[c].l = st[c].l * alpha + ps;
        st[c].m = mnew;
        // half v: keys 32v + 4q + r (block 2v) then 32v + 16 + 4q + r (block 2v + 1)
        pb[c][0] = pack8(pv);
        pb[c][1] = pack8(pv + 8);
#pragma unroll
        for (int dt = 0; dt < HD / 16; ++dt)
#pragma unroll
          for (int r = 0; r < 4; ++r) st[c].o[dt][r] *= alpha;
      }
      // O^T += V^T P^T for both halves; V^T read once for both column tiles
#pragma unroll
      for (int v = 0; v < 2; ++v) {
#pragma unroll
        for (int dt = 0; dt < HD / 16; ++dt) {
          const uint2 lo = lds_tr(vt, (32 * v + row0) * VSTR + dt * 32 + colb);
          const uint2 hi = lds_tr(vt, (32 * v + 16 + row0) * VSTR + dt * 32 + colb);
          uint4 u4;
          u4.x = lo.x; u4.y = lo.y; u4.z = hi.x; u4.w = hi.y;
          const bf16x8 va = as_bf16x8(u4);
#pragma unroll
          for (int c = 0; c < 2; ++c) st[c].o[dt] = mfma16(va, pb[c][v], st[c].o[dt]);
        }
      }
    }
    if (more) stash((sidx + 1) & 1);
    __syncthreads();
  }
#pragma unroll
  for (int c = 0; c < 2; ++c) finish_col<HD>(st[c], a, orow[c], rvalid[c]);
}

// Work carried by an instantiation: dense tiles, sparse tokens, or both.  The
// sparse-only kernel needs neither the dense path's LDS nor its registers,
// so three of its workgroups fit on a CU instead of two.
constexpr int kDenseWork = 1, kSparseWork = 2, kBothWork = 3;
constexpr int kSparseLds = 4 * 32 * VSTR + 2048 * 4;

template <int HD, int WORK>
__global__ __launch_bounds__(MT, WORK == kSparseWork ? 3 : 2) void k_attn_mfma(MfmaArgs a) {
  constexpr int T = HD / 32;
  // sparse: per-wave value tile + the token's index row; dense: double-
  // buffered key and value tiles (the two uses share the LDS)
  constexpr int kLds = (WORK & kDenseWork) ? (kDenseLds > kSparseLds ? kDenseLds : kSparseLds)
                                           : kSparseLds;
  __shared__ __attribute__((aligned(16))) char smem[kLds];
  char (*vt)[32 * VSTR] = reinterpret_cast<char (*)[32 * VSTR]>(smem);
  int* ilist = reinterpret_cast<int*>(smem + 4 * 32 * VSTR);
  __shared__ int s_nd, s_lastv;
  __shared__ int s_pair;

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int q = lane >> 4, i = lane & 15;
  const int Gh = a.Hq / a.Hkv;

  // number of dense (b, h) pairs
  if (threadIdx.x == 0) {
    int nd = 0;
    if (a.route)
      for (int x = 0; x < a.B * a.Hq; ++x) nd += a.route[x] == 0;
    s_nd = nd;
  }
  __syncthreads();
  const int nd = s_nd;
  const long long n_dense_items = (long long)nd * a.qtiles;
  const long long item = blockIdx.x;

  if ((WORK & kDenseWork) && item < n_dense_items) {
    // ------------------------------------------------------------ dense query tile
    const int tile = a.qtiles - 1 - (int)(item / nd);   // longest tiles first
    const int d_idx = (int)(item % nd);
    if (threadIdx.x == 0) {
      int c = -1, x = 0;
      for (; x < a.B * a.Hq; ++x)
        if (a.route[x] == 0 && ++c == d_idx) break;
      s_pair = x;
    }
    __syncthreads();
    const int pair = s_pair;
    const int b = pair / a.Hq, h = pair - b * a.Hq;
    if constexpr ((WORK & kDenseWork) != 0) dense_tile<HD>(a, b, h, tile, smem);
    return;
  }

  // -------------------------------------------------------------- sparse token
  const long long sidx = item - n_dense_items;
  // sparse items in (sequence, block of sgpl KV heads, token) order: the
  // workgroups resident at one time gather from one or two blocks of K/V
  const int nblk = a.Hkv / a.sgpl;
  if (!(WORK & kSparseWork) || !a.do_sparse || sidx >= (long long)a.B * nblk * a.R) return;
  const int b = (int)(sidx / ((long long)nblk * a.R));
  const int rem = (int)(sidx - (long long)b * nblk * a.R);
  const int gblk = rem / a.R, r_loc = rem - gblk * a.R;
  const int n = a.n0 + r_loc;
  const int p = a.L - a.N + n;
  // index row into LDS; the last valid entry bounds the loop
  const int32_t* irow = a.topk + ((size_t)b * a.idx_rows_per_b + (n - a.idx_n_base)) * a.K;
  if (threadIdx.x == 0) s_lastv = -1;
  __syncthreads();
  int lastv = -1;
  const int kpad = (a.K + 31) / 32 * 32;
  for (int e = threadIdx.x; e < kpad; e += MT) {
    int j = (e < a.K) ? irow[e] : -1;
    if (j < 0 || j > p) j = -1;
    ilist[e] = j;
    if (j >= 0) lastv = e;
  }
  if (lastv >= 0) atomicMax(&s_lastv, lastv);
  __syncthreads();
  const int nsteps = (s_lastv + 32) / 32;
  char* vtile = vt[w];
  const size_t rstride = (size_t)a.Hkv * HD;
  // (KV head, 16-head chunk) pairs spread over the four waves
  const int nhc = (Gh + 15) / 16;
  for (int pi = w; pi < a.sgpl * nhc; pi += 4) {
    const int g = gblk * a.sgpl + pi / nhc;
    {
      const int hc = (pi % nhc) * 16;
      int myh = -1, cnt = 0;
      for (int x = hc; x < min(Gh, hc + 16); ++x) {
        const int h = g * Gh + x;
        const bool sp = a.route ? a.route[(size_t)b * a.Hq + h] != 0 : true;
        if (sp) {
          if (cnt == i) myh = h;
          ++cnt;
        }
      }
      if (cnt == 0) continue;
      bf16x8 qb[T];
      {
        const bf16_bits* qr = a.q + (((size_t)b * a.N + n) * a.Hq + (myh < 0 ? 0 : myh)) * HD;
#pragma unroll
        for (int t = 0; t < T; ++t) {
          uint4 u = (myh >= 0) ? *reinterpret_cast<const uint4*>(qr + t * 32 + q * 8)
                               : make_uint4(0, 0, 0, 0);
          qb[t] = as_bf16x8(u);
        }
      }
      ColState<HD> st;
      st.m = -INFINITY;
      st.l = 0.f;
#pragma unroll
      for (int dt = 0; dt < HD / 16; ++dt) st.o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const bf16_bits* kbase = a.k + ((size_t)b * a.L * a.Hkv + g) * HD;
      const bf16_bits* vbase = a.v + ((size_t)b * a.L * a.Hkv + g) * HD;
      for (int sidx2 = 0; sidx2 < nsteps; ++sidx2) {
        const int e0 = sidx2 * 32;
        // key rows straight into the A operand (the four lane quads of a key
        // read 64 contiguous bytes), issued before the value rows
        uint4 ka[2][T];
        bool kval[2][4];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int j = ilist[e0 + u * 16 + i];
#pragma unroll
          for (int t = 0; t < T; ++t)
            ka[u][t] = (j >= 0) ? *reinterpret_cast<const uint4*>(kbase + (size_t)j * rstride +
                                                                   t * 32 + q * 8)
                                : make_uint4(0, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) kval[u][r] = ilist[e0 + u * 16 + 4 * q + r] >= 0;
        }
        // value rows of the 32 keys -> this wave's LDS tile
        constexpr int CPR = HD / 8;
        uint4 vv[32 * CPR / 64];
#pragma unroll
        for (int x = 0; x < 32 * CPR / 64; ++x) {
          const int cidx = x * 64 + lane;
          const int r = cidx / CPR, cc = cidx - r * CPR;
          const int j = ilist[e0 + r];
          vv[x] = (j >= 0) ? *reinterpret_cast<const uint4*>(vbase + (size_t)j * rstride + cc * 8)
                           : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int x = 0; x < 32 * CPR / 64; ++x) {
          const int cidx = x * 64 + lane;
          const int r = cidx / CPR, cc = cidx - r * CPR;
          *reinterpret_cast<uint4*>(vtile + r * VSTR + cc * 16) = vv[x];
        }
        __builtin_amdgcn_s_waitcnt(0);   // this wave's LDS tile is complete
        __builtin_amdgcn_wave_barrier();
        step_core<HD>(ka, qb, kval, vtile, a.scale_log2, st);
        __builtin_amdgcn_wave_barrier();
      }
      const size_t orow = ((size_t)b * a.N + n) * a.Hq + (myh < 0 ? 0 : myh);
      finish_col<HD>(st, a, orow, myh >= 0);
    }
  }
}

}  // namespace

bool mfma_attention_supported(const Dims& D) {
  // one selected set per token (per-head sets take the other kernels)
  return D.qkv_bf16 && (D.d == 64 || D.d == 128) && D.K <= 2048 && D.Hq / D.Hkv >= 1 &&
         D.IH == 1;
}

hipError_t launch_attention_mfma(const Dims& D, const AttnArgs& aa, hipStream_t s) {
  if (D.B == 0 || aa.R == 0) return hipSuccess;
  MfmaArgs a{};
  a.q = (const bf16_bits*)aa.q; a.k = (const bf16_bits*)aa.k; a.v = (const bf16_bits*)aa.v;
  a.topk = aa.topk; a.idx_rows_per_b = aa.idx_rows_per_b; a.idx_n_base = aa.idx_n_base;
  a.gate = aa.gate; a.y2 = aa.y2; a.route = aa.route; a.out = aa.out;
  a.B = D.B; a.N = D.N; a.L = D.L; a.Hq = D.Hq; a.Hkv = D.Hkv; a.K = D.K;
  a.n0 = aa.n0; a.R = aa.R;
  a.qtiles = aa.skip_dense ? 0 : (aa.R + DROWS - 1) / DROWS;
  a.do_sparse = aa.skip_sparse ? 0 : 1;
  a.sgpl = (aa.sparse_heads_per_item > 0 && D.Hkv % aa.sparse_heads_per_item == 0)
               ? aa.sparse_heads_per_item : D.Hkv;
  a.scale_log2 = D.scale * kLog2e;
  const long long dense_max = aa.route ? (long long)D.B * D.Hq * a.qtiles : 0;
  const long long blocks =
      dense_max + (aa.skip_sparse ? 0 : (long long)D.B * (D.Hkv / a.sgpl) * aa.R);
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  const int work = (dense_max > 0 ? kDenseWork : 0) | (aa.skip_sparse ? 0 : kSparseWork);
  const dim3 g((unsigned)blocks), t(MT);
  ProfScope ps(s, kStageAttention);
#define DSA_ATTN_MFMA(HDV)                                                                  \
  if (work == kDenseWork) hipLaunchKernelGGL((k_attn_mfma<HDV, kDenseWork>), g, t, 0, s, a); \
  else if (work == kSparseWork)                                                            \
    hipLaunchKernelGGL((k_attn_mfma<HDV, kSparseWork>), g, t, 0, s, a);                     \
  else hipLaunchKernelGGL((k_attn_mfma<HDV, kBothWork>), g, t, 0, s, a);
  if (D.d == 128) {
    DSA_ATTN_MFMA(128)
  } else {
    DSA_ATTN_MFMA(64)
  }
#undef DSA_ATTN_MFMA
  return hipGetLastError();
}

}  // namespace dsa
