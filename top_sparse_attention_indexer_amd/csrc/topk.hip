// Exact top-K per query row with ties to the lower position.
//
// Selection rule of the page "超大规模MoE架构中稀疏注意力机制的演进与实践"
// (§二.1: keep the K = 2048 best-scoring past positions whatever the context
// length) and of "混合注意力架构演进：从线性注意力到稀疏门控的技术权衡" (§三,
// an index array of shape [L, top_k]); rows with at most K visible keys keep
// all of them.
//
// Method: radix select on the order-preserving 32-bit key of each float score
// in three digit levels (11, 11, 10 bits) with LDS histograms, which yields
// the exact K-th key T and the number kk of keys equal to T that are still
// needed; every key > T and the first kk keys == T are then written in
// ascending position order.  Rows up to 65536 keys are read once into a
// candidate list in LDS (k_topk_cand); wider rows, and lists that overflow,
// take the multi-pass path (row_stream); few long rows can be split over
// workgroups (k_split_*).
#include "common.h"
#include "launch.h"

namespace dsa {
namespace {

constexpr int kShift[3] = {21, 10, 0};
constexpr int kBins[3] = {2048, 2048, 1024};

__device__ __forceinline__ bool row_has_sparse(const uint8_t* route, int b, int Hq) {
  if (!route) return true;
  for (int h = 0; h < Hq; ++h)
    if (route[(size_t)b * Hq + h]) return true;
  return false;
}

// Finds the bin t holding the kk-th largest element of hist[0..nb) (counting
// from the top) and the count of elements in bins above t.  Every thread of
// the block must call it; the result lands in res[0] (bin) and res[1] (count
// above).  nb must be a multiple of NT.
template <int NT>
__device__ void pick_bin(const uint32_t* hist, int nb, uint32_t kk, uint32_t* scratch,
                         uint32_t* res) {
  const int per = nb / NT;
  const int base = threadIdx.x * per;
  uint32_t mine = 0;
  for (int i = 0; i < per; ++i) mine += hist[base + i];
  uint32_t total;
  const uint32_t pre = block_excl_scan<NT>(mine, scratch, total);
  uint32_t running = total - pre - mine;  // elements in bins above this thread's bins
  for (int i = per - 1; i >= 0; --i) {
    const uint32_t c = hist[base + i];
    if (running < kk && running + c >= kk) {
      res[0] = (uint32_t)(base + i);
      res[1] = running;
    }
    running += c;
  }
  __syncthreads();
}

// ---------------------------------------------------------------- one row per workgroup
constexpr int RT = 1024;

// Three digit passes over a row held in memory, then an ordered compaction
// (block ranks in position order).  Used for rows the faster kernels below
// do not take.
template <int NT>
__device__ void row_stream(const float* __restrict__ row, int vis, int K, int32_t* __restrict__ o,
                           uint32_t* hist, uint32_t* scratch, uint32_t* res) {
  uint32_t prefix = 0, mask = 0, kk = (uint32_t)K;
  for (int lv = 0; lv < 3; ++lv) {
    const int shift = kShift[lv], nb = kBins[lv];
    for (int i = threadIdx.x; i < nb; i += NT) hist[i] = 0;
    __syncthreads();
    for (int j = threadIdx.x; j < vis; j += NT) {
      const uint32_t u = radix_key(row[j]);
      if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & (nb - 1)], 1u);
    }
    __syncthreads();
    pick_bin<NT>(hist, nb, kk, scratch, res);
    const uint32_t t = res[0], above = res[1];
    prefix |= t << shift;
    mask |= (uint32_t)(nb - 1) << shift;
    kk -= above;
    __syncthreads();
  }
  const uint32_t T = prefix;
  uint32_t base_sel = 0, base_tie = 0;
  for (int start = 0; start < vis; start += NT) {
    const int j = start + threadIdx.x;
    const uint32_t u = (j < vis) ? radix_key(row[j]) : 0u;
    const bool gt = (j < vis) && u > T;
    const bool eq = (j < vis) && u == T;
    uint32_t tie_tot, sel_tot;
    const uint32_t tie_rank = block_rank<NT>(eq, scratch, tie_tot);
    const bool sel = gt || (eq && base_tie + tie_rank < kk);
    const uint32_t pos = block_rank<NT>(sel, scratch, sel_tot);
    if (sel && base_sel + pos < (uint32_t)K) o[base_sel + pos] = j;
    base_tie += tie_tot;
    base_sel += sel_tot;
  }
}

__global__ __launch_bounds__(RT) void k_topk_rows(const float* __restrict__ scores, size_t ld,
                                                  int N, int L, int K, int n0, int R,
                                                  int32_t* __restrict__ topk, int idx_rows_per_b,
                                                  int idx_n_base, const uint8_t* __restrict__ route,
                                                  int Hq, int rpt) {
  const int r = blockIdx.x, b = blockIdx.y;
  const int n = n0 + r;
  int32_t* o = topk + ((size_t)b * idx_rows_per_b + (n - idx_n_base)) * K;
  const int vis = L - N + n / rpt + 1;
  if (!row_has_sparse(route, b, Hq)) {
    for (int i = threadIdx.x; i < K; i += RT) o[i] = -1;
    return;
  }
  if (vis <= K) {
    for (int i = threadIdx.x; i < K; i += RT) o[i] = (i < vis) ? i : -1;
    return;
  }
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t scratch[RT / DSA_WAVE + 1];
  __shared__ uint32_t res[2];
  row_stream<RT>(scores + ((size_t)b * R + r) * ld, vis, K, o, hist, scratch, res);
}

// ------------------------------------------------ one row per workgroup, one read of the row
// A sample of one key per thread (positions spread over the row) gives a
// lower bound b_lo for the first-level bin of the K-th key, set so that about
// 1.5 K keys are expected at or above it.  One coalesced pass then histograms
// those keys and appends them (key, position) to a candidate list in LDS
// (one LDS atomic per wave and load for the slots).  The three digit levels
// run on the list; the selected positions go to two bitmaps (keys above T,
// keys equal to T) that are read in position order with one block scan for
// each, the first kk keys equal to T being taken.  A list that overflows, or
// that holds fewer than K keys (bound too high), sends the row to the
// multi-pass path, so the result is exact either way.
// Instantiations: rows up to 32768 keys with 512 threads and 6144 list slots
// (two rows per CU); rows up to 65536 keys with 1024 threads and 8192 slots.
constexpr int kMaxWords = 2048;         // bitmap words: rows up to 65536 positions

template <int CT, int kCandCap>
__global__ __launch_bounds__(CT) void k_topk_cand(const float* __restrict__ scores, size_t ld,
                                                  int N, int L, int K, int n0, int R,
                                                  int32_t* __restrict__ topk, int idx_rows_per_b,
                                                  int idx_n_base, const uint8_t* __restrict__ route,
                                                  int Hq, int rpt) {
  const int r = blockIdx.x, b = blockIdx.y;
  const int n = n0 + r;
  int32_t* o = topk + ((size_t)b * idx_rows_per_b + (n - idx_n_base)) * K;
  const int vis = L - N + n / rpt + 1;
  if (!row_has_sparse(route, b, Hq)) {
    for (int i = threadIdx.x; i < K; i += CT) o[i] = -1;
    return;
  }
  if (vis <= K) {
    for (int i = threadIdx.x; i < K; i += CT) o[i] = (i < vis) ? i : -1;
    return;
  }
  const float* row = scores + ((size_t)b * R + r) * ld;
  __shared__ uint32_t hist[2048];
  __shared__ uint64_t cand[kCandCap];
  __shared__ uint32_t bm_gt[kMaxWords], bm_eq[kMaxWords];
  __shared__ uint32_t scratch[CT / DSA_WAVE + 1];
  __shared__ uint32_t res[3];
  const int lane = threadIdx.x & (DSA_WAVE - 1);
  // bound from the sample
  for (int i = threadIdx.x; i < 2048; i += CT) hist[i] = 0;
  if (threadIdx.x == 0) {
    res[0] = 0;
    res[2] = 0;   // candidate count
  }
  __syncthreads();
  uint32_t b_lo = 0;
  const long long want = (3LL * K * CT) / (2LL * vis) + 8;
  if (want < CT / 2) {
    const int j = (int)(((long long)threadIdx.x * vis) / CT);
    atomicAdd(&hist[radix_key(row[j]) >> 21], 1u);
    __syncthreads();
    pick_bin<CT>(hist, 2048, (uint32_t)want, scratch, res);
    b_lo = res[0];
    for (int i = threadIdx.x; i < 2048; i += CT) hist[i] = 0;
  }
  const int nwords = (vis + 31) / 32;
  for (int i = threadIdx.x; i < nwords; i += CT) {
    bm_gt[i] = 0;
    bm_eq[i] = 0;
  }
  __syncthreads();
  // one pass: first-level histogram of the keys >= b_lo, and the list.  A
  // round of loads is counted first, so that the list slots cost one wave
  // scan and one LDS atomic per wave and round.
  auto append = [&](const uint32_t* u, const int* jv, int cnt_n) {
    uint32_t mine = 0;
    for (int x = 0; x < cnt_n; ++x) mine += (jv[x] < vis && (u[x] >> 21) >= b_lo);
    const uint32_t incl = wave_incl_scan(mine);
    uint32_t base = 0;
    if (lane == DSA_WAVE - 1 && incl) base = atomicAdd(&res[2], incl);
    base = __shfl(base, DSA_WAVE - 1, DSA_WAVE);
    uint32_t slot = base + incl - mine;
    for (int x = 0; x < cnt_n; ++x) {
      if (jv[x] < vis && (u[x] >> 21) >= b_lo) {
        atomicAdd(&hist[u[x] >> 21], 1u);
        if (slot < (uint32_t)kCandCap) cand[slot] = ((uint64_t)u[x] << 32) | (uint32_t)jv[x];
        ++slot;
      }
    }
  };
  if ((ld & 3) == 0) {
    // 16-byte loads, four per thread in flight (16384 positions per round);
    // whole vectors inside the row's ld columns are read unconditionally
    for (int j0 = 0; j0 < vis; j0 += CT * 16) {
      uint32_t u[16];
      int jv[16];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int j = j0 + (x * CT + threadIdx.x) * 4;
        float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
        if (j + 3 < (int)ld) f = *reinterpret_cast<const float4*>(row + j);
        else if (j < vis)
          for (int y = 0; y < 4; ++y) (&f.x)[y] = (j + y < vis) ? row[j + y] : 0.f;
        u[4 * x] = radix_key(f.x); u[4 * x + 1] = radix_key(f.y);
        u[4 * x + 2] = radix_key(f.z); u[4 * x + 3] = radix_key(f.w);
#pragma unroll
        for (int y = 0; y < 4; ++y) jv[4 * x + y] = j + y;
      }
      append(u, jv, 16);
    }
  } else {
    for (int j0 = 0; j0 < vis; j0 += CT * 16) {
      uint32_t u[16];
      int jv[16];
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const int j = j0 + x * CT + threadIdx.x;
        u[x] = (j < vis) ? radix_key(row[j]) : 0u;
        jv[x] = j;
      }
      append(u, jv, 16);
    }
  }
  __syncthreads();
  const uint32_t nc = res[2];
  if (nc > (uint32_t)kCandCap || nc < (uint32_t)K) {
    __syncthreads();
    row_stream<CT>(row, vis, K, o, hist, scratch, res);
    return;
  }
  // three digit levels on the list
  uint32_t kk = (uint32_t)K;
  pick_bin<CT>(hist, 2048, kk, scratch, res);
  const uint32_t t0 = res[0];
  kk -= res[1];
  __syncthreads();
  for (int i = threadIdx.x; i < 2048; i += CT) hist[i] = 0;
  __syncthreads();
  for (uint32_t i = threadIdx.x; i < nc; i += CT) {
    const uint32_t u = (uint32_t)(cand[i] >> 32);
    if ((u >> 21) == t0) atomicAdd(&hist[(u >> 10) & 2047u], 1u);
  }
  __syncthreads();
  pick_bin<CT>(hist, 2048, kk, scratch, res);
  const uint32_t pfx = (t0 << 11) | res[0];
  kk -= res[1];
  __syncthreads();
  for (int i = threadIdx.x; i < 1024; i += CT) hist[i] = 0;
  __syncthreads();
  for (uint32_t i = threadIdx.x; i < nc; i += CT) {
    const uint32_t u = (uint32_t)(cand[i] >> 32);
    if ((u >> 10) == pfx) atomicAdd(&hist[u & 1023u], 1u);
  }
  __syncthreads();
  pick_bin<CT>(hist, 1024, kk, scratch, res);
  const uint32_t T = (pfx << 10) | res[0];
  kk -= res[1];   // keys equal to T still to take, lowest positions first
  // selected positions into the bitmaps
  for (uint32_t i = threadIdx.x; i < nc; i += CT) {
    const uint64_t cd = cand[i];
    const uint32_t u = (uint32_t)(cd >> 32), j = (uint32_t)cd;
    if (u > T) atomicOr(&bm_gt[j >> 5], 1u << (j & 31));
    else if (u == T) atomicOr(&bm_eq[j >> 5], 1u << (j & 31));
  }
  __syncthreads();
  // ordered write: each thread owns a contiguous run of bitmap words
  const int wpt = (nwords + CT - 1) / CT;
  const int w0 = threadIdx.x * wpt;
  uint32_t ngt = 0, neq = 0;
  for (int w = w0; w < min(nwords, w0 + wpt); ++w) {
    ngt += __popc(bm_gt[w]);
    neq += __popc(bm_eq[w]);
  }
  uint32_t tot_eq, tot_sel;
  const uint32_t eq_before = block_excl_scan<CT>(neq, scratch, tot_eq);
  uint32_t take = (eq_before >= kk) ? 0u : min(neq, kk - eq_before);
  uint32_t pos = block_excl_scan<CT>(ngt + take, scratch, tot_sel);
  for (int w = w0; w < min(nwords, w0 + wpt); ++w) {
    uint32_t eqw = bm_eq[w];
    uint32_t keep = 0;   // the lowest `take` bits of eqw
    while (eqw && take) {
      const uint32_t low = eqw & (0u - eqw);
      keep |= low;
      eqw ^= low;
      --take;
    }
    uint32_t m = bm_gt[w] | keep;
    while (m) {
      const int bit = __ffs((int)m) - 1;
      if (pos < (uint32_t)K) o[pos] = w * 32 + bit;
      ++pos;
      m &= m - 1;
    }
  }
}

// ---------------------------------------------------------------- rows split over workgroups
constexpr int ST = 256;      // threads per workgroup
constexpr int SCH = 8192;    // scores per chunk
constexpr int kHistWords = 2048 + 2048 + 1024;

struct SplitWs {
  uint32_t* hist;   // [rows][5120]
  uint32_t* cnt;    // [rows][nchunks][2]  (count > T, count == T)
  uint32_t* state;  // [rows][2]           (T, kk)
  int nchunks;
};

__device__ __forceinline__ uint32_t* level_hist(uint32_t* h, int lv) {
  return h + (lv == 0 ? 0 : (lv == 1 ? 2048 : 4096));
}

// Rebuilds (prefix, mask, kk) after `levels` digit passes from the global
// histograms of one row.  Every thread of the block must call it.
__device__ void split_state(const uint32_t* ghist, int levels, int K, uint32_t* lhist,
                            uint32_t* scratch, uint32_t* res, uint32_t& prefix, uint32_t& mask,
                            uint32_t& kk) {
  prefix = 0;
  mask = 0;
  kk = (uint32_t)K;
  for (int lv = 0; lv < levels; ++lv) {
    const int nb = kBins[lv];
    const uint32_t* g = ghist + (lv == 0 ? 0 : (lv == 1 ? 2048 : 4096));
    for (int i = threadIdx.x; i < nb; i += ST) lhist[i] = g[i];
    __syncthreads();
    pick_bin<ST>(lhist, nb, kk, scratch, res);
    prefix |= res[0] << kShift[lv];
    mask |= (uint32_t)(nb - 1) << kShift[lv];
    kk -= res[1];
    __syncthreads();
  }
}

template <int LV>
__global__ __launch_bounds__(ST) void k_split_hist(const float* __restrict__ scores, size_t ld,
                                                   int N, int L, int K, int n0, int R,
                                                   SplitWs ws, const uint8_t* __restrict__ route,
                                                   int Hq, int rpt) {
  const int c = blockIdx.x, row = blockIdx.y;  // row = b * R + r
  const int b = row / R, r = row - b * R;
  const int vis = L - N + (n0 + r) / rpt + 1;
  if (vis <= K || !row_has_sparse(route, b, Hq)) return;
  const int j0 = c * SCH, j1 = min(vis, j0 + SCH);
  if (j0 >= j1) return;
  __shared__ uint32_t lhist[2048];
  __shared__ uint32_t scratch[ST / DSA_WAVE + 1];
  __shared__ uint32_t res[2];
  uint32_t* gh = ws.hist + (size_t)row * kHistWords;
  uint32_t prefix, mask, kk;
  split_state(gh, LV, K, lhist, scratch, res, prefix, mask, kk);
  const int nb = kBins[LV], shift = kShift[LV];
  for (int i = threadIdx.x; i < nb; i += ST) lhist[i] = 0;
  __syncthreads();
  const float* srow = scores + (size_t)row * ld;
  for (int j = j0 + threadIdx.x; j < j1; j += ST) {
    const uint32_t u = radix_key(srow[j]);
    if ((u & mask) == prefix) atomicAdd(&lhist[(u >> shift) & (nb - 1)], 1u);
  }
  __syncthreads();
  uint32_t* g = level_hist(gh, LV);
  for (int i = threadIdx.x; i < nb; i += ST) {
    const uint32_t v = lhist[i];
    if (v) atomicAdd(&g[i], v);
  }
}

__global__ __launch_bounds__(ST) void k_split_count(const float* __restrict__ scores, size_t ld,
                                                    int N, int L, int K, int n0, int R,
                                                    SplitWs ws, const uint8_t* __restrict__ route,
                                                    int Hq, int rpt) {
  const int c = blockIdx.x, row = blockIdx.y;
  const int b = row / R, r = row - b * R;
  const int vis = L - N + (n0 + r) / rpt + 1;
  if (vis <= K || !row_has_sparse(route, b, Hq)) return;
  const int j0 = c * SCH, j1 = min(vis, j0 + SCH);
  __shared__ uint32_t lhist[2048];
  __shared__ uint32_t scratch[ST / DSA_WAVE + 1];
  __shared__ uint32_t res[2];
  uint32_t prefix, mask, kk;
  split_state(ws.hist + (size_t)row * kHistWords, 3, K, lhist, scratch, res, prefix, mask, kk);
  const uint32_t T = prefix;
  uint32_t gt = 0, eq = 0;
  const float* srow = scores + (size_t)row * ld;
  for (int j = j0 + threadIdx.x; j < j1; j += ST) {
    const uint32_t u = radix_key(srow[j]);
    gt += (u > T);
    eq += (u == T);
  }
  uint32_t tgt, teq;
  block_excl_scan<ST>(gt, scratch, tgt);
  block_excl_scan<ST>(eq, scratch, teq);
  if (threadIdx.x == 0) {
    uint32_t* cc = ws.cnt + ((size_t)row * ws.nchunks + c) * 2;
    cc[0] = tgt;
    cc[1] = teq;
    if (c == 0) {
      ws.state[(size_t)row * 2 + 0] = T;
      ws.state[(size_t)row * 2 + 1] = kk;
    }
  }
}

__global__ __launch_bounds__(ST) void k_split_compact(const float* __restrict__ scores, size_t ld,
                                                      int N, int L, int K, int n0, int R,
                                                      SplitWs ws, int32_t* __restrict__ topk,
                                                      int idx_rows_per_b, int idx_n_base,
                                                      const uint8_t* __restrict__ route, int Hq,
                                                      int rpt) {
  const int c = blockIdx.x, row = blockIdx.y;
  const int b = row / R, r = row - b * R;
  const int n = n0 + r;
  const int vis = L - N + n / rpt + 1;
  int32_t* o = topk + ((size_t)b * idx_rows_per_b + (n - idx_n_base)) * K;
  if (!row_has_sparse(route, b, Hq)) {
    if (c == 0)
      for (int i = threadIdx.x; i < K; i += ST) o[i] = -1;
    return;
  }
  if (vis <= K) {
    const int i0 = c * SCH, i1 = min(vis, i0 + SCH);
    for (int i = i0 + threadIdx.x; i < i1; i += ST) o[i] = i;
    if (c == 0)
      for (int i = vis + threadIdx.x; i < K; i += ST) o[i] = -1;
    return;
  }
  const int j0 = c * SCH, j1 = min(vis, j0 + SCH);
  if (j0 >= j1) return;
  __shared__ uint32_t scratch[ST / DSA_WAVE + 1];
  __shared__ uint32_t bases[2];
  const uint32_t T = ws.state[(size_t)row * 2 + 0];
  const uint32_t kk = ws.state[(size_t)row * 2 + 1];
  if (threadIdx.x == 0) {
    uint32_t sel_base = 0, tie_base = 0;
    const uint32_t* cc = ws.cnt + (size_t)row * ws.nchunks * 2;
    for (int i = 0; i < c; ++i) {
      const uint32_t g = cc[2 * i], e = cc[2 * i + 1];
      const uint32_t take = (kk > tie_base) ? min(e, kk - tie_base) : 0u;
      sel_base += g + take;
      tie_base += e;
    }
    bases[0] = sel_base;
    bases[1] = tie_base;
  }
  __syncthreads();
  uint32_t base_sel = bases[0], base_tie = bases[1];
  const float* srow = scores + (size_t)row * ld;
  for (int start = j0; start < j1; start += ST) {
    const int j = start + threadIdx.x;
    const uint32_t u = (j < j1) ? radix_key(srow[j]) : 0u;
    const bool gt = (j < j1) && u > T;
    const bool eq = (j < j1) && u == T;
    uint32_t tie_tot, sel_tot;
    const uint32_t tie_rank = block_rank<ST>(eq, scratch, tie_tot);
    const bool sel = gt || (eq && base_tie + tie_rank < kk);
    const uint32_t pos = block_rank<ST>(sel, scratch, sel_tot);
    if (sel && base_sel + pos < (uint32_t)K) o[base_sel + pos] = j;
    base_tie += tie_tot;
    base_sel += sel_tot;
  }
}

__global__ void k_fill_u32(uint32_t* p, size_t n, uint32_t v) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

}  // namespace

hipError_t launch_fill_u32(uint32_t* p, size_t n, uint32_t value, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int blocks = (int)std::min<size_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(k_fill_u32, dim3(blocks), dim3(256), 0, s, p, n, value);
  return hipGetLastError();
}

hipError_t launch_topk_rows(const Dims& D, const float* scores, size_t ld, int n0, int R,
                            int32_t* topk, int idx_rows_per_b, int idx_n_base,
                            const uint8_t* route, hipStream_t s) {
  if (D.B == 0 || R == 0) return hipSuccess;
  // rows up to kMaxWords * 32 positions: one read of the row (candidate
  // list in LDS); longer rows: the multi-pass kernel
  const long long vmax = (long long)D.L - D.N + (n0 + R - 1) / D.IH + 1;
  const dim3 grid(R, D.B);
  ProfScope ps(s, kStageTopk);
  if (vmax <= 32768)
    hipLaunchKernelGGL((k_topk_cand<512, 6144>), grid, dim3(512), 0, s, scores, ld, D.N, D.L, D.K,
                       n0, R, topk, idx_rows_per_b, idx_n_base, route, D.Hq, D.IH);
  else if (vmax <= (long long)kMaxWords * 32)
    hipLaunchKernelGGL((k_topk_cand<1024, 8192>), grid, dim3(1024), 0, s, scores, ld, D.N, D.L,
                       D.K, n0, R, topk, idx_rows_per_b, idx_n_base, route, D.Hq, D.IH);
  else
    hipLaunchKernelGGL(k_topk_rows, grid, dim3(RT), 0, s, scores, ld, D.N, D.L, D.K, n0, R, topk,
                       idx_rows_per_b, idx_n_base, route, D.Hq, D.IH);
  return hipGetLastError();
}

size_t split_topk_ws_bytes(const Dims& D, int R) {
  const size_t rows = (size_t)D.B * R;
  const size_t nch = ((size_t)D.L + SCH - 1) / SCH;
  return rows * (kHistWords + nch * 2 + 2) * sizeof(uint32_t);
}

hipError_t launch_topk_split(const Dims& D, const float* scores, size_t ld, int n0, int R,
                             int32_t* topk, int idx_rows_per_b, int idx_n_base,
                             const uint8_t* route, void* wsp, hipStream_t s) {
  if (D.B == 0 || R == 0) return hipSuccess;
  const int rows = D.B * R;
  SplitWs ws;
  ws.nchunks = (D.L + SCH - 1) / SCH;
  ws.hist = (uint32_t*)wsp;
  ws.cnt = ws.hist + (size_t)rows * kHistWords;
  ws.state = ws.cnt + (size_t)rows * ws.nchunks * 2;
  ProfScope ps(s, kStageTopk);
  hipError_t e = launch_fill_u32(ws.hist, (size_t)rows * kHistWords, 0u, s);
  if (e != hipSuccess) return e;
  const dim3 grid(ws.nchunks, rows);
  hipLaunchKernelGGL(k_split_hist<0>, grid, dim3(ST), 0, s, scores, ld, D.N, D.L, D.K, n0, R, ws,
                     route, D.Hq, D.IH);
  hipLaunchKernelGGL(k_split_hist<1>, grid, dim3(ST), 0, s, scores, ld, D.N, D.L, D.K, n0, R, ws,
                     route, D.Hq, D.IH);
  hipLaunchKernelGGL(k_split_hist<2>, grid, dim3(ST), 0, s, scores, ld, D.N, D.L, D.K, n0, R, ws,
                     route, D.Hq, D.IH);
  hipLaunchKernelGGL(k_split_count, grid, dim3(ST), 0, s, scores, ld, D.N, D.L, D.K, n0, R, ws,
                     route, D.Hq, D.IH);
  hipLaunchKernelGGL(k_split_compact, grid, dim3(ST), 0, s, scores, ld, D.N, D.L, D.K, n0, R, ws,
                     topk, idx_rows_per_b, idx_n_base, route, D.Hq, D.IH);
  return hipGetLastError();
}

}  // namespace dsa
