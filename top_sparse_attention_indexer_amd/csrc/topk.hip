// Exact top-K per query row with ties to the lower position.
//
// Selection rule of the page "超大规模MoE架构中稀疏注意力机制的演进与实践"
// (§二.1: keep the K = 2048 best-scoring past positions whatever the context
// length) and of "混合注意力架构演进：从线性注意力到稀疏门控的技术权衡" (§三,
// an index array of shape [L, top_k]); rows with at most K visible keys keep
// all of them.
//
// Method: radix select on the order-preserving 32-bit key of each float score
// in three digit passes (11, 11, 10 bits) with LDS histograms, which yields the
// exact K-th key T and the number kk of keys equal to T that are still needed.
// An ordered compaction (wave ballots + popcounts, blocks scanned in position
// order) then writes every key > T and the first kk keys == T, ascending.
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

template <int NT>
__device__ __forceinline__ uint32_t block_sum_u32(uint32_t x, uint32_t* scratch) {
  uint32_t total;
  block_excl_scan<NT>(x, scratch, total);
  return total;
}

// ---------------------------------------------------------------- one row per workgroup
constexpr int RT = 1024;

__global__ __launch_bounds__(RT) void k_topk_rows(const float* __restrict__ scores, size_t ld,
                                                  int N, int L, int K, int n0, int R,
                                                  int32_t* __restrict__ topk, int idx_rows_per_b,
                                                  int idx_n_base, const uint8_t* __restrict__ route,
                                                  int Hq) {
  const int r = blockIdx.x, b = blockIdx.y;
  const int n = n0 + r;
  int32_t* o = topk + ((size_t)b * idx_rows_per_b + (n - idx_n_base)) * K;
  const int vis = L - N + n + 1;
  if (!row_has_sparse(route, b, Hq)) {
    for (int i = threadIdx.x; i < K; i += RT) o[i] = -1;
    return;
  }
  if (vis <= K) {
    for (int i = threadIdx.x; i < K; i += RT) o[i] = (i < vis) ? i : -1;
    return;
  }
  const float* row = scores + ((size_t)b * R + r) * ld;
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t scratch[RT / DSA_WAVE + 1];
  __shared__ uint32_t res[2];

  uint32_t prefix = 0, mask = 0, kk = (uint32_t)K;
  for (int lv = 0; lv < 3; ++lv) {
    const int shift = kShift[lv], nb = kBins[lv];
    for (int i = threadIdx.x; i < nb; i += RT) hist[i] = 0;
    __syncthreads();
    for (int j = threadIdx.x; j < vis; j += RT) {
      const uint32_t u = radix_key(row[j]);
      if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & (nb - 1)], 1u);
    }
    __syncthreads();
    pick_bin<RT>(hist, nb, kk, scratch, res);
    const uint32_t t = res[0], above = res[1];
    prefix |= t << shift;
    mask |= (uint32_t)(nb - 1) << shift;
    kk -= above;
    __syncthreads();
  }

  const uint32_t T = prefix;
  uint32_t base_sel = 0, base_tie = 0;
  for (int start = 0; start < vis; start += RT) {
    const int j = start + threadIdx.x;
    const uint32_t u = (j < vis) ? radix_key(row[j]) : 0u;
    const bool gt = (j < vis) && u > T;
    const bool eq = (j < vis) && u == T;
    uint32_t tie_tot, sel_tot;
    const uint32_t tie_rank = block_rank<RT>(eq, scratch, tie_tot);
    const bool sel = gt || (eq && base_tie + tie_rank < kk);
    const uint32_t pos = block_rank<RT>(sel, scratch, sel_tot);
    if (sel && base_sel + pos < (uint32_t)K) o[base_sel + pos] = j;
    base_tie += tie_tot;
    base_sel += sel_tot;
  }
}

// ------------------------------------------------ one row per workgroup, row in registers
// Rows of at most NT * E scores: each thread owns E consecutive positions.
// The keys are read with vector loads in chunks of EC per thread; when the
// row is one chunk (E <= 32) it is read once and every pass works from
// registers, otherwise each pass re-reads its chunks (one batch of loads per
// chunk, from cache).  The three digit levels histogram the keys in LDS and
// the ordered write needs one block scan, since positions are contiguous per
// thread.  The first-level histogram is kept in four copies (by wave) so that
// fewer waves contend for one bin.
constexpr int kCopies = 4;

template <int NT, int E>
__global__ __launch_bounds__(NT) void k_topk_rows_reg(const float* __restrict__ scores, size_t ld,
                                                      int N, int L, int K, int n0, int R,
                                                      int32_t* __restrict__ topk,
                                                      int idx_rows_per_b, int idx_n_base,
                                                      const uint8_t* __restrict__ route, int Hq) {
  constexpr int EC = E < 32 ? E : 32;   // keys per chunk
  constexpr int NCH = E / EC;
  const int r = blockIdx.x, b = blockIdx.y;
  const int n = n0 + r;
  int32_t* o = topk + ((size_t)b * idx_rows_per_b + (n - idx_n_base)) * K;
  const int vis = L - N + n + 1;
  if (!row_has_sparse(route, b, Hq)) {
    for (int i = threadIdx.x; i < K; i += NT) o[i] = -1;
    return;
  }
  if (vis <= K) {
    for (int i = threadIdx.x; i < K; i += NT) o[i] = (i < vis) ? i : -1;
    return;
  }
  __shared__ uint32_t hist[kCopies * 2048];
  __shared__ uint32_t scratch[NT / DSA_WAVE + 1];
  __shared__ uint32_t res[2];
  const float* row = scores + ((size_t)b * R + r) * ld;
  const int jt = threadIdx.x * E;   // this thread's positions [jt, jt + E)
  uint32_t key[EC];
  // keys of chunk c (positions jt + c * EC ..); 0 below every real key
  auto load_keys = [&](int c) {
    const int j0 = jt + c * EC;
    if ((ld & 3) == 0) {
      // whole vectors inside the row's ld columns are read unconditionally
      // (columns past vis exist in the buffer) and masked afterwards
#pragma unroll
      for (int x = 0; x < EC; x += 4) {
        const int j = j0 + x;
        float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
        if (j + 3 < (int)ld) f = *reinterpret_cast<const float4*>(row + j);
        else if (j < vis)
          for (int y = 0; y < 4; ++y) (&f.x)[y] = (j + y < vis) ? row[j + y] : 0.f;
        key[x] = (j < vis) ? radix_key(f.x) : 0u;
        key[x + 1] = (j + 1 < vis) ? radix_key(f.y) : 0u;
        key[x + 2] = (j + 2 < vis) ? radix_key(f.z) : 0u;
        key[x + 3] = (j + 3 < vis) ? radix_key(f.w) : 0u;
      }
    } else {
#pragma unroll
      for (int x = 0; x < EC; ++x) key[x] = (j0 + x < vis) ? radix_key(row[j0 + x]) : 0u;
    }
  };
  auto nvalid = [&](int c) { return max(0, min(EC, vis - (jt + c * EC))); };
  if (NCH == 1) load_keys(0);
  // A lower bound for the first-level bin of the K-th key from one key per
  // thread: bins below b_lo are then left out of the histogram, which keeps
  // the many keys far under the threshold (the crowded bins) away from the
  // LDS atomics.  If fewer than K keys reach b_lo the bound was too high and
  // the full histogram is built instead, so the result is exact either way.
  for (int i = threadIdx.x; i < kCopies * 2048; i += NT) hist[i] = 0;
  if (threadIdx.x == 0) res[0] = 0;
  __syncthreads();
  // samples: the first key of every thread holding positions; about
  // 1.5 K * nsamp / vis of them are expected at or above the K-th key's bin
  const long long nsamp = min((long long)NT, ((long long)vis + E - 1) / E);
  const long long want = (3LL * K * nsamp) / (2LL * vis) + 8;
  if (want < nsamp / 2) {
    if (NCH > 1) load_keys(0);
    if (nvalid(0) > 0) atomicAdd(&hist[2048 + (key[0] >> 21)], 1u);
    __syncthreads();
    pick_bin<NT>(hist + 2048, 2048, (uint32_t)want, scratch, res);
    if (threadIdx.x < 2048 / 2) {   // clear the sample histogram for level 0
      hist[2048 + 2 * threadIdx.x] = 0;
      hist[2048 + 2 * threadIdx.x + 1] = 0;
    }
    __syncthreads();
  }
  uint32_t b_lo = res[0];
  // level 0: top 11 bits of the keys in bins >= b_lo, four histogram copies
  uint32_t nhi = 0;
  {
    uint32_t* hc = hist + ((threadIdx.x / DSA_WAVE) % kCopies) * 2048;
    for (int c = 0; c < NCH; ++c) {
      if (NCH > 1) load_keys(c);
      const int nv = nvalid(c);
#pragma unroll
      for (int x = 0; x < EC; ++x)
        if (x < nv && (key[x] >> 21) >= b_lo) {
          atomicAdd(&hc[key[x] >> 21], 1u);
          ++nhi;
        }
    }
    if (b_lo > 0 && block_sum_u32<NT>(nhi, scratch) < (uint32_t)K) {
      // the bound was too high: add the keys below it
      for (int c = 0; c < NCH; ++c) {
        if (NCH > 1) load_keys(c);
        const int nv = nvalid(c);
#pragma unroll
        for (int x = 0; x < EC; ++x)
          if (x < nv && (key[x] >> 21) < b_lo) atomicAdd(&hc[key[x] >> 21], 1u);
      }
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 2048; i += NT) {
    uint32_t t = 0;
#pragma unroll
    for (int c = 0; c < kCopies; ++c) t += hist[c * 2048 + i];
    hist[i] = t;
  }
  __syncthreads();
  uint32_t kk = (uint32_t)K;
  pick_bin<NT>(hist, 2048, kk, scratch, res);
  const uint32_t t0 = res[0];
  kk -= res[1];
  __syncthreads();
  // level 1: next 11 bits of the keys in bin t0
  for (int i = threadIdx.x; i < 2048; i += NT) hist[i] = 0;
  __syncthreads();
  for (int c = 0; c < NCH; ++c) {
    if (NCH > 1) load_keys(c);
    const int nv = nvalid(c);
#pragma unroll
    for (int x = 0; x < EC; ++x)
      if (x < nv && (key[x] >> 21) == t0) atomicAdd(&hist[(key[x] >> 10) & 2047u], 1u);
  }
  __syncthreads();
  pick_bin<NT>(hist, 2048, kk, scratch, res);
  const uint32_t pfx = (t0 << 11) | res[0];
  kk -= res[1];
  __syncthreads();
  // level 2: last 10 bits of the keys sharing the top 22
  for (int i = threadIdx.x; i < 1024; i += NT) hist[i] = 0;
  __syncthreads();
  for (int c = 0; c < NCH; ++c) {
    if (NCH > 1) load_keys(c);
    const int nv = nvalid(c);
#pragma unroll
    for (int x = 0; x < EC; ++x)
      if (x < nv && (key[x] >> 10) == pfx) atomicAdd(&hist[key[x] & 1023u], 1u);
  }
  __syncthreads();
  pick_bin<NT>(hist, 1024, kk, scratch, res);
  const uint32_t T = (pfx << 10) | res[0];
  kk -= res[1];   // keys equal to T still to take, lowest positions first
  // ordered write: keys > T, and the first kk keys == T
  uint32_t ngt = 0, neq = 0;
  for (int c = 0; c < NCH; ++c) {
    if (NCH > 1) load_keys(c);
    const int nv = nvalid(c);
#pragma unroll
    for (int x = 0; x < EC; ++x) {
      ngt += (x < nv && key[x] > T);
      neq += (x < nv && key[x] == T);
    }
  }
  uint32_t tot_eq;
  const uint32_t eq_before = block_excl_scan<NT>(neq, scratch, tot_eq);
  const uint32_t take_eq = (eq_before >= kk) ? 0u : min(neq, kk - eq_before);
  uint32_t tot_sel;
  uint32_t pos = block_excl_scan<NT>(ngt + take_eq, scratch, tot_sel);
  uint32_t eq_seen = 0;
  for (int c = 0; c < NCH; ++c) {
    if (NCH > 1) load_keys(c);
    const int nv = nvalid(c);
#pragma unroll
    for (int x = 0; x < EC; ++x) {
      const bool v = x < nv;
      const bool eq = v && key[x] == T;
      const bool sel = (v && key[x] > T) || (eq && eq_seen < take_eq);
      eq_seen += eq;
      if (sel && pos < (uint32_t)K) o[pos] = jt + c * EC + x;
      pos += sel;
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
                                                   int Hq) {
  const int c = blockIdx.x, row = blockIdx.y;  // row = b * R + r
  const int b = row / R, r = row - b * R;
  const int vis = L - N + n0 + r + 1;
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
                                                    int Hq) {
  const int c = blockIdx.x, row = blockIdx.y;
  const int b = row / R, r = row - b * R;
  const int vis = L - N + n0 + r + 1;
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
                                                      const uint8_t* __restrict__ route, int Hq) {
  const int c = blockIdx.x, row = blockIdx.y;
  const int b = row / R, r = row - b * R;
  const int n = n0 + r;
  const int vis = L - N + n + 1;
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
  // the longest row of the launch decides how many scores each thread holds
  const long long vmax = (long long)D.L - D.N + n0 + R;
  const dim3 grid(R, D.B);
#define DSA_TOPK_REG(NT, E)                                                                  \
  hipLaunchKernelGGL((k_topk_rows_reg<NT, E>), grid, dim3(NT), 0, s, scores, ld, D.N, D.L, D.K, \
                     n0, R, topk, idx_rows_per_b, idx_n_base, route, D.Hq)
  if (vmax <= 1024LL * 8) DSA_TOPK_REG(1024, 8);
  else if (vmax <= 1024LL * 16) DSA_TOPK_REG(1024, 16);
  else if (vmax <= 1024LL * 32) DSA_TOPK_REG(1024, 32);
  else
    hipLaunchKernelGGL(k_topk_rows, grid, dim3(RT), 0, s, scores, ld, D.N, D.L, D.K, n0, R, topk,
                       idx_rows_per_b, idx_n_base, route, D.Hq);
#undef DSA_TOPK_REG
  return hipGetLastError();
}

int split_topk_chunk() { return SCH; }

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
  hipError_t e = launch_fill_u32(ws.hist, (size_t)rows * kHistWords, 0u, s);
  if (e != hipSuccess) return e;
  const dim3 grid(ws.nchunks, rows);
  hipLaunchKernelGGL(k_split_hist<0>, grid, dim3(ST), 0, s, scores, ld, D.N, D.L, D.K, n0, R, ws,
                     route, D.Hq);
  hipLaunchKernelGGL(k_split_hist<1>, grid, dim3(ST), 0, s, scores, ld, D.N, D.L, D.K, n0, R, ws,
                     route, D.Hq);
  hipLaunchKernelGGL(k_split_hist<2>, grid, dim3(ST), 0, s, scores, ld, D.N, D.L, D.K, n0, R, ws,
                     route, D.Hq);
  hipLaunchKernelGGL(k_split_count, grid, dim3(ST), 0, s, scores, ld, D.N, D.L, D.K, n0, R, ws,
                     route, D.Hq);
  hipLaunchKernelGGL(k_split_compact, grid, dim3(ST), 0, s, scores, ld, D.N, D.L, D.K, n0, R, ws,
                     topk, idx_rows_per_b, idx_n_base, route, D.Hq);
  return hipGetLastError();
}

}  // namespace dsa
