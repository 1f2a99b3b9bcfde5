// Indexer scores and exact top-K for prefill without a score matrix in HBM.
//
// The indexer product of "超大规模MoE架构中稀疏注意力机制的演进与实践" §二.1-§二.2
// (q_idx . k_idx over every visible position, no rotary term) and its top-K,
// computed blockwise and kept on chip, as "大模型推理架构演进：从稀疏注意力到隐式
// 专家路由" §2.2-§2.3 describes (per query, a selection made without writing
// the whole query x key matrix).
//
// Four kernels, all computing scores on MFMA with the same instruction,
// operands and accumulation order as the materialising indexer (so the same
// float values):
//   k_idx_tau: per query row, a strided sample of its visible keys gives its
//     score range and a 256-bin histogram; the threshold tau is the lower
//     edge of the bin that brings the count from the top to about
//     1.5 K * samples / visible (no threshold when that covers every key).
//   k_idx_scan<false>: workgroups of 128 rows x 256 keys (each wave two
//     16-row MFMA column blocks on one key operand) count, per (row, key
//     chunk), the scores >= tau; k_idx_offsets turns the counts into each
//     chunk's offset in the row's candidate list;
//   k_idx_scan<true>: the same tiles again, appending (score, position) of
//     every score >= tau at its offset, so the list is in position order.
// k_topk_cands: one workgroup per row.  If the list holds at least K keys and
// did not overflow, it holds every key >= tau, hence every key >= the K-th
// largest score (which is >= tau): the exact selection (radix digits 11/11/10
// on the order-preserving key, ties to the lower position) runs on the list,
// and an ordered compaction writes the positions ascending.  Otherwise the
// row falls back to the same selection streamed over recomputed scores.
#include "common.h"
#include "launch.h"
#include "mfma.h"
#include "attn_tile.h"

namespace dsa {
namespace {

constexpr int FT = 256;           // threads of the filter (4 waves)
constexpr int kRowsPerWg = 64;
constexpr int kScanRows = 128;     // rows per scan workgroup (two 16-row blocks per wave)
constexpr int kSamples = 2048;    // sampled keys per row (at most)
constexpr int kBins = 256;
constexpr int CT = 512;           // threads of the selection
constexpr int kShift[3] = {21, 10, 0};
constexpr int kDigitBins[3] = {2048, 2048, 1024};

__device__ __forceinline__ bool any_sparse(const uint8_t* route, int b, int Hq) {
  if (!route) return true;
  for (int h = 0; h < Hq; ++h)
    if (route[(size_t)b * Hq + h]) return true;
  return false;
}

constexpr int KC = 256;           // keys per scan tile

struct FilterArgs {
  const bf16_bits* q_idx; const bf16_bits* k_idx; const uint8_t* route;
  float2* cand;       // [B * R][cap] (score, position as float bits)
  int32_t* count;     // [B * R] keys >= tau (may exceed cap)
  float* tau;         // [B * R] threshold (-inf: every visible key)
  int32_t* ccnt;      // [B * R][nkc] per key chunk: count, then offset
  int N, L, K, Hq;
  int n0, R;          // query rows [n0, n0 + R) of each sequence
  int cap, nkc;       // list capacity; key chunks of the longest row
  long long B_rows;   // B * R
  int rpt;            // virtual rows per token (indexer heads)
};

// Scores of 16 keys (rows of the A operand: key j0 + i for lane i of each
// quad) against the 16 query columns held in qb; lane (q, i) receives the
// scores of keys j0 + 4q .. j0 + 4q + 3 for column i.  Keys at or beyond
// `lim` read as zero rows.
template <int DIDX>
__device__ __forceinline__ f32x4 score16(const bf16_bits* kseq, int j0, int lim,
                                         const bf16x8 (&qb)[DIDX / 32]) {
  constexpr int T = DIDX / 32;
  const int lane = threadIdx.x & 63;
  const int q = lane >> 4, i = lane & 15;
  const int jk = j0 + i;
  uint4 kb[T];
#pragma unroll
  for (int t = 0; t < T; ++t)
    kb[t] = jk < lim ? *reinterpret_cast<const uint4*>(kseq + (size_t)jk * DIDX + t * 32 + q * 8)
                     : make_uint4(0, 0, 0, 0);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < T; ++t) acc = mfma16(as_bf16x8(kb[t]), qb[t], acc);
  return acc;
}

// Per-row threshold from a strided sample (one workgroup per 64 rows).
template <int DIDX>
__global__ __launch_bounds__(FT) void k_idx_tau(FilterArgs a) {
  constexpr int T = DIDX / 32;
  // per wave: 16 rows x kBins counters, two 16-bit counts per word
  __shared__ uint32_t hist[4][16][kBins / 2];
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int q = lane >> 4, i = lane & 15;
  const int r0 = blockIdx.x * kRowsPerWg + w * 16;
  if (r0 >= a.R) return;                       // wave-uniform; no block barrier below
  const int r = r0 + i;
  const bool rv = r < a.R;
  const int p = a.L - a.N + (a.n0 + (rv ? r : r0)) / a.rpt;   // this column's last visible key
  const int vis = p + 1;
  const int p_hi = a.L - a.N + (a.n0 + min(a.R - 1, r0 + 15)) / a.rpt;
  const bool need = rv && vis > a.K && any_sparse(a.route, b, a.Hq);
  if (p_hi + 1 <= a.K || !any_sparse(a.route, b, a.Hq)) {
    if (rv && q == 0) a.tau[(size_t)b * a.R + r] = -INFINITY;
    return;
  }
  bf16x8 qb[T];
  {
    const bf16_bits* qr = a.q_idx + ((size_t)b * a.N * a.rpt + a.n0 + (rv ? r : r0)) * DIDX;
#pragma unroll
    for (int t = 0; t < T; ++t)
      qb[t] = as_bf16x8(*reinterpret_cast<const uint4*>(qr + t * 32 + q * 8));
  }
  const bf16_bits* kseq = a.k_idx + (size_t)b * a.L * DIDX;
  // sample: keys s * stride, s = 0 .. ns - 1, over the wave's range
  const int stride = max(1, (p_hi + kSamples) / kSamples);
  const int ns = p_hi / stride + 1;            // samples of the longest row
  // scores of the sample blocks s0 .. s0 + 16 SU - 1 (A operand rows: sample
  // keys (s0 + 16 uu + i) * stride), SU blocks of loads in flight together
  constexpr int SU = 8;
  auto sample_scores = [&](int s0, f32x4 (&acc)[SU]) {
    uint4 kb[SU][T];
#pragma unroll
    for (int uu = 0; uu < SU; ++uu) {
      const int sx = s0 + uu * 16 + i;
      const size_t js = (size_t)min(sx, ns - 1) * stride;
#pragma unroll
      for (int t = 0; t < T; ++t)
        kb[uu][t] = *reinterpret_cast<const uint4*>(kseq + js * DIDX + t * 32 + q * 8);
    }
#pragma unroll
    for (int uu = 0; uu < SU; ++uu) {
      acc[uu] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < T; ++t) acc[uu] = mfma16(as_bf16x8(kb[uu][t]), qb[t], acc[uu]);
    }
  };
  float mn = INFINITY, mx = -INFINITY;
  for (int s0 = 0; s0 < ns; s0 += 16 * SU) {
    f32x4 acc[SU];
    sample_scores(s0, acc);
#pragma unroll
    for (int uu = 0; uu < SU; ++uu)
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int sidx = s0 + uu * 16 + 4 * q + x;
        if (sidx < ns && sidx * stride <= p) {
          mn = fminf(mn, acc[uu][x]);
          mx = fmaxf(mx, acc[uu][x]);
        }
      }
  }
  mn = -max_xor32(max_xor16(-mn));
  mx = max_xor32(max_xor16(mx));
  // histogram of the samples over [mn, mx] in kBins bins
  for (int e = lane; e < 16 * kBins / 2; e += 64) hist[w][e / (kBins / 2)][e % (kBins / 2)] = 0;
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  const float span = mx - mn;
  const float scale = span > 0.f ? (float)kBins / span : 0.f;
  for (int s0 = 0; s0 < ns; s0 += 16 * SU) {
    f32x4 acc[SU];
    sample_scores(s0, acc);
#pragma unroll
    for (int uu = 0; uu < SU; ++uu)
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int sidx = s0 + uu * 16 + 4 * q + x;
        if (need && sidx < ns && sidx * stride <= p) {
          const int bin = min(kBins - 1, max(0, (int)((acc[uu][x] - mn) * scale)));
          atomicAdd(&hist[w][i][bin >> 1], 1u << (16 * (bin & 1)));
        }
      }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  // threshold: lower edge of the bin where the count from the top reaches
  // about 1.5 K * (samples of this row) / visible (lane quad 0 scans)
  if (rv && q == 0) {
    float tau = -INFINITY;
    if (need && span > 0.f) {
      const int nsr = p / stride + 1;
      const int want = (int)((3LL * a.K * nsr + 2LL * vis - 1) / (2LL * vis)) + 2;
      int run = 0, bin = -1;
      for (int bb = kBins - 1; bb >= 0; --bb) {
        const uint32_t wd = hist[w][i][bb >> 1];
        run += (int)((wd >> (16 * (bb & 1))) & 0xffffu);
        if (run >= want) {
          bin = bb;
          break;
        }
      }
      if (bin > 0) tau = mn + (float)bin / scale;
    }
    a.tau[(size_t)b * a.R + r] = tau;
  }
}

// One tile of 64 rows x KC keys: per (row, chunk) the count of scores >= tau
// (WRITE = false), or the candidates themselves at the chunk's offset in the
// row's list (WRITE = true).  The tile's key rows go once into LDS (direct
// loads, whole rows per lane group, chunks permuted as kt_swz) and the four
// waves read their MFMA operands there.  Within a chunk, the four lane quads
// of a column hold keys 4q .. 4q + 3 of each 16-key block, so a prefix over
// the quads per block keeps the list in position order.
template <int DIDX, bool WRITE>
__global__ __launch_bounds__(FT) void k_idx_scan(FilterArgs a) {
  constexpr int T = DIDX / 32;
  constexpr int CPR = DIDX / 8;                  // 16-byte chunks per key row
  constexpr int RPI = 64 / CPR;                  // key rows per direct load
  constexpr int RB = kScanRows / 64;             // 16-row blocks per wave
  __shared__ __attribute__((aligned(16))) char ktile[KC * DIDX * 2];
  const int b = blockIdx.z, kc = blockIdx.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int q = lane >> 4, i = lane & 15;
  const int rb0 = blockIdx.x * kScanRows;
  // block-uniform exits: the block's last row bounds the keys it scans
  const int p_blk = a.L - a.N + (a.n0 + min(a.R - 1, rb0 + kScanRows - 1)) / a.rpt;
  const int j_lo = kc * KC;
  if (j_lo > p_blk || p_blk + 1 <= a.K || !any_sparse(a.route, b, a.Hq)) return;
  const int j_hi = min(j_lo + KC, p_blk + 1);   // keys [j_lo, j_hi) of this tile
  const bf16_bits* kseq = a.k_idx + (size_t)b * a.L * DIDX;
  // the tile's key rows into LDS (rows past j_hi read the last one; masked)
#pragma unroll
  for (int m = w; m < KC / RPI; m += 4) {
    const int rr = m * RPI + lane / CPR, pc = lane % CPR;
    const size_t j = (size_t)min(j_lo + rr, j_hi - 1);
    const int lc = pc ^ (rr & (CPR - 1));
    __builtin_amdgcn_global_load_lds((const void*)(kseq + j * DIDX + lc * 8),
                                     (__attribute__((address_space(3))) void*)(ktile + m * 1024),
                                     16, 0, 0);
  }
  // this wave's rows: block u holds rows r0 + 16 u + i (one MFMA column each)
  const int r0 = rb0 + w * 16 * RB;
  bool need[RB];
  float tau[RB];
  int lim[RB];                                    // keys below lim are visible
  size_t row[RB];
  bf16x8 qb[RB][T];
#pragma unroll
  for (int u = 0; u < RB; ++u) {
    const int r = r0 + 16 * u + i;
    const bool rv = r < a.R;
    row[u] = (size_t)b * a.R + (rv ? r : 0);
    const int p = a.L - a.N + (a.n0 + (rv ? r : 0)) / a.rpt;
    need[u] = rv && p + 1 > a.K && j_lo <= p;
    // a row without a list has tau = +inf, so no score passes it
    tau[u] = need[u] ? a.tau[row[u]] : INFINITY;
    lim[u] = need[u] ? p + 1 : 0;
    const bf16_bits* qr = a.q_idx + ((size_t)b * a.N * a.rpt + a.n0 + (rv ? r : 0)) * DIDX;
#pragma unroll
    for (int t = 0; t < T; ++t)
      qb[u][t] = as_bf16x8(rv ? *reinterpret_cast<const uint4*>(qr + t * 32 + q * 8)
                              : make_uint4(0, 0, 0, 0));
  }
  int run[RB];
#pragma unroll
  for (int u = 0; u < RB; ++u) run[u] = (WRITE && need[u]) ? a.ccnt[row[u] * a.nkc + kc] : 0;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();                               // the whole tile has landed
  // this wave's rows see keys up to p_w; keys up to p_w0 (its first row's
  // position) are visible to every row of the wave (wave-uniform values)
  const int p_w = __builtin_amdgcn_readfirstlane(
      a.L - a.N + (a.n0 + min(a.R - 1, r0 + 16 * RB - 1)) / a.rpt);
  const int p_w0 = __builtin_amdgcn_readfirstlane(a.L - a.N + (a.n0 + r0) / a.rpt);
  // the scores of a 16-key block for both row blocks, the key operand read
  // from LDS once
  auto scores = [&](int j0, f32x4 (&acc)[RB]) __attribute__((always_inline)) {
    const int u16 = (j0 - j_lo) >> 4;
    uint4 kv[T];
#pragma unroll
    for (int t = 0; t < T; ++t)
      kv[t] = *reinterpret_cast<const uint4*>(ktile + kt_swz<DIDX>(u16 * 16 + i, 4 * t + q));
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < T; ++t) acc[u] = mfma16(as_bf16x8(kv[t]), qb[u][t], acc[u]);
    }
  };
  if (!WRITE) {
    // counts only: per lane over the tiles, across the quads once at the end
    uint32_t cnt[RB];
#pragma unroll
    for (int u = 0; u < RB; ++u) cnt[u] = 0;
    if (r0 < a.R && j_lo <= p_w) {
      for (int j0 = j_lo; j0 < j_hi && j0 <= p_w; j0 += 16) {
        f32x4 acc[RB];
        scores(j0, acc);
        if (j0 + 15 <= p_w0) {
#pragma unroll
          for (int u = 0; u < RB; ++u)
#pragma unroll
            for (int x = 0; x < 4; ++x) cnt[u] += acc[u][x] >= tau[u] ? 1u : 0u;
        } else {
#pragma unroll
          for (int u = 0; u < RB; ++u)
#pragma unroll
            for (int x = 0; x < 4; ++x)
              cnt[u] += (j0 + 4 * q + x < lim[u] && acc[u][x] >= tau[u]) ? 1u : 0u;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      uint32_t c = cnt[u];
      c += __shfl_xor(c, 16, 64);
      c += __shfl_xor(c, 32, 64);
      if (need[u] && q == 0) a.ccnt[row[u] * a.nkc + kc] = (int)c;
    }
    return;
  }
  if (r0 < a.R && j_lo <= p_w) {
    for (int j0 = j_lo; j0 < j_hi && j0 <= p_w; j0 += 16) {
      f32x4 acc[RB];
      scores(j0, acc);
#pragma unroll
      for (int u = 0; u < RB; ++u) {
        uint32_t bits = 0;
#pragma unroll
        for (int x = 0; x < 4; ++x)
          bits |= (j0 + 4 * q + x < lim[u] && acc[u][x] >= tau[u]) ? (1u << x) : 0u;
        const uint32_t c = __popc(bits);
        // the partner lanes' counts by the gfx950 lane swaps (VALU, no LDS
        // round trip): each swap hands both lanes of a pair both values
        const auto s16 = __builtin_amdgcn_permlane16_swap(c, c, false, false);
        const uint32_t c1 = (q & 1) ? s16[0] : s16[1];         // quad q ^ 1
        const uint32_t pair = c + c1;
        const auto s32 = __builtin_amdgcn_permlane32_swap(pair, pair, false, false);
        const uint32_t pair2 = (q & 2) ? s32[0] : s32[1];      // the other pair
        // counts of the column's quads (lane 16 q + i): prefix over q
        const uint32_t before = ((q & 1) ? c1 : 0u) + ((q & 2) ? pair2 : 0u);
        uint32_t slot = (uint32_t)run[u] + before;
        float2* clist = a.cand + row[u] * a.cap;
        while (bits) {
          const int x = __ffs(bits) - 1;
          bits &= bits - 1;
          if (slot < (uint32_t)a.cap)
            clist[slot] = make_float2(acc[u][x], __int_as_float(j0 + 4 * q + x));
          ++slot;
        }
        run[u] += (int)(pair + pair2);
      }
    }
  }
}

// Counts of a row's key chunks -> their offsets in the row's list (in
// place), and the row's total.  One wave per row.
__global__ __launch_bounds__(FT) void k_idx_offsets(FilterArgs a) {
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (long long)a.B_rows) return;
  const int b = (int)(row / a.R), r = (int)(row - (long long)b * a.R);
  const int p = a.L - a.N + (a.n0 + r) / a.rpt;
  if (p + 1 <= a.K) return;
  const int nk = p / KC + 1;
  int32_t* cc = a.ccnt + (size_t)row * a.nkc;
  int base = 0;
  for (int k0 = 0; k0 < nk; k0 += 64) {
    const int k = k0 + lane;
    const uint32_t v = k < nk ? (uint32_t)cc[k] : 0u;
    const uint32_t incl = wave_incl_scan(v);
    if (k < nk) cc[k] = base + (int)(incl - v);
    base += (int)__builtin_amdgcn_readlane((int)incl, 63);
  }
  if (lane == 0) a.count[row] = base;
}

// kk-th largest over hist[0..nb) from the top: bin and count above it.
__device__ void pick_bin_ct(const uint32_t* hist, int nb, uint32_t kk, uint32_t* scratch,
                            uint32_t* res) {
  const int per = nb / CT;
  const int base = threadIdx.x * per;
  uint32_t mine = 0;
  for (int x = 0; x < per; ++x) mine += hist[base + x];
  uint32_t total;
  const uint32_t pre = block_excl_scan<CT>(mine, scratch, total);
  uint32_t running = total - pre - mine;
  for (int x = per - 1; x >= 0; --x) {
    const uint32_t c = hist[base + x];
    if (running < kk && running + c >= kk) {
      res[0] = (uint32_t)(base + x);
      res[1] = running;
    }
    running += c;
  }
  __syncthreads();
}

struct SelectArgs {
  const bf16_bits* q_idx; const bf16_bits* k_idx; const uint8_t* route;
  const float2* cand; const int32_t* count;
  int32_t* topk; int idx_rows_per_b, idx_n_base;
  int N, L, K, Hq;
  int n0, R, cap;
  int rpt;            // virtual rows per token (indexer heads)
};

constexpr int kCandLds = 6144;   // list entries held in LDS (cap must not exceed it)

// Exact selection streamed over the row's scores, recomputed per pass on MFMA
// exactly as the filter computes them (fallback for rows whose list cannot
// be used).  Passes: three digit levels, then the ordered compaction.
template <int DIDX>
__device__ void select_stream(const SelectArgs& a, int b, int n, int vis, int32_t* o,
                              uint32_t* hist, float* sc, uint32_t* scratch, uint32_t* res) {
  constexpr int T = DIDX / 32;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int q = lane >> 4, i = lane & 15;
  constexpr int NW = CT / 64;
  bf16x8 qb[T];
  {
    const bf16_bits* qr = a.q_idx + ((size_t)b * a.N * a.rpt + n) * DIDX;
#pragma unroll
    for (int t = 0; t < T; ++t)
      qb[t] = as_bf16x8(*reinterpret_cast<const uint4*>(qr + t * 32 + q * 8));
  }
  const bf16_bits* kseq = a.k_idx + (size_t)b * a.L * DIDX;
  // scores of keys [j0, j0 + 16 NW) into sc[] (wave w takes 16 of them)
  auto fill = [&](int j0) {
    const f32x4 acc = score16<DIDX>(kseq, j0 + 16 * w, vis, qb);
    if (i == 0) {
#pragma unroll
      for (int x = 0; x < 4; ++x) sc[16 * w + 4 * q + x] = acc[x];
    }
    __syncthreads();
  };
  uint32_t prefix = 0, mask = 0, kk = (uint32_t)a.K;
  for (int lv = 0; lv < 3; ++lv) {
    const int shift = kShift[lv], nb = kDigitBins[lv];
    for (int x = threadIdx.x; x < nb; x += CT) hist[x] = 0;
    __syncthreads();
    for (int j0 = 0; j0 < vis; j0 += 16 * NW) {
      fill(j0);
      const int j = j0 + (int)threadIdx.x;
      if (threadIdx.x < 16 * NW && j < vis) {
        const uint32_t u = radix_key(sc[threadIdx.x]);
        if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & (nb - 1)], 1u);
      }
      __syncthreads();
    }
    pick_bin_ct(hist, nb, kk, scratch, res);
    prefix |= res[0] << shift;
    mask |= (uint32_t)(nb - 1) << shift;
    kk -= res[1];
    __syncthreads();
  }
  const uint32_t Tk = prefix;
  uint32_t base_sel = 0, base_tie = 0;
  for (int j0 = 0; j0 < vis; j0 += 16 * NW) {
    fill(j0);
    const int j = j0 + (int)threadIdx.x;
    const bool in = threadIdx.x < 16 * NW && j < vis;
    const uint32_t u = in ? radix_key(sc[threadIdx.x]) : 0u;
    const bool gt = in && u > Tk, eq = in && u == Tk;
    uint32_t tie_tot, sel_tot;
    const uint32_t tie_rank = block_rank<CT>(eq, scratch, tie_tot);
    const bool sel = gt || (eq && base_tie + tie_rank < kk);
    const uint32_t pos = block_rank<CT>(sel, scratch, sel_tot);
    if (sel && base_sel + pos < (uint32_t)a.K) o[base_sel + pos] = j;
    base_tie += tie_tot;
    base_sel += sel_tot;
  }
}

template <int DIDX>
__global__ __launch_bounds__(CT) void k_topk_cands(SelectArgs a) {
  __shared__ uint32_t hist[2048];
  // keys only: the positions are read again from the list (in L2) by the
  // final compaction, which halves the LDS and doubles the resident rows
  __shared__ uint32_t ckey[kCandLds];
  __shared__ float sc[16 * (CT / 64)];
  __shared__ uint32_t scratch[CT / 64 + 1];
  __shared__ uint32_t wcnt[2 * (CT / 64)];
  __shared__ uint32_t res[2];
  const int r = blockIdx.x, b = blockIdx.y;
  const int n = a.n0 + r;
  int32_t* o = a.topk + ((size_t)b * a.idx_rows_per_b + (n - a.idx_n_base)) * a.K;
  const int vis = a.L - a.N + n / a.rpt + 1;
  if (!any_sparse(a.route, b, a.Hq)) {
    for (int x = threadIdx.x; x < a.K; x += CT) o[x] = -1;
    return;
  }
  if (vis <= a.K) {
    for (int x = threadIdx.x; x < a.K; x += CT) o[x] = (x < vis) ? x : -1;
    return;
  }
  const int cnt = a.count[(size_t)b * a.R + r];
  if (cnt < a.K || cnt > a.cap) {
    select_stream<DIDX>(a, b, n, vis, o, hist, sc, scratch, res);
    return;
  }
  // the list into LDS (order-preserving keys), first digit counted on the way
  const float2* cl = a.cand + ((size_t)b * a.R + r) * a.cap;
  for (int x = threadIdx.x; x < 2048; x += CT) hist[x] = 0;
  __syncthreads();
  for (int x = threadIdx.x; x < cnt; x += CT) {
    const float2 e = cl[x];
    const uint32_t u = radix_key(e.x);
    ckey[x] = u;
    atomicAdd(&hist[u >> 21], 1u);
  }
  __syncthreads();
  uint32_t kk = (uint32_t)a.K;
  pick_bin_ct(hist, 2048, kk, scratch, res);
  const uint32_t t0 = res[0];
  kk -= res[1];
  __syncthreads();
  for (int x = threadIdx.x; x < 2048; x += CT) hist[x] = 0;
  __syncthreads();
  for (int x = threadIdx.x; x < cnt; x += CT) {
    const uint32_t u = ckey[x];
    if ((u >> 21) == t0) atomicAdd(&hist[(u >> 10) & 2047u], 1u);
  }
  __syncthreads();
  pick_bin_ct(hist, 2048, kk, scratch, res);
  const uint32_t pfx = (t0 << 11) | res[0];
  kk -= res[1];
  __syncthreads();
  for (int x = threadIdx.x; x < 1024; x += CT) hist[x] = 0;
  __syncthreads();
  for (int x = threadIdx.x; x < cnt; x += CT) {
    const uint32_t u = ckey[x];
    if ((u >> 10) == pfx) atomicAdd(&hist[u & 1023u], 1u);
  }
  __syncthreads();
  pick_bin_ct(hist, 1024, kk, scratch, res);
  const uint32_t Tk = (pfx << 10) | res[0];
  kk -= res[1];   // keys equal to Tk still to take, lowest positions first
  // ordered compaction (the list is in position order).  Wave w takes the
  // entries [w * span, (w + 1) * span) in rounds of 64: a count pass of its
  // keys above Tk and equal to Tk, one exchange of the waves' counts, then
  // the write pass.  An entry's output slot is the number of selected
  // entries before it: every key above Tk, and the first kk keys equal to Tk.
  {
    constexpr int NW = CT / 64;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int span = (cnt + NW * 64 - 1) / (NW * 64) * 64;
    const int xb = w * span, xe = min(cnt, xb + span);
    uint32_t ngt = 0, neq = 0;
    for (int x0 = xb; x0 < xe; x0 += 64) {
      const int x = x0 + lane;
      const uint32_t u = x < xe ? ckey[x] : 0u;
      ngt += (uint32_t)__popcll(__ballot(x < xe && u > Tk));
      neq += (uint32_t)__popcll(__ballot(x < xe && u == Tk));
    }
    if (lane == 0) {
      wcnt[w] = ngt;
      wcnt[NW + w] = neq;
    }
    __syncthreads();
    uint32_t gtb = 0, tb = 0;   // keys above / equal to Tk before this wave's span
    for (int v = 0; v < w; ++v) {
      gtb += wcnt[v];
      tb += wcnt[NW + v];
    }
    const uint64_t below = lanemask_lt();
    for (int x0 = xb; x0 < xe; x0 += 64) {
      const int x = x0 + lane;
      const bool in = x < xe;
      const uint32_t u = in ? ckey[x] : 0u;
      const bool gt = in && u > Tk, eq = in && u == Tk;
      const uint64_t mgt = __ballot(gt), meq = __ballot(eq);
      const uint32_t g0 = gtb + (uint32_t)__popcll(mgt & below);
      const uint32_t t0l = tb + (uint32_t)__popcll(meq & below);
      const bool sel = gt || (eq && t0l < kk);
      const uint32_t pos = g0 + min(t0l, kk);
      if (sel && pos < (uint32_t)a.K) o[pos] = __float_as_int(cl[x].y);
      gtb += (uint32_t)__popcll(mgt);
      tb += (uint32_t)__popcll(meq);
    }
  }
}

}  // namespace

bool idx_topk_supported(const Dims& D) {
  return D.idx_bf16 && (D.didx == 32 || D.didx == 64 || D.didx == 128) && D.K <= kCandLds / 3;
}

int idx_topk_cap(const Dims& D) { return std::min(kCandLds, 3 * D.K); }

// Workspace: candidate lists, then per row the threshold, the total, and the
// per-chunk counts / offsets.
size_t idx_topk_ws_bytes(const Dims& D, int R) {
  auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
  const size_t rows = (size_t)D.B * R;
  const size_t nkc = ((size_t)D.L + KC - 1) / KC;
  return al(rows * idx_topk_cap(D) * sizeof(float2)) + al(rows * 4) + al(rows * 4) +
         al(rows * nkc * 4);
}

hipError_t launch_idx_topk(const Dims& D, const void* q_idx, const void* k_idx, int n0, int R,
                           int32_t* topk, int idx_rows_per_b, int idx_n_base,
                           const uint8_t* route, void* ws, hipStream_t s) {
  if (D.B == 0 || R == 0) return hipSuccess;
  auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
  const size_t rows = (size_t)D.B * R;
  FilterArgs f{};
  f.q_idx = (const bf16_bits*)q_idx; f.k_idx = (const bf16_bits*)k_idx; f.route = route;
  f.cap = idx_topk_cap(D);
  f.nkc = (D.L + KC - 1) / KC;
  char* w = (char*)ws;
  f.cand = (float2*)w;                 w += al(rows * f.cap * sizeof(float2));
  f.tau = (float*)w;                   w += al(rows * 4);
  f.count = (int32_t*)w;               w += al(rows * 4);
  f.ccnt = (int32_t*)w;
  f.N = D.N; f.L = D.L; f.K = D.K; f.Hq = D.Hq; f.n0 = n0; f.R = R;
  f.B_rows = (long long)rows;
  f.rpt = D.IH;
  SelectArgs sa{};
  sa.q_idx = f.q_idx; sa.k_idx = f.k_idx; sa.route = route;
  sa.cand = f.cand; sa.count = f.count;
  sa.topk = topk; sa.idx_rows_per_b = idx_rows_per_b; sa.idx_n_base = idx_n_base;
  sa.N = D.N; sa.L = D.L; sa.K = D.K; sa.Hq = D.Hq; sa.n0 = n0; sa.R = R; sa.cap = f.cap;
  sa.rpt = D.IH;
  const int rb = (R + kRowsPerWg - 1) / kRowsPerWg;
  const int nk_used = (D.L - D.N + (n0 + R - 1) / D.IH) / KC + 1;   // chunks the last row sees
  const int rbs = (R + kScanRows - 1) / kScanRows;
  const dim3 gt(rb, D.B), gscan(rbs, nk_used, D.B), gs(R, D.B);
  const dim3 goff((unsigned)((rows + 3) / 4));
  {
    ProfScope ps(s, kStageIndexer);
#define DSA_IDX_PASSES(DI)                                                          \
  hipLaunchKernelGGL(k_idx_tau<DI>, gt, dim3(FT), 0, s, f);                         \
  hipLaunchKernelGGL((k_idx_scan<DI, false>), gscan, dim3(FT), 0, s, f);            \
  hipLaunchKernelGGL(k_idx_offsets, goff, dim3(FT), 0, s, f);                       \
  hipLaunchKernelGGL((k_idx_scan<DI, true>), gscan, dim3(FT), 0, s, f);
    if (D.didx == 32) { DSA_IDX_PASSES(32) }
    else if (D.didx == 64) { DSA_IDX_PASSES(64) }
    else { DSA_IDX_PASSES(128) }
#undef DSA_IDX_PASSES
  }
  {
    ProfScope ps(s, kStageTopk);
    if (D.didx == 32) hipLaunchKernelGGL(k_topk_cands<32>, gs, dim3(CT), 0, s, sa);
    else if (D.didx == 64) hipLaunchKernelGGL(k_topk_cands<64>, gs, dim3(CT), 0, s, sa);
    else hipLaunchKernelGGL(k_topk_cands<128>, gs, dim3(CT), 0, s, sa);
  }
  return hipGetLastError();
}

}  // namespace dsa
