// Decode path in one cooperative launch: indexer scan, exact top-K, ordered
// index rows, gathered attention and gate, for few query rows per sequence.
//
// Steps of the gated sparse forward on the page "超大规模MoE架构中稀疏注意力机制的
// 演进与实践" (§二.1 indexer + top-K, §二.2 no rotary term, §四.1 gather ->
// attention -> gate) for the case where every sequence has a few new tokens
// and a long cache.  Blockwise selection without a global score matrix, in
// the spirit of the page "大模型推理架构演进：从稀疏注意力到隐式专家路由"
// §2.2-§2.3, with scores kept in LDS.
//
// Every workgroup owns one chunk of one sequence's keys (its "unit") for the
// whole launch.  The grid is sized to what the device holds at once (from the
// occupancy query).  All data that workgroups exchange belongs to one
// sequence, so the phases are separated by barriers of the sequence's units
// only (two levels, every wait bounded).
//   P1  stream k_idx once: scores of the chunk's keys for all N rows into LDS.
// Single-row sequences (N == 1), when the LDS holds every chunk's candidates:
//   C1  each chunk passes on its M largest keys under (key descending,
//       position ascending), as order values key << 32 | ~position in
//       position order; atomics keep the row's largest (M+1)-th value and
//       the key range of its candidates.  The first digit of the chunk's
//       selection is counted during P1.
//   C2  after one barrier, every unit with an attention item loads the row's
//       candidates, finds their K-th largest value cK and checks that cK is
//       above every chunk's (M+1)-th value; if so the index list is the
//       candidates at or above cK in position order, built in LDS, and the
//       unit goes straight to its attention items.  Otherwise the sequence
//       takes the histogram phases below.
// Histogram phases (N > 1, or the fallback above):
//   H1  first-digit (top 11 key bits) histogram per row -> global.
//   H2  bin t0 holding the K-th key; per chunk the count of keys above t0;
//       keys in t0 appended to the candidate region of the chunk's group
//       (16 groups per row), their second digit (next 11 bits) histogrammed.
//   H3  each unit resolves its row's exact K-th key T and the tie cut P*
//       (t1 from the second histogram; then a rank count, or the last digit
//       and a radix on positions, over the few candidates sharing the top 22
//       bits) and writes its chunk's selected positions, in order, at its
//       prefix offset -> ascending index rows.
//   Attention items (row, KV head, split of 256 keys, chunk of heads), taken
//       by the units of the item's sequence: each wave takes 64 keys per pass
//       (bf16: MFMA with the heads as the 16 columns; fp32: lane = key for
//       scores, lane = value slice for PV), online softmax; the last split
//       of a (row, KV head, head chunk) to finish merges the partials and
//       applies the gate.
#include <unistd.h>

#include <atomic>
#include <chrono>
#include <cmath>
#include <mutex>

#include <hip/hip_ext.h>

#include "common.h"
#include "launch.h"
#include "mfma.h"

namespace dsa {
namespace {

constexpr int DT = 256;        // threads per workgroup
constexpr int DSC = 8192;      // LDS score capacity per workgroup (floats)
constexpr int kLdsFloats = 16384 + 8 * 128 + 64;  // value tiles / scores + q + (max, sum)
constexpr int DMAXCH = 2048;   // max chunks per sequence
constexpr int kMaxGrid = 4096;  // largest grid the control block is sized for
constexpr float kLog2e = 1.4426950408889634f;

struct DecodeArgs {
  const void* q_idx; const void* k_idx; const void* q; const void* k; const void* v;
  const float* gate; const float* y2; const uint8_t* route; float* out; int32_t* list;
  uint64_t* ctl;     // epoch-tagged barrier counters and error word
  uint64_t* rowtag;  // [rows] epoch-tagged state of the row's zeroed arrays
  uint32_t* hist0;   // [rows][2048] first-digit histogram   (zeroed in-kernel)
  uint32_t* hist1;   // [rows][2048] second-digit histogram  (zeroed in-kernel)
  uint32_t* ticket;  // [rows][Hkv][nhc] finished splits     (zeroed in-kernel)
  uint32_t* cand_n;  // [rows][kCandGroups] candidates per group   (zeroed in-kernel)
  uint32_t* cnt;     // [rows][nch] per chunk: keys above the first-digit bin t0
  uint64_t* cand;    // [rows][cand_cap] key << 32 | position, one region per group
  float* part;       // [rows][Hq][S][HD+4]: max, sum, 2 pad, accumulator
  uint64_t* fcand;   // [rows][Cpad] each chunk's M largest order values, in position order
  uint64_t* sgslot;  // [B][ngroups][8] epoch-tagged group slots of the sequence barriers
  uint64_t* verdict; // [B][8] epoch-tagged: 1 = candidates hold the top K, 2 = they may not
  uint64_t* seqerr;  // [B][8] epoch-tagged: 1 = a unit of the sequence gave up waiting
  int B, N, L, Hq, Hkv, K, CH, nch, S, nhc, cand_cap;
  uint64_t* fstat;   // [rows][nch][4 waves][2]: (largest | smallest << 32) candidate key of
                     // the wave's share of the chunk, and the chunk's (M+1)-th value
  int M, Cpad;       // candidates per chunk (0: histogram selection only), padded row size
  int ccnt;          // candidates present per row
  float scale_log2;
  uint32_t epoch;    // distinct per launch; tags every control word
  const uint32_t* epw;  // under stream capture: device word with the launch's epoch
  uint32_t spin_limit;  // polls before a wait gives up (0: give up at the first wait)
};

__device__ __forceinline__ bool seq_sparse(const uint8_t* route, int b, int Hq) {
  if (!route) return true;
  for (int h = 0; h < Hq; ++h)
    if (route[(size_t)b * Hq + h]) return true;
  return false;
}

// Cross-workgroup data is written with device-scope atomic stores and read
// with device-scope atomic loads: both bypass the per-XCD L2 copies, so no
// L2 writeback / invalidate (the expensive part of a device-scope fence) is
// needed around the sequence barriers.  Counters and histograms use atomic RMWs.
__device__ __forceinline__ void st_dev(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_dev(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_dev64(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_devf(float* p, float v) { st_dev((uint32_t*)p, __float_as_uint(v)); }
__device__ __forceinline__ float ld_devf(const float* p) { return __uint_as_float(ld_dev((const uint32_t*)p)); }

constexpr int kBarGroup = 16;   // workgroups per first-level barrier group
// Candidates of a row are appended to kCandGroups regions, one per group of
// consecutive chunks, each with its own counter: few chunks contend for a
// counter and the regions stay contiguous for the readers.
constexpr int kCandGroups = 16;
// Control block of 64-bit words, each (launch epoch << 32 | value); a word
// whose epoch is not the current launch's means "nothing yet", so the block
// is never cleared.  Layout: [0] error word; [1] (seed, count) and [2] epoch
// of captured launches (k_decode_epoch); member slots from word 8 (one
// per workgroup).  The sequence barriers' group slots and the verdict words
// are tagged the same way.
size_t ctl_words64(int grid) { return 8 + (size_t)grid; }

__device__ __forceinline__ bool tagged(uint64_t v, uint32_t epoch, uint32_t at_least) {
  return (uint32_t)(v >> 32) == epoch && (uint32_t)v >= at_least;
}

__device__ __forceinline__ void raise_error(const DecodeArgs& a, uint32_t ep, int b) {
  const uint64_t tag = ((uint64_t)ep << 32) | 1ull;
  st_dev64(a.seqerr + 8 * b, tag);
  st_dev64(a.ctl, tag);
}

// Bounded wait of one thread for a tagged word of sequence b; false when the
// wait gives up (after spin_limit polls, at once when spin_limit is 0) or
// when another unit of the sequence already gave up.  A give-up is recorded
// in the sequence's abort word and in the launch's error word (control word
// 0), which the host reads back through dsa_exec_status.
__device__ __forceinline__ bool wait_tag(const DecodeArgs& a, uint32_t ep, int b, const uint64_t* p,
                                         uint32_t at_least) {
  if (a.spin_limit == 0) {
    raise_error(a, ep, b);
    return false;
  }
  uint32_t spins = 0;
  while (!tagged(ld_dev64(p), ep, at_least)) {
    if (tagged(ld_dev64(a.seqerr + 8 * b), ep, 1u)) return false;
    __builtin_amdgcn_s_sleep(1);
    if (++spins > a.spin_limit) {
      raise_error(a, ep, b);
      return false;
    }
  }
  return true;
}

// Barrier of the units of one sequence (workgroups [b * nch, (b + 1) * nch)):
// all data exchanged between workgroups belongs to one sequence, so no
// workgroup waits for another sequence's.  No shared counters: every unit
// writes its own arrival slot, the first unit of each group of 16 (counted
// within the sequence) waits for its members and writes the group slot, and
// every unit waits for the sequence's group slots.  Each thread first waits
// for its own outstanding memory operations, so the stores before the
// barrier have completed when the slot is written.
__device__ __forceinline__ bool seq_sync(const DecodeArgs& a, uint32_t ep, int b, uint32_t phase,
                                         int* flag) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const int u0 = b * a.nch;
  const int lu = (int)blockIdx.x - u0;
  const int ngs = (a.nch + kBarGroup - 1) / kBarGroup;
  const int gi = lu / kBarGroup;
  uint64_t* mslot = a.ctl + 8;
  uint64_t* gslot = a.sgslot + (size_t)b * ngs * 8;
  const uint64_t tag = ((uint64_t)ep << 32) | phase;
  if (threadIdx.x == 0) {
    *flag = 1;
    st_dev64(mslot + blockIdx.x, tag);
  }
  __syncthreads();
  if (lu == gi * kBarGroup) {
    const int gsize = min(kBarGroup, a.nch - gi * kBarGroup);
    if ((int)threadIdx.x < gsize &&
        !wait_tag(a, ep, b, mslot + u0 + gi * kBarGroup + threadIdx.x, phase))
      *flag = 0;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0 && *flag) st_dev64(gslot + 8 * gi, tag);
  }
  if ((int)threadIdx.x < ngs && !wait_tag(a, ep, b, gslot + 8 * threadIdx.x, phase)) *flag = 0;
  __syncthreads();
  return *flag != 0;
}

// Row accumulators (both histograms, candidate count, merge tickets) are
// cleared at the start of every launch by the first unit of the sequence;
// the row's tag then reads "ready" for this launch.
__device__ __forceinline__ void clear_rows(const DecodeArgs& a, uint32_t ep, int b) {
  const int nt = a.Hkv * a.nhc;
  for (int n = 0; n < a.N; ++n) {
    const int row = b * a.N + n;
    uint32_t* h0 = a.hist0 + (size_t)row * 2048;
    uint32_t* h1 = a.hist1 + (size_t)row * 2048;
    for (int i = threadIdx.x; i < 2048; i += DT) {
      st_dev(h0 + i, 0u);
      st_dev(h1 + i, 0u);
    }
    for (int i = threadIdx.x; i < nt; i += DT) st_dev(a.ticket + (size_t)row * nt + i, 0u);
    if (threadIdx.x < kCandGroups) st_dev(a.cand_n + (size_t)row * kCandGroups + threadIdx.x, 0u);

  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x < a.N)
    st_dev64(a.rowtag + b * a.N + threadIdx.x, ((uint64_t)ep << 32) | 2ull);
}

// Waits until the rows of sequence b are cleared for this launch.
__device__ __forceinline__ bool rows_ready(const DecodeArgs& a, uint32_t ep, int b, int* flag) {
  __syncthreads();
  if (threadIdx.x == 0) *flag = 1;
  __syncthreads();
  if ((int)threadIdx.x < a.N && !wait_tag(a, ep, b, a.rowtag + b * a.N + threadIdx.x, 2u)) *flag = 0;
  __syncthreads();
  return *flag != 0;
}

// A unit that gave up waiting leaves its sequence's results undefined: it
// marks them so (NaN outputs, index rows of -1) before it returns.  Units of
// the sequence cannot pass the wait it gave up at, so no valid result of the
// sequence is written after these.
template <int HD>
__device__ __attribute__((noinline)) void abandon_rows(float* out, int32_t* list, int N, int Hq,
                                                      int K, int b) {
  const size_t n_out = (size_t)N * Hq * HD;
  float* o = out + (size_t)b * n_out;
  const float qnan = __uint_as_float(0x7fc00000u);
  for (size_t i = threadIdx.x; i < n_out; i += DT) o[i] = qnan;
  int32_t* l = list + (size_t)b * N * K;
  for (size_t i = threadIdx.x; i < (size_t)N * K; i += DT) l[i] = -1;
}
template <int HD>
__device__ __forceinline__ void abandon(const DecodeArgs& a, int b) {
  abandon_rows<HD>(a.out, a.list, a.N, a.Hq, a.K, b);
}

// kk-th largest (from the top) over hist[0..nb): bin and count above it.
__device__ __forceinline__ void pick_top(const uint32_t* hist, int nb, uint32_t kk, uint32_t* scratch,
                         uint32_t* res) {
  const int per = nb / DT;
  const int base = threadIdx.x * per;
  uint32_t mine = 0;
  for (int i = 0; i < per; ++i) mine += hist[base + i];
  uint32_t total;
  const uint32_t pre = block_excl_scan<DT>(mine, scratch, total);
  uint32_t running = total - pre - mine;
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

// kk-th smallest (from the bottom) over hist[0..nb): bin and count below it.
__device__ __forceinline__ void pick_low(const uint32_t* hist, int nb, uint32_t kk, uint32_t* scratch,
                         uint32_t* res) {
  const int per = nb / DT;
  const int base = threadIdx.x * per;
  uint32_t mine = 0;
  for (int i = 0; i < per; ++i) mine += hist[base + i];
  uint32_t total;
  uint32_t running = block_excl_scan<DT>(mine, scratch, total);
  for (int i = 0; i < per; ++i) {
    const uint32_t c = hist[base + i];
    if (running < kk && running + c >= kk) {
      res[0] = (uint32_t)(base + i);
      res[1] = running;
    }
    running += c;
  }
  __syncthreads();
}

__device__ __forceinline__ uint32_t block_sum(uint32_t x, uint32_t* scratch) {
  uint32_t total;
  block_excl_scan<DT>(x, scratch, total);
  return total;
}

// Word of bin b in the selection histogram: one pad word after every 32
// bins, so that lanes reading 32 consecutive bins each (lane l the chunk of
// bins 32 c_l .. 32 c_l + 31, word 33 c_l + j) hit different LDS banks.
constexpr int kHistWords = 2048 + 64;
__device__ __forceinline__ int hslot(uint32_t b) { return (int)(b + (b >> 5)); }

// The kk-th largest (1 <= kk <= m) of the order values get(0), ..., get(n - 1)
// (key << 32 | ~position, distinct; 0 marks an empty slot, so a value is
// present iff its low word is nonzero).  m values are present, their keys
// are at least hmin and (value - (hmin << 32)) < 2^hi.  Digits of
// (value - (hmin << 32)) are fixed from the top, 11 bits at a time, with
// 32-bit arithmetic while they lie in the key word; once at most DT values
// share the digits fixed so far they are gathered and the kk-th is found by
// ranking them.  Each level costs two barriers: wave 0 alone turns the
// histogram into the digit (32 bins per lane, one DPP scan) and clears the
// bins it read.
// Caller: buf[0 .. DT) and res[2] must be zero and hist[0 .. kHistWords) either
// zero or, with hist_ready, the counts of the first digit (bin b at word
// hslot(b)), all visible to every
// thread (written before a barrier).  On return hist is zero again; buf and
// res[2] are not.
// LDS: hist (2048 words), buf (DT values), red (1 value), res (4 words).
template <class Get>
__device__ __forceinline__ uint64_t kth_largest(int n, uint32_t kk, Get get, uint32_t hmin, int hi,
                                                uint32_t m, bool hist_ready, uint32_t* hist,
                                                uint64_t* buf, uint64_t* red, uint32_t* res) {
  const int iters = (n + 8 * DT - 1) / (8 * DT);   // the same for every thread
  auto load8 = [&](int k, uint64_t* vv) {
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      // read at a clamped index unconditionally, then mask
      const int i = (int)threadIdx.x + k * 8 * DT + x * DT;
      const uint64_t v = get(min(i, n - 1));
      vv[x] = i < n ? v : 0ull;
    }
    // keep the reads together: without this the scheduler puts each read
    // next to its use and waits for it
    __builtin_amdgcn_sched_barrier(0);
  };
  const int lane = threadIdx.x & 63;
  uint64_t prefix = 0;   // (value - (hmin << 32)) >> hi of the kk-th
  const uint64_t hbase = (uint64_t)hmin << 32;
  // a present value whose digits above bit hi equal the prefix (all present
  // values while hi = 64; keys are at least hmin, so the difference is the
  // offset of the value above hbase)
  auto matches = [&](uint64_t v) -> bool {
    return (uint32_t)v != 0u && (hi >= 64 || ((v - hbase) >> hi) == prefix);
  };
  while (m > (uint32_t)DT && hi > 0) {
    const int bits = min(11, hi);
    const int sh = hi - bits;
    const uint32_t nbm = (1u << bits) - 1u;
    for (int k = 0; k < (hist_ready ? 0 : iters); ++k) {
      uint64_t vv[8];
      load8(k, vv);
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const uint64_t v = vv[x];
        if (matches(v)) atomicAdd(&hist[hslot((uint32_t)((v - hbase) >> sh) & nbm)], 1u);
      }
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      // lane l holds bins [top_l - per, top_l), lane 0 the highest; an
      // inclusive scan of the lanes' counts finds the lane whose bins hold
      // the kk-th value from the top, a second scan over that lane's bins
      // (one per lane) the bin.  The bins read are cleared.
      const int nb = 1 << bits;
      const int per = max(1, nb >> 6);
      const int top = nb - per * lane;
      uint32_t sum = 0;
      if (per == 32) {
        // an 11-bit digit: bins top - 32 .. top - 1, all reads in flight together
        uint32_t hv[32];
#pragma unroll
        for (int j = 0; j < 32; ++j) hv[j] = hist[hslot((uint32_t)(top - 32 + j))];
#pragma unroll
        for (int j = 0; j < 32; ++j) sum += hv[j];
      } else {
#pragma unroll 1
        for (int j = 0; j < per; ++j) {
          const int bin = top - 1 - j;
          sum += bin >= 0 ? hist[hslot((uint32_t)bin)] : 0u;
        }
      }
      const uint32_t incl = wave_incl_scan(sum);          // values in bins >= this lane's lowest
      const int L = __ffsll((long long)__ballot(incl >= kk)) - 1;
      const int topL = __builtin_amdgcn_readlane(top, L);
      const uint32_t aboveL = (uint32_t)__builtin_amdgcn_readlane((int)(incl - sum), L);
      const int bin = topL - 1 - lane;
      const uint32_t cnt = (lane < per && bin >= 0) ? hist[hslot((uint32_t)bin)] : 0u;
      const uint32_t ci = aboveL + wave_incl_scan(cnt);
      const int J = __ffsll((long long)__ballot(ci >= kk)) - 1;
      if (lane == J) {
        res[0] = (uint32_t)bin;
        res[1] = ci - cnt;
        res[3] = cnt;
      }
      if (per == 32) {
#pragma unroll
        for (int j = 0; j < 32; ++j) hist[hslot((uint32_t)(top - 32 + j))] = 0u;
      } else {
#pragma unroll 1
        for (int j = 0; j < per; ++j) {
          const int b2 = top - 1 - j;
          if (b2 >= 0) hist[hslot((uint32_t)b2)] = 0u;
        }
      }
    }
    __syncthreads();
    const uint32_t d = res[0];
    kk -= res[1];
    m = res[3];
    prefix = (prefix << bits) | d;
    hi = sh;
    hist_ready = false;
  }
  if (hist_ready) {
    // counts handed in but no level needed: leave the histogram cleared
    for (int i = threadIdx.x; i < kHistWords; i += DT) hist[i] = 0;
  }
  // gather: one LDS atomic per wave and group of eight values for the slots
  for (int k = 0; k < iters; ++k) {
    uint64_t vv[8];
    load8(k, vv);
    uint32_t msk = 0;
#pragma unroll
    for (int x = 0; x < 8; ++x) msk |= (matches(vv[x]) ? 1u : 0u) << x;
    const uint32_t c8 = (uint32_t)__popc(msk);
    const uint32_t incl = wave_incl_scan(c8);
    const uint32_t wt = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
    if (wt) {
      uint32_t wb = 0;
      if (lane == 63) wb = atomicAdd(&res[2], wt);
      uint32_t sl = (uint32_t)__builtin_amdgcn_readlane((int)wb, 63) + incl - c8;
#pragma unroll
      for (int x = 0; x < 8; ++x)
        if ((msk >> x) & 1u) {
          if (sl < (uint32_t)DT) buf[sl] = vv[x];
          ++sl;
        }
    }
  }
  __syncthreads();
  const uint32_t mm = min(res[2], (uint32_t)DT);
  if (threadIdx.x < mm) {
    const uint64_t me = buf[threadIdx.x];
    uint32_t r = 0;
    for (uint32_t x = 0; x < mm; x += 16) {   // buf beyond mm is zero, below every value
      uint64_t o[16];
#pragma unroll
      for (int y = 0; y < 16; ++y) o[y] = buf[x + y];
#pragma unroll
      for (int y = 0; y < 16; ++y) r += o[y] > me;
    }
    if (r + 1 == kk) red[0] = me;
  }
  __syncthreads();
  return red[0];
}

__device__ __forceinline__ uint4 raw16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void widen(const uint4& u, float* o, const bf16_bits*) {
  o[0] = __uint_as_float(u.x << 16); o[1] = __uint_as_float(u.x & 0xffff0000u);
  o[2] = __uint_as_float(u.y << 16); o[3] = __uint_as_float(u.y & 0xffff0000u);
  o[4] = __uint_as_float(u.z << 16); o[5] = __uint_as_float(u.z & 0xffff0000u);
  o[6] = __uint_as_float(u.w << 16); o[7] = __uint_as_float(u.w & 0xffff0000u);
}
__device__ __forceinline__ void widen(const uint4& u, float* o, const float*) {
  o[0] = __uint_as_float(u.x); o[1] = __uint_as_float(u.y);
  o[2] = __uint_as_float(u.z); o[3] = __uint_as_float(u.w);
}

// One attention pass of an item: heads hsel[0..nh) of KV head g, keys given
// by the index-row segment [e0, e1) (sparse) or positions [e0, e1) (dense).
// Each wave takes 64 keys at a time: scores with lane = key (all key-row
// loads in flight together), online softmax per wave, PV with lane = (key
// slot, 16-byte slice of the value row).  bf16 value rows go straight from
// memory into this wave's LDS tile (no registers), issued before the scores
// are computed.  The four waves are merged through LDS; one partial
// (max, sum, acc) per head is written for split s.
// LDS use: [0, 16384) floats value tiles (4 x 16 KB, later the merge
// buffer), then q (HCT x HD) and the per-wave (max, sum).
template <typename TQ, int HD, int HCT>
__device__ __forceinline__ void attend(const DecodeArgs& a, int row, int b, int n, int g, int s, bool dense,
                       int e0, int e1, const int* hsel, int nh, float* lds, bool q_ready,
                       const uint32_t* llist) {
  constexpr int EPV = 16 / (int)sizeof(TQ);   // elements per 16-byte load
  constexpr int LPR = HD / EPV;               // lanes per value row
  constexpr int KPI = 64 / LPR;               // value rows per load instruction
  constexpr int NKL = HD / EPV;               // 16-byte loads per key row
  constexpr bool VLDS = sizeof(TQ) == 2;      // value rows staged in LDS
  constexpr int BATCH = 8;
  const TQ* K = (const TQ*)a.k;
  const TQ* V = (const TQ*)a.v;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int p = a.L - a.N + n;
  char* vtile = (char*)lds + w * 64 * HD * 2;  // this wave's 64 value rows (bf16)
  float* wb = lds;                             // [4][HCT][HD], after the key loop
  float* qs = lds + 16384;                     // [HCT][HD]
  float* wml = qs + HCT * HD;                  // [4][HCT][2]
  if (!q_ready) {
    for (int e = threadIdx.x; e < HCT * HD; e += DT) {
      const int hh = e / HD, c = e - hh * HD;
      float x = 0.f;
      if (hh < nh) x = ld_f((const TQ*)a.q, (((size_t)b * a.N + n) * a.Hq + hsel[hh]) * HD + c) *
                       a.scale_log2;
      qs[e] = x;
    }
    __syncthreads();
  }
  float m_w[HCT], l_w[HCT], acc[HCT][EPV];
#pragma unroll
  for (int h = 0; h < HCT; ++h) {
    m_w[h] = -INFINITY;
    l_w[h] = 0.f;
#pragma unroll
    for (int i = 0; i < EPV; ++i) acc[h][i] = 0.f;
  }
  const uint32_t* lrow = (const uint32_t*)a.list + (size_t)row * a.K;
  const int ks = lane / LPR, dc = lane % LPR;
  const TQ* vseq = V + ((size_t)b * a.L * a.Hkv + g) * HD;
  for (int t0 = e0 + w * 64; t0 < e1; t0 += 4 * 64) {
    const int e = t0 + lane;
    int j = -1;
    if (e < e1) {
      j = dense ? e : (int)(llist ? llist[e] : ld_dev(lrow + e));
      if (j < 0 || j > p) j = -1;
    }
    if constexpr (VLDS) {
      // rows r = m*KPI + lane/LPR of this wave's tile, 16-byte slice lane%LPR
#pragma unroll
      for (int m = 0; m < 64 / KPI; ++m) {
        const int jr = __shfl(j, m * KPI + ks, 64);
        const TQ* src = vseq + (size_t)(jr < 0 ? 0 : jr) * a.Hkv * HD + dc * EPV;
        __builtin_amdgcn_global_load_lds(
            (const void*)src, (__attribute__((address_space(3))) void*)(vtile + m * 1024), 16, 0, 0);
      }
    }
    float sc[HCT];
#pragma unroll
    for (int h = 0; h < HCT; ++h) sc[h] = 0.f;
    const TQ* kr = K + (((size_t)b * a.L + (j < 0 ? 0 : j)) * a.Hkv + g) * HD;
#pragma unroll 1
    for (int c0 = 0; c0 < NKL; c0 += BATCH) {
      uint4 raw[BATCH];
#pragma unroll
      for (int i = 0; i < BATCH; ++i)
        raw[i] = (j >= 0) ? raw16(kr + (c0 + i) * EPV) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < BATCH; ++i) {
        float kv[EPV];
        widen(raw[i], kv, (const TQ*)nullptr);
#pragma unroll
        for (int h = 0; h < HCT; ++h) {
          float t = sc[h];
#pragma unroll
          for (int x = 0; x < EPV; ++x) t = fmaf(qs[h * HD + (c0 + i) * EPV + x], kv[x], t);
          sc[h] = t;
        }
      }
    }
    float pr[HCT];
#pragma unroll
    for (int h = 0; h < HCT; ++h) {
      const float sv = (j >= 0 && h < nh) ? sc[h] : -INFINITY;
      const float mt = wave_max(sv);
      const float mnew = fmaxf(m_w[h], mt);
      float alpha = 1.f, pv = 0.f;
      if (mnew != -INFINITY) {
        alpha = exp2f(m_w[h] - mnew);
        pv = exp2f(sv - mnew);
      }
      l_w[h] = l_w[h] * alpha + wave_sum(pv);
      m_w[h] = mnew;
      pr[h] = pv;
#pragma unroll
      for (int i = 0; i < EPV; ++i) acc[h][i] *= alpha;
    }
    // PV: lane = (key slot ks, dims dc*EPV ..)
    if constexpr (VLDS) {
      __builtin_amdgcn_s_waitcnt(0);      // this wave's value tile has arrived
      __builtin_amdgcn_wave_barrier();
#pragma unroll 4
      for (int t = 0; t < 64; t += KPI) {
        const uint4 u = *reinterpret_cast<const uint4*>(vtile + (t + ks) * (HD * 2) + dc * 16);
        float vv[EPV];
        widen(u, vv, (const TQ*)nullptr);
#pragma unroll
        for (int h = 0; h < HCT; ++h) {
          const float pv = __shfl(pr[h], t + ks, 64);
#pragma unroll
          for (int x = 0; x < EPV; ++x) acc[h][x] = fmaf(pv, vv[x], acc[h][x]);
        }
      }
      __builtin_amdgcn_s_waitcnt(0);      // tile reads done before it is refilled
      __builtin_amdgcn_wave_barrier();
    } else {
#pragma unroll 1
      for (int t = 0; t < 64; t += KPI * 8) {
        uint4 raw[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int jv = __shfl(j, t + i * KPI + ks, 64);
          raw[i] = (jv >= 0) ? raw16(V + (((size_t)b * a.L + jv) * a.Hkv + g) * HD + dc * EPV)
                             : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float vv[EPV];
          widen(raw[i], vv, (const TQ*)nullptr);
#pragma unroll
          for (int h = 0; h < HCT; ++h) {
            const float pv = __shfl(pr[h], t + i * KPI + ks, 64);
#pragma unroll
            for (int x = 0; x < EPV; ++x) acc[h][x] = fmaf(pv, vv[x], acc[h][x]);
          }
        }
      }
    }
  }
  // reduce over key slots
#pragma unroll
  for (int o = LPR; o < 64; o <<= 1)
#pragma unroll
    for (int h = 0; h < HCT; ++h)
#pragma unroll
      for (int i = 0; i < EPV; ++i) acc[h][i] += __shfl_xor(acc[h][i], o, 64);
  __syncthreads();   // value tiles are dead; their LDS becomes the merge buffer
  if (lane < LPR) {
#pragma unroll
    for (int h = 0; h < HCT; ++h)
#pragma unroll
      for (int i = 0; i < EPV; ++i) wb[(w * HCT + h) * HD + lane * EPV + i] = acc[h][i];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < HCT; ++h) {
      wml[(w * HCT + h) * 2 + 0] = m_w[h];
      wml[(w * HCT + h) * 2 + 1] = l_w[h];
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < nh * HD; e += DT) {
    const int hh = e / HD, c = e - hh * HD;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, wml[(ww * HCT + hh) * 2]);
    float l = 0.f, s_acc = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) {
        const float mw = wml[(ww * HCT + hh) * 2];
        const float f = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
        l = fmaf(f, wml[(ww * HCT + hh) * 2 + 1], l);
        s_acc = fmaf(f, wb[(ww * HCT + hh) * HD + c], s_acc);
      }
    }
    float* pp = a.part + (((size_t)row * a.Hq + hsel[hh]) * a.S + s) * (HD + 4);
    st_devf(pp + 4 + c, s_acc);
    if (c == 0) {
      st_devf(pp + 0, M);
      st_devf(pp + 1, l);
    }
  }
  __syncthreads();
}


// bf16 keys and values on MFMA: one pass of a wave covers 64 keys as four
// blocks of 16.  S^T = K Q^T with the item's heads as the 16 columns (lane
// column i = head i), the online softmax per column in registers, then
// O^T += V^T P^T with V^T read from this wave's LDS value tile by the
// transposing LDS read.  The d axis is taken in 32-dim chunks, so the four
// lane quads of one key read 64 contiguous bytes of its row.  The four waves
// are merged through LDS; one partial (max, sum, acc) per head is written
// for split s.
template <int HD>
__device__ __forceinline__ void attend_mfma(const DecodeArgs& a, int row, int b, int n, int g, int s, bool dense,
                            int e0, int e1, const int* hsel, int nh, float* lds,
                            const uint32_t* llist) {
  constexpr int T = HD / 32;
  constexpr int NC = 16;                      // columns (heads) per item
  constexpr int LPR = HD / 8;                 // lanes per value row (16-byte pieces)
  constexpr int KPI = 64 / LPR;               // value rows per load instruction
  const bf16_bits* K = (const bf16_bits*)a.k;
  const bf16_bits* V = (const bf16_bits*)a.v;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int q = lane >> 4, i = lane & 15;
  const int p = a.L - a.N + n;
  char* vtile = (char*)lds + w * 64 * HD * 2;  // this wave's 64 value rows
  float* wb = lds;                             // [4][NC][HD], after the key loop
  float* wml = lds + 16384;                    // [4][NC][2]
  bf16x8 qb[T];
  {
    const bool hv = i < nh;
    const bf16_bits* qr =
        (const bf16_bits*)a.q + (((size_t)b * a.N + n) * a.Hq + (hv ? hsel[i] : 0)) * HD;
#pragma unroll
    for (int t = 0; t < T; ++t)
      qb[t] = as_bf16x8(hv ? *reinterpret_cast<const uint4*>(qr + t * 32 + q * 8)
                           : make_uint4(0, 0, 0, 0));
  }
  float m_c = -INFINITY, l_c = 0.f;
  f32x4 o[HD / 16];
#pragma unroll
  for (int dt = 0; dt < HD / 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint32_t* lrow = (const uint32_t*)a.list + (size_t)row * a.K;
  const bf16_bits* kseq = K + ((size_t)b * a.L * a.Hkv + g) * HD;
  const bf16_bits* vseq = V + ((size_t)b * a.L * a.Hkv + g) * HD;
  const size_t rs = (size_t)a.Hkv * HD;        // elements between token rows
  const int ks = lane / LPR, dc = lane % LPR;
  const int row0 = 4 * q + (i >> 2), colb = (i & 3) * 8;
  for (int t0 = e0 + w * 64; t0 < e1; t0 += 4 * 64) {
    int jl = -1;   // position of key t0 + lane
    {
      const int e = t0 + lane;
      if (e < e1) {
        jl = dense ? e : (int)(llist ? llist[e] : ld_dev(lrow + e));
        if (jl < 0 || jl > p) jl = -1;
      }
    }
    const uint64_t vm = __ballot(jl >= 0);
#pragma unroll
    for (int m = 0; m < 64 / KPI; ++m) {
      const int jr = __shfl(jl, m * KPI + ks, 64);
      const bf16_bits* src = vseq + (size_t)(jr < 0 ? 0 : jr) * rs + dc * 8;
      __builtin_amdgcn_global_load_lds(
          (const void*)src, (__attribute__((address_space(3))) void*)(vtile + m * 1024), 16, 0, 0);
    }
    uint4 ka[4][T];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int ju = __shfl(jl, 16 * u + i, 64);
#pragma unroll
      for (int t = 0; t < T; ++t)
        ka[u][t] = (ju >= 0) ? *reinterpret_cast<const uint4*>(kseq + (size_t)ju * rs + t * 32 + q * 8)
                             : make_uint4(0, 0, 0, 0);
    }
    float sv[16];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < T; ++t) acc = mfma16(as_bf16x8(ka[u][t]), qb[t], acc);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        sv[u * 4 + r] = ((vm >> (16 * u + 4 * q + r)) & 1ull) ? acc[r] * a.scale_log2 : -INFINITY;
    }
    float mt = sv[0];
#pragma unroll
    for (int x = 1; x < 16; ++x) mt = fmaxf(mt, sv[x]);
    mt = max_xor16(mt);
    mt = max_xor32(mt);
    const float mnew = fmaxf(m_c, mt);
    float alpha = 1.f, pv[16];
    if (mnew == -INFINITY) {
#pragma unroll
      for (int x = 0; x < 16; ++x) pv[x] = 0.f;
    } else {
      alpha = exp2_fast(m_c - mnew);
#pragma unroll
      for (int x = 0; x < 16; ++x) pv[x] = exp2_fast(sv[x] - mnew);
    }
    float ps = 0.f;
#pragma unroll
    for (int x = 0; x < 16; ++x) ps += pv[x];
    l_c = l_c * alpha + ps;
    m_c = mnew;
    // P^T for keys 32v + 4q + r (block 2v) and 32v + 16 + 4q + r (block 2v + 1)
    const bf16x8 pb0 = pack8(pv), pb1 = pack8(pv + 8);
#pragma unroll
    for (int dt = 0; dt < HD / 16; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) o[dt][r] *= alpha;
    __builtin_amdgcn_s_waitcnt(0);      // this wave's value tile has arrived
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int v = 0; v < 2; ++v) {
#pragma unroll
      for (int dt = 0; dt < HD / 16; ++dt) {
        const uint2 lo = lds_tr(vtile, (32 * v + row0) * (HD * 2) + dt * 32 + colb);
        const uint2 hi = lds_tr(vtile, (32 * v + 16 + row0) * (HD * 2) + dt * 32 + colb);
        uint4 u4;
        u4.x = lo.x; u4.y = lo.y; u4.z = hi.x; u4.w = hi.y;
        o[dt] = mfma16(as_bf16x8(u4), v ? pb1 : pb0, o[dt]);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);      // tile reads done before it is refilled
    __builtin_amdgcn_wave_barrier();
  }
  l_c = sum_xor16(l_c);
  l_c = sum_xor32(l_c);
  __syncthreads();   // value tiles are dead; their LDS becomes the merge buffer
  if (i < nh) {
#pragma unroll
    for (int dt = 0; dt < HD / 16; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) wb[(w * NC + i) * HD + dt * 16 + 4 * q + r] = o[dt][r];
    if (q == 0) {
      wml[(w * NC + i) * 2 + 0] = m_c;
      wml[(w * NC + i) * 2 + 1] = l_c;
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < nh * HD; e += DT) {
    const int hh = e / HD, c = e - hh * HD;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, wml[(ww * NC + hh) * 2]);
    float l = 0.f, s_acc = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) {
        const float mw = wml[(ww * NC + hh) * 2];
        const float f = (mw == -INFINITY) ? 0.f : exp2_fast(mw - M);
        l = fmaf(f, wml[(ww * NC + hh) * 2 + 1], l);
        s_acc = fmaf(f, wb[(ww * NC + hh) * HD + c], s_acc);
      }
    }
    float* pp = a.part + (((size_t)row * a.Hq + hsel[hh]) * a.S + s) * (HD + 4);
    st_devf(pp + 4 + c, s_acc);
    if (c == 0) {
      st_devf(pp + 0, M);
      st_devf(pp + 1, l);
    }
  }
  __syncthreads();
}

// Attention item `it`: (row, KV head g, key split s, head chunk hci), the
// split index varying fastest so that the splits of one (row, KV head, head
// chunk) run side by side.
struct Item {
  int row, g, s, hci;
};
__device__ __forceinline__ Item item_of(const DecodeArgs& a, int it) {
  Item t;
  int rem = it;
  t.s = rem % a.S; rem /= a.S;
  t.hci = rem % a.nhc; rem /= a.nhc;
  t.g = rem % a.Hkv; rem /= a.Hkv;
  t.row = rem;
  return t;
}

// The item's query heads by route: sparse ones in hsel[0], dense ones in
// hsel[1] (thread 0 writes them; the caller synchronises).
template <int HCT>
__device__ void item_heads(const DecodeArgs& a, const Item& t, int rb, int (*hsel)[HCT],
                           int* nsel) {
  if (threadIdx.x != 0) return;
  const int G_heads = a.Hq / a.Hkv;
  int ns = 0, nd = 0;
  for (int i = t.hci * HCT; i < min(G_heads, t.hci * HCT + HCT); ++i) {
    const int h = t.g * G_heads + i;
    const bool sparse = a.route ? (a.route[(size_t)rb * a.Hq + h] != 0) : true;
    if (sparse) hsel[0][ns++] = h;
    else hsel[1][nd++] = h;
  }
  nsel[0] = ns;
  nsel[1] = nd;
}

template <typename TI, int DIDX, typename TQ, int HD, int HCT>
__global__ __launch_bounds__(DT, 2) void k_decode(DecodeArgs a) {
  __shared__ float4 lds4[kLdsFloats / 4];
  float* lds = reinterpret_cast<float*>(lds4);
  __shared__ uint32_t hist[kHistWords];
  __shared__ uint32_t scratch[DT / DSA_WAVE + 1];
  __shared__ uint32_t res[4];
  __shared__ int flag;
  __shared__ int hsel[2][HCT];
  __shared__ int nsel[2];
  __shared__ uint32_t t0s[4], kk0s[4];
  __shared__ uint64_t red[16];

  const int u = blockIdx.x;
  const bool has_unit = u < a.B * a.nch;
  const int b = has_unit ? u / a.nch : 0;
  const int c = has_unit ? u - b * a.nch : 0;
  const int j0 = c * a.CH;
  const int clen = has_unit ? min(a.CH, a.L - j0) : 0;
  const bool sp = has_unit && seq_sparse(a.route, b, a.Hq);
  const int N = a.N, K = a.K;

  // the launch's epoch: a kernel argument, or under stream capture (where
  // every replay of the graph would see the same argument) a word that the
  // captured k_decode_epoch advanced just before
  const uint32_t ep = a.epw ? ld_dev(a.epw) : a.epoch;
  if (has_unit && c == 0) clear_rows(a, ep, b);
  // single-row sequence on the candidate selection
  const bool cand_sel = a.M > 0 && sp && a.L > K;

  // ---------------------------------------------------------------- P1 scan
  if (sp) {
    constexpr int EPL = 16 / (int)sizeof(TI);
    constexpr int LPK = DIDX / EPL;
    constexpr int KPW = 64 / LPK;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int sub = lane % LPK, kin = lane / LPK;
    const TI* qi = (const TI*)a.q_idx;
    const TI* ki = (const TI*)a.k_idx;
    float qv[4][EPL];
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int e = 0; e < EPL; ++e)
        qv[n][e] = (n < N) ? ld_f(qi, ((size_t)b * N + n) * DIDX + sub * EPL + e) : 0.f;
    constexpr int U = 8;
    for (int base = w * KPW; base < clen; base += 4 * KPW * U) {
      uint4 raw[U];
#pragma unroll
      for (int uu = 0; uu < U; ++uu) {
        const int jj = base + kin + uu * 4 * KPW;
        raw[uu] = (jj < clen) ? raw16(ki + ((size_t)b * a.L + j0 + jj) * DIDX + sub * EPL)
                              : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int uu = 0; uu < U; ++uu) {
        const int jj = base + kin + uu * 4 * KPW;
        float kv[EPL];
        widen(raw[uu], kv, (const TI*)nullptr);
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          if (n >= N) break;
          float s = 0.f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) s = fmaf(qv[n][e], kv[e], s);
          if constexpr (LPK <= 16) {
            s = group_sum_dpp<LPK>(s);
          } else {
#pragma unroll
            for (int o = LPK / 2; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
          }
          if (sub == 0 && jj < clen) lds[n * a.CH + jj] = s;
        }
      }
    }
  }
  if (!has_unit) return;   // a workgroup without a chunk has no further work
  if (a.M) {
    // state the candidate selection expects (published by the barriers below)
    for (int i = threadIdx.x; i < kHistWords; i += DT) hist[i] = 0;
    reinterpret_cast<uint64_t*>(lds + a.CH)[threadIdx.x] = 0;
    if (threadIdx.x == 0) res[2] = 0;
  }
  // the sequence's per-row accumulators are cleared by its first unit
  if (!rows_ready(a, ep, b, &flag)) {
    abandon<HD>(a, b);
    return;
  }

  // ------------------------------------------------ histogram selection phases
  // H1: first-digit (top 11 key bits) histogram of every row -> global.
  auto build_hist0 = [&]() {
    if (sp) {
      __syncthreads();
      for (int n = 0; n < N; ++n) {
        const int vis = a.L - N + n + 1;
        if (vis <= K) continue;
        const int lim = min(clen, vis - j0);
        for (int i = threadIdx.x; i < 2048; i += DT) hist[i] = 0;
        __syncthreads();
        for (int jj = threadIdx.x; jj < lim; jj += DT)
          atomicAdd(&hist[radix_key(lds[n * a.CH + jj]) >> 21], 1u);
        __syncthreads();
        uint32_t* gh = a.hist0 + ((size_t)b * N + n) * 2048;
        for (int i = threadIdx.x; i < 2048; i += DT)
          if (hist[i]) atomicAdd(&gh[i], hist[i]);
        __syncthreads();
      }
    }
  };
  // H2: t0 = bin of the K-th key; keys above it are counted per chunk, keys in
  // it become candidates and feed the second-digit histogram.
  auto cand_phase = [&]() {
    // t0 = bin of the K-th key; keys above it are counted per chunk, keys in it
    // become candidates and feed the second-digit histogram.
    if (sp) {
      for (int n = 0; n < N; ++n) {
        const int vis = a.L - N + n + 1;
        if (vis <= K) continue;
        const int row = b * N + n;
        const uint32_t* gh = a.hist0 + (size_t)row * 2048;
  #pragma unroll
        for (int i = 0; i < 2048 / DT; ++i) hist[threadIdx.x + i * DT] = ld_dev(gh + threadIdx.x + i * DT);
        __syncthreads();
        pick_top(hist, 2048, (uint32_t)K, scratch, res);
        const uint32_t t0 = res[0];
        if (threadIdx.x == 0) {
          t0s[n] = t0;
          kk0s[n] = (uint32_t)K - res[1];
        }
        const int lim = min(clen, vis - j0);
        uint32_t above = 0, ncand = 0;
        for (int jj = threadIdx.x; jj < lim; jj += DT) {
          const uint32_t bin = radix_key(lds[n * a.CH + jj]) >> 21;
          above += bin > t0;
          ncand += bin == t0;
        }
        uint32_t tot_c;
        const uint32_t pre = block_excl_scan<DT>(ncand, scratch, tot_c);
        const uint32_t tot_a = block_sum(above, scratch);
        const int upg = (a.nch + kCandGroups - 1) / kCandGroups;   // chunks per group
        const int grp = c / upg;
        uint32_t base_slot = 0;
        if (threadIdx.x == 0) {
          // reserve this unit's slots in its group's region; the reply is
          // needed only after the second-digit histogram below
          if (tot_c) base_slot = atomicAdd(&a.cand_n[(size_t)row * kCandGroups + grp], tot_c);
          st_dev(&a.cnt[(size_t)row * a.nch + c], tot_a);
        }
        for (int i = threadIdx.x; i < 2048; i += DT) hist[i] = 0;
        __syncthreads();
        for (int jj = threadIdx.x; jj < lim; jj += DT) {
          const uint32_t key = radix_key(lds[n * a.CH + jj]);
          if ((key >> 21) == t0) atomicAdd(&hist[(key >> 10) & 2047u], 1u);
        }
        if (threadIdx.x == 0) res[2] = base_slot;
        __syncthreads();
        uint32_t slot = res[2] + pre;
        uint64_t* cr = (uint64_t*)a.cand + (size_t)row * a.cand_cap + (size_t)grp * upg * a.CH;
        for (int jj = threadIdx.x; jj < lim; jj += DT) {
          const uint32_t key = radix_key(lds[n * a.CH + jj]);
          if ((key >> 21) == t0) {
            st_dev64(cr + slot, ((uint64_t)key << 32) | (uint32_t)(j0 + jj));
            ++slot;
          }
        }
        __syncthreads();
        uint32_t* gh1 = a.hist1 + (size_t)row * 2048;
        for (int i = threadIdx.x; i < 2048; i += DT)
          if (hist[i]) atomicAdd(&gh1[i], hist[i]);
        __syncthreads();
      }
    }
  };
  // H3 (ordered rows): every unit resolves its row's exact threshold itself:
  // t1 from the second-digit histogram, then the few candidates sharing the
  // top two digits give the exact K-th key T and the position cut P* for
  // ties.  The unit's offset in the index row is the number of selected keys
  // in the chunks before it.
  auto select_phase = [&]() {
    // Every unit resolves its row's exact threshold itself (no further
    // barrier): t1 from the second-digit histogram, then the few candidates
    // sharing the top two digits give the exact K-th key T and the position cut
    // P* for ties.  The unit's offset in the index row is the number of
    // selected keys in the chunks before it.
    if (has_unit) {
      for (int n = 0; n < N; ++n) {
        const int row = b * N + n;
        const int vis = a.L - N + n + 1;
        uint32_t* lr = (uint32_t*)a.list + (size_t)row * K;
        if (!sp) {
          if (c == 0)
            for (int i = threadIdx.x; i < K; i += DT) st_dev(lr + i, 0xffffffffu);
          continue;
        }
        if (vis <= K) {
          const int lim = min(clen, vis - j0);
          for (int jj = threadIdx.x; jj < lim; jj += DT) st_dev(lr + j0 + jj, (uint32_t)(j0 + jj));
          if (c == 0)
            for (int i = vis + threadIdx.x; i < K; i += DT) st_dev(lr + i, 0xffffffffu);
          continue;
        }
        const uint32_t t0 = t0s[n];
        uint32_t kk = kk0s[n];
        // one round trip: second-digit histogram, the groups' candidate counts
        // and the keys above bin t0 in the chunks before this one
        const uint32_t* gh1 = a.hist1 + (size_t)row * 2048;
        const uint32_t* cnt_row = a.cnt + (size_t)row * a.nch;
        uint32_t* gpre = reinterpret_cast<uint32_t*>(lds + DSC);   // [kCandGroups + 1]
        uint64_t* cl = reinterpret_cast<uint64_t*>(lds + DSC + 64);
        const int cap_lds = (kLdsFloats - DSC - 64) / 2;
        const int upg = (a.nch + kCandGroups - 1) / kCandGroups;
        uint32_t before = 0;
        {
          uint32_t h8[2048 / DT];
  #pragma unroll
          for (int x = 0; x < 2048 / DT; ++x) h8[x] = ld_dev(gh1 + threadIdx.x + x * DT);
          uint32_t gc = 0;
          if (threadIdx.x < kCandGroups) gc = ld_dev(a.cand_n + (size_t)row * kCandGroups + threadIdx.x);
          for (int u = threadIdx.x; u < c; u += DT) before += ld_dev(cnt_row + u);
  #pragma unroll
          for (int x = 0; x < 2048 / DT; ++x) hist[threadIdx.x + x * DT] = h8[x];
          if (threadIdx.x < kCandGroups) gpre[threadIdx.x + 1] = gc;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
          uint32_t acc = 0;
          gpre[0] = 0;
          for (int g2 = 1; g2 <= kCandGroups; ++g2) {
            acc += gpre[g2];
            gpre[g2] = acc;
          }
        }
        __syncthreads();
        const int nc = (int)gpre[kCandGroups];
        pick_top(hist, 2048, kk, scratch, res);
        const uint32_t t1 = res[0];
        kk -= res[1];
        const uint32_t m = hist[t1];              // candidates sharing digits t0, t1
        const uint64_t* crg = (const uint64_t*)a.cand + (size_t)row * a.cand_cap;
        // flat candidate index -> slot: the last group whose first index is <= f
        // (a fixed-step search, so that several of them interleave)
        auto grp_of = [&](uint32_t f) -> int {
          int lo = 0;
  #pragma unroll
          for (int st = kCandGroups / 2; st > 0; st >>= 1)
            if (gpre[lo + st] <= f) lo += st;
          return lo;
        };
        auto cand_slot = [&](uint32_t f) -> size_t {
          const int g2 = grp_of(f);
          return (size_t)g2 * upg * a.CH + (f - gpre[g2]);
        };
        const uint32_t pfx = (t0 << 11) | t1;      // top 22 bits of T
        const bool in_lds = m <= (uint32_t)cap_lds;
        if (threadIdx.x == 0) res[3] = 0;
        __syncthreads();
        // one pass over the row's candidates: selected-for-sure ones before this
        // chunk, and the ones sharing the top two digits (kept in LDS)
        for (int i0 = 0; i0 < nc; i0 += DT * 8) {
          size_t sl8[8];
  #pragma unroll
          for (int x = 0; x < 8; ++x) sl8[x] = cand_slot((uint32_t)(i0 + x * DT + threadIdx.x));
          uint64_t v8[8];
  #pragma unroll
          for (int x = 0; x < 8; ++x) {
            const int f = i0 + x * DT + threadIdx.x;
            v8[x] = (f < nc) ? ld_dev64(crg + sl8[x]) : 0ull;
          }
  #pragma unroll
          for (int x = 0; x < 8; ++x) {
            const int f = i0 + x * DT + threadIdx.x;
            if (f >= nc) continue;
            const uint32_t key = (uint32_t)(v8[x] >> 32), pos = (uint32_t)v8[x];
            const uint32_t top = key >> 10;
            if (top > pfx && pos < (uint32_t)j0) ++before;
            if (top == pfx && in_lds) cl[atomicAdd(&res[3], 1u)] = v8[x];
          }
        }
        __syncthreads();
        auto cand = [&](uint32_t i) -> uint64_t {
          return in_lds ? cl[i] : ld_dev64(crg + cand_slot(i));
        };
        const uint32_t nl = in_lds ? m : (uint32_t)nc;   // entries to scan for the last digit
        // T, the K-th key, and P*, the last position taken among keys equal to T
        uint32_t T, pstar;
        if (in_lds && m <= (uint32_t)DT) {
          // few candidates share the top 22 bits: the kk-th of them under
          // (key descending, position ascending) by counting the ones before it
          if (threadIdx.x < m) {
            const uint64_t me = cl[threadIdx.x];
            const uint32_t key = (uint32_t)(me >> 32), pos = (uint32_t)me;
            uint32_t r = 0;
  #pragma unroll 8
            for (uint32_t i = 0; i < m; ++i) {
              const uint64_t o = cl[i];
              const uint32_t ok = (uint32_t)(o >> 32), op = (uint32_t)o;
              r += (ok > key) || (ok == key && op < pos);
            }
            if (r + 1 == kk) {
              res[0] = key;
              res[1] = pos;
            }
          }
          __syncthreads();
          T = res[0];
          pstar = res[1];
          __syncthreads();
        } else {
          // digit 3: key bits 9..0 among the candidates with prefix pfx
          for (int i = threadIdx.x; i < 1024; i += DT) hist[i] = 0;
          __syncthreads();
          for (uint32_t i = threadIdx.x; i < nl; i += DT) {
            const uint32_t key = (uint32_t)(cand(i) >> 32);
            if ((key >> 10) == pfx) atomicAdd(&hist[key & 1023u], 1u);
          }
          __syncthreads();
          pick_top(hist, 1024, kk, scratch, res);
          const uint32_t t2 = res[0];
          kk -= res[1];
          const uint32_t ties = hist[t2];
          T = (pfx << 10) | t2;
          __syncthreads();
          pstar = 0x7fffffffu;
          if (kk < ties) {
            // kk-th smallest position among the keys equal to T
            uint32_t pprefix = 0, pmask = 0;
            const int pshift[3] = {20, 10, 0};
            const int pbins[3] = {2048, 1024, 1024};
            for (int lv = 0; lv < 3; ++lv) {
              const int nb = pbins[lv], sh = pshift[lv];
              for (int i = threadIdx.x; i < nb; i += DT) hist[i] = 0;
              __syncthreads();
              for (uint32_t i = threadIdx.x; i < nl; i += DT) {
                const uint64_t cd = cand(i);
                const uint32_t key = (uint32_t)(cd >> 32), pos = (uint32_t)cd;
                if (key == T && (pos & pmask) == pprefix) atomicAdd(&hist[(pos >> sh) & (nb - 1)], 1u);
              }
              __syncthreads();
              pick_low(hist, nb, kk, scratch, res);
              pprefix |= res[0] << sh;
              pmask |= (uint32_t)(nb - 1) << sh;
              kk -= res[1];
              __syncthreads();
            }
            pstar = pprefix;
          }
        }
        // selected candidates with the top-two-digit prefix before this chunk
        for (uint32_t i = threadIdx.x; i < nl; i += DT) {
          const uint64_t cd = cand(i);
          const uint32_t key = (uint32_t)(cd >> 32), pos = (uint32_t)cd;
          if ((key >> 10) == pfx && pos < (uint32_t)j0 && (key > T || (key == T && pos <= pstar)))
            ++before;
        }
        uint32_t base = block_sum(before, scratch);
        const int lim = min(clen, vis - j0);
        // each thread takes 8 consecutive keys: one block scan per 8 * DT keys
        for (int s0 = 0; s0 < lim; s0 += DT * 8) {
          const int jb = s0 + threadIdx.x * 8;
          uint32_t m8 = 0, c8 = 0;
  #pragma unroll
          for (int x = 0; x < 8; ++x) {
            const int jj = jb + x;
            if (jj < lim) {
              const uint32_t key = radix_key(lds[n * a.CH + jj]);
              if (key > T || (key == T && (uint32_t)(j0 + jj) <= pstar)) {
                m8 |= 1u << x;
                ++c8;
              }
            }
          }
          uint32_t tot;
          uint32_t o = base + block_excl_scan<DT>(c8, scratch, tot);
  #pragma unroll
          for (int x = 0; x < 8; ++x)
            if ((m8 >> x) & 1u) {
              if (o < (uint32_t)K) st_dev(lr + o, (uint32_t)(j0 + jb + x));
              ++o;
            }
          base += tot;
        }
      }
    }
  };

  // ------------------------------------------------ attention items
  // The last split of a (row, KV head, head chunk) to finish merges the
  // partials and applies the gate (ticket counter), so no barrier follows.
  // llist: the item row's index list in LDS, or null to read the global one.
  constexpr bool kMfma = sizeof(TQ) == 2;   // bf16 keys/values: MFMA attention
  const int per_s = ((K + a.S - 1) / a.S + 63) / 64 * 64;
  const int per_d = ((a.L + a.S - 1) / a.S + 63) / 64 * 64;
  auto run_item = [&](int it, const uint32_t* llist) {
    const Item t = item_of(a, it);
    const int row = t.row, g = t.g, s = t.s, hci = t.hci;
    const int rb = row / N, rn = row - rb * N;
    item_heads<HCT>(a, t, rb, hsel, nsel);
    __syncthreads();
    const int ns = nsel[0], nd = nsel[1];
    if (llist && g == 0 && hci == 0) {
      // this split's part of the row's index list, from the LDS copy
      const int e0 = s * per_s, e1 = min(K, e0 + per_s);
      int32_t* lo = a.list + (size_t)row * K;
      for (int e = e0 + (int)threadIdx.x; e < e1; e += DT) lo[e] = (int32_t)llist[e];
    }
    const int vis = a.L - N + rn + 1;
    if (ns > 0) {
      const int e0 = s * per_s, e1 = min(K, e0 + per_s);
      if constexpr (kMfma)
        attend_mfma<HD>(a, row, rb, rn, g, s, false, e0, e1, hsel[0], ns, lds, llist);
      else
        attend<TQ, HD, HCT>(a, row, rb, rn, g, s, false, e0, e1, hsel[0], ns, lds, false, llist);
    }
    if (nd > 0) {
      const int e0 = s * per_d, e1 = min(vis, e0 + per_d);
      if constexpr (kMfma)
        attend_mfma<HD>(a, row, rb, rn, g, s, true, e0, e1, hsel[1], nd, lds, nullptr);
      else
        attend<TQ, HD, HCT>(a, row, rb, rn, g, s, true, e0, e1, hsel[1], nd, lds, false, nullptr);
    }
    // ticket: the last split of this (row, g, hci) merges
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
      const uint32_t tk = atomicAdd(&a.ticket[((size_t)row * a.Hkv + g) * a.nhc + hci], 1u);
      res[0] = (tk + 1 == (uint32_t)a.S) ? 1u : 0u;
    }
    __syncthreads();
    if (res[0]) {
      // One round of loads per 8 splits: this thread's accumulator elements
      // (registers) and every (head, split) max and sum (to LDS), together
      // with the gate and second-branch values; then each thread merges its
      // (head, dim) elements over the splits with a running max.
      constexpr int PS = HD + 4;                   // floats per partial
      constexpr int NE = (HCT * HD + DT - 1) / DT;
      constexpr int MB = 8;                        // splits per round
      const int nh = ns + nd;
      const int S = a.S;
      float* mls = lds;                            // [nh][MB] (max, sum)
      float Mx[NE], Lx[NE], Ax[NE], gv[NE], yv[NE];
#pragma unroll
      for (int k = 0; k < NE; ++k) {
        Mx[k] = -INFINITY;
        Lx[k] = 0.f;
        Ax[k] = 0.f;
        gv[k] = 1.f;
        yv[k] = 0.f;
      }
      for (int s0 = 0; s0 < S; s0 += MB) {
        const int sb = min(MB, S - s0);
        float av[NE][MB];
#pragma unroll
        for (int k = 0; k < NE; ++k) {
          const int e = threadIdx.x + k * DT;
          const bool ok = e < nh * HD;
          const int hh = e / HD, cth = e - hh * HD;
          const int h = !ok ? 0 : (hh < ns ? hsel[0][hh] : hsel[1][hh - ns]);
          const size_t orow = (size_t)row * a.Hq + h;
          const float* pk = a.part + (orow * S + s0) * PS + 4 + cth;
#pragma unroll
          for (int x = 0; x < MB; ++x) av[k][x] = (ok && x < sb) ? ld_devf(pk + (size_t)x * PS) : 0.f;
          if (s0 == 0 && ok && a.gate) {
            gv[k] = a.gate[orow];
            yv[k] = a.y2[orow * HD + cth];
          }
        }
        // every slot of [nh][MB] is written (unused splits as max -inf,
        // sum 0) so that the reads below need no predicate
        for (int i2 = threadIdx.x; i2 < nh * MB; i2 += DT) {
          const int hh = i2 / MB, sl = i2 - hh * MB;
          float mval = -INFINITY, lval = 0.f;
          if (sl < sb) {
            const int h = hh < ns ? hsel[0][hh] : hsel[1][hh - ns];
            const float* ps = a.part + (((size_t)row * a.Hq + h) * S + s0 + sl) * PS;
            mval = ld_devf(ps);
            lval = ld_devf(ps + 1);
          }
          mls[2 * i2] = mval;
          mls[2 * i2 + 1] = lval;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < NE; ++k) {
          const int e = threadIdx.x + k * DT;
          if (e >= nh * HD) continue;
          const float* ml = mls + 2 * (e / HD) * MB;
          float mv[MB], lv[MB];
#pragma unroll
          for (int x = 0; x < MB; ++x) {
            mv[x] = ml[2 * x];
            lv[x] = ml[2 * x + 1];
          }
          float mb = Mx[k];
#pragma unroll
          for (int x = 0; x < MB; ++x) mb = fmaxf(mb, mv[x]);
          if (mb == -INFINITY) continue;
          const float f0 = (Mx[k] == -INFINITY) ? 0.f : exp2f(Mx[k] - mb);
          float l = Lx[k] * f0, acc = Ax[k] * f0;
#pragma unroll
          for (int x = 0; x < MB; ++x) {
            const float f = exp2f(mv[x] - mb);   // 0 for an unused or empty split
            l = fmaf(f, lv[x], l);
            acc = fmaf(f, av[k][x], acc);
          }
          Mx[k] = mb;
          Lx[k] = l;
          Ax[k] = acc;
        }
        __syncthreads();
      }
#pragma unroll
      for (int k = 0; k < NE; ++k) {
        const int e = threadIdx.x + k * DT;
        if (e >= nh * HD) continue;
        const int hh = e / HD, cth = e - hh * HD;
        const int h = hh < ns ? hsel[0][hh] : hsel[1][hh - ns];
        const size_t orow = (size_t)row * a.Hq + h;
        float val = (Lx[k] > 0.f) ? Ax[k] / Lx[k] : 0.f;
        if (a.gate) val = fmaf(gv[k], val, (1.f - gv[k]) * yv[k]);
        a.out[orow * HD + cth] = val;
      }
    }
    __syncthreads();
  };

  const int items_seq = N * a.Hkv * a.S * a.nhc;   // items of this sequence
  uint32_t ph = 1;                                  // sequence barrier phase
  const uint32_t* llist = nullptr;
  bool slow = a.M == 0;
  if (!slow) {
    // ---------------------------------------------- candidate selection (N == 1)
    // C1: the chunk's M largest keys under (key descending, position
    // ascending), as order values key << 32 | ~position, go to the row's
    // candidate array in position order, with the key range of each wave's
    // share and the chunk's (M+1)-th value.
    const int row = b;
    const bool need = cand_sel;
    uint64_t* cbuf = reinterpret_cast<uint64_t*>(lds + a.CH);
    auto ord_at = [&](int jj) -> uint64_t {
      return ((uint64_t)radix_key(lds[jj]) << 32) | (uint32_t)~(uint32_t)(j0 + jj);
    };
    if (need) {
      __syncthreads();
      uint64_t e = 0;
      if (clen > a.M)
        e = kth_largest(clen, (uint32_t)a.M + 1, ord_at, 0u, 64, (uint32_t)clen, false, hist, cbuf,
                        red, res);
      uint64_t* cw = a.fcand + (size_t)row * a.Cpad + (size_t)c * a.M;
      uint32_t base = 0;
      uint32_t kmx = 0, kmn = 0xffffffffu;
      for (int s0 = 0; s0 < clen; s0 += DT * 8) {
        const int jb = s0 + (int)threadIdx.x * 8;
        uint64_t v8[8];
        uint32_t c8 = 0;
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          const uint64_t v = ord_at(min(jb + x, clen - 1));
          v8[x] = jb + x < clen ? v : 0ull;
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int x = 0; x < 8; ++x) c8 += v8[x] > e;
        uint32_t tot;
        uint32_t o = base + block_excl_scan<DT>(c8, scratch, tot);
#pragma unroll
        for (int x = 0; x < 8; ++x)
          if (v8[x] > e) {
            if (o < (uint32_t)a.M) st_dev64(cw + o, v8[x]);
            ++o;
            kmx = max(kmx, (uint32_t)(v8[x] >> 32));
            kmn = min(kmn, (uint32_t)(v8[x] >> 32));
          }
        base += tot;
      }
      // this wave's candidate key range and the chunk's (M+1)-th value
      kmx = wave_max_u32(kmx);
      kmn = wave_min_u32(kmn);
      if ((threadIdx.x & 63) == 0) {
        uint64_t* fs = a.fstat + (((size_t)row * a.nch + c) * 4 + (threadIdx.x >> 6)) * 2;
        st_dev64(fs, (uint64_t)kmx | ((uint64_t)kmn << 32));
        st_dev64(fs + 1, e);
      }
      for (int o = (int)base + (int)threadIdx.x; o < a.M; o += DT) st_dev64(cw + o, 0ull);
    }
    if (!seq_sync(a, ep, b, ph++, &flag)) {
      abandon<HD>(a, b);
      return;
    }
    // C2: every unit with an attention item loads the row's candidates,
    // counting their first digit as they arrive, and finds their K-th
    // largest value cK.  The candidates hold the row's top K when cK is above
    // every chunk's (M+1)-th value (a key left out of a chunk is below that
    // chunk's (M+1)-th, hence below cK, and K candidates are at or above cK);
    // then the index list is the candidates at or above cK in position
    // order, built in LDS.  Otherwise the sequence falls back to the
    // histogram phases.
    const int items_row = items_seq;
    uint32_t* llw = hist;
    if (!need) {
      if (c >= items_row) return;
      __syncthreads();
      for (int e = threadIdx.x; e < K; e += DT) llw[e] = (sp && e < a.L) ? (uint32_t)e : 0xffffffffu;
      __syncthreads();
      llist = llw;
    } else if (c < items_row) {
      const int C = a.nch * a.M;
      const uint64_t* cr = a.fcand + (size_t)row * a.Cpad;
      // the row's candidate key range and largest left-out value, from the
      // per-wave records of C1 (loaded together with the candidates)
      const int nst = a.nch * 4;
      const uint64_t* fs = a.fstat + (size_t)row * nst * 2;
      uint32_t kmax = 0, kmin = 0xffffffffu;
      uint64_t emax = 0;
      uint64_t v16[16];
      auto load16 = [&](int i0) __attribute__((always_inline)) {
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          const int i = i0 + x * DT + (int)threadIdx.x;
          const uint64_t v = ld_dev64(cr + min(i, C - 1));
          v16[x] = i < C ? v : 0ull;
        }
        __builtin_amdgcn_sched_barrier(0);
      };
      load16(0);
      // the records, four per thread and round (one round for up to 256
      // chunks), reduced while the candidates are in flight
      for (int q0 = 0; q0 * DT < nst; q0 += 4) {
        uint64_t sw[4][2];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int i = min((int)threadIdx.x + (q0 + q) * DT, nst - 1);
          sw[q][0] = ld_dev64(fs + 2 * i);
          sw[q][1] = ld_dev64(fs + 2 * i + 1);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if ((int)threadIdx.x + (q0 + q) * DT < nst) {
            kmax = max(kmax, (uint32_t)sw[q][0]);
            kmin = min(kmin, (uint32_t)(sw[q][0] >> 32));
            emax = max(emax, sw[q][1]);
          }
      }
      kmax = wave_max_u32(kmax);
      kmin = wave_min_u32(kmin);
      emax = wave_max_u64(emax);
      if ((threadIdx.x & 63) == 0) {
        red[threadIdx.x >> 6] = kmax;
        red[4 + (threadIdx.x >> 6)] = kmin;
        red[8 + (threadIdx.x >> 6)] = emax;
      }
      cbuf[a.Cpad + threadIdx.x] = 0;   // the selection's gather buffer
      if (threadIdx.x == 0) res[2] = 0;
      __syncthreads();
      kmax = (uint32_t)max(max(red[0], red[1]), max(red[2], red[3]));
      kmin = (uint32_t)min(min(red[4], red[5]), min(red[6], red[7]));
      emax = max(max(red[8], red[9]), max(red[10], red[11]));
      // first digit over the key range the candidates take, counted as the
      // candidates are stored
      const int chi = kmax > kmin ? 64 - __clz(kmax - kmin) : 32;
      const int bits = min(11, chi);
      const int sh = chi - bits;
      const uint32_t nbm = (1u << bits) - 1u;
      for (int i0 = 0; i0 < a.Cpad; i0 += DT * 16) {
        if (i0) load16(i0);
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          const int i = i0 + x * DT + (int)threadIdx.x;
          const uint64_t v = v16[x];
          if (i < a.Cpad) cbuf[i] = v;
          if ((uint32_t)v != 0u)
            atomicAdd(&hist[hslot((uint32_t)((v - ((uint64_t)kmin << 32)) >> sh) & nbm)], 1u);
        }
      }
      const uint64_t ck =
          a.ccnt >= K ? kth_largest(a.Cpad, (uint32_t)K, [&](int i) { return cbuf[i]; }, kmin, chi,
                                    (uint32_t)a.ccnt, true, hist, cbuf + a.Cpad, red, res)
                      : 0ull;
      const bool valid = ck != 0 && ck > emax;
      if (c == 0 && threadIdx.x == 0)
        st_dev64(a.verdict + 8 * b, ((uint64_t)ep << 32) | (valid ? 1u : 2u));
      if (valid) {
        // the list: the candidates at or above cK in position order.  Wave
        // w takes entries [w * Cpad / 4, (w + 1) * Cpad / 4) in rounds of 64
        // consecutive ones (a count pass, a scan of the four waves' counts,
        // then the write pass with lane offsets from the round's ballot)
        const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
        const int span = a.Cpad / 4;                   // a multiple of 256
        const uint64_t* wsrc = cbuf + (size_t)w * span + lane;
        uint32_t cntw = 0;
        for (int r0 = 0; r0 < span; r0 += 64 * 4) {
          uint64_t v4[4];
#pragma unroll
          for (int x = 0; x < 4; ++x) v4[x] = wsrc[r0 + 64 * x];
#pragma unroll
          for (int x = 0; x < 4; ++x) cntw += (uint32_t)__popcll(__ballot(v4[x] >= ck));
        }
        if (lane == 0) scratch[w] = cntw;
        __syncthreads();
        uint32_t o = 0;
        for (int x = 0; x < w; ++x) o += scratch[x];
        for (int r0 = 0; r0 < span; r0 += 64 * 4) {
          uint64_t v4[4];
#pragma unroll
          for (int x = 0; x < 4; ++x) v4[x] = wsrc[r0 + 64 * x];
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const bool in = v4[x] >= ck;
            const uint64_t mk = __ballot(in);
            if (in) llw[o + (uint32_t)__popcll(mk & lanemask_lt())] = ~(uint32_t)v4[x];
            o += (uint32_t)__popcll(mk);
          }
        }
        __syncthreads();
        llist = llw;
      } else {
        slow = true;
      }
    } else {
      // no attention item here: this unit is needed again only if the
      // sequence falls back (unit 0 publishes the verdict)
      if (threadIdx.x == 0) {
        res[0] = 0;
        if (wait_tag(a, ep, b, a.verdict + 8 * b, 1u)) res[0] = (uint32_t)ld_dev64(a.verdict + 8 * b);
      }
      __syncthreads();
      const uint32_t vd = res[0];
      __syncthreads();
      if (vd == 0u) abandon<HD>(a, b);   // the wait gave up
      if (vd != 2u) return;
      slow = true;
    }
  }
  if (slow) {
    build_hist0();
    bool ok = seq_sync(a, ep, b, ph++, &flag);
    if (ok) {
      cand_phase();
      ok = seq_sync(a, ep, b, ph++, &flag);
    }
    if (ok) {
      select_phase();
      ok = seq_sync(a, ep, b, ph++, &flag);
    }
    if (!ok) {
      abandon<HD>(a, b);
      return;
    }
    llist = nullptr;
  }
  for (int il = c; il < items_seq; il += a.nch) run_item(b * items_seq + il, llist);
}

template <typename TI, int DIDX, typename TQ, int HD>
const void* decode_kernel(int G) {
  if constexpr (sizeof(TQ) == 2) {
    (void)G;
    return reinterpret_cast<const void*>(&k_decode<TI, DIDX, TQ, HD, 16>);
  } else {
    if (G <= 4) return reinterpret_cast<const void*>(&k_decode<TI, DIDX, TQ, HD, 4>);
    return reinterpret_cast<const void*>(&k_decode<TI, DIDX, TQ, HD, 8>);
  }
}

template <typename TI, typename TQ, int HD>
const void* pick_didx(int didx, int G) {
  switch (didx) {
    case 16: return decode_kernel<TI, 16, TQ, HD>(G);
    case 32: return decode_kernel<TI, 32, TQ, HD>(G);
    case 64: return decode_kernel<TI, 64, TQ, HD>(G);
    default: return decode_kernel<TI, 128, TQ, HD>(G);
  }
}

const void* select_kernel(const Dims& D) {
  const int G = D.Hq / D.Hkv;
  if (D.idx_bf16) {
    if (D.qkv_bf16) return D.d == 128 ? pick_didx<bf16_bits, bf16_bits, 128>(D.didx, G)
                                      : pick_didx<bf16_bits, bf16_bits, 64>(D.didx, G);
    return D.d == 128 ? pick_didx<bf16_bits, float, 128>(D.didx, G)
                      : pick_didx<bf16_bits, float, 64>(D.didx, G);
  }
  if (D.qkv_bf16) return D.d == 128 ? pick_didx<float, bf16_bits, 128>(D.didx, G)
                                    : pick_didx<float, bf16_bits, 64>(D.didx, G);
  return D.d == 128 ? pick_didx<float, float, 128>(D.didx, G)
                    : pick_didx<float, float, 64>(D.didx, G);
}

// Occupancy per (kernel, device), cached in a fixed table: the library keeps
// no static object whose destructor would run at process exit, and a call
// after the first for a kernel allocates nothing.
struct GridEntry {
  const void* fn;
  int dev, grid;
};
std::mutex g_grid_mu;
GridEntry g_grid[128];
int g_grid_n = 0;

int coresident_blocks(const void* fn) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(g_grid_mu);
  for (int x = 0; x < g_grid_n; ++x)
    if (g_grid[x].fn == fn && g_grid[x].dev == dev) return g_grid[x].grid;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  int per = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, fn, DT, 0) != hipSuccess) return 0;
  per = std::min(per, 2);
  if (g_grid_n < 128) g_grid[g_grid_n++] = GridEntry{fn, dev, cus * per};
  return cus * per;
}

}  // namespace

bool decode_plan(const Dims& D, int grid, DecodePlan& P) {
  if (D.N < 1 || D.N > 4 || grid <= 0 || grid > kMaxGrid) return false;
  if (D.IH != 1) return false;   // one selected set per token only
  const int rows = D.B * D.N;
  if (rows > grid) return false;
  // smallest chunk (multiple of 256) with one unit per workgroup
  long long ch = ((long long)D.B * D.L + grid - 1) / grid;
  ch = std::max<long long>(256, (ch + 255) / 256 * 256);
  while ((long long)D.B * ((D.L + ch - 1) / ch) > grid) ch += 256;
  if (ch * D.N > DSC) return false;
  const int nch = (int)((D.L + ch - 1) / ch);
  if (nch > DMAXCH) return false;
  P.grid = grid;
  P.CH = (int)ch;
  P.nch = nch;
  const int G = D.Hq / D.Hkv;
  const int hct = D.qkv_bf16 ? 16 : (G <= 4 ? 4 : 8);   // heads per attention item
  P.nhc = (G + hct - 1) / hct;
  // one split per 256 keys: every split keeps the four waves of its
  // workgroup busy with one 64-key pass each
  P.S = std::max(1, (D.K + 255) / 256);
  P.cand_cap = kCandGroups * ((nch + kCandGroups - 1) / kCandGroups) * (int)ch;
  // One-exchange selection for single-row sequences: each chunk passes on
  // its M largest keys.  A chunk's count of top-K keys is close to binomial
  // with mean `share` for keys in no particular order, so share plus four
  // standard deviations plus 8 is exceeded with probability below 1e-6 per
  // chunk; capped by what the LDS holds next to the chunk's scores.
  P.M = 0;
  P.Cpad = 0;
  // (the per-wave records of a row, 4 per chunk, are read 8 per thread)
  if (D.N == 1 && D.K <= 2048 && nch * 4 <= 8 * DT) {
    const int avail = (kLdsFloats - (int)ch - 2 * DT) / 2;   // 8-byte slots left in LDS
    const int share = (D.K + nch - 1) / nch;
    int M = (int)std::min<long long>(ch, share + (int)std::ceil(4.0 * std::sqrt((double)share)) + 8);
    // padded to whole blocks of 4 * DT slots: the list pass reads an even
    // count of at most 32 per thread
    auto padded = [&](int m) { return ((long long)nch * m + 4 * DT - 1) / (4 * DT) * (4 * DT); };
    while (M > 0 && (padded(M) > avail || padded(M) > 32 * DT)) --M;
    if (M > 0 && (long long)M * nch >= D.K && (M == ch || 2 * M >= 3 * share)) {
      P.M = M;
      P.Cpad = (int)padded(M);
    }
  }
  return true;
}

int decode_grid(const Dims& D) { return coresident_blocks(select_kernel(D)); }

size_t decode_ws_bound(const Dims& D) {
  DecodePlan P;
  P.nch = (int)std::min<long long>(DMAXCH, ((long long)D.L + 255) / 256);
  P.S = (D.K + 63) / 64;
  P.nhc = D.Hq;
  P.cand_cap = D.L + kCandGroups * DSC;   // groups * (chunks per group) * CH < L + groups * CH
  P.Cpad = D.N == 1 ? (kLdsFloats - 256 - 2 * DT) / 2 : 0;
  return decode_ws_bytes(D, P);
}

// Workspace layout (all offsets 256-byte aligned): the zeroed block (control
// words, both digit histograms, candidate counts, tickets), then per-chunk
// counts, candidates and attention partials.
struct DecodeLayout {
  size_t ctl, rowtag, sgslot, verdict, seqerr, hist0, hist1, cand_n, ticket, cnt, cand, fcand, fstat,
      part, total;
};

DecodeLayout decode_layout(const Dims& D, const DecodePlan& P) {
  const size_t rows = (size_t)D.B * D.N;
  auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
  DecodeLayout Lo;
  size_t off = 0;
  Lo.ctl = off;    off = al(off + ctl_words64(kMaxGrid) * 8);
  Lo.rowtag = off; off = al(off + rows * 8);
  Lo.sgslot = off; off = al(off + (size_t)D.B * ((P.nch + kBarGroup - 1) / kBarGroup) * 64);
  Lo.verdict = off; off = al(off + (size_t)D.B * 64);
  Lo.seqerr = off; off = al(off + (size_t)D.B * 64);
  Lo.hist0 = off;  off = al(off + rows * 2048 * 4);
  Lo.hist1 = off;  off = al(off + rows * 2048 * 4);
  Lo.cand_n = off; off = al(off + rows * kCandGroups * 4);
  Lo.ticket = off; off = al(off + rows * D.Hkv * (size_t)P.nhc * 4);
  Lo.cnt = off;    off = al(off + rows * (size_t)P.nch * 4);
  Lo.cand = off;   off = al(off + rows * (size_t)P.cand_cap * 8);
  Lo.fcand = off;  off = al(off + rows * (size_t)P.Cpad * 8);
  Lo.fstat = off;  off = al(off + (P.Cpad ? rows * (size_t)P.nch * 64 : 0));
  Lo.part = off;   off = al(off + rows * D.Hq * (size_t)P.S * (D.d + 4) * 4);
  Lo.total = off;
  return Lo;
}

size_t decode_ws_bytes(const Dims& D, const DecodePlan& P) { return decode_layout(D, P).total; }

// Launches of this kernel are ordered across streams: all of its workgroups
// must be resident at once, so two of them must not share the GPU.
struct StreamOrder {
  std::mutex mu;
  hipStream_t last = nullptr;
  bool have_last = false;
  hipEvent_t done = nullptr;
  uint32_t epoch = 0;
};

// A fresh, nonzero launch epoch; the first one is drawn from the clock and
// the process id so that control words left by another process do not match.
uint32_t next_epoch(StreamOrder& so) {
  if (so.epoch == 0) {
    const uint64_t t = (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count();
    so.epoch = (uint32_t)(t ^ (t >> 32) ^ ((uint64_t)getpid() << 16));
  }
  if (++so.epoch == 0) ++so.epoch;
  return so.epoch;
}

StreamOrder& stream_order(int dev) {
  static StreamOrder orders[64];
  return orders[dev & 63];
}

// Polls a decode wait makes before it gives up; see dsa_set_wait_limit.
std::atomic<uint32_t> g_wait_limit{kDefaultWaitLimit};

// Epoch of the last decode launch per workspace (its control block sits at
// the workspace's start), so that dsa_exec_status can tell this launch's
// error word from one left by an earlier launch.  A fixed table of the last
// kWsSlots workspaces (oldest replaced first).
constexpr int kWsSlots = 64;
struct WsEntry {
  const void* ws;
  uint32_t epoch;   // the launch's epoch, or kDeviceEpoch: read it from the workspace
};
constexpr uint32_t kDeviceEpoch = 0xffffffffu;
std::mutex g_ws_mu;
WsEntry g_ws[kWsSlots];
int g_ws_next = 0;

void record_launch(const void* ws, uint32_t epoch) {
  std::lock_guard<std::mutex> lock(g_ws_mu);
  for (WsEntry& e : g_ws)
    if (e.ws == ws) {
      e.epoch = epoch;
      return;
    }
  g_ws[g_ws_next] = WsEntry{ws, epoch};
  g_ws_next = (g_ws_next + 1) % kWsSlots;
}

void set_wait_limit(uint32_t polls) { g_wait_limit.store(polls, std::memory_order_relaxed); }

int decode_exec_status(const void* ws, hipStream_t s, hipError_t* err) {
  *err = hipSuccess;
  uint32_t epoch = 0;
  {
    std::lock_guard<std::mutex> lock(g_ws_mu);
    for (const WsEntry& e : g_ws)
      if (e.ws == ws && ws) epoch = e.epoch;
    if (epoch == 0) return 0;
  }
  *err = hipStreamSynchronize(s);
  if (*err != hipSuccess) return 0;
  // control words 0 (error) .. 2 (the device epoch of captured launches)
  uint64_t words[3] = {0, 0, 0};
  *err = hipMemcpy(words, ws, sizeof(words), hipMemcpyDeviceToHost);
  if (*err != hipSuccess) return 0;
  if (epoch == kDeviceEpoch) epoch = (uint32_t)words[2];
  return words[0] == (((uint64_t)epoch << 32) | 1ull) ? 1 : 0;
}

void forget_launch(const void* ws) {
  std::lock_guard<std::mutex> lock(g_ws_mu);
  for (WsEntry& e : g_ws)
    if (e.ws == ws) e = WsEntry{nullptr, 0};
}

hipError_t decode_setup() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  StreamOrder& so = stream_order(dev);
  std::lock_guard<std::mutex> lock(so.mu);
  if (!so.done) e = hipEventCreateWithFlags(&so.done, hipEventDisableTiming);
  return e;
}

// Under stream capture the epoch cannot travel as a kernel argument: every
// replay of the graph would reuse it, and control words left by the previous
// replay would then pass for this one's.  This one-thread kernel, captured
// just before the decode kernel, keeps (seed, count) in control words 1-2 and
// writes the epoch for the launch: a new seed (a new capture) restarts the
// count, every replay advances it.
__global__ void k_decode_epoch(uint32_t* w, uint32_t seed) {
  if (threadIdx.x == 0) {
    const uint32_t cnt = (w[0] == seed) ? w[1] + 1u : 1u;
    uint32_t e = seed ^ (cnt * 0x9E3779B9u);
    if (e == 0) e = 1;
    w[0] = seed;
    w[1] = cnt;
    w[2] = e;   // low half of control word 2
  }
}

hipError_t launch_decode(const Dims& D, const DecodePlan& P, const void* q_idx, const void* k_idx,
                         const void* q, const void* k, const void* v, const float* gate,
                         const float* y2, const uint8_t* route, float* out, int32_t* list,
                         void* ws, hipStream_t s) {
  char* w = (char*)ws;
  const DecodeLayout Lo = decode_layout(D, P);
  DecodeArgs a{};
  a.q_idx = q_idx; a.k_idx = k_idx; a.q = q; a.k = k; a.v = v;
  a.gate = gate; a.y2 = y2; a.route = route; a.out = out; a.list = list;
  a.ctl = (uint64_t*)(w + Lo.ctl);
  a.rowtag = (uint64_t*)(w + Lo.rowtag);
  a.hist0 = (uint32_t*)(w + Lo.hist0);
  a.hist1 = (uint32_t*)(w + Lo.hist1);
  a.ticket = (uint32_t*)(w + Lo.ticket);
  a.cand_n = (uint32_t*)(w + Lo.cand_n);
  a.cnt = (uint32_t*)(w + Lo.cnt);
  a.cand = (uint64_t*)(w + Lo.cand);
  a.part = (float*)(w + Lo.part);
  a.fcand = (uint64_t*)(w + Lo.fcand);
  a.sgslot = (uint64_t*)(w + Lo.sgslot);
  a.verdict = (uint64_t*)(w + Lo.verdict);
  a.seqerr = (uint64_t*)(w + Lo.seqerr);
  a.M = P.M; a.Cpad = P.Cpad;
  a.ccnt = P.M ? (P.nch - 1) * P.M + std::min(D.L - (P.nch - 1) * P.CH, P.M) : 0;
  a.fstat = (uint64_t*)(w + Lo.fstat);
  a.B = D.B; a.N = D.N; a.L = D.L; a.Hq = D.Hq; a.Hkv = D.Hkv; a.K = D.K;
  a.CH = P.CH; a.nch = P.nch; a.S = P.S; a.nhc = P.nhc; a.cand_cap = P.cand_cap;
  a.scale_log2 = D.scale * kLog2e;

  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  e = hipStreamIsCapturing(s, &cs);
  if (e != hipSuccess) return e;
  const bool capturing = cs == hipStreamCaptureStatusActive;
  StreamOrder& so = stream_order(dev);
  std::lock_guard<std::mutex> lock(so.mu);
  if (!so.done) {
    if (capturing) return hipErrorStreamCaptureUnsupported;   // set-up must precede capture
    e = hipEventCreateWithFlags(&so.done, hipEventDisableTiming);
    if (e != hipSuccess) return e;
  }
  // eager launches on another stream wait for the last one; a captured graph
  // is ordered against other decode launches by whoever replays it
  if (!capturing && so.have_last && so.last != s) {
    e = hipStreamWaitEvent(s, so.done, 0);
    if (e != hipSuccess) return e;
  }
  a.epoch = next_epoch(so);
  a.epw = nullptr;
  a.spin_limit = g_wait_limit.load(std::memory_order_relaxed);
  void* args[] = {&a};
  if (capturing) {
    uint32_t* w32 = reinterpret_cast<uint32_t*>(a.ctl + 1);   // control words 1-2
    hipLaunchKernelGGL(k_decode_epoch, dim3(1), dim3(64), 0, s, w32, a.epoch);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    a.epw = w32 + 2;
    record_launch(ws, kDeviceEpoch);
    ProfScope ps(s, kStageDecode);
    e = hipLaunchKernel(select_kernel(D), dim3(P.grid), dim3(DT), args, 0, s);
    return e;
  }
  record_launch(ws, a.epoch);
  // the completion event rides on the kernel's own dispatch
  {
    ProfScope ps(s, kStageDecode);
    e = hipExtLaunchKernel(select_kernel(D), dim3(P.grid), dim3(DT), args, 0, s, nullptr, so.done, 0);
  }
  so.last = s;
  so.have_last = true;
  return e;
}

}  // namespace dsa
