// Prefill attention for both routes in one launch, blocked by key range so
// that the keys and values a group of workgroups gathers stay in one XCD's L2.
//
// What it computes: for a sparse head, softmax(q k^T * scale) v over the
// selected rows of the query token ("混合注意力架构演进：从线性注意力到稀疏门控
// 的技术权衡" §三; steps 3-4 of the gated forward on "超大规模MoE架构中稀疏注意力
// 机制的演进与实践" §四.1); for a dense head the same over every visible key
// ("Advanced Attention Mechanisms" article §2.1), both followed by the gate
// blend of step 5.  The page "Elastic Attention：动态路由优化大模型长文本处理"
// §3.1 puts both kinds of head in one fused op with load balancing by the
// actual route; here they are items of one persistent grid.
//
// Why key ranges.  A sparse token reads 2048 scattered 256-byte key and value
// rows per KV head; gathered from a whole 65536-token sequence they come from
// HBM / the Infinity Cache (about 7.5-8.7 TB/s on MI355X), while gathered from
// a region that fits one XCD's 4 MB L2 they come at about 27 TB/s (measured
// with a plain gather kernel).  So the keys are cut into ranges of RC
// positions and the work into slices (sequence, KV head, range): the K/V of
// one slice (RC * d * 4 bytes; 4 MB for RC = 8192, d = 128) is what the
// workgroups of an XCD gather from while they work through that slice.
// Every (query row, head) gets one partial result per range it sees (its
// online-softmax state: log2-sum-exp and normalised output), merged by
// k_merge_ranges; rows that see a single range write the output directly.
// The range length trades L2 locality against the per-(row, range) costs
// (partials, their merge, each range's pipeline start): on the 64K elastic
// prefill 8192 keys beat 4096 (attention 84 vs 91 ms, merge 4.1 vs 5.8 ms)
// and 16384 (87 ms).
//
// Scheduling.  k_sched lists the non-empty slices in (sequence, KV head,
// range) order and deals them to the 8 XCDs round robin; each XCD has a
// queue of items (dense query tiles and sparse query blocks of its slices,
// the two kinds interleaved evenly within a slice so that MFMA-bound and
// gather-bound work run side by side).  The attention grid is persistent:
// each workgroup reads its XCD id from the hardware register and takes items
// from that XCD's queue with an atomic counter, then from the other queues
// once its own is empty.  The mapping only decides cache locality; every item
// is taken exactly once whatever XCD a workgroup runs on.
#include "attn_tile.h"
#include "common.h"
#include "launch.h"
#include "mfma.h"

namespace dsa {
namespace {

constexpr int ST = 256;             // threads (4 waves)
constexpr int kXcd = 8;             // XCDs (queues)
constexpr int kQB = 16;             // query rows per sparse item
constexpr int DROWS = 128;          // query rows per dense tile
constexpr int DKEYS = 64;           // keys per dense step
constexpr int kDenseLds = 4 * DKEYS * 256;   // K and V, double-buffered, 64 rows of <= 256 B
constexpr int kSeg = 256;           // index entries staged per wave at a time
// fourth word of a raw buffer resource on gfx9-family GPUs (32-bit data)
constexpr int kBufWord3 = 0x00020000;
constexpr int kSparseLds = 4 * 2 * 32 * 256 + 4 * kSeg * 4;   // per wave: key and value tiles, entries
constexpr int kLds = kDenseLds > kSparseLds ? kDenseLds : kSparseLds;

struct SliceArgs {
  const bf16_bits* q; const bf16_bits* k; const bf16_bits* v;
  const int32_t* topk; int idx_rows_per_b, idx_n_base;
  const float* gate; const float* y2; const uint8_t* route;
  float* out;
  const int32_t* off;   // [B * R][NC + 1] index-row offsets of the ranges
  const int32_t* sched; // queue tables (k_sched)
  uint32_t* ctr;        // [kXcd] queue counters, zeroed by k_sched
  float* part_o;        // [B * R][NC][Hq][HD] normalised partial outputs
  float* part_lse;      // [B * R][NC][Hq] log2-sum-exp of the partials
  int B, N, L, Hq, Hkv, K;
  int n0, R;            // query rows [n0, n0 + R) of each sequence
  int RC, NC;           // keys per range; ranges seen by the chunk's last row
  int cap;              // slices per queue table
  float scale_log2;
  int IH;               // index rows per token (indexer heads); head h uses h / (Hq / IH)
};

// Queue tables: [0, 8) slice counts, [8, 16) item totals, then per queue the
// slice ids (cap each) and the exclusive prefix of their item counts.
__device__ __forceinline__ const int32_t* q_sid(const SliceArgs& a, int x) {
  return a.sched + 16 + (size_t)x * a.cap;
}
__device__ __forceinline__ const int32_t* q_pre(const SliceArgs& a, int x) {
  return a.sched + 16 + (size_t)(kXcd + x) * a.cap;
}

// Query heads of group g of sequence b by route.
__device__ __forceinline__ bool head_sparse(const SliceArgs& a, int b, int h) {
  return a.route ? a.route[(size_t)b * a.Hq + h] != 0 : true;
}

struct SliceItems {
  int r_c;      // first chunk row that sees the range
  int nsp;      // sparse heads in the group
  int nt;       // dense tiles per dense head
  int n_dense;  // dense items
  int n_sparse; // sparse items
};

__device__ __forceinline__ SliceItems slice_items(const SliceArgs& a, int b, int g, int c) {
  SliceItems s;
  const int G = a.Hq / a.Hkv;
  const int off = a.L - a.N + a.n0;   // position of chunk row 0
  s.r_c = max(0, c * a.RC - off);
  s.nsp = 0;
  for (int x = 0; x < G; ++x) s.nsp += head_sparse(a, b, g * G + x) ? 1 : 0;
  if (s.r_c >= a.R) {
    s.nt = s.n_dense = s.n_sparse = 0;
    return s;
  }
  s.nt = (a.R + DROWS - 1) / DROWS - s.r_c / DROWS;
  s.n_dense = (G - s.nsp) * s.nt;
  s.n_sparse = s.nsp > 0 ? (a.R - s.r_c + kQB - 1) / kQB : 0;
  return s;
}

// One workgroup: the queue tables and zeroed counters.
__global__ __launch_bounds__(ST) void k_sched(SliceArgs a, int32_t* sched) {
  const int lane = threadIdx.x & 63, x = threadIdx.x >> 6;
  const int nslices = a.B * a.Hkv * a.NC;
  // waves 0..3 take queues x and x + 4
  for (int qx = x; qx < kXcd; qx += 4) {
    int cnt = 0, tot = 0;
    for (int base = qx; base < nslices; base += kXcd * 64) {
      const int s = base + lane * kXcd;
      int items = 0;
      if (s < nslices) {
        const int c = s % a.NC, bg = s / a.NC;
        const SliceItems it = slice_items(a, bg / a.Hkv, bg % a.Hkv, c);
        items = it.n_dense + it.n_sparse;
      }
      // order-preserving compaction of the non-empty slices
      const uint64_t m = __ballot(items > 0);
      const int rank = __popcll(m & lanemask_lt());
      const uint32_t incl = wave_incl_scan((uint32_t)items);
      if (items > 0) {
        sched[16 + (size_t)qx * a.cap + cnt + rank] = s;
        sched[16 + (size_t)(kXcd + qx) * a.cap + cnt + rank] = tot + (int)(incl - items);
      }
      cnt += __popcll(m);
      tot += (int)__builtin_amdgcn_readlane((int)incl, 63);
    }
    if (lane == 0) {
      sched[qx] = cnt;
      sched[kXcd + qx] = tot;
      a.ctr[qx] = 0u;
    }
  }
}

// One wave per index row (token row and indexer head): offsets of the ranges
// in the row.  off[c] = number of valid entries (in [0, p]) below c * RC,
// for c = 0 .. nr (nr = p / RC + 1).  The row lists its valid entries in
// ascending order before any padding, so the entries of range c are
// [off[c], off[c + 1]) and off[c] is where the row's range index first
// reaches c: found by comparing each entry's range with its predecessor's
// (no atomics).
__global__ __launch_bounds__(ST) void k_range_offsets(SliceArgs a) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const long long row = (long long)blockIdx.x * 4 + w;   // ((b * R + r) * IH + ih)
  if (row >= (long long)a.B * a.R * a.IH) return;   // wave-uniform
  const int ih = (int)(row % a.IH);
  const long long br = row / a.IH;
  const int b = (int)(br / a.R), r = (int)(br - (long long)b * a.R);
  const int n = a.n0 + r, p = a.L - a.N + n;
  const int nr = p / a.RC + 1;
  const int32_t* irow =
      a.topk + (((size_t)b * a.idx_rows_per_b + (n - a.idx_n_base)) * a.IH + ih) * a.K;
  int32_t* o = const_cast<int32_t*>(a.off) + (size_t)row * (a.NC + 1);
  // range index of an entry; padding, entries past p and the slot past the
  // row's end count as range nr
  auto range_of = [&](int j) { return (j >= 0 && j <= p) ? j / a.RC : nr; };
  // 64 consecutive entries per round (lane = entry, coalesced); a lane whose
  // entry starts a new range writes that range's offset (and those of any
  // empty ranges before it); the slot at index K closes the remaining ranges
  int carry = -1;                                // range of the entry before the round
  for (int e0 = 0; e0 <= a.K; e0 += 64) {
    const int e = e0 + lane;
    const int cur = (e < a.K) ? range_of(irow[e]) : nr;
    int prev = __shfl_up(cur, 1, 64);
    if (lane == 0) prev = carry;
    if (e <= a.K)
      for (int cc = prev + 1; cc <= cur; ++cc) o[cc] = e;
    carry = __builtin_amdgcn_readlane(cur, 63);
  }
}

// Result of one (row, head) column: the final gated output when the row sees a
// single range, else the partial of range c.  l is already summed over quads.
template <int HD>
__device__ __forceinline__ void emit_col(const SliceArgs& a, const ColState<HD>& st, float l,
                                         int b, int r, int h, int c, int nr) {
  const int lane = threadIdx.x & 63;
  const int q = lane >> 4;
  const int n = a.n0 + r;
  const float inv = (l > 0.f) ? 1.f / l : 0.f;
  if (nr == 1) {
    const size_t orow = ((size_t)b * a.N + n) * a.Hq + h;
    const float g = a.gate ? a.gate[orow] : 1.f;
#pragma unroll
    for (int dt = 0; dt < HD / 16; ++dt) {
      const int d0 = dt * 16 + 4 * q;
      float4 v;
      float* vv = &v.x;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        float val = st.o[dt][x] * inv;
        if (a.gate) val = fmaf(g, val, (1.f - g) * a.y2[orow * HD + d0 + x]);
        vv[x] = val;
      }
      *reinterpret_cast<float4*>(a.out + orow * HD + d0) = v;
    }
    return;
  }
  const size_t slot = (((size_t)b * a.R + r) * a.NC + c) * a.Hq + h;
#pragma unroll
  for (int dt = 0; dt < HD / 16; ++dt) {
    const int d0 = dt * 16 + 4 * q;
    float4 v = make_float4(st.o[dt][0] * inv, st.o[dt][1] * inv, st.o[dt][2] * inv,
                           st.o[dt][3] * inv);
    *reinterpret_cast<float4*>(a.part_o + slot * HD + d0) = v;
  }
  if (q == 0) a.part_lse[slot] = (l > 0.f) ? st.m + __builtin_amdgcn_logf(l) : -INFINITY;
}

// Dense query tile of a slice: 128 chunk rows of one dense head, 32 per wave as
// two 16-column MFMA tiles, against the range's keys in 64-key steps.  Key and
// value tiles go from memory straight into LDS (direct loads, double-buffered:
// step s + 1 is in flight while step s computes; one barrier per step).  Rows
// are stored back to back with their 16-byte chunks permuted so that both
// the key reads (16 rows, one chunk) and the transposing value reads are
// free of bank conflicts.
template <int HD>
__device__ void dense_tile(const SliceArgs& a, int b, int h, int tile, int c, char* smem) {
  constexpr int T = HD / 32;
  constexpr int CPR = HD / 8;                    // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;                  // rows per direct load
  constexpr int TB = DKEYS * HD * 2;             // bytes of one 64-row tile
  char* kbuf0 = smem;
  char* vbuf0 = smem + 2 * TB;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int q = lane >> 4, i = lane & 15;
  const int g = h / (a.Hq / a.Hkv);
  const int rbase = tile * DROWS;
  const int off = a.L - a.N + a.n0;              // position of chunk row 0
  const int rlast = min(a.R - 1, rbase + DROWS - 1);
  const int pmax = off + rlast;                  // last key any row of the tile sees
  const int kb = c * a.RC;
  const int ke = min(kb + a.RC, pmax + 1);       // keys [kb, ke) of the range
  const int wlast = min(a.R - 1, rbase + w * 32 + 31);
  // wave-uniform (read from lane 0 so that the branches on it stay scalar)
  const int pmax_wave = __builtin_amdgcn_readfirstlane(off + wlast);
  const int pmin_wave = __builtin_amdgcn_readfirstlane(off + rbase + w * 32);
  bf16x8 qb[2][T];
  int prow[2];
  bool rvalid[2];
#pragma unroll
  for (int cc = 0; cc < 2; ++cc) {
    const int r = rbase + w * 32 + cc * 16 + i;
    rvalid[cc] = r < a.R && off + r >= kb;
    prow[cc] = rvalid[cc] ? off + r : -1;
    const size_t orow = ((size_t)b * a.N + a.n0 + (rvalid[cc] ? r : 0)) * a.Hq + h;
    const bf16_bits* qr = a.q + orow * HD;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      uint4 u = rvalid[cc] ? *reinterpret_cast<const uint4*>(qr + q * (HD / 4) + t * 8)
                           : make_uint4(0, 0, 0, 0);
      qb[cc][t] = as_bf16x8(u);
    }
  }
  ColState<HD> st[2];
  // softmax denominators on the matrix cores: an all-ones A operand against
  // the same P^T operand the output MFMA takes gives every lane its
  // column's sum of the (bf16) weights, so the VALU does no per-score adds
  // and numerator and denominator use the same rounded weights
  f32x4 lacc[2];
  bf16x8 ones;
#pragma unroll
  for (int x = 0; x < 8; ++x) ones[x] = (__bf16)1.0f;
#pragma unroll
  for (int cc = 0; cc < 2; ++cc) {
    st[cc].m = -INFINITY;
    st[cc].l = 0.f;
    lacc[cc] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < HD / 16; ++dt) st[cc].o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const bf16_bits* kbase = a.k + ((size_t)b * a.L * a.Hkv + g) * HD;
  const bf16_bits* vbase = a.v + ((size_t)b * a.L * a.Hkv + g) * HD;
  // each step reads through buffer resources based at its first row, so
  // each lane's row and chunk is a fixed vector offset and the range check
  // (which covers the vector offset) turns rows past the sequence into
  // zeros; rows past the range are real keys of the sequence (their scores
  // are masked, their values weighted 0)
  const uint32_t rs_bytes = (uint32_t)(a.Hkv * HD * 2);
  const size_t rstride = (size_t)a.Hkv * HD;
  constexpr int MPW = DKEYS / RPI / 4;           // direct loads per wave and buffer
  const int wu = __builtin_amdgcn_readfirstlane(w);
  uint32_t ko[MPW], vo[MPW];
#pragma unroll
  for (int x = 0; x < MPW; ++x) {
    const int rr = (wu + 4 * x) * RPI + lane / CPR, pc = lane % CPR;
    ko[x] = (uint32_t)rr * rs_bytes + (uint32_t)((pc ^ (rr & (CPR - 1))) * 16);
    vo[x] = (uint32_t)rr * rs_bytes + (uint32_t)((pc ^ ((rr & (CPR / 2 - 1)) << 1)) * 16);
  }
  // the 64 key and value rows from j0 into buffer buf
  auto issue = [&](int j0, int buf) {
    const int nrec = (int)((uint32_t)(a.L - 1 - j0) * rs_bytes + HD * 2);
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(kbase + (size_t)j0 * rstride), (short)0, nrec, kBufWord3);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(vbase + (size_t)j0 * rstride), (short)0, nrec, kBufWord3);
#pragma unroll
    for (int x = 0; x < MPW; ++x) {
      const int m = wu + 4 * x;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          krs, (__attribute__((address_space(3))) void*)(kbuf0 + buf * TB + m * 1024), 16, ko[x], 0,
          0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          vrs, (__attribute__((address_space(3))) void*)(vbuf0 + buf * TB + m * 1024), 16, vo[x], 0,
          0, 0);
    }
  };
  const int nsteps = (ke - kb + DKEYS - 1) / DKEYS;
  issue(kb, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const int row0 = 4 * q + (i >> 2);   // value row this lane points at (transposing read)
  const int colb = (i & 3) * 8;
  // steps whose keys this wave's rows reach: a prefix of the tile's steps
  // (the rest only load for the other waves), so the step body below runs
  // unconditionally and the accumulators stay in place across iterations
  const int nsteps_w = pmax_wave < kb ? 0 : min(nsteps, (pmax_wave - kb) / DKEYS + 1);
  for (int sidx = 0; sidx < nsteps_w; ++sidx) {
    const int j0 = kb + sidx * DKEYS;
    if (sidx + 1 < nsteps) issue(j0 + DKEYS, (sidx + 1) & 1);
    {
      const char* kt = kbuf0 + (sidx & 1) * TB;
      const char* vt = vbuf0 + (sidx & 1) * TB;
      f32x4 sacc[2][4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        bf16x8 ka[T];
#pragma unroll
        for (int t = 0; t < T; ++t)
          ka[t] = as_bf16x8(*reinterpret_cast<const uint4*>(kt + kt_swz<HD>(u * 16 + i, q * (CPR / 4) + t)));
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int t = 0; t < T; ++t) acc = mfma16(ka[t], qb[cc][t], acc);
          sacc[cc][u] = acc;
        }
      }
      // raw scores; masks only where a key can lie past a row's position or
      // the range (the wave's first row has the smallest position).  The
      // test is wave-uniform and the masked form uses plain selects, so the
      // step has no per-element branches.
      const bool interior = j0 + DKEYS - 1 <= pmin_wave && j0 + DKEYS <= ke;
      bf16x8 pb[2][2];
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        float sv[16];
        if (interior) {
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) sv[u * 4 + rr] = sacc[cc][u][rr];
        } else {
          // keys below lim are visible; key j0 + 4q + (16u + rr) is this
          // lane's score [u][rr]
          const int dl = min(prow[cc] + 1, ke) - j0 - 4 * q;
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
              sv[u * 4 + rr] = u * 16 + rr < dl ? sacc[cc][u][rr] : -INFINITY;
        }
        float mt = sv[0];
#pragma unroll
        for (int x = 1; x < 16; ++x) mt = fmaxf(mt, sv[x]);
        mt = max_xor32(max_xor16(mt)) * a.scale_log2;
        // lazy maximum (see kLazyLog2)
        const bool bump = mt > st[cc].m + kLazyLog2;
        if (__builtin_amdgcn_ballot_w64(bump)) {
          const float mnew = bump ? mt : st[cc].m;
          const float alpha = exp2_fast(st[cc].m - mnew);
#pragma unroll
          for (int dt = 0; dt < HD / 16; ++dt)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) st[cc].o[dt][rr] *= alpha;
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) lacc[cc][rr] *= alpha;
          st[cc].m = mnew;
        }
        // a column whose maximum is still -inf has only masked scores, which
        // give exp2(-inf) = 0 against any finite subtrahend
        const float msub = st[cc].m == -INFINITY ? 0.f : st[cc].m;
        float pv[16];
#pragma unroll
        for (int x = 0; x < 16; ++x) pv[x] = exp2_fast(fmaf(sv[x], a.scale_log2, -msub));
        pb[cc][0] = pack8(pv);
        pb[cc][1] = pack8(pv + 8);
        lacc[cc] = mfma16(ones, pb[cc][0], lacc[cc]);
        lacc[cc] = mfma16(ones, pb[cc][1], lacc[cc]);
      }
#pragma unroll
      for (int v = 0; v < 2; ++v) {
#pragma unroll
        for (int dt = 0; dt < HD / 16; ++dt) {
          const uint2 lo = lds_tr(vt, vt_swz<HD>(32 * v + row0, dt * 32 + colb));
          const uint2 hi = lds_tr(vt, vt_swz<HD>(32 * v + 16 + row0, dt * 32 + colb));
          uint4 u4;
          u4.x = lo.x; u4.y = lo.y; u4.z = hi.x; u4.w = hi.y;
          const bf16x8 va = as_bf16x8(u4);
#pragma unroll
          for (int cc = 0; cc < 2; ++cc) st[cc].o[dt] = mfma16(va, pb[cc][v], st[cc].o[dt]);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);   // this wave's loads of the next step have landed
    __syncthreads();
  }
  for (int sidx = nsteps_w; sidx < nsteps; ++sidx) {
    if (sidx + 1 < nsteps) issue(kb + (sidx + 1) * DKEYS, (sidx + 1) & 1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
#pragma unroll
  for (int cc = 0; cc < 2; ++cc) {
    const float l = lacc[cc][0];
    if (rvalid[cc]) {
      const int r = rbase + w * 32 + cc * 16 + i;
      emit_col<HD>(a, st[cc], l, b, r, h, c, prow[cc] / a.RC + 1);
    }
  }
}

// Sparse query block of a slice: up to kQB chunk rows; wave w takes rows
// w, w + 4, ...  For each row and each chunk of up to 16 sparse heads of the
// group (the MFMA columns), the row's entries of this range are staged in the
// wave's LDS (up to kSeg at a time, one round of loads), then consumed 32 per
// step through the wave's LDS key and value tiles (see the pipeline below).
template <int HD>
__device__ void sparse_block(const SliceArgs& a, int b, int g, int c, int r0, char* smem) {
  constexpr int T = HD / 32;
  constexpr int CPR = HD / 8;
  constexpr int NG = 64 / CPR;              // lane groups (one 16-byte chunk per lane)
  constexpr int RPG = 32 / NG;              // rows each lane group stages per step
  constexpr int TB = 32 * HD * 2;           // bytes of one 32-row tile
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int q = lane >> 4, i = lane & 15;
  const int G = a.Hq / a.Hkv;
  char* ktile = smem + w * 2 * (32 * 256);
  char* vtile = ktile + TB;
  int* wl = reinterpret_cast<int*>(smem + 4 * 2 * 32 * 256) + w * kSeg;
  const bf16_bits* kbase = a.k + ((size_t)b * a.L * a.Hkv + g) * HD;
  const bf16_bits* vbase = a.v + ((size_t)b * a.L * a.Hkv + g) * HD;
  // buffer resources over this (sequence, KV head)'s rows: 32-bit offsets,
  // and a read past the last row returns zeros instead of faulting
  const uint32_t rs_bytes = (uint32_t)(a.Hkv * HD * 2);
  const int nrec = (int)((uint32_t)(a.L - 1) * rs_bytes + HD * 2);
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)kbase, (short)0, nrec, kBufWord3);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)vbase, (short)0, nrec, kBufWord3);
  const int gi = lane / CPR, ch = lane % CPR;
  // staging lane (gi, ch) fetches chunk ch ^ sp_f(R) of tile row R =
  // gi * RPG + m and stores it at chunk ch of that row (see sp_f); sp_f is
  // linear, so the fetched chunk is cfix ^ sp_f(m)
  const uint32_t cfix = (uint32_t)((ch ^ sp_f<HD>(gi * RPG)) << 4);
  char* kst = ktile + gi * RPG * (HD * 2) + ch * 16;
  char* vst = vtile + gi * RPG * (HD * 2) + ch * 16;
  const int kb = c * a.RC;
  const int r1 = min(a.R, r0 + kQB);
  const int HPS = a.Hq / a.IH;              // query heads per index row
  for (int r = r0 + w; r < r1; r += 4) {
    const int n = a.n0 + r, p = a.L - a.N + n;
    const int ke = min(kb + a.RC, p + 1);
    const int nr = p / a.RC + 1;
    // heads of the group by index row (set ih = h / HPS), up to 16 per chunk
    for (int h0 = g * G; h0 < g * G + G;) {
      const int ih = h0 / HPS;
      const int hend = min(g * G + G, (ih + 1) * HPS);
      const int hc0 = h0;
      h0 = min(hend, hc0 + 16);
      const int32_t* orow = a.off + (((size_t)b * a.R + r) * a.IH + ih) * (a.NC + 1);
      const int lo = min(max(orow[c], 0), a.K);
      const int hi = min(max(orow[c + 1], lo), a.K);
      const int32_t* irow =
          a.topk + (((size_t)b * a.idx_rows_per_b + (n - a.idx_n_base)) * a.IH + ih) * a.K;
      int myh = -1, cnt = 0;
      for (int h = hc0; h < h0; ++h) {
        if (head_sparse(a, b, h)) {
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
      for (int s0 = lo; s0 < hi; s0 += kSeg) {
        const int sn = min(kSeg, hi - s0);
        // stage this part of the segment, each entry checked against the range
        // and the row (entries past the segment read as -1): the byte offset
        // of the entry's row, or INT_MIN for an entry outside this range
        // (less than 2^31 by the launch's limit on L * Hkv * d * 2)
        int jv[kSeg / 64];
#pragma unroll
        for (int x = 0; x < kSeg / 64; ++x) {
          const int e = x * 64 + lane;
          jv[x] = (e < sn) ? irow[s0 + e] : -1;
        }
#pragma unroll
        for (int x = 0; x < kSeg / 64; ++x) {
          const int j = jv[x];
          wl[x * 64 + lane] = (j >= kb && j < ke) ? (int)((uint32_t)j * rs_bytes) : INT_MIN;
        }
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_wave_barrier();
        // register-staged pipeline: the 32 key and value rows of step e0 are
        // loaded into registers (whole 256-byte rows per lane group, the
        // access pattern the L2 serves fastest; buffer loads with 32-bit
        // offsets) while step e0 - 32 computes, then written to the wave's
        // LDS tiles (chunks permuted by sp_f) and read back as MFMA
        // operands.  Lane group gi = lane / CPR stages rows gi * RPG ..
        // gi * RPG + RPG - 1.  Masked entries (INT_MIN) read row 0.  The
        // loads' register results order the staging stores after them; the
        // stores and the step's reads of the tiles are LDS operations of one
        // wave, which the LDS performs in order.
        u32x4 kr[RPG], vr[RPG];
        {
          int jr[RPG];
#pragma unroll
          for (int m = 0; m < RPG; m += 4)
            *reinterpret_cast<int4*>(&jr[m]) = *reinterpret_cast<const int4*>(wl + gi * RPG + m);
#pragma unroll
          for (int m = 0; m < RPG; ++m) {
            const uint32_t off = ((uint32_t)jr[m] & 0x7fffffffu) | (cfix ^ (uint32_t)(sp_f<HD>(m) << 4));
            kr[m] = __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0);
            vr[m] = __builtin_amdgcn_raw_buffer_load_b128(vrs, off, 0, 0);
          }
        }
        for (int e0 = 0; e0 < sn; e0 += 32) {
#pragma unroll
          for (int m = 0; m < RPG; ++m) {
            *reinterpret_cast<u32x4*>(kst + m * (HD * 2)) = kr[m];
            *reinterpret_cast<u32x4*>(vst + m * (HD * 2)) = vr[m];
          }
          bool kval[2][4];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int4 e4 = *reinterpret_cast<const int4*>(wl + e0 + u * 16 + 4 * q);
            kval[u][0] = e4.x >= 0; kval[u][1] = e4.y >= 0;
            kval[u][2] = e4.z >= 0; kval[u][3] = e4.w >= 0;
          }
          __builtin_amdgcn_wave_barrier();
          if (e0 + 32 < sn) {
            int jr[RPG];
#pragma unroll
            for (int m = 0; m < RPG; m += 4)
              *reinterpret_cast<int4*>(&jr[m]) =
                  *reinterpret_cast<const int4*>(wl + e0 + 32 + gi * RPG + m);
#pragma unroll
            for (int m = 0; m < RPG; ++m) {
              const uint32_t off = ((uint32_t)jr[m] & 0x7fffffffu) | (cfix ^ (uint32_t)(sp_f<HD>(m) << 4));
              kr[m] = __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0);
              vr[m] = __builtin_amdgcn_raw_buffer_load_b128(vrs, off, 0, 0);
            }
          }
          step32_lds<HD>(ktile, vtile, qb, kval, a.scale_log2, st);
          __builtin_amdgcn_wave_barrier();   // tile reads are consumed by the MFMAs above
        }
      }
      const float l = sum_xor32(sum_xor16(st.l));
      if (myh >= 0) emit_col<HD>(a, st, l, b, r, myh, c, nr);
    }
  }
}

template <int HD>
__global__ __launch_bounds__(ST, 2) void k_attn_slices(SliceArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[kLds];
  __shared__ int s_item[4];
  const uint32_t xcc = __builtin_amdgcn_s_getreg((3 << 11) | 20) & (kXcd - 1);  // HW_REG_XCC_ID
  int qx = (int)xcc, tried = 0;
  for (;;) {
    if (threadIdx.x == 0) {
      int found = 0;
      while (tried < kXcd) {
        const int total = a.sched[kXcd + qx];
        if (total > 0 && a.ctr[qx] < (uint32_t)total) {
          const uint32_t t = atomicAdd(&a.ctr[qx], 1u);
          if (t < (uint32_t)total) {
            // the queue's slice holding item t (binary search over the prefix)
            const int cnt = a.sched[qx];
            const int32_t* pre = q_pre(a, qx);
            int lo = 0, hi = cnt - 1;
            while (lo < hi) {
              const int mid = (lo + hi + 1) >> 1;
              if (pre[mid] <= (int)t) lo = mid;
              else hi = mid - 1;
            }
            s_item[0] = q_sid(a, qx)[lo];
            s_item[1] = (int)t - pre[lo];
            found = 1;
            break;
          }
        }
        qx = (qx + 1) & (kXcd - 1);
        ++tried;
      }
      s_item[2] = found;
      s_item[3] = tried;
    }
    __syncthreads();
    const int found = s_item[2];
    const int s = s_item[0], it = s_item[1];
    tried = s_item[3];
    qx = (int)((xcc + tried) & (kXcd - 1));
    __syncthreads();
    if (!found) return;
    const int c = s % a.NC, bg = s / a.NC;
    const int b = bg / a.Hkv, g = bg - b * a.Hkv;
    const SliceItems S = slice_items(a, b, g, c);
    // dense items spread evenly through the slice's item sequence
    const int tot = S.n_dense + S.n_sparse;
    const long long dk0 = (long long)it * S.n_dense / tot;
    const long long dk1 = (long long)(it + 1) * S.n_dense / tot;
    if (dk1 > dk0) {
      const int d = (int)dk0;                 // dense item index
      const int hi = d / S.nt, tile = S.r_c / DROWS + d % S.nt;
      // the hi-th dense head of the group
      const int G = a.Hq / a.Hkv;
      int h = -1, k = 0;
      for (int x = 0; x < G; ++x)
        if (!head_sparse(a, b, g * G + x) && k++ == hi) {
          h = g * G + x;
          break;
        }
      dense_tile<HD>(a, b, h, tile, c, smem);
    } else {
      const int sp = it - (int)dk1;           // sparse item index
      sparse_block<HD>(a, b, g, c, S.r_c + sp * kQB, smem);
    }
    __syncthreads();
  }
}

// Merge of the per-range partials of rows that see more than one range: one
// workgroup per (sequence, row); thread t takes head t / 8 (in rounds of 32
// heads), dims 16 * (t % 8) .. + 16.
template <int HD>
__global__ __launch_bounds__(ST) void k_merge_ranges(SliceArgs a) {
  const int r = blockIdx.x, b = blockIdx.y;
  const int n = a.n0 + r, p = a.L - a.N + n;
  const int nr = p / a.RC + 1;
  if (nr == 1) return;
  constexpr int TPH = HD / 4;             // threads per head: one float4 of the output each
  constexpr int HPR = ST / TPH;           // heads per round
  constexpr int MR = 8;                   // ranges held in registers at once
  const int hl = threadIdx.x / TPH, d4 = threadIdx.x % TPH;
  for (int h0 = 0; h0 < a.Hq; h0 += HPR) {
    const int h = h0 + hl;
    if (h >= a.Hq) break;
    const size_t slot0 = ((size_t)b * a.R + r) * a.NC * a.Hq + h;   // range c at + c * Hq
    float m = -INFINITY, wsum = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    // up to MR ranges per round, every load of the round in flight together
    // (the range count is the same for the whole workgroup)
    for (int c0 = 0; c0 < nr; c0 += MR) {
      float lv[MR];
      float4 ov[MR];
#pragma unroll
      for (int x = 0; x < MR; ++x) {
        if (c0 + x < nr) {
          const size_t slot = slot0 + (size_t)(c0 + x) * a.Hq;
          lv[x] = a.part_lse[slot];
          ov[x] = reinterpret_cast<const float4*>(a.part_o + slot * HD)[d4];
        } else {
          lv[x] = -INFINITY;
          ov[x] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
      float mb = m;
#pragma unroll
      for (int x = 0; x < MR; ++x) mb = fmaxf(mb, lv[x]);
      if (mb == -INFINITY) continue;
      // a range without entries has lse = -inf (weight 0) and a zero output
      const float f0 = m == -INFINITY ? 0.f : exp2_fast(m - mb);
      wsum *= f0;
      acc.x *= f0; acc.y *= f0; acc.z *= f0; acc.w *= f0;
#pragma unroll
      for (int x = 0; x < MR; ++x) {
        const float wg = lv[x] == -INFINITY ? 0.f : exp2_fast(lv[x] - mb);
        wsum += wg;
        acc.x = fmaf(wg, ov[x].x, acc.x);
        acc.y = fmaf(wg, ov[x].y, acc.y);
        acc.z = fmaf(wg, ov[x].z, acc.z);
        acc.w = fmaf(wg, ov[x].w, acc.w);
      }
      m = mb;
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    const size_t orow = ((size_t)b * a.N + n) * a.Hq + h;
    float o[4] = {acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv};
    if (a.gate) {
      const float gt = a.gate[orow];
      const float4 y = reinterpret_cast<const float4*>(a.y2 + orow * HD)[d4];
      const float yv[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
      for (int x = 0; x < 4; ++x) o[x] = fmaf(gt, o[x], (1.f - gt) * yv[x]);
    }
    reinterpret_cast<float4*>(a.out + orow * HD)[d4] = make_float4(o[0], o[1], o[2], o[3]);
  }
}

int g_grid_cache[64][2];

}  // namespace

SlicePlan slice_plan(const Dims& D, int R) {
  SlicePlan P;
  P.RC = kSliceKeys;
  const int p_last = D.L - 1;   // bound for any chunk
  P.NC = p_last / P.RC + 1;
  (void)R;
  const long long nslices = (long long)D.B * D.Hkv * P.NC;
  P.cap = (int)((nslices + kXcd - 1) / kXcd);
  return P;
}

size_t slice_ws_bytes(const Dims& D, int R) {
  const SlicePlan P = slice_plan(D, R);
  auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
  size_t b = 0;
  b += al((size_t)D.B * R * D.IH * (P.NC + 1) * 4);              // offsets
  b += al((16 + (size_t)2 * kXcd * P.cap) * 4);                   // queue tables
  b += al(kXcd * 4 * 16);                                         // counters
  b += al((size_t)D.B * R * P.NC * D.Hq * D.d * 4);               // partial outputs
  b += al((size_t)D.B * R * P.NC * D.Hq * 4);                     // partial lse
  return b;
}

bool slice_attention_supported(const Dims& D) {
  // 32-bit byte offsets within one sequence's keys (buffer loads)
  return D.qkv_bf16 && (D.d == 64 || D.d == 128) && D.L <= 256 * kSliceKeys &&
         (long long)D.L * D.Hkv * D.d * 2 < (1ll << 31);
}

hipError_t launch_attention_slices(const Dims& D, const AttnArgs& aa, void* ws, hipStream_t s) {
  if (D.B == 0 || aa.R == 0) return hipSuccess;
  const SlicePlan P = slice_plan(D, aa.R);
  SliceArgs a{};
  a.q = (const bf16_bits*)aa.q; a.k = (const bf16_bits*)aa.k; a.v = (const bf16_bits*)aa.v;
  a.topk = aa.topk; a.idx_rows_per_b = aa.idx_rows_per_b; a.idx_n_base = aa.idx_n_base;
  a.gate = aa.gate; a.y2 = aa.y2; a.route = aa.route; a.out = aa.out;
  a.B = D.B; a.N = D.N; a.L = D.L; a.Hq = D.Hq; a.Hkv = D.Hkv; a.K = D.K;
  a.n0 = aa.n0; a.R = aa.R;
  a.RC = P.RC;
  // ranges seen by the chunk's last row bound the partial slots
  a.NC = (D.L - D.N + aa.n0 + aa.R - 1) / P.RC + 1;
  a.cap = P.cap;
  a.scale_log2 = D.scale * kLog2e;
  a.IH = D.IH;
  auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
  char* w = (char*)ws;
  size_t o = 0;
  a.off = (const int32_t*)(w + o);   o += al((size_t)D.B * aa.R * D.IH * (P.NC + 1) * 4);
  int32_t* sched = (int32_t*)(w + o); o += al((16 + (size_t)2 * kXcd * P.cap) * 4);
  a.sched = sched;
  a.ctr = (uint32_t*)(w + o);        o += al(kXcd * 4 * 16);
  a.part_o = (float*)(w + o);        o += al((size_t)D.B * aa.R * P.NC * D.Hq * D.d * 4);
  a.part_lse = (float*)(w + o);
  const long long rows = (long long)D.B * aa.R * D.IH;   // index rows
  {
    ProfScope ps(s, kStagePrep);
    hipLaunchKernelGGL(k_range_offsets, dim3((unsigned)((rows + 3) / 4)), dim3(ST), 0, s, a);
    hipLaunchKernelGGL(k_sched, dim3(1), dim3(ST), 0, s, a, sched);
  }
  // persistent grid: what the device holds at once
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  int& grid = g_grid_cache[dev & 63][D.d == 128 ? 1 : 0];
  if (grid == 0) {
    int cus = 0, per = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    e = D.d == 128 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, k_attn_slices<128>, ST, 0)
                   : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, k_attn_slices<64>, ST, 0);
    if (e != hipSuccess) return e;
    grid = cus * std::max(1, per);
  }
  {
    ProfScope ps(s, kStageAttention);
    if (D.d == 128) hipLaunchKernelGGL(k_attn_slices<128>, dim3(grid), dim3(ST), 0, s, a);
    else hipLaunchKernelGGL(k_attn_slices<64>, dim3(grid), dim3(ST), 0, s, a);
  }
  {
    ProfScope ps(s, kStageMerge);
    if (D.d == 128) hipLaunchKernelGGL(k_merge_ranges<128>, dim3(aa.R, D.B), dim3(ST), 0, s, a);
    else hipLaunchKernelGGL(k_merge_ranges<64>, dim3(aa.R, D.B), dim3(ST), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace dsa
