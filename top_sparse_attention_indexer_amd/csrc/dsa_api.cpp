// C ABI of libdsa: argument checks, workspace planning and kernel dispatch.
// Every check runs before anything is enqueued.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/dsa.h"
#include "launch.h"

namespace {

thread_local std::string g_err;

dsa_status fail(dsa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

dsa_status ok() {
  g_err.clear();
  return DSA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Query rows per sequence at or below which the streaming indexer and the
// split-row top-k are used (decode and short speculative batches).
constexpr int kDecodeRows = 8;
// Budget of materialised prefill scores per chunk of query rows (floats).
constexpr size_t kScoreBudget = size_t(64) << 20;

dsa_status check_problem(const dsa_problem* p, dsa::Dims& D) {
  if (!p) return fail(DSA_ERR_INVALID_ARG, "problem pointer is null");
  if (p->batch < 0 || p->n_q < 0) return fail(DSA_ERR_INVALID_ARG, "batch and n_q must be >= 0");
  if (p->batch > 65535) return fail(DSA_ERR_INVALID_ARG, "batch %d exceeds 65535", p->batch);
  if (p->kv_len < 1) return fail(DSA_ERR_INVALID_ARG, "kv_len must be >= 1");
  if (p->n_q > p->kv_len)
    return fail(DSA_ERR_INVALID_ARG, "n_q (%d) exceeds kv_len (%d)", p->n_q, p->kv_len);
  if (p->h_q < 1 || p->h_kv < 1) return fail(DSA_ERR_INVALID_ARG, "head counts must be >= 1");
  if (p->h_q % p->h_kv != 0)
    return fail(DSA_ERR_INVALID_ARG, "h_q (%d) is not a multiple of h_kv (%d)", p->h_q, p->h_kv);
  if (p->top_k < 1) return fail(DSA_ERR_INVALID_ARG, "top_k must be >= 1");
  if (p->head_dim < 1 || p->idx_dim < 1) return fail(DSA_ERR_INVALID_ARG, "dims must be >= 1");
  if (!std::isfinite(p->softmax_scale)) return fail(DSA_ERR_INVALID_ARG, "softmax_scale is not finite");
  if (p->qkv_dtype != DSA_FP32 && p->qkv_dtype != DSA_BF16)
    return fail(DSA_ERR_UNSUPPORTED, "qkv_dtype %d is not fp32 (0) or bf16 (1)", p->qkv_dtype);
  if (p->idx_dtype != DSA_FP32 && p->idx_dtype != DSA_BF16)
    return fail(DSA_ERR_UNSUPPORTED, "idx_dtype %d is not fp32 (0) or bf16 (1)", p->idx_dtype);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(DSA_ERR_UNSUPPORTED, "head_dim %d not in {64, 128}", p->head_dim);
  if (p->idx_dim != 16 && p->idx_dim != 32 && p->idx_dim != 64 && p->idx_dim != 128)
    return fail(DSA_ERR_UNSUPPORTED, "idx_dim %d not in {16, 32, 64, 128}", p->idx_dim);
  if (p->h_q / p->h_kv > 256)
    return fail(DSA_ERR_UNSUPPORTED, "more than 256 query heads per KV head");
  if ((long long)p->h_q * p->head_dim > (1ll << 20))
    return fail(DSA_ERR_UNSUPPORTED, "h_q * head_dim too large");
  if (p->idx_heads < 0) return fail(DSA_ERR_INVALID_ARG, "idx_heads must be >= 0");
  const int ih = p->idx_heads > 1 ? p->idx_heads : 1;
  if (p->h_q % ih != 0)
    return fail(DSA_ERR_INVALID_ARG, "h_q (%d) is not a multiple of idx_heads (%d)", p->h_q, ih);
  if ((long long)p->n_q * ih > (1ll << 30))
    return fail(DSA_ERR_UNSUPPORTED, "n_q * idx_heads too large");
  D.B = p->batch;
  D.N = p->n_q;
  D.L = p->kv_len;
  D.Hq = p->h_q;
  D.Hkv = p->h_kv;
  D.d = p->head_dim;
  D.didx = p->idx_dim;
  D.K = p->top_k;
  D.qkv_bf16 = p->qkv_dtype == DSA_BF16;
  D.idx_bf16 = p->idx_dtype == DSA_BF16;
  D.scale = p->softmax_scale > 0.f ? p->softmax_scale : 1.0f / std::sqrt((float)p->head_dim);
  D.IH = ih;
  return DSA_OK;
}

bool is_empty(const dsa::Dims& D) { return D.B == 0 || D.N == 0; }

// The indexer and top-k stages see IH index rows per query token; few such
// rows take the streaming indexer and the split-row top-k.
bool few_index_rows(const dsa::Dims& D) { return (long long)D.N * D.IH <= kDecodeRows; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Workspace layout of one call.
struct Plan {
  bool fused_decode = false;  // one cooperative launch (few rows, scores in LDS)
  dsa::DecodePlan dp;
  size_t dec_off = 0, dec_bytes = 0;
  bool decode;     // streaming indexer + split-row top-k
  int R;           // query tokens per chunk (times IH index rows)
  size_t scores_off = 0, scores_bytes = 0, ld = 0;
  size_t tk_off = 0, tk_bytes = 0;      // split top-k scratch
  size_t idx_off = 0, idx_bytes = 0;    // internal index rows of one chunk
  size_t part_off = 0, part_bytes = 0;  // attention partials of one chunk
  int splits_sparse = 1, splits_dense = 1;
  bool slices = false;  // key-range blocked MFMA attention (prefill, bf16)
  int Ra = 0;           // query rows per attention launch on that path
  bool onchip = false;  // indexer + top-k without a score matrix
  int Rs = 0;           // query tokens per launch of that pair
  size_t it_off = 0, it_bytes = 0;
  size_t sl_off = 0, sl_bytes = 0;
  size_t total = 0;
};

// KV heads per sparse attention item: the largest divisor of Hkv whose K/V
// for one sequence stays within kGatherBudget (the 256 MB Infinity Cache has
// to hold what the resident workgroups gather); all heads when one sequence's
// whole K/V fits.
constexpr size_t kGatherBudget = size_t(160) << 20;
int sparse_heads_per_item(const dsa::Dims& D) {
  const size_t per_head = (size_t)D.L * D.d * (D.qkv_bf16 ? 2 : 4) * 2;
  int best = 1;
  for (int g = 1; g <= D.Hkv; ++g)
    if (D.Hkv % g == 0 && (size_t)g * per_head <= kGatherBudget) best = g;
  return best;
}

int prefill_chunk_rows(const dsa::Dims& D) {
  size_t per_row = (size_t)D.B * D.L * D.IH;
  size_t r = std::max<size_t>(64, kScoreBudget / std::max<size_t>(per_row, 1));
  r = r / 64 * 64;
  return (int)std::min<size_t>(r, (size_t)D.N);
}

// Budget of indexer candidate lists per launch of the on-chip indexer + top-k.
constexpr size_t kCandBudget = size_t(1) << 30;
// Budget of per-range attention partials per launch of the key-range path;
// rows per launch are a multiple of 1024 (or all rows).
constexpr size_t kPartialBudget = size_t(6) << 30;
int slice_chunk_rows(const dsa::Dims& D) {
  const size_t per_row = dsa::slice_ws_bytes(D, 1);
  size_t r = std::max<size_t>(1024, kPartialBudget / std::max<size_t>(per_row, 1)) / 1024 * 1024;
  return (int)std::min<size_t>(r, (size_t)D.N);
}

bool use_slices(const dsa::Dims& D) {
  return D.N > kDecodeRows && dsa::slice_attention_supported(D);
}

Plan plan_topk(const dsa::Dims& D) {
  Plan P;
  P.decode = few_index_rows(D);
  P.R = D.N;
  if (P.decode) P.tk_bytes = dsa::split_topk_ws_bytes(D, D.N * D.IH);
  P.total = align256(P.tk_bytes);
  return P;
}

Plan plan_attn(const dsa::Dims& D) {
  Plan P;
  P.decode = D.N <= kDecodeRows;
  P.R = D.N;
  if (use_slices(D)) {
    P.slices = true;
    P.Ra = slice_chunk_rows(D);
    P.sl_bytes = dsa::slice_ws_bytes(D, P.Ra);
    P.total = align256(P.sl_bytes);
    return P;
  }
  dsa::attn_pick_splits(D, D.N, P.splits_sparse, P.splits_dense);
  P.part_bytes = dsa::attn_part_bytes(D, D.N, std::max(P.splits_sparse, P.splits_dense));
  P.total = align256(P.part_bytes);
  return P;
}

// Few query rows: the single-launch decode kernel when its grid and LDS limits
// allow (needs a device to size the co-resident grid).
bool plan_fused_decode(const dsa::Dims& D, Plan& P) {
  if (D.N > 4 || D.IH != 1) return false;
  const int grid = dsa::decode_grid(D);
  if (grid <= 0 || !dsa::decode_plan(D, grid, P.dp)) return false;
  P.fused_decode = true;
  P.decode = true;
  P.R = D.N;
  size_t off = 0;
  P.dec_off = off;
  P.dec_bytes = dsa::decode_ws_bytes(D, P.dp);
  off = align256(off + P.dec_bytes);
  P.idx_off = off;
  P.idx_bytes = (size_t)D.B * D.N * D.K * sizeof(int32_t);
  off = align256(off + P.idx_bytes);
  P.total = off;
  return true;
}

Plan plan_fused(const dsa::Dims& D, bool allow_single_launch = true) {
  Plan P;
  if (allow_single_launch && plan_fused_decode(D, P)) return P;
  P.decode = few_index_rows(D);
  P.slices = use_slices(D);
  P.Ra = P.slices ? slice_chunk_rows(D) : D.N;
  P.onchip = P.slices && dsa::idx_topk_supported(D);
  P.R = P.decode ? D.N : std::min(P.Ra, prefill_chunk_rows(D));
  P.ld = (size_t)D.L;
  size_t off = 0;
  if (P.onchip) {
    // candidate lists of up to kCandBudget bytes per launch
    const size_t per_row = dsa::idx_topk_ws_bytes(D, D.IH);
    P.Rs = (int)std::min<size_t>((size_t)P.Ra, std::max<size_t>(64, kCandBudget / per_row));
    P.it_off = off;
    P.it_bytes = dsa::idx_topk_ws_bytes(D, P.Rs * D.IH);
    off = align256(off + P.it_bytes);
  } else {
    P.scores_off = off;
    P.scores_bytes = (size_t)D.B * P.R * D.IH * D.L * sizeof(float);
    off = align256(off + P.scores_bytes);
  }
  if (P.decode) {
    P.tk_off = off;
    P.tk_bytes = dsa::split_topk_ws_bytes(D, P.R * D.IH);
    off = align256(off + P.tk_bytes);
  }
  P.idx_off = off;
  P.idx_bytes = (size_t)D.B * (P.slices ? P.Ra : P.R) * D.IH * D.K * sizeof(int32_t);
  off = align256(off + P.idx_bytes);
  if (P.slices) {
    P.sl_off = off;
    P.sl_bytes = dsa::slice_ws_bytes(D, P.Ra);
    off = align256(off + P.sl_bytes);
  } else {
    dsa::attn_pick_splits(D, P.R, P.splits_sparse, P.splits_dense);
    P.part_off = off;
    P.part_bytes = dsa::attn_part_bytes(D, P.R, std::max(P.splits_sparse, P.splits_dense));
    off = align256(off + P.part_bytes);
  }
  P.total = off;
  return P;
}

dsa_status check_ws(const Plan& P, void* ws, size_t ws_bytes) {
  if (P.total == 0) return DSA_OK;
  if (!ws) return fail(DSA_ERR_WORKSPACE, "workspace is null but %zu bytes are needed", P.total);
  if (!aligned16(ws)) return fail(DSA_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
  if (ws_bytes < P.total)
    return fail(DSA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, P.total);
  return DSA_OK;
}

#define DSA_NEED(ptr, name)                                                       \
  do {                                                                            \
    if (!(ptr)) return fail(DSA_ERR_INVALID_ARG, "%s is null", name);             \
    if (!aligned16(ptr)) return fail(DSA_ERR_INVALID_ARG, "%s is not 16-byte aligned", name); \
  } while (0)

dsa_status hip_status(hipError_t e, const char* where) {
  if (e != hipSuccess) return fail(DSA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
  return ok();
}

dsa_status check_router(const dsa_router* r, dsa::RouterArgs& R) {
  if (!r) return fail(DSA_ERR_INVALID_ARG, "router is null");
  if (r->hidden < 1 || r->hidden > 65536)
    return fail(DSA_ERR_INVALID_ARG, "router hidden %d not in [1, 65536]", r->hidden);
  DSA_NEED(r->w1, "router w1");
  DSA_NEED(r->b1, "router b1");
  DSA_NEED(r->w2, "router w2");
  DSA_NEED(r->b2, "router b2");
  R.hidden = r->hidden;
  R.w1 = r->w1; R.b1 = r->b1; R.w2 = r->w2; R.b2 = r->b2;
  return DSA_OK;
}

dsa_status check_gate(const float* gate, const float* y2) {
  if (gate) {
    if (!aligned16(gate)) return fail(DSA_ERR_INVALID_ARG, "gate is not 16-byte aligned");
    DSA_NEED(y2, "y2 (required when gate is given)");
  }
  return DSA_OK;
}

}  // namespace

namespace dsa {

dsa_status fused_ws_need(const dsa_problem* p, size_t* bytes) {
  dsa::Dims D;
  dsa_status st = check_problem(p, D);
  if (st != DSA_OK) return st;
  *bytes = is_empty(D) ? 0 : plan_fused(D).total;
  return ok();
}

dsa_status report(dsa_status st, const char* msg) {
  if (st == DSA_OK) return ok();
  return fail(st, "%s", msg);
}

}  // namespace dsa

extern "C" {

dsa_status dsa_workspace_size(const dsa_problem* p, size_t* bytes) {
  dsa::Dims D;
  dsa_status st = check_problem(p, D);
  if (st != DSA_OK) return st;
  if (!bytes) return fail(DSA_ERR_INVALID_ARG, "bytes is null");
  if (is_empty(D)) {
    *bytes = 0;
    return ok();
  }
  size_t need = std::max({plan_topk(D).total, plan_attn(D).total, plan_fused(D, false).total});
  if (D.N <= 4)  // the single-launch decode plan, for any grid size
    need = std::max(need, align256(dsa::decode_ws_bound(D)) +
                              align256((size_t)D.B * D.N * D.K * sizeof(int32_t)));
  *bytes = need;
  return ok();
}

dsa_status dsa_indexer_scores(const dsa_problem* p, const void* q_idx, const void* k_idx,
                              float* scores, void* stream) {
  dsa::Dims D;
  dsa_status st = check_problem(p, D);
  if (st != DSA_OK) return st;
  if (is_empty(D)) return ok();
  DSA_NEED(q_idx, "q_idx");
  DSA_NEED(k_idx, "k_idx");
  DSA_NEED(scores, "scores");
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  const int rows = D.N * D.IH;   // index rows per sequence
  if (few_index_rows(D))
    e = dsa::launch_indexer_scan(D, q_idx, k_idx, 0, rows, D.L, scores, (size_t)D.L, true, nullptr, s);
  else
    e = dsa::launch_indexer_tiles(D, q_idx, k_idx, 0, rows, D.L, scores, (size_t)D.L, true, nullptr, s);
  return hip_status(e, "dsa_indexer_scores");
}

dsa_status dsa_topk(const dsa_problem* p, const float* scores, int32_t* topk_idx, void* ws,
                    size_t ws_bytes, void* stream) {
  dsa::Dims D;
  dsa_status st = check_problem(p, D);
  if (st != DSA_OK) return st;
  if (is_empty(D)) return ok();
  DSA_NEED(scores, "scores");
  DSA_NEED(topk_idx, "topk_idx");
  const Plan P = plan_topk(D);
  if ((st = check_ws(P, ws, ws_bytes)) != DSA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  const int rows = D.N * D.IH;   // index rows per sequence
  if (P.decode)
    e = dsa::launch_topk_split(D, scores, (size_t)D.L, 0, rows, topk_idx, rows, 0, nullptr,
                               (char*)ws + P.tk_off, s);
  else
    e = dsa::launch_topk_rows(D, scores, (size_t)D.L, 0, rows, topk_idx, rows, 0, nullptr, s);
  return hip_status(e, "dsa_topk");
}

dsa_status dsa_sparse_attn(const dsa_problem* p, const void* q, const void* k, const void* v,
                           const int32_t* topk_idx, const float* gate, const float* y2,
                           const uint8_t* route, float* out, void* ws, size_t ws_bytes,
                           void* stream) {
  dsa::Dims D;
  dsa_status st = check_problem(p, D);
  if (st != DSA_OK) return st;
  if (is_empty(D)) return ok();
  DSA_NEED(q, "q");
  DSA_NEED(k, "k");
  DSA_NEED(v, "v");
  DSA_NEED(topk_idx, "topk_idx");
  DSA_NEED(out, "out");
  if ((st = check_gate(gate, y2)) != DSA_OK) return st;
  const Plan P = plan_attn(D);
  if ((st = check_ws(P, ws, ws_bytes)) != DSA_OK) return st;
  if (P.slices) {
    hipError_t e = hipSuccess;
    for (int n0 = 0; n0 < D.N && e == hipSuccess; n0 += P.Ra) {
      dsa::AttnArgs a{};
      a.q = q; a.k = k; a.v = v;
      a.topk = topk_idx; a.idx_rows_per_b = D.N; a.idx_n_base = 0;
      a.gate = gate; a.y2 = y2; a.route = route; a.out = out;
      a.n0 = n0; a.R = std::min(P.Ra, D.N - n0);
      e = dsa::launch_attention_slices(D, a, (char*)ws + P.sl_off, (hipStream_t)stream);
    }
    return hip_status(e, "dsa_sparse_attn");
  }
  dsa::AttnArgs a{};
  a.q = q; a.k = k; a.v = v;
  a.topk = topk_idx; a.idx_rows_per_b = D.N; a.idx_n_base = 0;
  a.gate = gate; a.y2 = y2; a.route = route; a.out = out;
  a.part = P.part_bytes ? (float*)((char*)ws + P.part_off) : nullptr;
  a.n0 = 0; a.R = D.N;
  a.splits_sparse = P.splits_sparse;
  a.splits_dense = P.splits_dense;
  if (D.N > kDecodeRows && dsa::mfma_attention_supported(D))
    return hip_status(dsa::launch_attention_mfma(D, a, (hipStream_t)stream), "dsa_sparse_attn");
  return hip_status(dsa::launch_attention(D, a, (hipStream_t)stream), "dsa_sparse_attn");
}

dsa_status dsa_fused_forward(const dsa_problem* p, const void* q_idx, const void* k_idx,
                             const void* q, const void* k, const void* v, const float* gate,
                             const float* y2, const uint8_t* route, float* out,
                             int32_t* topk_idx_out, void* ws, size_t ws_bytes, void* stream) {
  dsa::Dims D;
  dsa_status st = check_problem(p, D);
  if (st != DSA_OK) return st;
  if (is_empty(D)) return ok();
  DSA_NEED(q_idx, "q_idx");
  DSA_NEED(k_idx, "k_idx");
  DSA_NEED(q, "q");
  DSA_NEED(k, "k");
  DSA_NEED(v, "v");
  DSA_NEED(out, "out");
  if (topk_idx_out && !aligned16(topk_idx_out))
    return fail(DSA_ERR_INVALID_ARG, "topk_idx_out is not 16-byte aligned");
  if (route && !aligned16(route)) return fail(DSA_ERR_INVALID_ARG, "route is not 16-byte aligned");
  if ((st = check_gate(gate, y2)) != DSA_OK) return st;
  const Plan P = plan_fused(D);
  if ((st = check_ws(P, ws, ws_bytes)) != DSA_OK) return st;

  hipStream_t s = (hipStream_t)stream;
  char* w = (char*)ws;
  if (P.fused_decode) {
    // the decode control block (and its error word) sits at the workspace start
    int32_t* list = topk_idx_out ? topk_idx_out : (int32_t*)(w + P.idx_off);
    return hip_status(dsa::launch_decode(D, P.dp, q_idx, k_idx, q, k, v, gate, y2, route, out,
                                         list, w + P.dec_off, s),
                      "dsa_fused_forward");
  }
  dsa::forget_launch(ws);
  float* scores = (float*)(w + P.scores_off);
  int32_t* idx_chunk = (int32_t*)(w + P.idx_off);
  hipError_t e = hipSuccess;
  if (P.slices) {
    // all index rows of an attention launch first (indexer and top-k per
    // chunk of score rows), then one launch for both routes over them
    for (int na = 0; na < D.N && e == hipSuccess; na += P.Ra) {
      const int Rc = std::min(P.Ra, D.N - na);
      int32_t* idx = topk_idx_out ? topk_idx_out : idx_chunk;
      const int rows_per_b = topk_idx_out ? D.N : P.Ra;
      const int n_base = topk_idx_out ? 0 : na;
      // the indexer and top-k count index rows (IH per token)
      const int H = D.IH;
      if (P.onchip) {
        for (int n0 = na; n0 < na + Rc && e == hipSuccess; n0 += P.Rs) {
          const int R = std::min(P.Rs, na + Rc - n0);
          e = dsa::launch_idx_topk(D, q_idx, k_idx, n0 * H, R * H, idx, rows_per_b * H,
                                   n_base * H, route, w + P.it_off, s);
        }
      } else {
        for (int n0 = na; n0 < na + Rc && e == hipSuccess; n0 += P.R) {
          const int R = std::min(P.R, na + Rc - n0);
          const int ncols = D.L - D.N + n0 + R;  // keys visible to the last row of the chunk
          e = dsa::launch_indexer_tiles(D, q_idx, k_idx, n0 * H, R * H, ncols, scores, P.ld, false,
                                        route, s);
          if (e == hipSuccess)
            e = dsa::launch_topk_rows(D, scores, P.ld, n0 * H, R * H, idx, rows_per_b * H,
                                      n_base * H, route, s);
        }
      }
      if (e != hipSuccess) break;
      dsa::AttnArgs a{};
      a.q = q; a.k = k; a.v = v;
      a.topk = idx; a.idx_rows_per_b = rows_per_b; a.idx_n_base = n_base;
      a.gate = gate; a.y2 = y2; a.route = route; a.out = out;
      a.n0 = na; a.R = Rc;
      e = dsa::launch_attention_slices(D, a, w + P.sl_off, s);
    }
    return hip_status(e, "dsa_fused_forward");
  }
  float* part = P.part_bytes ? (float*)(w + P.part_off) : nullptr;
  for (int n0 = 0; n0 < D.N && e == hipSuccess; n0 += P.R) {
    const int R = std::min(P.R, D.N - n0);
    const int ncols = D.L - D.N + n0 + R;  // keys visible to the last row of the chunk
    int32_t* idx = topk_idx_out ? topk_idx_out : idx_chunk;
    const int rows_per_b = topk_idx_out ? D.N : R;
    const int n_base = topk_idx_out ? 0 : n0;
    const int H = D.IH;   // index rows per token in the indexer and top-k
    if (P.decode) {
      e = dsa::launch_indexer_scan(D, q_idx, k_idx, n0 * H, R * H, ncols, scores, P.ld, false,
                                   route, s);
      if (e == hipSuccess)
        e = dsa::launch_topk_split(D, scores, P.ld, n0 * H, R * H, idx, rows_per_b * H,
                                   n_base * H, route, w + P.tk_off, s);
    } else {
      e = dsa::launch_indexer_tiles(D, q_idx, k_idx, n0 * H, R * H, ncols, scores, P.ld, false,
                                    route, s);
      if (e == hipSuccess)
        e = dsa::launch_topk_rows(D, scores, P.ld, n0 * H, R * H, idx, rows_per_b * H,
                                  n_base * H, route, s);
    }
    if (e != hipSuccess) break;
    dsa::AttnArgs a{};
    a.q = q; a.k = k; a.v = v;
    a.topk = idx; a.idx_rows_per_b = rows_per_b; a.idx_n_base = n_base;
    a.gate = gate; a.y2 = y2; a.route = route; a.out = out; a.part = part;
    a.n0 = n0; a.R = R;
    a.splits_sparse = P.splits_sparse;
    a.splits_dense = P.splits_dense;
    if (D.N > kDecodeRows && dsa::mfma_attention_supported(D)) {
      a.sparse_heads_per_item = sparse_heads_per_item(D);
      e = dsa::launch_attention_mfma(D, a, s);
    } else {
      e = dsa::launch_attention(D, a, s);
    }
  }
  return hip_status(e, "dsa_fused_forward");
}

dsa_status dsa_route_workspace_size(const dsa_problem* p, const dsa_router* r, size_t* bytes) {
  dsa::Dims D;
  dsa_status st = check_problem(p, D);
  if (st != DSA_OK) return st;
  dsa::RouterArgs R;
  if ((st = check_router(r, R)) != DSA_OK) return st;
  if (!bytes) return fail(DSA_ERR_INVALID_ARG, "bytes is null");
  size_t fwd = 0;   // what every other entry point accepts, the forward included
  if ((st = dsa_workspace_size(p, &fwd)) != DSA_OK) return st;
  *bytes = is_empty(D) ? 0 : std::max(dsa::route_ws_bytes(D, R.hidden), fwd);
  return ok();
}

dsa_status dsa_route_heads(const dsa_problem* p, const dsa_router* r, const void* k,
                           uint8_t* route, float* logits, void* ws, size_t ws_bytes,
                           void* stream) {
  dsa::Dims D;
  dsa_status st = check_problem(p, D);
  if (st != DSA_OK) return st;
  dsa::RouterArgs R;
  if ((st = check_router(r, R)) != DSA_OK) return st;
  if (is_empty(D)) return ok();
  DSA_NEED(k, "k");
  if (!route) return fail(DSA_ERR_INVALID_ARG, "route is null");
  if (logits && !aligned16(logits)) return fail(DSA_ERR_INVALID_ARG, "logits is not 16-byte aligned");
  Plan P;
  P.total = dsa::route_ws_bytes(D, R.hidden);
  if ((st = check_ws(P, ws, ws_bytes)) != DSA_OK) return st;
  return hip_status(dsa::launch_route(D, R, k, route, logits, ws, (hipStream_t)stream),
                    "dsa_route_heads");
}

dsa_status dsa_fused_forward_routed(const dsa_problem* p, const dsa_router* r, const void* q_idx,
                                    const void* k_idx, const void* q, const void* k,
                                    const void* v, const float* gate, const float* y2,
                                    uint8_t* route_out, float* out, int32_t* topk_idx_out,
                                    void* ws, size_t ws_bytes, void* stream) {
  dsa::Dims D;
  dsa_status st = check_problem(p, D);
  if (st != DSA_OK) return st;
  dsa::RouterArgs R;
  if ((st = check_router(r, R)) != DSA_OK) return st;
  if (is_empty(D)) return ok();
  DSA_NEED(route_out, "route_out");
  DSA_NEED(k, "k");
  // every check of the forward runs before the router is enqueued
  size_t need = 0;
  if ((st = dsa::fused_ws_need(p, &need)) != DSA_OK) return st;
  Plan P;
  P.total = std::max(dsa::route_ws_bytes(D, R.hidden), need);
  if ((st = check_ws(P, ws, ws_bytes)) != DSA_OK) return st;
  DSA_NEED(q_idx, "q_idx");
  DSA_NEED(k_idx, "k_idx");
  DSA_NEED(q, "q");
  DSA_NEED(v, "v");
  DSA_NEED(out, "out");
  if (topk_idx_out && !aligned16(topk_idx_out))
    return fail(DSA_ERR_INVALID_ARG, "topk_idx_out is not 16-byte aligned");
  if ((st = check_gate(gate, y2)) != DSA_OK) return st;
  hipError_t e = dsa::launch_route(D, R, k, route_out, nullptr, ws, (hipStream_t)stream);
  if (e != hipSuccess) return hip_status(e, "dsa_fused_forward_routed");
  return dsa_fused_forward(p, q_idx, k_idx, q, k, v, gate, y2, route_out, out, topk_idx_out, ws,
                           ws_bytes, stream);
}

dsa_status dsa_exec_status(const void* ws, void* stream) {
  if (!ws) return fail(DSA_ERR_INVALID_ARG, "workspace is null");
  hipError_t e;
  const int gave_up = dsa::decode_exec_status(ws, (hipStream_t)stream, &e);
  if (e != hipSuccess) return fail(DSA_ERR_HIP, "dsa_exec_status: %s", hipGetErrorString(e));
  if (gave_up)
    return fail(DSA_ERR_EXEC,
                "the last decode launch on this workspace gave up waiting for its workgroups "
                "(other work kept some of them from running); its outputs are NaN");
  return ok();
}

void dsa_set_wait_limit(uint32_t polls) { dsa::set_wait_limit(polls); }

dsa_status dsa_profile_start(int32_t max_launches) {
  if (max_launches < 1 || max_launches > (1 << 20))
    return fail(DSA_ERR_INVALID_ARG, "max_launches %d not in [1, 2^20]", max_launches);
  return hip_status(dsa::prof_start(max_launches), "dsa_profile_start");
}

dsa_status dsa_profile_stop(double* ms, int32_t* launches, int32_t n_stages, int64_t* dropped) {
  if (n_stages < 0) return fail(DSA_ERR_INVALID_ARG, "n_stages is negative");
  long long d = 0;
  const hipError_t e = dsa::prof_stop(ms, launches, n_stages, &d);
  if (dropped) *dropped = d;
  return hip_status(e, "dsa_profile_stop");
}

const char* dsa_last_error(void) { return g_err.c_str(); }

}  // extern "C"
