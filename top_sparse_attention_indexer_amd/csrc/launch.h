// Host-side launchers of the libdsa kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/dsa.h"

namespace dsa {

struct Dims {
  int B, N, L, Hq, Hkv, d, didx, K;
  bool qkv_bf16, idx_bf16;
  float scale;  // resolved softmax scale (> 0)
  // indexer heads: 1 = one selected set per token shared by every head; IH
  // > 1 = one set per (token, indexer head), query head h using set
  // h / (Hq / IH).  The indexer and top-k stages then work on IH "virtual
  // rows" per token: q_idx row and index row n * IH + i, visible prefix that
  // of token n.  Their n0 / R / index-row arguments count virtual rows.
  int IH = 1;
};

// ---- indexer ---------------------------------------------------------------
// Scores of query rows [n0, n0 + R) of every sequence into
// out[(b * R + r) * ld + j] for j < ncols.  Masked entries (j > p) are written
// as -inf only if write_masked; tiles that are wholly masked are skipped
// otherwise.  route (nullable) skips sequences whose heads are all dense.
hipError_t launch_indexer_tiles(const Dims& D, const void* q_idx, const void* k_idx,
                                int n0, int R, int ncols, float* out, size_t ld,
                                bool write_masked, const uint8_t* route, hipStream_t s);

// Indexer and exact top-K of query rows [n0, n0 + R) without a score matrix
// (bf16 indexer inputs, d_idx in {32, 64, 128}, K <= 2048): MFMA scores
// filtered against a sampled per-row threshold into candidate lists in `ws`
// (idx_topk_ws_bytes), then the exact selection on the lists.  Index rows as
// for launch_topk_rows.
bool idx_topk_supported(const Dims& D);
size_t idx_topk_ws_bytes(const Dims& D, int R);
hipError_t launch_idx_topk(const Dims& D, const void* q_idx, const void* k_idx, int n0, int R,
                           int32_t* topk, int idx_rows_per_b, int idx_n_base,
                           const uint8_t* route, void* ws, hipStream_t s);

// Streaming variant for few query rows per sequence (R <= 8): one thread per
// key, every key row read once for all R rows.
hipError_t launch_indexer_scan(const Dims& D, const void* q_idx, const void* k_idx,
                               int n0, int R, int ncols, float* out, size_t ld,
                               bool write_masked, const uint8_t* route, hipStream_t s);

// ---- top-k -----------------------------------------------------------------
// One workgroup per row: rows r of query rows [n0, n0 + R) of each sequence,
// scores at scores[(b * R + r) * ld]; index row of query n of sequence b at
// topk[(b * idx_rows_per_b + n - idx_n_base) * K].
hipError_t launch_topk_rows(const Dims& D, const float* scores, size_t ld, int n0, int R,
                            int32_t* topk, int idx_rows_per_b, int idx_n_base,
                            const uint8_t* route, hipStream_t s);

// Rows split across workgroups (few, long rows).  Uses `ws` (split_topk_ws_bytes).
size_t split_topk_ws_bytes(const Dims& D, int R);
hipError_t launch_topk_split(const Dims& D, const float* scores, size_t ld, int n0, int R,
                             int32_t* topk, int idx_rows_per_b, int idx_n_base,
                             const uint8_t* route, void* ws, hipStream_t s);

// ---- attention -------------------------------------------------------------
struct AttnArgs {
  const void* q; const void* k; const void* v;
  const int32_t* topk;      // rows at topk[(b * idx_rows_per_b + n - idx_n_base) * K]
  int idx_rows_per_b, idx_n_base;
  const float* gate; const float* y2; const uint8_t* route;
  float* out;
  float* part;              // partials for split keys (nullable when splits == 1)
  int n0, R;                // query rows handled: [n0, n0 + R) of each sequence
  int splits_sparse, splits_dense;
  // MFMA attention only: which work the launch carries (both by default),
  // and how many KV heads one sparse item takes (0: all).  Items run in
  // (sequence, block of KV heads, token) order, so fewer heads per item keep
  // the K/V that the resident workgroups gather cache-sized.
  bool skip_dense = false, skip_sparse = false;
  int sparse_heads_per_item = 0;
};
size_t attn_part_bytes(const Dims& D, int R, int splits);
void attn_pick_splits(const Dims& D, int R, int& splits_sparse, int& splits_dense);
hipError_t launch_attention(const Dims& D, const AttnArgs& a, hipStream_t s);
// bf16 MFMA attention for prefill-shaped calls (both routes in one launch;
// no partials).  Supported for bf16 q/k/v, d in {64, 128}, K <= 2048.
bool mfma_attention_supported(const Dims& D);
hipError_t launch_attention_mfma(const Dims& D, const AttnArgs& a, hipStream_t s);

// bf16 MFMA attention blocked by key range (prefill): both routes in one
// persistent launch whose workgroups take (sequence, KV head, key range)
// slices XCD by XCD, per-range partials merged afterwards.  Needs
// slice_ws_bytes(D, R) of workspace for a launch over R query rows, and index
// rows that are ascending in their valid entries (as dsa_topk writes them).
constexpr int kSliceKeys = 8192;    // keys per range
struct SlicePlan {
  int RC = 0;    // keys per range
  int NC = 0;    // ranges of the longest row
  int cap = 0;   // slices per XCD queue table
};
SlicePlan slice_plan(const Dims& D, int R);
size_t slice_ws_bytes(const Dims& D, int R);
bool slice_attention_supported(const Dims& D);
hipError_t launch_attention_slices(const Dims& D, const AttnArgs& a, void* ws, hipStream_t s);

// ---- fused decode (one cooperative launch) ----------------------------------
struct DecodePlan {
  int grid = 0;      // co-resident workgroups
  int CH = 0;        // keys per chunk (one chunk per workgroup)
  int nch = 0;       // chunks per sequence
  int S = 1;         // attention key splits
  int nhc = 1;       // head chunks per KV head
  int cand_cap = 0;  // candidate slots per row (histogram selection)
  int M = 0;         // candidates per chunk for the one-exchange selection (0: not used)
  int Cpad = 0;      // candidate slots per row for it (nch * M, padded)
};
// Co-resident grid for the decode kernel of these dims on the current device
// (0 if it cannot be determined, e.g. without a GPU).
int decode_grid(const Dims& D);
bool decode_plan(const Dims& D, int grid, DecodePlan& P);
size_t decode_ws_bytes(const Dims& D, const DecodePlan& P);
// Upper bound of decode_ws_bytes over every grid size.
size_t decode_ws_bound(const Dims& D);
hipError_t launch_decode(const Dims& D, const DecodePlan& P, const void* q_idx, const void* k_idx,
                         const void* q, const void* k, const void* v, const float* gate,
                         const float* y2, const uint8_t* route, float* out, int32_t* list,
                         void* ws, hipStream_t s);

// Failure reporting of the decode kernel: every wait between its workgroups
// is bounded by a number of polls (kDefaultWaitLimit unless changed; 0 makes
// every wait give up at once).  decode_exec_status synchronises `s` and
// returns 1 if the last decode launch on workspace `ws` gave up, else 0
// (also when no decode launch used `ws`); forget_launch drops that record.
constexpr uint32_t kDefaultWaitLimit = 1u << 24;
void set_wait_limit(uint32_t polls);
int decode_exec_status(const void* ws, hipStream_t s, hipError_t* err);
void forget_launch(const void* ws);
// Creates, on the current device, what the first decode launch would
// otherwise create (the cross-stream ordering event).
hipError_t decode_setup();

// ---- route producer (route.hip) -----------------------------------------------
// Weights of the two-layer router (device pointers, fp32): W1 [Hkv*d, hidden],
// b1 [hidden], W2 [hidden, Hq, 2], b2 [Hq, 2] (column 0 full, 1 sparse).
struct RouterArgs {
  int hidden;
  const float *w1, *b1, *w2, *b2;
};
size_t route_ws_bytes(const Dims& D, int hidden);
// route [B, Hq] (1 = sparse) and, if logits != nullptr, logits [B, Hq, 2]
// from the keys k [B, L, Hkv, d] of the last N positions of each sequence.
hipError_t launch_route(const Dims& D, const RouterArgs& r, const void* k, uint8_t* route,
                        float* logits, void* ws, hipStream_t s);

// ---- stage timing (dsa_profile_start / dsa_profile_stop) -----------------------
enum Stage { kStageIndexer = 0, kStageTopk = 1, kStageAttention = 2, kStageMerge = 3,
             kStageDecode = 4, kStagePrep = 5, kStageRoute = 6, kStages = 7 };
void prof_begin(hipStream_t s, int stage);
void prof_end(hipStream_t s);
hipError_t prof_start(int max_launches);
hipError_t prof_stop(double* ms, int32_t* launches, int n_stages, long long* dropped);
// Marks the launches enqueued during its lifetime as one timed launch of `stage`.
struct ProfScope {
  hipStream_t s;
  ProfScope(hipStream_t s_, int stage) : s(s_) { prof_begin(s, stage); }
  ~ProfScope() { prof_end(s); }
};

// ---- entry-point helpers (dsa_api.cpp) -----------------------------------------
// Workspace bytes dsa_fused_forward needs for *p (checks *p like the entry
// points; the plan the call will take, including the single-launch decode).
dsa_status fused_ws_need(const dsa_problem* p, size_t* bytes);
// Sets the thread's last-error message and returns st.
dsa_status report(dsa_status st, const char* msg);

// ---- misc ------------------------------------------------------------------
hipError_t launch_fill_u32(uint32_t* p, size_t n, uint32_t value, hipStream_t s);

}  // namespace dsa
