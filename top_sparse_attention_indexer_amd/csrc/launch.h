// Host-side launchers of the libdsa kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

struct Dims {
  int B, N, L, Hq, Hkv, d, didx, K;
  bool qkv_bf16, idx_bf16;
  float scale;  // resolved softmax scale (> 0)
};

// ---- indexer ---------------------------------------------------------------
// Scores of query rows [n0, n0 + R) of every sequence into
// out[(b * R + r) * ld + j] for j < ncols.  Masked entries (j > p) are written
// as -inf only if write_masked; tiles that are wholly masked are skipped
// otherwise.  route (nullable) skips sequences whose heads are all dense.
hipError_t launch_indexer_tiles(const Dims& D, const void* q_idx, const void* k_idx,
                                int n0, int R, int ncols, float* out, size_t ld,
                                bool write_masked, const uint8_t* route, hipStream_t s);

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

// ---- misc ------------------------------------------------------------------
hipError_t launch_fill_u32(uint32_t* p, size_t n, uint32_t value, hipStream_t s);

}  // namespace dsa
