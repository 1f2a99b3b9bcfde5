/*
 * dsa.h — C ABI of libdsa.so: indexer + top-k sparse attention with a gate
 * blend and a per-head full/sparse route, for AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages, cited by title and section):
 *   [EA]   "Elastic Attention：动态路由优化大模型长文本处理"
 *          §2.2 per-head route decision, §3.1 one fused op for both routes.
 *   [GDSA] "超大规模MoE架构中稀疏注意力机制的演进与实践"
 *          §二.1 indexer + top-K (K = 2048), §二.2 no RoPE in the indexer,
 *          §二.3 gate, §四.1 pseudo-code of the gated sparse forward.
 *   [HYB]  "混合注意力架构演进：从线性注意力到稀疏门控的技术权衡"
 *          §三 indexer scores -> top-k index array [L, top_k] -> gather ->
 *          softmax(Q K_sel^T / sqrt(d)) V_sel; §五.5 fallback to full attention.
 *   [AAM]  "Advanced Attention Mechanisms" article (wmrh.cn)
 *          §2.1 scaled dot-product attention and the causal mask,
 *          §3.2 tiled attention with online normalisation, §3.4 sigmoid gate.
 *
 * Problem.  B sequences; each has L keys and its last N positions are the
 * queries (N <= L).  Query row n sits at position p = L - N + n and sees keys
 * 0..p (bottom-right causal alignment, own key included).  One indexer query
 * per token and one indexer key per position: the selected set is shared by
 * all heads of a token.  Query head h reads key/value head h / (Hq / Hkv).
 *
 * Layouts (all row-major, contiguous, every pointer 16-byte aligned):
 *   q_idx  [B, N, d_idx]      qidx dtype (fp32 or bf16)
 *   k_idx  [B, L, d_idx]      qidx dtype
 *   q      [B, N, Hq, d]      qkv dtype
 *   k, v   [B, L, Hkv, d]     qkv dtype (token-major: one selected position
 *                             is one contiguous Hkv*d row)
 *   scores [B, N, L]          float32
 *   topk   [B, N, K]          int32, ascending, -1 padded
 *   gate   [B, N, Hq]         float32, post-sigmoid g in [0, 1]
 *   y2     [B, N, Hq, d]      float32 second-branch output
 *   route  [B, Hq]            uint8, 1 = top-k sparse, 0 = full causal
 *   out    [B, N, Hq, d]      float32
 * bf16 tensors are passed as their 16-bit patterns.
 *
 * Ownership.  Every tensor pointer is device memory owned by the caller; the
 * library allocates nothing, frees nothing and keeps no pointer after a call
 * returns.  Scratch memory is the caller's workspace (size from
 * dsa_workspace_size).  `stream` is a hipStream_t (NULL = the null stream).
 * Calls only enqueue work: they never synchronise or copy to the host.
 *
 * Errors.  All checks run before anything is enqueued; on a non-OK status
 * nothing was enqueued and dsa_last_error() (thread-local) says why.
 * Execution faults surface at the caller's next synchronisation.  Calls are
 * re-entrant across threads and streams if their workspaces are distinct.
 * Preconditions the library cannot check: finite inputs (NaN/Inf give
 * undefined selections); device pointers of the stated sizes.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = 1, /* null required pointer, bad size, misalignment   */
  DSA_ERR_UNSUPPORTED = 2, /* head_dim / idx_dim / dtype outside the built set */
  DSA_ERR_WORKSPACE = 3,   /* workspace pointer null or smaller than needed    */
  DSA_ERR_HIP = 4          /* a launch failed (hipGetLastError)                */
} dsa_status;

typedef enum { DSA_FP32 = 0, DSA_BF16 = 1 } dsa_dtype;

typedef struct {
  int32_t batch;     /* B >= 0 (0 makes every call a no-op)                   */
  int32_t n_q;       /* N >= 0 query tokens per sequence (0: no-op)           */
  int32_t kv_len;    /* L >= N, L >= 1 keys per sequence                      */
  int32_t h_q;       /* Hq >= 1, a multiple of h_kv                           */
  int32_t h_kv;      /* Hkv >= 1                                              */
  int32_t head_dim;  /* d in {64, 128}                                        */
  int32_t idx_dim;   /* d_idx in {16, 32, 64, 128}                            */
  int32_t top_k;     /* K >= 1; rows with at most K visible keys keep them all */
  int32_t qkv_dtype; /* dsa_dtype of q, k, v                                  */
  int32_t idx_dtype; /* dsa_dtype of q_idx, k_idx                             */
  float softmax_scale; /* <= 0 selects 1 / sqrt(head_dim)                     */
} dsa_problem;

/* Bytes of workspace every entry point below accepts for problem *p
 * (the largest need of any of them).  Host-only; enqueues nothing. */
dsa_status dsa_workspace_size(const dsa_problem* p, size_t* bytes);

/* Indexer scores ([GDSA] §二.1-§二.2, [HYB] §三):
 *   scores[b,n,j] = sum_c q_idx[b,n,c] * k_idx[b,j,c]  for j <= p,
 *   scores[b,n,j] = -inf                               for j >  p.
 * Plain product, no scale, no rotary term, float32 accumulation (exact for
 * integer-valued inputs whose products sum below 2^24).  Needs no workspace. */
dsa_status dsa_indexer_scores(const dsa_problem* p, const void* q_idx,
                              const void* k_idx, float* scores, void* stream);

/* Top-K per query row ([GDSA] §二.1, [HYB] §三) from scores [B,N,L]:
 * the K_eff = min(K, p+1) visible positions with the largest score, ties to
 * the lower position, -0.0 equal to +0.0, written ascending and padded with
 * -1 to K.  Entries of scores beyond p are not read.  Selection compares the
 * float32 bits exactly, so the set is unique. */
dsa_status dsa_topk(const dsa_problem* p, const float* scores, int32_t* topk_idx,
                    void* ws, size_t ws_bytes, void* stream);

/* Attention over the selected rows plus gate ([HYB] §三, [AAM] §2.1,
 * [GDSA] §四.1 steps 3-5, [EA] §2.2):
 *   sparse head (route[b,h] = 1, or route == NULL):
 *     a = softmax_j(q . k_j * scale) v_j over j in topk_idx[b,n,:];
 *     entries outside [0, p] (padding) are skipped; a row with no valid entry
 *     gives a = 0;
 *   dense head (route[b,h] = 0): the same over every j in 0..p, topk ignored;
 *   out = g*a + (1-g)*y2 with g = gate[b,n,h]; gate == NULL gives out = a
 *   (y2 may then be NULL).
 * float32 accumulation for bf16 and fp32 inputs. */
dsa_status dsa_sparse_attn(const dsa_problem* p, const void* q, const void* k,
                           const void* v, const int32_t* topk_idx,
                           const float* gate, const float* y2,
                           const uint8_t* route, float* out,
                           void* ws, size_t ws_bytes, void* stream);

/* The whole path in one call ([GDSA] §四.1): indexer, top-k, gather,
 * attention, gate, with the route of dsa_sparse_attn.  topk_idx_out
 * (nullable) receives the index rows; sequences whose heads are all dense
 * skip the indexer and top-k and get index rows of -1. */
dsa_status dsa_fused_forward(const dsa_problem* p, const void* q_idx,
                             const void* k_idx, const void* q, const void* k,
                             const void* v, const float* gate, const float* y2,
                             const uint8_t* route, float* out,
                             int32_t* topk_idx_out, void* ws, size_t ws_bytes,
                             void* stream);

/* Message for the last non-OK status on this thread ("" if none). */
const char* dsa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
