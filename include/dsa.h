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
 * 0..p (bottom-right causal alignment, own key included).  One indexer key
 * per position.  With idx_heads H <= 1 there is one indexer query per token
 * and the selected set is shared by all heads of the token ([GDSA] §二.1).
 * With H > 1 ([GDSA] §四.1, whose scores and indices carry a head axis) each
 * token has H indexer queries, indexer head i selects its own set from its
 * own scores, and query head h attends over set h / (Hq / H).  Query head h
 * reads key/value head h / (Hq / Hkv).
 *
 * Layouts (all row-major, contiguous, every pointer 16-byte aligned):
 *   q_idx  [B, N, H, d_idx]   qidx dtype (fp32 or bf16); H = max(1, idx_heads)
 *   k_idx  [B, L, d_idx]      qidx dtype
 *   q      [B, N, Hq, d]      qkv dtype
 *   k, v   [B, L, Hkv, d]     qkv dtype (token-major: one selected position
 *                             is one contiguous Hkv*d row)
 *   scores [B, N, H, L]       float32
 *   topk   [B, N, H, K]       int32, ascending, -1 padded
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
 *
 * Co-residency.  dsa_fused_forward with at most 4 query rows per sequence
 * (decode) runs as one launch whose workgroups exchange data while they run,
 * so all of them must be resident on the device at once; the grid is sized
 * from the occupancy query to fill the whole device, and the library orders
 * its own such launches across streams.  Other work running on the device at
 * the same time (another stream of the caller, another process) can keep
 * some workgroups from starting.  Every wait between workgroups is bounded:
 * a wait that gives up makes the outputs of its sequence NaN and its index
 * rows -1, and dsa_exec_status() then returns DSA_ERR_EXEC.
 *
 * Stream capture.  The entry points enqueue only kernels (no copies,
 * memsets or allocations), so a call can be captured into a HIP graph after
 * one eager call on the same device (which creates the library's event).
 * A captured single-launch decode adds a one-thread kernel that advances
 * the launch tag on the device, so every replay is a fresh launch; replays
 * of a graph are not ordered by the library against other decode launches.
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
  DSA_ERR_HIP = 4,         /* a launch failed (hipGetLastError)                */
  DSA_ERR_EXEC = 5         /* a launch ran but gave up (see dsa_exec_status)   */
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
  int32_t idx_heads; /* H >= 0 indexer heads; 0 or 1: one set per token shared
                        by all heads; H > 1 (h_q a multiple of H): one set per
                        indexer head, query head h using set h / (h_q / H)   */
} dsa_problem;

/* Bytes of workspace every entry point below accepts for problem *p
 * (the largest need of any of them).  Host-only; enqueues nothing. */
dsa_status dsa_workspace_size(const dsa_problem* p, size_t* bytes);

/* Indexer scores ([GDSA] §二.1-§二.2, [HYB] §三), per indexer head i:
 *   scores[b,n,i,j] = sum_c q_idx[b,n,i,c] * k_idx[b,j,c]  for j <= p,
 *   scores[b,n,i,j] = -inf                                 for j >  p.
 * Plain product, no scale, no rotary term, float32 accumulation (exact for
 * integer-valued inputs whose products sum below 2^24).  Needs no workspace. */
dsa_status dsa_indexer_scores(const dsa_problem* p, const void* q_idx,
                              const void* k_idx, float* scores, void* stream);

/* Top-K per index row ([GDSA] §二.1, [HYB] §三) from scores [B,N,H,L]:
 * the K_eff = min(K, p+1) visible positions with the largest score, ties to
 * the lower position, -0.0 equal to +0.0, written ascending and padded with
 * -1 to K.  Entries of scores beyond p are not read.  Selection compares the
 * float32 bits exactly, so the set is unique. */
dsa_status dsa_topk(const dsa_problem* p, const float* scores, int32_t* topk_idx,
                    void* ws, size_t ws_bytes, void* stream);

/* Attention over the selected rows plus gate ([HYB] §三, [AAM] §2.1,
 * [GDSA] §四.1 steps 3-5, [EA] §2.2):
 *   sparse head (route[b,h] = 1, or route == NULL):
 *     a = softmax_j(q . k_j * scale) v_j over j in topk_idx[b,n,h/(Hq/H),:];
 *     entries outside [0, p] (padding) are skipped; a row with no valid entry
 *     gives a = 0.  Precondition: each index row lists its entries in
 *     [0, p] in ascending order, before any padding (the layout dsa_topk
 *     writes); prefill shapes read each key range's entries as one
 *     contiguous run of the row, so other orders can drop entries;
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

/* dsa_fused_forward for callers that cannot allocate (code under graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * arguments and results, but no workspace argument.  Scratch memory is a
 * fixed 64 MiB device array inside the library (one per device, held until
 * the process ends); problems whose dsa_fused_forward workspace exceeds it
 * are rejected with DSA_ERR_WORKSPACE before anything is enqueued (decode
 * batches fit; long prefills do not).  The call allocates nothing: the
 * array's device address is looked up on the first call made on a device.
 * Every call on a device shares that device's array, so calls that overlap
 * on one device (other streams, other threads) race and must be ordered by
 * the caller.  dsa_exec_status() takes the array's address as `ws`; it is
 * not exposed, so that call does not apply here. */
dsa_status dsa_fused_forward_noalloc(const dsa_problem* p, const void* q_idx,
                                     const void* k_idx, const void* q, const void* k,
                                     const void* v, const float* gate, const float* y2,
                                     const uint8_t* route, float* out,
                                     int32_t* topk_idx_out, void* stream);

/* Weights of the per-head route producer ([EA] §2.2): a two-layer router
 * on the keys of the call's tokens.  Device pointers, fp32, row-major,
 * 16-byte aligned, owned by the caller:
 *   w1 [Hkv*d, hidden], b1 [hidden], w2 [hidden, Hq, 2], b2 [Hq, 2]
 * (last axis: column 0 full attention, column 1 sparse). */
typedef struct {
  int32_t hidden;    /* 1 <= hidden <= 65536 */
  const float* w1;
  const float* b1;
  const float* w2;
  const float* b2;
} dsa_router;

/* Bytes of workspace dsa_route_heads and dsa_fused_forward_routed accept for
 * *p and *r (the larger need of the two).  Host-only; enqueues nothing. */
dsa_status dsa_route_workspace_size(const dsa_problem* p, const dsa_router* r, size_t* bytes);

/* Route producer ([EA] §2.2: the router reads the current key hidden states,
 * is a two-layer MLP and takes one full/sparse decision per head, hard at
 * inference).  For each sequence b:
 *   x = mean of the key rows k[b, j, :, :] (Hkv*d values) over the call's
 *       tokens j = L - N .. L - 1;
 *   z = max(0, x w1 + b1) w2 + b2         ([Hq, 2], fp32 accumulation);
 *   route[b, h] = 1 (sparse) if z[h][1] > z[h][0], else 0 (full; a tie
 *   keeps full attention).
 * k [B, L, Hkv, d] in qkv dtype; route [B, Hq] uint8; logits [B, Hq, 2]
 * float32 (nullable).  The summation order is fixed, so equal inputs give
 * equal decisions. */
dsa_status dsa_route_heads(const dsa_problem* p, const dsa_router* r, const void* k,
                           uint8_t* route, float* logits, void* ws, size_t ws_bytes,
                           void* stream);

/* dsa_route_heads followed on the same stream by dsa_fused_forward with
 * route = route_out: the decision is made on the device and read there by
 * the indexer, top-k and attention launches (no host round trip).
 * route_out [B, Hq] receives the decision (required, 16-byte aligned). */
dsa_status dsa_fused_forward_routed(const dsa_problem* p, const dsa_router* r,
                                    const void* q_idx, const void* k_idx, const void* q,
                                    const void* k, const void* v, const float* gate,
                                    const float* y2, uint8_t* route_out, float* out,
                                    int32_t* topk_idx_out, void* ws, size_t ws_bytes,
                                    void* stream);

/* Execution status of the last dsa_fused_forward on workspace `ws`:
 * synchronises `stream` (the stream that call used), then returns
 * DSA_ERR_EXEC if that call was a single-launch decode and one of its waits
 * between workgroups gave up (its results are not valid; see Co-residency),
 * DSA_ERR_HIP if the synchronisation or the read-back failed, else DSA_OK.
 * Other launch kinds have no waits and always report DSA_OK here.  Host
 * call; blocks until the stream is idle. */
dsa_status dsa_exec_status(const void* ws, void* stream);

/* Number of polls a wait between decode workgroups makes before it gives up
 * (default 16777216, i.e. seconds).  0 makes every such wait give up at
 * once: the failure path is then exercised deterministically (used by the
 * tests).  Process-wide; applies to launches enqueued after the call. */
void dsa_set_wait_limit(uint32_t polls);

/* Stage timing (tracing).  Between dsa_profile_start and dsa_profile_stop,
 * every kernel the entry points enqueue is bracketed by two HIP events on its
 * launch stream (up to max_launches launches; later ones are counted as
 * dropped).  dsa_profile_stop synchronises on those events and returns, per
 * stage, the summed GPU time in milliseconds and the number of launches:
 *   0 indexer scores, 1 top-k selection, 2 attention (both routes),
 *   3 merge of split/range partials, 4 single-launch decode (the whole
 *   path), 5 preparation (range offsets, work queues), 6 route producer.
 * ms and launches have n_stages entries (either may be NULL); dropped
 * (nullable) receives the count of launches not timed.  Host calls; the
 * events are created by start and destroyed by stop. */
#define DSA_PROFILE_STAGES 7
dsa_status dsa_profile_start(int32_t max_launches);
dsa_status dsa_profile_stop(double* ms, int32_t* launches, int32_t n_stages,
                            int64_t* dropped);

/* Message for the last non-OK status on this thread ("" if none). */
const char* dsa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
