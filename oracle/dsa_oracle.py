"""CPU oracle for indexer + top-k sparse attention with gate and per-head route.

TEST INFRASTRUCTURE ONLY.  This module is imported by the tests, by the smoke
check and by the bench's CPU-baseline leg, and by nothing else.  The HIP
library shares no code with it, and it imports nothing from the product.

It is the plain definition, written out slowly in float64 with numpy, one
query row at a time.  Sources are web pages, cited by title and section:

  [EA]   "Elastic Attention：动态路由优化大模型长文本处理"
         §2.2 per-head router decision (full or sparse), §3.1 one fused op
         carrying both kinds of head.
  [GDSA] "超大规模MoE架构中稀疏注意力机制的演进与实践"
         §二.1 indexer + top-K with K = 2048, §二.2 indexer without RoPE,
         §二.3 learned gate, §四.1 pseudo-code of the gated sparse forward
         (indexer product, top-k, gather of keys and values, scaled
         dot-product attention, gate blend with the linear branch).
  [HYB]  "混合注意力架构演进：从线性注意力到稀疏门控的技术权衡"
         §三 two-stage sparse forward (indexer scores, top-k index array of
         shape [L, top_k] shared by the heads, gather, softmax(Q K_sel^T /
         sqrt(d)) V_sel), §五.5 keep a switch back to full attention.
  [AAM]  the "Advanced Attention Mechanisms" article (wmrh.cn)
         §2.1 scaled dot-product attention and the lower-triangular causal
         mask, §3.4 a gate g = sigmoid(W x) in [0, 1] blending two branches.

Readings taken where the pages are silent (each is listed with its reason in
the design notes of the repository):
  * bottom-right causal alignment: query row n of N sits at absolute position
    p = L - N + n and sees keys 0..p (its own key included);
  * one indexer query per token and one indexer key per position, so the
    selected set is shared by every head of the token ([HYB] §三); or, with
    idx_heads > 1, one indexer query per (token, indexer head) and one set
    per indexer head, query head h using set h // (Hq / idx_heads)
    ([GDSA] §四.1 pseudo-code, top-k indices [batch, heads, top_k]);
  * the indexer score is a plain dot product (no scale, no RoPE, [GDSA] §二.2);
  * ties at the K-th score go to the lower position; -0.0 equals +0.0;
  * if the visible count is <= K every visible key is selected; index rows
    are ascending and padded with -1;
  * softmax scale 1/sqrt(d) unless given; query head h reads KV head
    h // (Hq / Hkv);
  * gate given post-sigmoid, blended as g*a + (1-g)*y2 for both routes;
  * route[b, h] = 1 means top-k sparse, 0 means full causal attention;
  * the route producer ([EA] §2.2): the router's input is the mean over the
    tokens of the call (positions L - N .. L - 1) of their keys, one vector
    of Hkv * d; the 2-layer MLP is linear, ReLU, linear with two logits per
    query head (column 0 full, column 1 sparse); inference takes the hard
    decision of the Gumbel-Softmax/straight-through training, the larger
    logit, a tie going to full attention.

Pins (tests, CPU): closed forms for the indexer, brute force over all
subsets for tiny top-k rows plus the closed-form orderings, the special case
K >= visible against torch's scaled_dot_product_attention in float64 (and a
boolean-mask SDPA for the sparse case), hand-derived worked examples under
tests/golden, the exact gate end points, and for the router a hand-derived
example (ReLU cut, bias, tie), invariances and torch's linear layers in
float64.  Nothing here is unpinned.
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence, Tuple

import numpy as np


def visible_count(n: int, n_q: int, kv_len: int) -> int:
    """Keys visible to query row n: bottom-right causal alignment.

    [AAM] §2.1: a query sees only its left context (lower-triangular mask).
    With N queries that are the last N of L positions, row n sits at
    p = L - N + n and sees positions 0..p.
    """
    return kv_len - n_q + n + 1


def indexer_scores(q_idx_row: np.ndarray, k_idx_seq: np.ndarray, vis: int) -> np.ndarray:
    """Indexer scores of one query token against its visible keys.

    [GDSA] §二.1/§二.2 and [HYB] §三: a cheap relevance score of the query
    against every historical position, a plain product with no rotary term.
    s[j] = sum_c q_idx[c] * k_idx[j, c] for j < vis, in float64.
    """
    q = q_idx_row.astype(np.float64)
    k = k_idx_seq[:vis].astype(np.float64)
    return k @ q


def select_top_k(scores: np.ndarray, top_k: int) -> np.ndarray:
    """The top-K positions of one row, ascending, padded with -1.

    [GDSA] §二.1: keep the K highest-scoring historical positions (at most K
    whatever the context length).  Order used: score descending, position
    ascending (ties go to the lower position); if the row has at most K
    entries all of them are kept.
    """
    vis = scores.shape[0]
    out = np.full(top_k, -1, dtype=np.int64)
    if vis <= top_k:
        out[:vis] = np.arange(vis)
        return out
    positions = np.arange(vis)
    # np.lexsort sorts by the last key first: -score ascending, then position.
    order = np.lexsort((positions, -scores))
    out[:] = np.sort(order[:top_k])
    return out


def softmax_attention(q_vec: np.ndarray, keys: np.ndarray, values: np.ndarray,
                      scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """softmax(q . k_j * scale) weighted sum of v_j, two-pass, float64.

    [HYB] §三 and [AAM] §2.1: softmax(Q K^T / sqrt(d)) V over the given rows.
    Returns the output vector and the weights.
    """
    t = (keys.astype(np.float64) @ q_vec.astype(np.float64)) * scale
    m = np.max(t)
    e = np.exp(t - m)
    w = e / np.sum(e)
    return w @ values.astype(np.float64), w


def gate_blend(a: np.ndarray, g: float, y2: np.ndarray) -> np.ndarray:
    """[GDSA] §四.1 step 5 and [AAM] §3.4: g * attention + (1 - g) * other."""
    return g * a + (1.0 - g) * y2.astype(np.float64)


def forward_row(b: int, n: int, *, n_q: int, kv_len: int, h_q: int, h_kv: int,
                head_dim: int, top_k: int, q_idx: np.ndarray, k_idx: np.ndarray,
                q: np.ndarray, k: np.ndarray, v: np.ndarray,
                gate: Optional[np.ndarray] = None, y2: Optional[np.ndarray] = None,
                route: Optional[np.ndarray] = None,
                softmax_scale: Optional[float] = None,
                idx_heads: int = 1) -> Tuple[np.ndarray, np.ndarray]:
    """The whole path for query token (b, n): returns (out [Hq, d], idx).

    Steps in the order of [GDSA] §四.1: indexer scores, top-k, gather of the
    selected key/value rows, attention per head, gate blend.  Heads with
    route 0 attend to every visible key instead ([EA] §2.2, [HYB] §五.5).
    Rows whose heads are all dense skip the indexer; their index row is -1.

    idx_heads = 1: one indexer query per token (q_idx [B, N, d_idx]) and one
    selected set shared by every head; idx is [K].  idx_heads = H > 1: the
    per-head selection of the [GDSA] §四.1 pseudo-code (scores and top-k
    indices carry a head axis): q_idx is [B, N, H, d_idx], indexer head i
    selects its own set from its own scores against the shared k_idx, and
    query head h uses set h // (Hq / H); idx is [H, K].
    """
    vis = visible_count(n, n_q, kv_len)
    scale = 1.0 / math.sqrt(head_dim) if not softmax_scale or softmax_scale <= 0 else float(softmax_scale)
    group = h_q // h_kv
    sparse_heads = [h for h in range(h_q) if route is None or route[b, h] != 0]
    nsets = max(1, idx_heads)
    idx = np.full((nsets, top_k), -1, dtype=np.int64)
    if sparse_heads:
        for i in range(nsets):
            qi = q_idx[b, n] if idx_heads <= 1 else q_idx[b, n, i]
            idx[i] = select_top_k(indexer_scores(qi, k_idx[b], vis), top_k)
    out = np.zeros((h_q, head_dim), dtype=np.float64)
    for h in range(h_q):
        g_kv = h // group
        if h in sparse_heads:
            sel = idx[h // (h_q // nsets)]
            rows = sel[sel >= 0]
        else:
            rows = np.arange(vis)
        a, _ = softmax_attention(q[b, n, h], k[b, rows, g_kv], v[b, rows, g_kv], scale)
        if gate is not None:
            a = gate_blend(a, float(gate[b, n, h]), y2[b, n, h])
        out[h] = a
    return out, (idx[0] if idx_heads <= 1 else idx)


def forward(params, inputs: Dict[str, np.ndarray], rows: Optional[Sequence[int]] = None,
            batches: Optional[Sequence[int]] = None, use_gate: bool = True,
            use_route: bool = True, softmax_scale: Optional[float] = None
            ) -> Tuple[np.ndarray, np.ndarray]:
    """Run ``forward_row`` over the chosen (batch, row) pairs.

    ``params`` carries batch, n_q, kv_len, h_q, h_kv, head_dim, top_k (and
    optionally idx_heads) as attributes.  Returns out [nb, nr, Hq, d] and
    idx [nb, nr, K] ([nb, nr, H, K] with idx_heads = H > 1).
    """
    bs = list(range(params.batch)) if batches is None else list(batches)
    ns = list(range(params.n_q)) if rows is None else list(rows)
    ih = getattr(params, "idx_heads", 1)
    out = np.zeros((len(bs), len(ns), params.h_q, params.head_dim), dtype=np.float64)
    ishape = (len(bs), len(ns), params.top_k) if ih <= 1 else (len(bs), len(ns), ih, params.top_k)
    idx = np.zeros(ishape, dtype=np.int64)
    for i, b in enumerate(bs):
        for r, n in enumerate(ns):
            out[i, r], idx[i, r] = forward_row(
                b, n, n_q=params.n_q, kv_len=params.kv_len, h_q=params.h_q,
                h_kv=params.h_kv, head_dim=params.head_dim, top_k=params.top_k,
                q_idx=inputs["q_idx"], k_idx=inputs["k_idx"], q=inputs["q"],
                k=inputs["k"], v=inputs["v"],
                gate=inputs.get("gate") if use_gate else None,
                y2=inputs.get("y2") if use_gate else None,
                route=inputs.get("route") if use_route else None,
                softmax_scale=softmax_scale, idx_heads=ih)
    return out, idx


def dense_causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                           softmax_scale: Optional[float] = None) -> np.ndarray:
    """Full causal attention for one sequence, written independently.

    q [N, Hq, d], k/v [L, Hkv, d] -> [N, Hq, d] in float64.  Builds the whole
    score matrix, masks j > L - N + n with -inf ([AAM] §2.1), and normalises
    each row with its own maximum.  Used by the self-checks of the sparse path.
    """
    n_q, h_q, d = q.shape
    kv_len, h_kv, _ = k.shape
    scale = 1.0 / math.sqrt(d) if not softmax_scale or softmax_scale <= 0 else float(softmax_scale)
    group = h_q // h_kv
    pos = np.arange(kv_len)[None, :]
    last = (kv_len - n_q + np.arange(n_q))[:, None]
    mask = pos <= last
    out = np.empty((n_q, h_q, d), dtype=np.float64)
    for h in range(h_q):
        kh = k[:, h // group].astype(np.float64)
        vh = v[:, h // group].astype(np.float64)
        logits = (q[:, h].astype(np.float64) @ kh.T) * scale
        logits = np.where(mask, logits, -np.inf)
        logits -= logits.max(axis=1, keepdims=True)
        p = np.exp(logits)
        p /= p.sum(axis=1, keepdims=True)
        out[:, h] = p @ vh
    return out


def route_heads(k_current: np.ndarray, w1: np.ndarray, b1: np.ndarray, w2: np.ndarray,
                b2: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per-head route of one sequence from the attention router, in float64.

    [EA] §2.2: a light router in every layer takes the current key hidden
    states, is a two-layer MLP and decides per attention head between full
    and sparse attention; it is trained through Gumbel-Softmax with a
    straight-through estimator, so at inference the decision is hard: the
    option with the larger logit.

    k_current [n, Hkv, d]: keys of the tokens of the call.  w1 [Hkv*d, Hr],
    b1 [Hr], w2 [Hr, Hq, 2], b2 [Hq, 2]; column 0 of the last axis is full
    attention, column 1 sparse.  Returns (logits [Hq, 2], route [Hq] uint8
    with 1 = sparse); a tie keeps full attention.
    """
    n = k_current.shape[0]
    x = k_current.reshape(n, -1).astype(np.float64).sum(axis=0) / n   # mean key vector
    hidden = x @ w1.astype(np.float64) + b1.astype(np.float64)
    hidden = np.where(hidden > 0.0, hidden, 0.0)                      # ReLU
    h_r, h_q = w2.shape[0], w2.shape[1]
    logits = (hidden @ w2.reshape(h_r, h_q * 2).astype(np.float64)).reshape(h_q, 2)
    logits = logits + b2.astype(np.float64)
    route = (logits[:, 1] > logits[:, 0]).astype(np.uint8)
    return logits, route


def route_batch(params, k: np.ndarray, router: Dict[str, np.ndarray]
                ) -> Tuple[np.ndarray, np.ndarray]:
    """route_heads for every sequence: the current tokens are the last n_q
    positions of each sequence's keys.  Returns logits [B, Hq, 2] and
    route [B, Hq]."""
    L, N = params.kv_len, params.n_q
    logits = np.zeros((params.batch, params.h_q, 2), dtype=np.float64)
    route = np.zeros((params.batch, params.h_q), dtype=np.uint8)
    for b in range(params.batch):
        logits[b], route[b] = route_heads(k[b, L - N:L], router["w1"], router["b1"],
                                          router["w2"], router["b2"])
    return logits, route
