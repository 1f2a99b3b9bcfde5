"""Seeded synthetic inputs for indexer + top-k sparse attention.

This module only draws random numbers and shapes them; it holds none of the
method's arithmetic.  Both the HIP path (through the tests and the bench) and
the CPU oracle are fed from it, so it imports nothing but numpy.

Workloads are named by what they are.  Their shapes follow the Gated-DSA
configuration on the page "超大规模MoE架构中稀疏注意力机制的演进与实践"
(§二.1: K = 2048 per query token; §三: a context of 1,048,576 tokens) and the
per-head full/sparse routing of the page "Elastic Attention：动态路由优化大模型
长文本处理" (§2.2).  No dataset is used; every tensor is drawn here.

Recipe (one PCG64 stream per tensor, spawned from SeedSequence(seed) in the
fixed order q_idx, k_idx, q, k, v, gate_z, y2, route, planted):
  * indexer entries: integers uniform on [lo, hi] inclusive, stored as float
    (exact in bf16), so every indexer score is an exact integer; with
    idx_heads > 1 every token has one indexer query per indexer head;
  * q, k, v, y2: N(0, 1) drawn in float32; q/k/v rounded to bf16 (round to
    nearest even) when the workload is bf16;
  * gate: z ~ N(0, 1) in float32, g = 1 / (1 + exp(-z)) evaluated in float64
    and rounded to float32 (the gate is handed over post-sigmoid);
  * route: per (sequence, query head), 1 = top-k sparse with probability
    ``route_sparse_p``, else 0 = full causal; all ones when ``route_sparse_p``
    is None;
  * planted rows: ``planted`` distinct key positions drawn uniformly from
    [0, L); their indexer rows are multiplied by ``planted_scale``.

All floating tensors are returned as float32 arrays whose values are exactly
representable in the workload's storage dtype; ``to_bf16_bits`` gives the
16-bit patterns for device upload.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Tuple

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int          # B sequences
    n_q: int            # N query tokens per sequence (the last N positions)
    kv_len: int         # L keys per sequence
    h_q: int            # query heads
    h_kv: int           # key/value heads
    head_dim: int       # d
    idx_dim: int        # d_idx
    top_k: int          # K
    qkv_dtype: str      # "fp32" | "bf16"
    idx_dtype: str      # "fp32" | "bf16"
    idx_range: Tuple[int, int]
    route_sparse_p: Optional[float] = None
    planted: int = 0
    planted_scale: int = 1
    seed: int = 0
    idx_heads: int = 1  # indexer query heads (1: one selected set shared by all heads)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def rows(self) -> int:
        return self.batch * self.n_q


# The five workloads.  Seeds are 1000 + ordinal.
WORKLOADS: Dict[str, Workload] = {
    w.name: w for w in [
        Workload("tiny_prefill_fp32", 1, 512, 512, 4, 1, 64, 32, 64,
                 "fp32", "fp32", (-8, 8), seed=1001),
        Workload("decode_b8_ctx128k", 8, 1, 131072, 32, 8, 128, 64, 2048,
                 "bf16", "bf16", (-4, 4), seed=1002),
        Workload("prefill_32k", 1, 32768, 32768, 32, 8, 128, 64, 2048,
                 "bf16", "bf16", (-4, 4), seed=1003),
        Workload("decode_ctx1m_mqa", 1, 1, 1048576, 64, 1, 128, 64, 2048,
                 "bf16", "bf16", (-4, 4), planted=16, planted_scale=3,
                 seed=1004),
        Workload("elastic_prefill_64k", 2, 65536, 65536, 32, 8, 128, 64, 2048,
                 "bf16", "bf16", (-4, 4), route_sparse_p=0.7, seed=1005),
    ]
}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    # in place on 32-bit patterns: for every finite or infinite value the
    # rounding increment cannot carry past bit 31
    u = np.array(x, dtype=np.float32, copy=True).view(np.uint32)
    r = u >> 16
    r &= 1
    r += 0x7FFF
    u += r
    u &= np.uint32(0xFFFF0000)
    return u.view(np.float32)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """16-bit patterns of float32 values that are already bf16-exact."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("values are not bf16-exact")
    return (u >> 16).astype(np.uint16)


def _normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return round_to_bf16(x) if dtype == "bf16" else x


def make_inputs(w: Workload, seed: Optional[int] = None,
                parts: Tuple[str, ...] = ("q_idx", "k_idx", "q", "k", "v",
                                          "gate", "y2", "route")
                ) -> Dict[str, np.ndarray]:
    """Draw the inputs of workload ``w``.

    Shapes: q_idx [B,N,d_idx] ([B,N,H_idx,d_idx] with idx_heads > 1),
    k_idx [B,L,d_idx], q [B,N,Hq,d],
    k/v [B,L,Hkv,d], gate [B,N,Hq], y2 [B,N,Hq,d], route [B,Hq] (uint8).
    ``parts`` limits which tensors are drawn (each has its own stream, so a
    subset is identical to the same tensors of a full draw).  Planted rows
    (if any) are applied to k_idx and their positions returned as ``planted``.
    """
    seed = w.seed if seed is None else seed
    streams = np.random.SeedSequence(seed).spawn(9)
    rng = {name: np.random.Generator(np.random.PCG64(s)) for name, s in zip(
        ("q_idx", "k_idx", "q", "k", "v", "gate", "y2", "route", "planted"),
        streams)}
    B, N, L = w.batch, w.n_q, w.kv_len
    lo, hi = w.idx_range
    out: Dict[str, np.ndarray] = {}
    if "q_idx" in parts:
        shape = (B, N, w.idx_dim) if w.idx_heads <= 1 else (B, N, w.idx_heads, w.idx_dim)
        out["q_idx"] = rng["q_idx"].integers(lo, hi + 1, size=shape,
                                             dtype=np.int8).astype(np.float32)
    if "k_idx" in parts:
        k_idx = rng["k_idx"].integers(lo, hi + 1, size=(B, L, w.idx_dim),
                                      dtype=np.int8).astype(np.float32)
        if w.planted:
            pos = np.sort(rng["planted"].choice(L, size=w.planted, replace=False))
            k_idx[:, pos, :] *= w.planted_scale
            out["planted"] = pos.astype(np.int64)
        out["k_idx"] = k_idx
    if "q" in parts:
        out["q"] = _normal(rng["q"], (B, N, w.h_q, w.head_dim), w.qkv_dtype)
    if "k" in parts:
        out["k"] = _normal(rng["k"], (B, L, w.h_kv, w.head_dim), w.qkv_dtype)
    if "v" in parts:
        out["v"] = _normal(rng["v"], (B, L, w.h_kv, w.head_dim), w.qkv_dtype)
    if "gate" in parts:
        z = rng["gate"].standard_normal(size=(B, N, w.h_q), dtype=np.float32)
        out["gate"] = (1.0 / (1.0 + np.exp(-z.astype(np.float64)))).astype(np.float32)
    if "y2" in parts:
        out["y2"] = rng["y2"].standard_normal(size=(B, N, w.h_q, w.head_dim),
                                              dtype=np.float32)
    if "route" in parts:
        if w.route_sparse_p is None:
            out["route"] = np.ones((B, w.h_q), dtype=np.uint8)
        else:
            out["route"] = (rng["route"].random(size=(B, w.h_q))
                            < w.route_sparse_p).astype(np.uint8)
    return out


def make_router(w: Workload, hidden: int = 256, sparse_share: float = 0.7,
                seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Seeded random weights of the two-layer attention router (no trained
    weights exist here), float32: w1 [Hkv*d, hidden], b1 [hidden],
    w2 [hidden, Hq, 2], b2 [Hq, 2] (column 0 full, column 1 sparse).

    Scales: the mean of n iid N(0, 1) keys has per-component variance 1/n,
    so w1 ~ N(0, n / (Hkv*d)) gives pre-activations of unit variance;
    b1 ~ N(0, 0.1^2); w2 ~ N(0, 1 / hidden) gives logit differences of
    about unit variance; b2 shifts the sparse column by the normal quantile
    of ``sparse_share``, so that about that share of heads goes sparse.
    """
    import statistics
    seed = w.seed + 500 if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    c = w.h_kv * w.head_dim
    n = max(1, w.n_q)
    w1 = rng.standard_normal((c, hidden)) * math.sqrt(n / c)
    b1 = rng.standard_normal(hidden) * 0.1
    w2 = rng.standard_normal((hidden, w.h_q, 2)) / math.sqrt(hidden)
    b2 = np.zeros((w.h_q, 2))
    b2[:, 1] = statistics.NormalDist().inv_cdf(sparse_share)
    return {k: v.astype(np.float32) for k, v in
            (("w1", w1), ("b1", b1), ("w2", w2), ("b2", b2))}


def sample_rows(w: Workload, count: int, seed: int = 7) -> np.ndarray:
    """A seeded, stratified sample of query rows (n indices, ascending).

    The first 16 rows, the 17 rows around the point where the visible length
    crosses K, the last 16 rows, plus ``count`` further rows drawn uniformly
    from the rest (all rows when the workload has no more).
    """
    N = w.n_q
    first_vis = w.kv_len - N + 1            # visible keys of query row 0
    cross = w.top_k - first_vis             # row whose visible length is K + 1
    picks = set(range(min(16, N)))
    picks.update(range(max(0, N - 16), N))
    for r in range(cross - 8, cross + 9):
        if 0 <= r < N:
            picks.add(r)
    rest = np.setdiff1d(np.arange(N), np.fromiter(picks, dtype=np.int64))
    rng = np.random.Generator(np.random.PCG64(seed))
    if count > 0 and rest.size:
        picks.update(rng.choice(rest, size=min(count, rest.size), replace=False).tolist())
    return np.array(sorted(picks), dtype=np.int64)
