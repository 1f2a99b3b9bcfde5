"""Throughput of the indexer + top-k sparse attention path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one dsa_fused_forward call (indexer, top-k, gather, attention,
gate) over one batch of seeded synthetic inputs already resident in HBM.
Prints one JSON line.  The default workload is the batch-8 decode over a
131072-token context (32 query / 8 KV heads, d = 128, d_idx = 64, K = 2048).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "query tokens/s (indexer+top-k+sparse attn) at K=2048; % HBM/MFMA peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16


def algorithmic_work(w, route):
    """Bytes the method must move and flops it must do for one step (no reuse model).

    Bytes: every indexer key row once per sequence (all query rows of a
    sequence share it), the selected key and value rows of every KV head that
    has a sparse head, once per query token; the whole causal key/value prefix
    once per (sequence, KV head) that has a dense head; q, q_idx, gate, y2
    and out once.  Flops: 2*d_idx per visible score, 4*d per (query head,
    attended key).
    """
    bq = 2 if w.qkv_dtype == "bf16" else 4
    bi = 2 if w.idx_dtype == "bf16" else 4
    B, N, L, K = w.batch, w.n_q, w.kv_len, w.top_k
    G = w.h_q // w.h_kv
    vis = L - N + 1 + np.arange(N, dtype=np.int64)
    keff = np.minimum(vis, K)
    r = route.reshape(B, w.h_kv, G)
    grp_sparse = r.any(axis=2).sum(axis=1)          # per sequence
    grp_dense = (~r.astype(bool)).any(axis=2).sum(axis=1)
    heads_sparse = r.sum(axis=(1, 2))
    heads_dense = w.h_q - heads_sparse
    seq_has_sparse = heads_sparse > 0
    byt = 0
    byt += int(seq_has_sparse.sum()) * L * w.idx_dim * bi                  # k_idx scan
    byt += B * N * w.idx_dim * bi                                          # q_idx
    byt += int(grp_sparse.sum()) * int(keff.sum()) * w.head_dim * 2 * bq   # gathered K and V
    byt += int(grp_dense.sum()) * L * w.head_dim * 2 * bq                  # dense prefixes
    byt += B * N * w.h_q * (w.head_dim * bq + 4 + 2 * 4 * w.head_dim)      # q, gate, y2, out
    flops = 0
    flops += int(seq_has_sparse.sum()) * int(vis.sum()) * 2 * w.idx_dim
    flops += int(heads_sparse.sum()) * int(keff.sum()) * 4 * w.head_dim
    flops += int(heads_dense.sum()) * int(vis.sum()) * 4 * w.head_dim
    return byt, flops


def measured_traffic(workload: str):
    """HBM bytes per launch of the dominant kernel from the counter runs kept in
    profiles/traffic.json (FETCH_SIZE and WRITE_SIZE, KiB per dispatch, each
    scaled by the factor a plain copy of known size gives).  None when no
    record exists or the kernel's source has changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None, None
    rec = json.load(open(path)).get(workload)
    if not rec:
        return None, None
    src = os.path.join(ROOT, rec["source"])
    if not os.path.exists(src):
        return None, rec
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if sha != rec["source_sha256"]:
        return None, rec
    byt = rec["fetch_kib"] * 1024 * rec["fetch_factor"] + rec["write_kib"] * 1024 * rec["write_factor"]
    return byt, rec


def cpu_baseline(w, x, budget_s):
    """The oracle as it stands, on whole query rows of the same workload, for ~budget_s."""
    from oracle import dsa_oracle as O
    try:
        import threadpoolctl
        cores = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] or [1])
    except Exception:
        cores = 1
    rows = 0
    t0 = time.perf_counter()
    pairs = [(b, n) for n in range(w.n_q) for b in range(w.batch)]
    while time.perf_counter() - t0 < budget_s:
        b, n = pairs[rows % len(pairs)]
        O.forward(w, x, rows=[n], batches=[b])
        rows += 1
    dt = time.perf_counter() - t0
    return {"value": rows / dt, "unit": "query tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{rows} whole query rows (all heads) of the same workload, {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_b8_ctx128k")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--stages", action="store_true", help="print per-stage GPU time")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="instead of the workload, copy this many bytes device to device "
                         "(a plain copy kernel of known size, for counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library runs on one GPU; it has no multi-GPU mode).", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_bytes:
        src = torch.ones(args.copy_bytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(max(1, args.steps)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": args.copy_bytes, "copies": max(1, args.steps)}))
        return
    from top_sparse_attention_indexer_amd import binding as B
    from top_sparse_attention_indexer_amd import synth
    from top_sparse_attention_indexer_amd.tensors import to_device

    w = synth.WORKLOADS[args.workload]
    x = synth.make_inputs(w)
    dev = to_device(w, x)
    p = B.problem_for(w)
    out = torch.empty((w.batch, w.n_q, w.h_q, w.head_dim), dtype=torch.float32, device="cuda")
    idx = torch.empty((w.batch, w.n_q, w.top_k), dtype=torch.int32, device="cuda")
    ws = torch.empty(max(1, B.dsa_workspace_size(p)), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        B.dsa_fused_forward(p, dev["q_idx"], dev["k_idx"], dev["q"], dev["k"], dev["v"],
                            dev["gate"], dev["y2"], dev["route"], out, idx, ws, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # timed region: K back-to-back steps between two events on the launch stream
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for _ in range(args.steps):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms = total_ms / args.steps
    # per-step spread from a second pass with events around every step
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(min(args.steps, 50))]
    for a, b_ in ev:
        a.record(stream)
        step()
        b_.record(stream)
    torch.cuda.synchronize()
    per = np.array([a.elapsed_time(b_) for a, b_ in ev])
    if args.stages:
        B.dsa_profile_start(1 << 16)
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        st, dropped = B.dsa_profile_stop()
        print(json.dumps({k: [v[0] / args.steps, v[1] / args.steps] for k, v in st.items()}),
              file=sys.stderr)
    tokens = w.batch * w.n_q
    byt, flops = algorithmic_work(w, x["route"])
    achieved = byt / (ms / 1e3) / 1e9
    traffic, rec = measured_traffic(w.name)
    if w.n_q <= 4:
        kernel = "k_decode (the step is this one launch)"
    else:
        kernel = "whole step (indexer, top-k and attention launches per chunk of rows)"
    res = {
        "metric": METRIC, "value": tokens / (ms / 1e3), "unit": "query tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16"
        if w.qkv_dtype == "bf16" else "fp32", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "n_q": w.n_q, "kv_len": w.kv_len,
                   "h_q": w.h_q, "h_kv": w.h_kv, "head_dim": w.head_dim, "idx_dim": w.idx_dim,
                   "top_k": w.top_k, "parallelism": "single GPU"},
        "step_ms_p10_p50_p90": [float(np.percentile(per, q)) for q in (10, 50, 90)],
        "roofline": {"bound": "hbm", "kernel": kernel, "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic, "algorithmic_bytes": byt, "algorithmic_flops": flops},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, x, args.cpu_seconds)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
