"""Throughput of the indexer + top-k sparse attention path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one dsa_fused_forward call (indexer, top-k, gather, attention,
gate) over one batch of seeded synthetic inputs already resident in HBM.
Prints one JSON line.  The headline workload is the largest configuration of
the set that fits one GPU: the elastic mixed-route prefill, B = 2 sequences
of 65536 causal tokens, 32 query / 8 KV heads, d = 128, d_idx = 64, K = 2048,
each (sequence, head) routed sparse with probability 0.7.  The decode and the
32K prefill workloads are measured too and reported as nested entries.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "query tokens/s (indexer+top-k+sparse attn) at K=2048; % HBM/MFMA peak"
HEADLINE = "elastic_prefill_64k"
OTHERS = ("decode_b8_ctx128k", "decode_ctx1m_mqa", "prefill_32k")
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 MFMA
# L2 read bandwidth from the unit counts: 8 XCDs x 16 channels x 128 B/clk
# x 2.4 GHz (the bound of a gather served from L2; no published figure)
L2_PEAK_GBS = 8 * 16 * 128 * 2.4
# VALU lane-operations per second (256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz):
# the bound of one compare per key for the top-k selection
ALU_PEAK_GOPS = 256 * 64 * 2.4


def work_model(w, route):
    """Algorithmic work of one forward, per stage (no reuse assumed).

    indexer: 2 * d_idx flops per visible (query, key) pair of every sequence
      with a sparse head; k_idx read once per sequence.
    topk: one compare per visible score.
    gather: the selected key and value rows of every KV head that has a
      sparse head, once per query token (Hkv_sparse * K_eff * d * 2 * 2 B).
    dense: 4 * d flops per (dense query head, visible key); the causal K/V
      prefix of every KV head with a dense head read once.
    streams: q, q_idx, gate, y2 and out once.
    """
    bq = 2 if w.qkv_dtype == "bf16" else 4
    bi = 2 if w.idx_dtype == "bf16" else 4
    B, N, L, K = w.batch, w.n_q, w.kv_len, w.top_k
    G = w.h_q // w.h_kv
    vis = L - N + 1 + np.arange(N, dtype=np.int64)
    keff = np.minimum(vis, K)
    r = route.reshape(B, w.h_kv, G).astype(bool)
    grp_sparse = int(r.any(axis=2).sum())
    grp_dense = int((~r).any(axis=2).sum())
    heads_sparse = int(r.sum())
    heads_dense = B * w.h_q - heads_sparse
    seq_sparse = int(r.any(axis=(1, 2)).sum())
    m = {}
    m["indexer_flops"] = seq_sparse * int(vis.sum()) * 2 * w.idx_dim
    m["indexer_bytes"] = seq_sparse * L * w.idx_dim * bi + B * N * w.idx_dim * bi
    m["topk_keys"] = seq_sparse * int(vis.sum())
    m["gather_bytes"] = grp_sparse * int(keff.sum()) * w.head_dim * 2 * bq
    m["sparse_flops"] = heads_sparse * int(keff.sum()) * 4 * w.head_dim
    m["dense_flops"] = heads_dense * int(vis.sum()) * 4 * w.head_dim
    m["dense_bytes"] = grp_dense * L * w.head_dim * 2 * bq
    m["stream_bytes"] = B * N * w.h_q * (w.head_dim * bq + 4 + 2 * 4 * w.head_dim)
    m["bytes"] = (m["indexer_bytes"] + m["gather_bytes"] + m["dense_bytes"] + m["stream_bytes"])
    m["flops"] = m["indexer_flops"] + m["sparse_flops"] + m["dense_flops"]
    return m


def measured_traffic(workload: str):
    """HBM bytes per launch of the dominant kernel from the counter runs kept in
    profiles/traffic.json (FETCH_SIZE and WRITE_SIZE, KiB per dispatch, each
    scaled by the factor a plain copy of known size gives).  None when no
    record exists or the kernel's source has changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(workload)
    if not rec:
        return None
    src = os.path.join(ROOT, rec["source"])
    if not os.path.exists(src):
        return None
    if hashlib.sha256(open(src, "rb").read()).hexdigest() != rec["source_sha256"]:
        return None
    return (rec["fetch_kib"] * 1024 * rec["fetch_factor"]
            + rec["write_kib"] * 1024 * rec["write_factor"]) / rec.get("launches_per_step", 1)


def stage_rooflines(w, m, stages, steps):
    """Per-stage time and roofline fraction from the stage timing of the timed
    region (GPU time of each stage's launches, summed, per step)."""
    out = {}
    per = {k: (v[0] / steps, v[1] / steps) for k, v in stages.items() if v[1] > 0}
    if "indexer" in per:
        t = per["indexer"][0] * 1e-3
        a = m["indexer_flops"] / t / 1e12
        out["indexer"] = {"ms": per["indexer"][0], "launches": per["indexer"][1], "bound": "mfma",
                          "achieved": a, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                          "frac": a / MFMA_BF16_PEAK_TFLOPS}
    if "topk" in per:
        t = per["topk"][0] * 1e-3
        a = m["topk_keys"] / t / 1e9
        out["topk"] = {"ms": per["topk"][0], "launches": per["topk"][1], "bound": "alu",
                       "achieved": a, "peak": ALU_PEAK_GOPS, "unit": "Gkeys/s",
                       "frac": a / ALU_PEAK_GOPS}
    if "attention" in per:
        t = per["attention"][0] * 1e-3
        t_mfma = m["dense_flops"] / (MFMA_BF16_PEAK_TFLOPS * 1e12)
        t_l2 = m["gather_bytes"] / (L2_PEAK_GBS * 1e9)
        if t_l2 >= t_mfma:
            a = m["gather_bytes"] / t / 1e9
            e = {"bound": "l2", "achieved": a, "peak": L2_PEAK_GBS, "unit": "GB/s"}
        else:
            a = m["dense_flops"] / t / 1e12
            e = {"bound": "mfma", "achieved": a, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s"}
        e["frac"] = max(t_l2, t_mfma) / t
        out["attention"] = dict({"ms": per["attention"][0], "launches": per["attention"][1]}, **e,
                                dense_tflops=m["dense_flops"] / t / 1e12,
                                dense_frac=m["dense_flops"] / t / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                                gather_gbs=m["gather_bytes"] / t / 1e9)
    if "merge" in per:
        out["merge"] = {"ms": per["merge"][0], "launches": per["merge"][1]}
    if "prep" in per:
        out["prep"] = {"ms": per["prep"][0], "launches": per["prep"][1]}
    if "route" in per and "route_bytes" in m:
        t = per["route"][0] * 1e-3
        a = m["route_bytes"] / t / 1e9
        out["route"] = {"ms": per["route"][0], "launches": per["route"][1], "bound": "hbm",
                        "achieved": a, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": a / HBM_PEAK_GBS}
    if "decode" in per:
        t = per["decode"][0] * 1e-3
        a = m["bytes"] / t / 1e9
        out["decode"] = {"ms": per["decode"][0], "launches": per["decode"][1], "bound": "hbm",
                         "achieved": a, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": a / HBM_PEAK_GBS}
    return out


def cpu_info():
    model = platform.processor() or "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        ncpu = len(os.sched_getaffinity(0))
    except AttributeError:
        ncpu = os.cpu_count() or 1
    return model, ncpu


def blas_threads():
    try:
        import threadpoolctl
        return max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] or [1])
    except Exception:
        return 1


def cpu_baseline(w, x, budget_s, rows=None, one_thread=False):
    """The oracle as it stands on whole query rows (all heads) of the same
    workload, for about budget_s seconds: query tokens/s."""
    import contextlib
    from oracle import dsa_oracle as O
    if one_thread:
        import threadpoolctl
        ctx = threadpoolctl.threadpool_limits(limits=1)
    else:
        ctx = contextlib.nullcontext()
    with ctx:
        threads = blas_threads()
        if rows is None:
            rows = list(range(w.n_q))
        pairs = [(b, n) for n in rows for b in range(w.batch)]
        done = 0
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < budget_s:
            b, n = pairs[done % len(pairs)]
            O.forward(w, x, rows=[n], batches=[b])
            done += 1
        dt = time.perf_counter() - t0
    return done / dt, done, dt, threads


class Runner:
    """Inputs on the GPU and one fused forward per call."""

    def __init__(self, w, seed=None):
        import torch
        from top_sparse_attention_indexer_amd import binding as B
        from top_sparse_attention_indexer_amd import synth
        from top_sparse_attention_indexer_amd.tensors import to_device
        self.B, self.w = B, w
        self.x = synth.make_inputs(w, seed=seed)
        self.dev = to_device(w, self.x)
        self.p = B.problem_for(w)
        self.out = torch.empty((w.batch, w.n_q, w.h_q, w.head_dim), dtype=torch.float32,
                               device="cuda")
        self.idx = torch.empty((w.batch, w.n_q, w.top_k), dtype=torch.int32, device="cuda")
        self.ws = torch.empty(max(1, B.dsa_workspace_size(self.p)), dtype=torch.uint8,
                              device="cuda")
        self.stream = torch.cuda.current_stream()

    def step(self):
        d = self.dev
        self.B.dsa_fused_forward(self.p, d["q_idx"], d["k_idx"], d["q"], d["k"], d["v"],
                                 d["gate"], d["y2"], d["route"], self.out, self.idx, self.ws,
                                 self.stream)


class RoutedRunner:
    """The forward with the route made on the device by the two-layer router
    (seeded random weights): dsa_fused_forward_routed, or the router alone."""

    def __init__(self, base, hidden=256, router_only=False):
        import torch
        from top_sparse_attention_indexer_amd import synth
        B, w = base.B, base.w
        self.B, self.w, self.base, self.router_only = B, w, base, router_only
        self.weights = {k: torch.from_numpy(v).cuda()
                        for k, v in synth.make_router(w, hidden=hidden).items()}
        self.r = B.router(self.weights["w1"], self.weights["b1"], self.weights["w2"],
                          self.weights["b2"])
        self.hidden = hidden
        self.route = torch.empty((w.batch, w.h_q), dtype=torch.uint8, device="cuda")
        self.ws = torch.empty(max(1, B.dsa_route_workspace_size(base.p, self.r)),
                              dtype=torch.uint8, device="cuda")
        self.stream = base.stream

    def step(self):
        b, d = self.base, self.base.dev
        if self.router_only:
            self.B.dsa_route_heads(b.p, self.r, d["k"], self.route, None, self.ws, self.stream)
        else:
            self.B.dsa_fused_forward_routed(b.p, self.r, d["q_idx"], d["k_idx"], d["q"], d["k"],
                                            d["v"], d["gate"], d["y2"], self.route, b.out,
                                            b.idx, self.ws, self.stream)

    def route_bytes(self):
        """Keys of the call's tokens once, the router weights once."""
        w = self.w
        c = w.h_kv * w.head_dim
        bq = 2 if w.qkv_dtype == "bf16" else 4
        weights = (c * self.hidden + self.hidden + self.hidden * 2 * w.h_q + 2 * w.h_q) * 4
        return w.batch * w.n_q * c * bq + weights


def timed(runners, steps, warmup):
    """Warm-up, then `steps` back-to-back steps (cycling over the runners)
    between two events on the launch stream; stage timing over the same
    region.  A step that is one timed launch group (the single-launch decode,
    the router) is timed without the per-launch events, which would add their
    own cost to a step of tens of microseconds: its stage time is then the
    region's time per step.  Returns ms per step, per-step spread and the
    stage sums."""
    import torch
    B = runners[0].B
    stream = runners[0].stream
    for i in range(warmup):
        runners[i % len(runners)].step()
    torch.cuda.synchronize()
    # launch groups per step, from one profiled step
    B.dsa_profile_start(1 << 10)
    runners[0].step()
    torch.cuda.synchronize()
    probe = {k: v for k, v in B.dsa_profile_stop()[0].items() if v[1] > 0}
    single = len(probe) == 1 and next(iter(probe.values()))[1] == 1
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    if not single:
        B.dsa_profile_start(1 << 17)
    t0.record(stream)
    for i in range(steps):
        runners[i % len(runners)].step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    if single:
        stages = {next(iter(probe)): (ms * steps, steps)}
    else:
        stages = B.dsa_profile_stop()[0]
    for r in runners:
        if isinstance(r, Runner):
            B.dsa_exec_status(r.ws, r.stream)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(min(steps, 20))]
    for i, (a, b_) in enumerate(ev):
        a.record(stream)
        runners[i % len(runners)].step()
        b_.record(stream)
    torch.cuda.synchronize()
    per = np.array([a.elapsed_time(b_) for a, b_ in ev])
    return ms, [float(np.percentile(per, q)) for q in (10, 50, 90)], stages


def graph_decode(w, steps, warmup):
    """The decode step captured once into a HIP graph (on a side stream) and
    replayed `steps` times back to back between two events; the replayed
    output is compared with the eager one."""
    import torch
    r = Runner(w)
    s = torch.cuda.Stream()
    r.stream = s
    with torch.cuda.stream(s):
        for _ in range(max(2, warmup)):
            r.step()
    torch.cuda.synchronize()
    ref = r.out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        r.step()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(s):
        for _ in range(3):
            g.replay()
        t0.record(s)
        for _ in range(steps):
            g.replay()
        t1.record(s)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    r.B.dsa_exec_status(r.ws, s)
    same = bool(torch.equal(r.out, ref))
    m = work_model(w, r.x["route"])
    return {"value": w.batch * w.n_q / (ms / 1e3), "unit": "query tokens/s", "ms_per_step": ms,
            "replays": steps, "replay_matches_eager": same, "config": config_of(w),
            "stages": {"decode": {"ms": ms, "launches": 1.0, "bound": "hbm",
                                  "achieved": m["bytes"] / (ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                                  "unit": "GB/s",
                                  "frac": m["bytes"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}}}


def config_of(w):
    return {"workload": w.name, "batch": w.batch, "n_q": w.n_q, "kv_len": w.kv_len,
            "h_q": w.h_q, "h_kv": w.h_kv, "head_dim": w.head_dim, "idx_dim": w.idx_dim,
            "top_k": w.top_k, "route_sparse_p": w.route_sparse_p, "parallelism": "single GPU"}


def progress(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def measure(w, steps, warmup, cold=False):
    """One workload: value, step time and per-stage rooflines.  cold: two input
    sets of the same shape used in alternation, so that consecutive steps do
    not find their inputs in the 256 MB Infinity Cache."""
    progress(f"{w.name}{' (two input sets)' if cold else ''}: inputs")
    runners = [Runner(w)] + ([Runner(w, seed=w.seed + 100)] if cold else [])
    progress(f"{w.name}: {warmup} warm-up + {steps} timed steps")
    ms, spread, stages = timed(runners, steps, warmup)
    progress(f"{w.name}: {ms:.4f} ms per step")
    m = work_model(w, runners[0].x["route"])
    res = {"value": w.batch * w.n_q / (ms / 1e3), "unit": "query tokens/s", "ms_per_step": ms,
           "step_ms_p10_p50_p90": spread, "config": config_of(w),
           "stages": stage_rooflines(w, m, stages, steps),
           "algorithmic_bytes": m["bytes"], "algorithmic_flops": m["flops"]}
    if cold:
        res["input_sets"] = 2
    return res, runners, m


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-others", action="store_true", help="only the headline workload")
    ap.add_argument("--router-only", action="store_true",
                    help="time only the route producer on the workload's keys (one JSON line)")
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
    from top_sparse_attention_indexer_amd import synth

    w = synth.WORKLOADS[args.workload]
    if args.router_only:
        progress(f"{w.name}: inputs")
        rr = RoutedRunner(Runner(w), router_only=True)
        ms_r, spread_r, stages_r = timed([rr], args.steps, args.warmup)
        mr = dict(work_model(w, rr.route.cpu().numpy()), route_bytes=rr.route_bytes())
        print(json.dumps({"workload": w.name, "router_ms": ms_r, "step_ms_p10_p50_p90": spread_r,
                          "stages": stage_rooflines(w, mr, stages_r, args.steps),
                          "hidden": rr.hidden, "route_bytes": rr.route_bytes()}))
        return
    head, runners, m = measure(w, args.steps, args.warmup)
    st = head["stages"]
    # dominant kernel: the stage with the largest GPU time
    dom = max((k for k in st if "ms" in st[k] and "bound" in st[k]), key=lambda k: st[k]["ms"])
    launches = max(1.0, st[dom]["launches"])
    roof = {k: st[dom][k] for k in ("bound", "achieved", "peak", "unit", "frac")}
    roof["kernel"] = {"attention": "k_attn_slices", "decode": "k_decode",
                      "indexer": "k_indexer_mfma", "topk": "k_topk_cand"}[dom]
    roof["stage"] = dom
    roof["launches_per_step"] = launches
    traffic = measured_traffic(w.name)
    roof["traffic"] = traffic
    res = {
        "metric": METRIC, "value": head["value"], "unit": "query tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.qkv_dtype == "bf16" else "fp32", "data": "synthetic",
        "config": head["config"],
        "step_ms_p10_p50_p90": head["step_ms_p10_p50_p90"],
        "roofline": roof,
        "stages": st,
        "algorithmic_bytes": head["algorithmic_bytes"],
        "algorithmic_flops": head["algorithmic_flops"],
    }
    x_head = runners[0].x
    others = {}
    if not args.no_others and args.workload == HEADLINE:
        # the route made on the device: the router alone, then the forward with it
        for key, only in (("route_producer", True), ("routed_forward", False)):
            progress(f"{w.name}: {key}")
            rr = RoutedRunner(runners[0], router_only=only)
            ms_r, spread_r, stages_r = timed([rr], args.steps if not only else 50, 3)
            mr = dict(work_model(w, rr.route.cpu().numpy()), route_bytes=rr.route_bytes())
            e = {"ms_per_step": ms_r, "step_ms_p10_p50_p90": spread_r,
                 "stages": stage_rooflines(w, mr, stages_r, args.steps if not only else 50),
                 "hidden": rr.hidden,
                 "sparse_share": float(rr.route.float().mean().item())}
            if not only:
                e["value"] = w.batch * w.n_q / (ms_r / 1e3)
                e["unit"] = "query tokens/s"
            progress(f"{w.name}: {key} {ms_r:.4f} ms")
            others[key] = e
            del rr
    del runners
    torch.cuda.empty_cache()
    if not args.no_others and args.workload == HEADLINE:
        for name in OTHERS:
            wo = synth.WORKLOADS[name]
            steps = 50 if wo.n_q == 1 else args.steps
            r, rr, _ = measure(wo, steps, max(args.warmup, 5 if wo.n_q == 1 else 1))
            r["traffic"] = measured_traffic(name)
            others[name] = r
            del rr
            torch.cuda.empty_cache()
        # the batch-8 decode captured into a HIP graph and replayed
        progress("decode_b8_ctx128k: graph capture and replay")
        r = graph_decode(synth.WORKLOADS["decode_b8_ctx128k"], 50, 5)
        progress(f"decode_b8_ctx128k (graph): {r['ms_per_step']:.4f} ms per step")
        others["decode_b8_ctx128k_graph"] = r
        torch.cuda.empty_cache()
        # the batch-8 decode with two input sets in alternation (403 MB of
        # inputs, above the 256 MB Infinity Cache)
        wo = synth.WORKLOADS["decode_b8_ctx128k"]
        r, rr, _ = measure(wo, 50, 6, cold=True)
        others["decode_b8_ctx128k_cold"] = r
        del rr
        torch.cuda.empty_cache()
        res["others"] = others
    if not args.no_cpu_baseline:
        model, ncpu = cpu_info()
        # rows spread evenly over the sequence: the mean cost of a row
        rows = np.linspace(0, w.n_q - 1, 257).astype(int).tolist()
        progress(f"oracle on the host, about {args.cpu_seconds:.0f} s")
        v, done, dt, threads = cpu_baseline(w, x_head, args.cpu_seconds, rows=rows)
        res["cpu_baseline"] = {
            "value": v, "unit": "query tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} whole query rows (all 32 heads, both routes) of {w.name}, "
                      f"spread evenly over the sequence, {dt:.1f} s",
            "host_cpus": ncpu, "cpu_model": model}
        one = {}
        for name in ("tiny_prefill_fp32", "decode_b8_ctx128k"):
            wo = synth.WORKLOADS[name]
            xo = synth.make_inputs(wo)
            v1, d1, t1, _ = cpu_baseline(wo, xo, 4.0, one_thread=True)
            one[name] = {"value": v1, "unit": "query tokens/s", "threads": 1,
                         "sample": f"{d1} whole query rows, {t1:.1f} s"}
        res["cpu_baseline"]["one_thread"] = one
    print(json.dumps(res))


if __name__ == "__main__":
    main()
