"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bars: top-k index rows bit-exact (integer-valued indexer inputs make every
score exact and the tie rule makes the set unique); outputs within max-abs
1e-4 for float32 workloads and 2e-2 for bf16 workloads (the oracle reads the
same bf16-rounded values and accumulates in float64).
"""
import numpy as np
import pytest
import torch

from oracle import dsa_oracle as O
from top_sparse_attention_indexer_amd import binding as B
from top_sparse_attention_indexer_amd import synth
from top_sparse_attention_indexer_amd.tensors import to_device

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-4, "bf16": 2e-2}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    yield
    torch.cuda.synchronize()


def idx_shape(w):
    """[B, N, K], or [B, N, H, K] with H = idx_heads > 1 indexer heads."""
    h = getattr(w, "idx_heads", 1)
    return (w.batch, w.n_q, w.top_k) if h <= 1 else (w.batch, w.n_q, h, w.top_k)


def run_fused(w, x, use_gate=True, use_route=True, want_idx=True, softmax_scale=0.0):
    p = B.problem_for(w, softmax_scale)
    dev = to_device(w, x)
    out = torch.empty((w.batch, w.n_q, w.h_q, w.head_dim), dtype=torch.float32, device="cuda")
    idx = (torch.full(idx_shape(w), -7, dtype=torch.int32, device="cuda")
           if want_idx else None)
    ws = torch.empty(max(1, B.dsa_workspace_size(p)), dtype=torch.uint8, device="cuda")
    B.dsa_fused_forward(p, dev["q_idx"], dev["k_idx"], dev["q"], dev["k"], dev["v"],
                        dev["gate"] if use_gate else None, dev["y2"] if use_gate else None,
                        dev["route"] if use_route else None, out, idx, ws)
    torch.cuda.synchronize()
    return out, idx


def check_rows(w, x, out, idx, rows, use_gate=True, use_route=True, batches=None):
    """Oracle on the chosen rows; exact index rows, outputs within tolerance."""
    bs = list(range(w.batch)) if batches is None else batches
    want_out, want_idx = O.forward(w, x, rows=rows, batches=bs, use_gate=use_gate,
                                   use_route=use_route)
    got_out = out[bs][:, rows].cpu().numpy() if not isinstance(out, np.ndarray) else out
    if idx is not None:
        got_idx = idx[bs][:, rows].cpu().numpy()
        bad = np.argwhere(np.any(got_idx != want_idx, axis=-1))
        assert bad.size == 0, f"index rows differ at (batch, row-sample) {bad[:5].tolist()}"
    err = np.max(np.abs(got_out.astype(np.float64) - want_out))
    assert err <= TOL[w.qkv_dtype], f"max-abs error {err}"
    return err


def check_index_structure(w, idx, batches=None):
    """Every row (of every indexer head): ascending ids in [0, p], count
    min(K, vis), then -1 padding."""
    N, L, K = w.n_q, w.kv_len, w.top_k
    H = max(1, getattr(w, "idx_heads", 1))
    vis = torch.arange(N, device="cuda", dtype=torch.int64) + (L - N + 1)
    vis = vis.repeat_interleave(H)
    cnt = torch.clamp(vis, max=K)
    pos = torch.arange(K, device="cuda")
    for b in (range(w.batch) if batches is None else batches):
        t = idx[b].reshape(N * H, K).to(torch.int64)
        valid = pos[None, :] < cnt[:, None]
        assert torch.all(torch.where(valid, t >= 0, t == -1)).item()
        assert torch.all(torch.where(valid, t < vis[:, None], True)).item()
        d = t[:, 1:] - t[:, :-1]
        both = valid[:, 1:]
        assert torch.all(torch.where(both, d > 0, True)).item()


# --------------------------------------------------------------------------- the five workloads
def test_tiny_prefill_fp32_all_rows(announce):
    w = synth.WORKLOADS["tiny_prefill_fp32"]
    x = synth.make_inputs(w)
    announce(f"fused_forward {w}")
    out, idx = run_fused(w, x)
    check_rows(w, x, out, idx, rows=list(range(w.n_q)))


def test_decode_b8_ctx128k_all_rows(announce):
    w = synth.WORKLOADS["decode_b8_ctx128k"]
    x = synth.make_inputs(w)
    announce(f"fused_forward {w}")
    out, idx = run_fused(w, x)
    check_rows(w, x, out, idx, rows=[0])


def test_decode_ctx1m_mqa_all_rows(announce):
    w = synth.WORKLOADS["decode_ctx1m_mqa"]
    x = synth.make_inputs(w)
    announce(f"fused_forward {w}")
    out, idx = run_fused(w, x)
    check_rows(w, x, out, idx, rows=[0])
    # planted rows are selected exactly when their score clears the threshold
    s = O.indexer_scores(x["q_idx"][0, 0], x["k_idx"][0], w.kv_len)
    sel = set(idx[0, 0].cpu().numpy().tolist())
    thr = s[sorted(sel)].min()
    for j in x["planted"]:
        if s[j] > thr:
            assert int(j) in sel
        elif s[j] < thr:
            assert int(j) not in sel


def test_prefill_32k_sampled_rows(announce):
    w = synth.WORKLOADS["prefill_32k"]
    x = synth.make_inputs(w)
    announce(f"fused_forward {w}")
    out, idx = run_fused(w, x)
    check_index_structure(w, idx)
    rows = synth.sample_rows(w, 64).tolist()
    announce(f"oracle on {len(rows)} sampled rows")
    check_rows(w, x, out, idx, rows=rows)


def test_elastic_prefill_64k_sampled_rows(announce):
    w = synth.WORKLOADS["elastic_prefill_64k"]
    x = synth.make_inputs(w)
    assert 0 < x["route"].sum() < x["route"].size     # both routes present
    announce(f"fused_forward {w}")
    out, idx = run_fused(w, x)
    # every index row of every sequence that has a sparse head
    sparse_seqs = [b for b in range(w.batch) if x["route"][b].any()]
    check_index_structure(w, idx, batches=sparse_seqs)
    # fixed rows (start, K boundary, end) plus 64 uniform rows of the interior
    rows = synth.sample_rows(w, 64).tolist()
    assert sum(2056 < r < w.n_q - 16 for r in rows) >= 60
    announce(f"oracle on {len(rows)} sampled rows x 2 sequences")
    check_rows(w, x, out, idx, rows=rows)
    del out, idx
    torch.cuda.empty_cache()


# --------------------------------------------------------------------------- edge cases, small shapes
def _w(B_, N, L, Hq, Hkv, d, didx, K, dt="bf16", route_p=None, seed=11):
    rng = (-4, 4) if dt == "bf16" else (-8, 8)
    return synth.Workload("edge", B_, N, L, Hq, Hkv, d, didx, K, dt, dt, rng,
                          route_sparse_p=route_p, seed=seed)


EDGE = [
    ("chunk_N_lt_L", _w(2, 100, 1000, 8, 2, 128, 64, 64)),
    ("K_ge_L", _w(1, 64, 64, 4, 1, 64, 32, 128)),
    ("K_eq_vis_boundary", _w(1, 40, 100, 4, 2, 64, 32, 70)),
    ("K_1", _w(2, 33, 77, 4, 4, 128, 16, 1)),
    ("ragged_decode_8193", _w(3, 1, 8193, 8, 2, 128, 64, 256)),
    ("ragged_decode_24577_spec3", _w(2, 3, 24577, 16, 2, 64, 128, 512)),
    ("decode_8_rows", _w(1, 8, 20000, 4, 1, 128, 64, 300)),
    ("prefill_9_rows_fp32", _w(1, 9, 3000, 4, 2, 128, 32, 200, dt="fp32")),
    ("mixed_route", _w(2, 70, 300, 8, 2, 128, 64, 32, route_p=0.5, seed=5)),
    ("fp32_d64", _w(1, 130, 130, 6, 3, 64, 64, 17, dt="fp32")),
    ("mqa_decode_many_heads", _w(1, 1, 50000, 64, 1, 128, 64, 2048)),
    ("spec_decode_4_rows", _w(2, 4, 30001, 8, 2, 128, 64, 1000)),
    ("decode_fp32_idx32", _w(3, 2, 9000, 4, 2, 64, 32, 333, dt="fp32")),
    ("decode_mixed_route", _w(4, 1, 12000, 8, 2, 128, 64, 500, route_p=0.5, seed=3)),
    ("decode_4_rows_long_ctx", _w(2, 4, 600000, 4, 1, 64, 64, 2048)),
    # dense-route heads over several 128-row tiles, ragged last tile and step
    ("mixed_route_3_tiles", _w(1, 300, 300, 8, 2, 128, 64, 48, route_p=0.5, seed=7)),
    ("mixed_route_d64_chunk", _w(2, 200, 461, 4, 1, 64, 32, 40, route_p=0.4, seed=9)),
    # single-row decode with fewer visible keys than K, and a short last chunk
    ("decode_L_lt_K", _w(2, 1, 300, 4, 2, 64, 32, 512)),
    ("decode_ragged_chunk", _w(5, 1, 3333, 8, 2, 128, 64, 700, seed=12)),
    # single-row decode: fp32 K/V (VALU attention reading the LDS index list),
    # K = 1, and a context that is one chunk
    ("decode_fp32_single_row", _w(3, 1, 9000, 4, 2, 64, 32, 333, dt="fp32")),
    ("decode_K_1", _w(3, 1, 5000, 4, 1, 64, 32, 1)),
    ("decode_one_chunk", _w(2, 1, 200, 4, 2, 64, 32, 100)),
]


@pytest.mark.parametrize("name,w", EDGE, ids=[e[0] for e in EDGE])
@pytest.mark.parametrize("use_gate", [True, False])
def test_edge_shapes(name, w, use_gate, announce):
    x = synth.make_inputs(w)
    announce(f"fused_forward {name} gate={use_gate} {w}")
    out, idx = run_fused(w, x, use_gate=use_gate)
    rows = list(range(w.n_q)) if w.n_q <= 320 else synth.sample_rows(w, 40).tolist()
    check_rows(w, x, out, idx, rows=rows, use_gate=use_gate)


@pytest.mark.parametrize("N,L", [(256, 300000), (64, 1048576)])
def test_long_context_prefill_chunk(N, L, announce):
    """A prefill chunk at the end of a long context (query rows over a long
    cache through the bottom-right causal alignment), up to a 1 M-token
    cache: rows wider than 65536 keys take the multi-pass top-k."""
    w = _w(1, N, L, 8, 2, 128, 64, 2048, seed=21)
    x = synth.make_inputs(w)
    announce(f"fused_forward {w}")
    out, idx = run_fused(w, x)
    check_index_structure(w, idx)
    check_rows(w, x, out, idx, rows=synth.sample_rows(w, 6).tolist())


@pytest.mark.parametrize("N,L", [(2, 20000), (200, 3000)])
def test_shared_key_indexer(N, L, announce):
    """The indexer run on the attention keys: the K cache itself is passed as
    k_idx (one KV head, d_idx = d).  The keys are integer-valued so that the
    scores, and with them the index rows, are exact."""
    w = _w(1, N, L, 8, 1, 128, 128, 256, seed=23)
    x = synth.make_inputs(w)
    x["k"] = x["k_idx"].reshape(1, L, 1, 128).astype(x["k"].dtype).copy()
    dev = to_device(w, x)
    p = B.problem_for(w)
    out = torch.empty((1, N, w.h_q, w.head_dim), dtype=torch.float32, device="cuda")
    idx = torch.full((1, N, w.top_k), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(1, B.dsa_workspace_size(p)), dtype=torch.uint8, device="cuda")
    announce(f"fused_forward, k_idx = K, {w}")
    B.dsa_fused_forward(p, dev["q_idx"], dev["k"], dev["q"], dev["k"], dev["v"], dev["gate"],
                        dev["y2"], None, out, idx, ws)
    torch.cuda.synchronize()
    rows = list(range(N)) if N <= 16 else synth.sample_rows(w, 16).tolist()
    check_rows(w, x, out, idx, rows=rows, use_route=False)


@pytest.mark.parametrize("kind", ["sampled_keys_high", "all_equal"])
def test_prefill_selection_fallback(kind, announce):
    """Prefill rows whose candidate list cannot be used must take the exact
    streamed selection.  sampled_keys_high: only every 4th key (the keys a
    strided sample of an 8192-key row sees) has a nonzero score, so the
    threshold estimated from the sample lets through fewer than K keys;
    all_equal: every score is equal, so every key is a candidate and the list
    overflows; the K lowest positions win."""
    w = _w(1, 64, 8192, 8, 2, 128, 64, 2048, seed=41)
    x = synth.make_inputs(w)
    if kind == "sampled_keys_high":
        x["q_idx"][:] = 1.0
        rng = np.random.default_rng(5)
        k = np.zeros_like(x["k_idx"])
        k[:, ::4, :] = rng.integers(0, 9, size=k[:, ::4, :].shape)
        k[:, ::4, 0] = np.maximum(k[:, ::4, 0], 1)      # every sampled key scores >= 1
        x["k_idx"] = k.astype(np.float32)
    else:
        x["q_idx"][:] = 1.0
        x["k_idx"][:] = 1.0
    announce(f"fused_forward prefill fallback {kind} {w}")
    out, idx = run_fused(w, x)
    check_index_structure(w, idx)
    if kind == "all_equal":
        assert torch.equal(idx[0, :, :].cpu(),
                           torch.arange(w.top_k, dtype=torch.int32).expand(w.n_q, -1))
    else:
        # the last rows see 2048 nonzero keys: exactly those are selected
        assert torch.all(idx[0, 60:] % 4 == 0).item()
    check_rows(w, x, out, idx, rows=[0, 1, 31, 62, 63])


def test_all_dense_route_skips_indexer(announce):
    w = _w(2, 50, 200, 4, 2, 128, 64, 16)
    x = synth.make_inputs(w)
    x["route"][:] = 0
    x["route"][1, 2] = 1      # sequence 1 keeps one sparse head
    announce(f"fused_forward all-dense seq 0 {w}")
    out, idx = run_fused(w, x)
    assert torch.all(idx[0] == -1).item()
    check_rows(w, x, out, idx, rows=list(range(w.n_q)))


@pytest.mark.parametrize("kind", ["window", "all_equal", "all_dense_seq"])
def test_decode_concentrated_top_k(kind, announce):
    """Single-row decode where each chunk passes on only its few largest keys.
    window: sequence 1's last 600 keys are boosted, so most of its top K sits
    in a few chunks; all_equal: every score of sequence 1 is equal, so its K
    lowest positions win.  Either way those chunks cannot pass on enough keys
    and sequence 1 must take the histogram phases while sequences 0 and 2 do
    not.  all_dense_seq: sequence 0 has only dense heads (no selection, index
    row all -1)."""
    w = _w(3, 1, 20000, 8, 2, 128, 64, 512, seed=13)
    x = synth.make_inputs(w)
    if kind == "window":
        x["k_idx"][1, -600:, :] *= 3
    elif kind == "all_equal":
        x["k_idx"][1] = 1.0
        x["q_idx"][1] = 1.0
    else:
        x["route"][0] = 0
    announce(f"fused_forward decode {kind} {w}")
    out, idx = run_fused(w, x)
    check_index_structure(w, idx, batches=[1, 2] if kind == "all_dense_seq" else None)
    if kind == "all_dense_seq":
        assert torch.all(idx[0] == -1).item()
    if kind == "all_equal":
        assert torch.equal(idx[1, 0].cpu(), torch.arange(w.top_k, dtype=torch.int32))
    check_rows(w, x, out, idx, rows=[0])


def test_custom_softmax_scale(announce):
    w = _w(1, 20, 90, 4, 1, 64, 32, 10, dt="fp32")
    x = synth.make_inputs(w)
    announce("fused_forward softmax_scale=0.05")
    out, idx = run_fused(w, x, softmax_scale=0.05)
    want, _ = O.forward(w, x, softmax_scale=0.05)
    assert np.max(np.abs(out.cpu().numpy() - want)) <= 1e-4


def test_gate_end_points_exact(announce):
    w = _w(1, 12, 60, 4, 2, 128, 64, 8)
    x = synth.make_inputs(w)
    x1 = dict(x, gate=np.ones_like(x["gate"]))
    announce("fused_forward gate=1 vs no gate")
    a1, _ = run_fused(w, x1)
    a, _ = run_fused(w, x, use_gate=False)
    assert torch.equal(a1, a)
    x0 = dict(x, gate=np.zeros_like(x["gate"]))
    a0, _ = run_fused(w, x0)
    assert np.array_equal(a0.cpu().numpy(), x["y2"])


def test_deterministic_repeat(announce):
    w = synth.WORKLOADS["decode_b8_ctx128k"].replace(kv_len=40000)
    x = synth.make_inputs(w)
    announce("fused_forward x3 determinism")
    o1, i1 = run_fused(w, x)
    o2, i2 = run_fused(w, x)
    o3, i3 = run_fused(w, x)
    assert torch.equal(o1, o2) and torch.equal(o1, o3)
    assert torch.equal(i1, i2) and torch.equal(i1, i3)


def run_entry_points(w, x):
    """The same forward through the three separate entry points (other
    kernels, other work split): scores, then top-k, then attention."""
    p = B.problem_for(w)
    dev = to_device(w, x)
    ws = torch.empty(max(1, B.dsa_workspace_size(p)), dtype=torch.uint8, device="cuda")
    scores = torch.empty((w.batch, w.n_q, w.kv_len), dtype=torch.float32, device="cuda")
    idx = torch.full((w.batch, w.n_q, w.top_k), -7, dtype=torch.int32, device="cuda")
    out = torch.empty((w.batch, w.n_q, w.h_q, w.head_dim), dtype=torch.float32, device="cuda")
    B.dsa_indexer_scores(p, dev["q_idx"], dev["k_idx"], scores)
    B.dsa_topk(p, scores, idx, ws)
    B.dsa_sparse_attn(p, dev["q"], dev["k"], dev["v"], idx, dev["gate"], dev["y2"], dev["route"],
                      out, ws)
    torch.cuda.synchronize()
    return out, idx


PLANS = [("decode_b8_ctx40k", synth.WORKLOADS["decode_b8_ctx128k"].replace(kv_len=40000)),
         ("decode_mqa_ctx200k", synth.WORKLOADS["decode_ctx1m_mqa"].replace(kv_len=200000)),
         ("prefill_3k_mixed_route", _w(2, 3000, 3000, 8, 2, 128, 64, 512, route_p=0.6, seed=31))]


@pytest.mark.parametrize("name,w", PLANS, ids=[p[0] for p in PLANS])
def test_same_result_under_another_plan(name, w, announce):
    """A race or an order-dependent reduction would show as a difference
    between two different work splits of the same problem: the fused call
    (one decode launch, or chunked prefill launches) against the separate
    entry points.  Index rows must agree bit for bit, outputs within the
    float tolerance (both are also compared with the oracle on some rows)."""
    x = synth.make_inputs(w)
    announce(f"fused_forward vs entry points {name} {w}")
    o1, i1 = run_fused(w, x)
    o2, i2 = run_entry_points(w, x)
    assert torch.equal(i1, i2)
    assert torch.max(torch.abs(o1 - o2)).item() <= TOL[w.qkv_dtype]
    rows = [0] if w.n_q == 1 else synth.sample_rows(w, 8).tolist()
    check_rows(w, x, o2, i2, rows=rows)


def test_decode_give_up_is_reported(announce):
    """A wait between decode workgroups that gives up must reach the caller:
    with a wait limit of 0 every wait gives up at once (every kernel still
    exits normally), the outputs are NaN, the index rows -1, and
    dsa_exec_status reports DSA_ERR_EXEC.  The next launch on the same
    workspace, with the default limit, is correct again."""
    w = synth.WORKLOADS["decode_b8_ctx128k"].replace(kv_len=30000)
    x = synth.make_inputs(w)
    p = B.problem_for(w)
    dev = to_device(w, x)
    ws = torch.empty(max(1, B.dsa_workspace_size(p)), dtype=torch.uint8, device="cuda")
    out = torch.zeros((w.batch, 1, w.h_q, w.head_dim), dtype=torch.float32, device="cuda")
    idx = torch.zeros((w.batch, 1, w.top_k), dtype=torch.int32, device="cuda")

    def fwd():
        B.dsa_fused_forward(p, dev["q_idx"], dev["k_idx"], dev["q"], dev["k"], dev["v"],
                            dev["gate"], dev["y2"], dev["route"], out, idx, ws)

    announce("decode with wait limit 0")
    B.dsa_set_wait_limit(0)
    try:
        fwd()
        with pytest.raises(B.DsaError) as ei:
            B.dsa_exec_status(ws)
        assert ei.value.status == B.DSA_ERR_EXEC
    finally:
        B.dsa_set_wait_limit(1 << 24)
    assert torch.all(torch.isnan(out)).item()
    assert torch.all(idx == -1).item()
    announce("decode again with the default limit")
    fwd()
    B.dsa_exec_status(ws)      # raises on failure
    check_rows(w, x, out, idx, rows=[0])


# --------------------------------------------------------------------------- single entry points
@pytest.mark.parametrize("N,L,didx,dt", [(1, 5000, 64, "bf16"), (5, 777, 32, "fp32"),
                                          (100, 333, 64, "bf16"), (64, 64, 128, "fp32"),
                                          # MFMA tiles: vector stores (L % 4 == 0), d_idx 32/128
                                          (130, 1000, 32, "bf16"), (70, 600, 128, "bf16")])
def test_indexer_scores_entry(N, L, didx, dt, announce):
    w = _w(2, N, L, 4, 1, 64, didx, 8, dt=dt)
    x = synth.make_inputs(w, parts=("q_idx", "k_idx"))
    dev = to_device(w, x)
    p = B.problem_for(w)
    scores = torch.empty((2, N, L), dtype=torch.float32, device="cuda")
    announce(f"indexer_scores N={N} L={L} didx={didx} {dt}")
    B.dsa_indexer_scores(p, dev["q_idx"], dev["k_idx"], scores)
    got = scores.cpu().numpy()
    for b in range(2):
        for n in range(N):
            vis = O.visible_count(n, N, L)
            want = O.indexer_scores(x["q_idx"][b, n], x["k_idx"][b], vis)
            assert np.array_equal(got[b, n, :vis].astype(np.float64), want)
            assert np.all(np.isneginf(got[b, n, vis:]))


def _adversarial_rows(L, rng):
    rows = [np.zeros(L, np.float32),                       # all equal
            np.arange(L, dtype=np.float32),                # s_j = j
            -np.arange(L, dtype=np.float32),               # s_j = -j
            np.where(rng.random(L) < 0.5, -0.0, 0.0).astype(np.float32),   # signed zeros
            rng.integers(-3, 4, size=L).astype(np.float32)]
    peaks = np.full(L, -5.0, np.float32)                   # maxima on chunk boundaries
    for j in range(0, L, 8192):
        peaks[j] = 9.0
        if j > 0:
            peaks[j - 1] = 9.0
    rows.append(peaks)
    rows.append(rng.standard_normal(L).astype(np.float32))  # non-integer scores
    return np.stack(rows)


@pytest.mark.parametrize("L,K", [(40000, 2048), (20000, 1), (3000, 2999), (3000, 3000),
                                  (3000, 3001), (16384, 8192)])
@pytest.mark.parametrize("n_rows", [7, 1, 9])      # split-row path (<= 8 rows), rows path (9)
def test_topk_entry_adversarial(L, K, n_rows, announce):
    rng = np.random.default_rng(L + K)
    base = _adversarial_rows(L, rng)
    extra = rng.integers(-2, 3, size=(max(0, n_rows - base.shape[0]), L)).astype(np.float32)
    rows = np.concatenate([base, extra])[:n_rows]
    w = _w(1, n_rows, L, 4, 1, 64, 32, K)
    sc = np.full((1, n_rows, L), -np.inf, np.float32)
    for n in range(n_rows):
        vis = O.visible_count(n, n_rows, L)
        sc[0, n, :vis] = rows[n, :vis]
    p = B.problem_for(w)
    ws = torch.empty(max(1, B.dsa_workspace_size(p)), dtype=torch.uint8, device="cuda")
    idx = torch.full((1, n_rows, K), -7, dtype=torch.int32, device="cuda")
    announce(f"topk L={L} K={K} rows={n_rows}")
    B.dsa_topk(p, torch.from_numpy(sc).cuda(), idx, ws)
    got = idx.cpu().numpy()
    for n in range(n_rows):
        vis = O.visible_count(n, n_rows, L)
        want = O.select_top_k(sc[0, n, :vis].astype(np.float64), K)
        assert np.array_equal(got[0, n], want), f"row {n}"


def test_topk_entry_many_rows(announce):
    """The one-row-per-workgroup path (N > 8) on prefill-shaped scores."""
    w = _w(2, 300, 5000, 4, 1, 64, 64, 700)
    x = synth.make_inputs(w, parts=("q_idx", "k_idx"))
    sc = np.full((2, 300, 5000), -np.inf, np.float32)
    for b in range(2):
        for n in range(300):
            vis = O.visible_count(n, 300, 5000)
            sc[b, n, :vis] = O.indexer_scores(x["q_idx"][b, n], x["k_idx"][b], vis)
    p = B.problem_for(w)
    ws = torch.empty(max(1, B.dsa_workspace_size(p)), dtype=torch.uint8, device="cuda")
    idx = torch.empty((2, 300, 700), dtype=torch.int32, device="cuda")
    announce("topk many rows")
    B.dsa_topk(p, torch.from_numpy(sc).cuda(), idx, ws)
    got = idx.cpu().numpy()
    for b in range(2):
        for n in range(0, 300, 7):
            vis = O.visible_count(n, 300, 5000)
            assert np.array_equal(got[b, n], O.select_top_k(sc[b, n, :vis].astype(np.float64), 700))


@pytest.mark.parametrize("N,L,K,route_p", [(1, 9000, 512, None), (40, 600, 64, 0.5),
                                            (4, 3000, 100, 0.5)])
def test_sparse_attn_entry_with_oracle_indices(N, L, K, route_p, announce):
    w = _w(2, N, L, 8, 2, 128, 64, K, route_p=route_p)
    x = synth.make_inputs(w)
    want_out, want_idx = O.forward(w, x)
    dev = to_device(w, x)
    p = B.problem_for(w)
    ws = torch.empty(max(1, B.dsa_workspace_size(p)), dtype=torch.uint8, device="cuda")
    idx = torch.from_numpy(want_idx.astype(np.int32)).cuda()
    out = torch.empty((2, N, 8, 128), dtype=torch.float32, device="cuda")
    announce(f"sparse_attn N={N} L={L} K={K}")
    B.dsa_sparse_attn(p, dev["q"], dev["k"], dev["v"], idx, dev["gate"], dev["y2"], dev["route"],
                      out, ws)
    torch.cuda.synchronize()
    assert np.max(np.abs(out.cpu().numpy() - want_out)) <= TOL["bf16"]


# --------------------------------------------------------------------------- per-head selection
# One indexer query per (token, indexer head) and one selected set per indexer
# head; query head h attends over set h / (Hq / idx_heads).
PER_HEAD = [
    # the 8-sequence decode shape (32 query, 8 KV heads) at a 32K context: sets
    # spanning two KV heads, and one set per query head
    ("decode_b8_ctx32k_ih4", synth.WORKLOADS["decode_b8_ctx128k"].replace(
        kv_len=32768, idx_heads=4)),
    ("decode_b8_ctx32k_ih32", synth.WORKLOADS["decode_b8_ctx128k"].replace(
        kv_len=32768, idx_heads=32)),
    # 2 tokens x 4 heads = 8 index rows: streaming indexer and split-row top-k
    ("spec_decode_ih4", _w(2, 2, 20000, 8, 2, 128, 64, 300).replace(idx_heads=4)),
    # prefill over several key ranges (key-range attention, on-chip indexer)
    ("prefill_ih2_mixed_route", _w(1, 600, 9000, 8, 2, 128, 64, 512, route_p=0.6,
                                   seed=31).replace(idx_heads=2)),
    ("prefill_ih8_one_set_per_head", _w(2, 300, 5000, 8, 4, 64, 32, 256,
                                        seed=32).replace(idx_heads=8)),
    # float32: score matrix, row top-k and the VALU attention
    ("prefill_fp32_ih2", _w(1, 70, 500, 4, 2, 64, 32, 40, dt="fp32").replace(idx_heads=2)),
    ("K_ge_L_ih4", _w(1, 64, 64, 4, 1, 64, 32, 128).replace(idx_heads=4)),
]


@pytest.mark.parametrize("name,w", PER_HEAD, ids=[e[0] for e in PER_HEAD])
def test_per_head_selection(name, w, announce):
    x = synth.make_inputs(w)
    announce(f"fused_forward per-head {name} {w}")
    out, idx = run_fused(w, x)
    sparse_seqs = [b for b in range(w.batch) if x["route"][b].any()]
    check_index_structure(w, idx, batches=sparse_seqs)
    rows = list(range(w.n_q)) if w.n_q <= 80 else synth.sample_rows(w, 24).tolist()
    check_rows(w, x, out, idx, rows=rows)
    # the sets differ between indexer heads (else the test would not tell them apart)
    if w.kv_len > w.top_k:
        t = idx[sparse_seqs[0], -1]
        assert not all(torch.equal(t[0], t[i]) for i in range(1, t.shape[0]))


def test_per_head_entry_points(announce):
    """dsa_indexer_scores -> dsa_topk -> dsa_sparse_attn with four indexer
    heads: scores [B,N,H,L] exact, index rows exact, outputs within tolerance."""
    w = _w(2, 40, 300, 8, 2, 128, 64, 32, route_p=0.7, seed=33).replace(idx_heads=4)
    x = synth.make_inputs(w)
    dev = to_device(w, x)
    p = B.problem_for(w)
    H = w.idx_heads
    announce(f"indexer/topk/sparse_attn per-head {w}")
    scores = torch.empty((w.batch, w.n_q, H, w.kv_len), dtype=torch.float32, device="cuda")
    B.dsa_indexer_scores(p, dev["q_idx"], dev["k_idx"], scores)
    ws = torch.empty(max(1, B.dsa_workspace_size(p)), dtype=torch.uint8, device="cuda")
    idx = torch.full(idx_shape(w), -7, dtype=torch.int32, device="cuda")
    B.dsa_topk(p, scores, idx, ws)
    out = torch.empty((w.batch, w.n_q, w.h_q, w.head_dim), dtype=torch.float32, device="cuda")
    B.dsa_sparse_attn(p, dev["q"], dev["k"], dev["v"], idx, dev["gate"], dev["y2"],
                      dev["route"], out, ws)
    torch.cuda.synchronize()
    got = scores.cpu().numpy()
    L, N = w.kv_len, w.n_q
    for b in range(w.batch):
        for n in range(N):
            vis = L - N + n + 1
            for i in range(H):
                want = O.indexer_scores(x["q_idx"][b, n, i], x["k_idx"][b], vis)
                assert np.array_equal(got[b, n, i, :vis], want[:vis].astype(np.float32))
                assert np.all(np.isneginf(got[b, n, i, vis:]))
    # the index rows of every head (route does not enter the top-k call)
    want_out, want_idx = O.forward(w, x, use_route=False)
    assert np.array_equal(idx.cpu().numpy(), want_idx)
    want_out, _ = O.forward(w, x)
    err = np.max(np.abs(out.cpu().numpy().astype(np.float64) - want_out))
    assert err <= TOL[w.qkv_dtype], f"max-abs error {err}"


# --------------------------------------------------------------------------- route producer
# Logits within ROUTE_TOL of the oracle (fp32 sums against float64; the router
# weights are scaled so that logits are of order one); the decision must match
# the oracle's wherever the oracle's two logits are more than 2 * ROUTE_TOL
# apart, and always match the kernel's own logits (larger logit, tie -> full).
ROUTE_TOL = 2e-3


def _router_dev(r):
    return {k: torch.from_numpy(v).cuda() for k, v in r.items()}


def run_route(w, x, r, want_logits=True):
    p = B.problem_for(w)
    rd = _router_dev(r)
    rr = B.router(rd["w1"], rd["b1"], rd["w2"], rd["b2"])
    k = to_device(w, {"k": x["k"]})["k"]
    route = torch.full((w.batch, w.h_q), 7, dtype=torch.uint8, device="cuda")
    logits = (torch.empty((w.batch, w.h_q, 2), dtype=torch.float32, device="cuda")
              if want_logits else None)
    ws = torch.empty(max(1, B.dsa_route_workspace_size(p, rr)), dtype=torch.uint8, device="cuda")
    B.dsa_route_heads(p, rr, k, route, logits, ws)
    torch.cuda.synchronize()
    return route.cpu().numpy(), (logits.cpu().numpy() if want_logits else None)


def check_route(w, x, r, route, logits):
    want_z, want_r = O.route_batch(w, x["k"], r)
    err = np.max(np.abs(logits.astype(np.float64) - want_z))
    assert err <= ROUTE_TOL, f"logit error {err}"
    np.testing.assert_array_equal(route, (logits[..., 1] > logits[..., 0]).astype(np.uint8))
    clear = np.abs(want_z[..., 1] - want_z[..., 0]) > 2 * ROUTE_TOL
    assert clear.mean() > 0.9
    np.testing.assert_array_equal(route[clear], want_r[clear])
    return err


ROUTE_CASES = [
    # 64K-token prefill of two sequences, 8 KV heads x 128 (the elastic workload)
    ("elastic_prefill_64k", synth.WORKLOADS["elastic_prefill_64k"], 256),
    # decode: one current token per sequence
    ("decode_b8", synth.WORKLOADS["decode_b8_ctx128k"].replace(kv_len=4096), 256),
    # fp32 keys, a hidden width and head count off the 64-lane grid
    ("fp32_odd_sizes", _w(3, 333, 1000, 6, 3, 64, 32, 16, dt="fp32"), 100),
    # rows wider than 2048 values (24 KV heads x 128), one hidden unit
    ("wide_rows", _w(2, 50, 70, 48, 24, 128, 64, 16), 1),
    # 192-value rows: 24 column groups, ten row lanes per workgroup
    ("row_192", _w(1, 1000, 1000, 9, 3, 64, 32, 16), 64),
]


@pytest.mark.parametrize("name,w,hidden", ROUTE_CASES, ids=[c[0] for c in ROUTE_CASES])
def test_route_heads_matches_oracle(name, w, hidden, announce):
    x = synth.make_inputs(w, parts=("k",))
    r = synth.make_router(w, hidden=hidden)
    announce(f"route_heads {name} hidden={hidden} {w}")
    route, logits = run_route(w, x, r)
    check_route(w, x, r, route, logits)
    # the same inputs give the same bits; logits are optional
    route2, logits2 = run_route(w, x, r)
    assert np.array_equal(logits2.view(np.uint32), logits.view(np.uint32))
    route3, _ = run_route(w, x, r, want_logits=False)
    np.testing.assert_array_equal(route3, route)


@pytest.mark.parametrize("shape", ["prefill", "decode"])
def test_fused_forward_routed(shape, announce):
    """The route made on the device feeds the forward: route_out equals
    dsa_route_heads' decision and the output is the oracle's under it."""
    if shape == "prefill":
        w = _w(2, 300, 5000, 8, 2, 128, 64, 256, seed=35)
    else:
        w = _w(4, 1, 20000, 8, 2, 128, 64, 512, seed=36)
    x = synth.make_inputs(w)
    r = synth.make_router(w, hidden=64)
    route_ref, _ = run_route(w, x, r, want_logits=False)
    assert 0 < route_ref.sum() < route_ref.size          # both routes present
    p = B.problem_for(w)
    rd = _router_dev(r)
    rr = B.router(rd["w1"], rd["b1"], rd["w2"], rd["b2"])
    dev = to_device(w, x)
    route = torch.full((w.batch, w.h_q), 7, dtype=torch.uint8, device="cuda")
    out = torch.empty((w.batch, w.n_q, w.h_q, w.head_dim), dtype=torch.float32, device="cuda")
    idx = torch.full(idx_shape(w), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(1, B.dsa_route_workspace_size(p, rr)), dtype=torch.uint8, device="cuda")
    announce(f"fused_forward_routed {shape} {w}")
    B.dsa_fused_forward_routed(p, rr, dev["q_idx"], dev["k_idx"], dev["q"], dev["k"], dev["v"],
                               dev["gate"], dev["y2"], route, out, idx, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(route.cpu().numpy(), route_ref)
    x["route"] = route_ref
    rows = list(range(w.n_q)) if w.n_q <= 16 else synth.sample_rows(w, 16).tolist()
    check_rows(w, x, out, idx, rows=rows)
