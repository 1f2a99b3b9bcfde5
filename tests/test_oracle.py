"""Pins of the CPU oracle against things other than itself (CPU only).

Each test ties one oracle function to a closed form, a brute-force search, a
library routine (torch's scaled_dot_product_attention in float64 on the CPU)
or a hand-derived worked example under tests/golden.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import dsa_oracle as O
from top_sparse_attention_indexer_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


class P:  # plain parameter bag for oracle.forward
    def __init__(self, **kw):
        self.__dict__.update(kw)


def _golden():
    with open(GOLDEN, encoding="utf-8") as f:
        return json.load(f)


# --------------------------------------------------------------------------- visibility
def test_visible_count_alignment():
    # prefill N == L: row n sees n + 1 keys; decode N == 1: sees all L
    assert [O.visible_count(n, 5, 5) for n in range(5)] == [1, 2, 3, 4, 5]
    assert O.visible_count(0, 1, 131072) == 131072
    # chunk of the last 3 of 10 positions
    assert [O.visible_count(n, 3, 10) for n in range(3)] == [8, 9, 10]


# --------------------------------------------------------------------------- indexer
def test_indexer_golden():
    g = _golden()["indexer"]
    s = O.indexer_scores(np.array(g["q_idx"], np.float32), np.array(g["k_idx"], np.float32), 4)
    assert s.tolist() == g["scores"]
    # a visible count of 2 drops the later keys
    assert O.indexer_scores(np.array(g["q_idx"]), np.array(g["k_idx"]), 2).tolist() == g["scores"][:2]


def test_indexer_one_hot_query_reads_a_column():
    rng = np.random.default_rng(0)
    k = rng.integers(-8, 9, size=(37, 32)).astype(np.float32)
    for c in (0, 5, 31):
        q = np.zeros(32, np.float32)
        q[c] = 1
        assert np.array_equal(O.indexer_scores(q, k, 37), k[:, c].astype(np.float64))
        q[c] = -3
        assert np.array_equal(O.indexer_scores(q, k, 37), -3 * k[:, c].astype(np.float64))


def test_indexer_closed_form_ramp():
    # k_j = j * (1, 2, ..., d); q = ones  =>  s_j = j * d (d + 1) / 2
    d = 64
    k = np.arange(50)[:, None] * np.arange(1, d + 1)[None, :]
    q = np.ones(d)
    assert np.array_equal(O.indexer_scores(q, k.astype(np.float32), 50), np.arange(50) * d * (d + 1) / 2)


def test_indexer_integer_inputs_give_exact_integers():
    w = synth.WORKLOADS["decode_b8_ctx128k"].replace(batch=1, kv_len=4096)
    x = synth.make_inputs(w, parts=("q_idx", "k_idx"))
    s = O.indexer_scores(x["q_idx"][0, 0], x["k_idx"][0], 4096)
    assert np.all(s == np.round(s)) and np.max(np.abs(s)) <= 64 * 16


# --------------------------------------------------------------------------- top-k
def _brute_force_top_k(s, k):
    """The unique k-subset S with: i in S, u not in S => s_i > s_u or (s_i == s_u and i < u)."""
    vis = len(s)
    if vis <= k:
        return list(range(vis))
    found = []
    for cand in itertools.combinations(range(vis), k):
        cs = set(cand)
        ok = all(s[i] > s[u] or (s[i] == s[u] and i < u)
                 for i in cand for u in range(vis) if u not in cs)
        if ok:
            found.append(list(cand))
    assert len(found) == 1
    return found[0]


def test_top_k_brute_force_tiny_rows():
    rng = np.random.default_rng(1)
    for trial in range(120):
        vis = int(rng.integers(1, 10))
        s = rng.integers(-2, 3, size=vis).astype(np.float64)   # many ties
        for k in range(1, 11):
            want = _brute_force_top_k(list(s), k)
            got = O.select_top_k(s, k)
            assert got.tolist() == want + [-1] * (k - len(want)), (s, k)


def test_top_k_golden():
    g = _golden()
    s = np.array(g["top_k"]["scores"], np.float64)
    for k, want in g["top_k"]["cases"]:
        assert O.select_top_k(s, k).tolist() == want
    z = g["top_k_signed_zero"]
    s = np.array([float(x) for x in z["scores"]])
    assert np.signbit(s[0]) and not np.signbit(s[1])
    assert O.select_top_k(s, z["k"]).tolist() == z["idx"]


@pytest.mark.parametrize("vis,k", [(100, 7), (2049, 2048), (5000, 2048), (64, 64), (65, 64)])
def test_top_k_closed_forms(vis, k):
    eq = np.zeros(vis)
    assert O.select_top_k(eq, k).tolist()[:min(k, vis)] == list(range(min(k, vis)))
    up = np.arange(vis, dtype=np.float64)
    want = list(range(max(0, vis - k), vis))
    assert O.select_top_k(up, k).tolist()[:len(want)] == want
    down = -np.arange(vis, dtype=np.float64)
    assert O.select_top_k(down, k).tolist()[:min(k, vis)] == list(range(min(k, vis)))


def test_top_k_invariants_random_rows():
    rng = np.random.default_rng(2)
    for vis, k in [(5000, 64), (3000, 2048), (2048, 2048), (2047, 2048), (9000, 1)]:
        s = rng.integers(-40, 41, size=vis).astype(np.float64)
        idx = O.select_top_k(s, k)
        sel = idx[idx >= 0]
        assert len(sel) == min(k, vis)
        assert np.all(np.diff(sel) > 0) and np.all(idx[len(sel):] == -1)
        if vis > k:
            mask = np.zeros(vis, bool)
            mask[sel] = True
            thr = s[sel].min()
            assert thr >= s[~mask].max()
            # ties at the threshold: every unselected tie sits above every selected tie
            tied_sel = np.nonzero(mask & (s == thr))[0]
            tied_un = np.nonzero(~mask & (s == thr))[0]
            if len(tied_un):
                assert tied_sel.max() < tied_un.min()


# --------------------------------------------------------------------------- attention
def _sdpa(q, k, v, mask):
    """torch SDPA in float64 on the CPU. q [N,Hq,d], k/v [L,Hkv,d], mask [N,L] bool."""
    tq = torch.from_numpy(q.astype(np.float64)).permute(1, 0, 2)[None]
    tk = torch.from_numpy(k.astype(np.float64)).permute(1, 0, 2)[None].contiguous()
    tv = torch.from_numpy(v.astype(np.float64)).permute(1, 0, 2)[None].contiguous()
    out = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=torch.from_numpy(mask)[None, None], enable_gqa=True)
    return out[0].permute(1, 0, 2).numpy()


def _bottom_right_mask(n_q, kv_len):
    return np.arange(kv_len)[None, :] <= (kv_len - n_q + np.arange(n_q))[:, None]


def _small(n_q, kv_len, h_q, h_kv, d, d_idx, k, seed, route=None):
    w = synth.Workload("t", 1, n_q, kv_len, h_q, h_kv, d, d_idx, k, "fp32", "fp32", (-3, 3),
                       route_sparse_p=route, seed=seed)
    return w, synth.make_inputs(w)


@pytest.mark.parametrize("n_q,kv_len,h_q,h_kv", [(9, 9, 4, 1), (5, 12, 4, 2), (1, 30, 6, 3), (7, 7, 2, 2)])
def test_dense_path_matches_sdpa(n_q, kv_len, h_q, h_kv):
    w, x = _small(n_q, kv_len, h_q, h_kv, 16, 8, 4, seed=3)
    got = O.dense_causal_attention(x["q"][0], x["k"][0], x["v"][0])
    want = _sdpa(x["q"][0], x["k"][0], x["v"][0], _bottom_right_mask(n_q, kv_len))
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("n_q,kv_len", [(12, 12), (4, 15), (1, 20)])
def test_sparse_with_k_at_least_visible_is_dense_causal(n_q, kv_len):
    w, x = _small(n_q, kv_len, 4, 2, 16, 8, kv_len, seed=4)
    out, idx = O.forward(w, x, use_gate=False)
    want = _sdpa(x["q"][0], x["k"][0], x["v"][0], _bottom_right_mask(n_q, kv_len))
    np.testing.assert_allclose(out[0], want, rtol=0, atol=1e-12)
    for n in range(n_q):
        vis = O.visible_count(n, n_q, kv_len)
        assert idx[0, n].tolist() == list(range(vis)) + [-1] * (kv_len - vis)


@pytest.mark.parametrize("n_q,kv_len,k", [(16, 16, 3), (6, 25, 5), (1, 40, 7)])
def test_sparse_matches_masked_sdpa(n_q, kv_len, k):
    """Sparse attention equals dense SDPA with every unselected key masked out."""
    w, x = _small(n_q, kv_len, 4, 2, 16, 8, k, seed=5)
    out, idx = O.forward(w, x, use_gate=False)
    mask = np.zeros((n_q, kv_len), bool)
    for n in range(n_q):
        sel = idx[0, n][idx[0, n] >= 0]
        mask[n, sel] = True
        # the selection itself: brute force on the exact integer scores
        vis = O.visible_count(n, n_q, kv_len)
        s = x["k_idx"][0, :vis].astype(np.int64) @ x["q_idx"][0, n].astype(np.int64)
        if vis <= 9:
            assert sel.tolist() == _brute_force_top_k(list(s), k)
    want = _sdpa(x["q"][0], x["k"][0], x["v"][0], mask)
    np.testing.assert_allclose(out[0], want, rtol=0, atol=1e-12)


def test_attention_golden_and_weights():
    g = _golden()["attention"]
    a, wts = O.softmax_attention(np.array(g["q"]), np.array(g["k"]), np.array(g["v"]), 0.5)
    np.testing.assert_allclose(wts, g["weights"], atol=1e-15)
    np.testing.assert_allclose(a, g["out"], atol=1e-14)


def test_attention_special_cases():
    rng = np.random.default_rng(6)
    q = rng.standard_normal(32)
    keys = rng.standard_normal((50, 32)) * 3
    # V == 1 gives 1; weights sum to 1
    a, wts = O.softmax_attention(q, keys, np.ones((50, 32)), 1 / math.sqrt(32))
    np.testing.assert_allclose(a, 1.0, atol=1e-13)
    assert abs(wts.sum() - 1) < 1e-12 and np.all(wts > 0)
    # one-hot V rows give the weight vector
    a, wts = O.softmax_attention(q, keys, np.eye(50), 1 / math.sqrt(32))
    np.testing.assert_allclose(a, wts, atol=1e-15)
    # larger logits get larger weights (monotone in the scaled product)
    t = keys @ q
    assert np.all(np.argsort(t) == np.argsort(wts))
    # a single visible key returns its value row
    a, wts = O.softmax_attention(q, keys[:1], keys[3:4], 0.1)
    np.testing.assert_allclose(a, keys[3], atol=0) and np.testing.assert_allclose(wts, [1.0])


# --------------------------------------------------------------------------- gate and route
def test_gate_golden_and_end_points():
    g = _golden()["gate"]
    np.testing.assert_allclose(O.gate_blend(np.array(g["a"]), g["g"], np.array(g["y2"])), g["out"], atol=0)
    rng = np.random.default_rng(7)
    a = rng.standard_normal(64)
    y2 = rng.standard_normal(64).astype(np.float32)
    assert np.array_equal(O.gate_blend(a, 1.0, y2), a)
    assert np.array_equal(O.gate_blend(a, 0.0, y2), y2.astype(np.float64))
    mid = O.gate_blend(a, 0.3, y2)
    assert np.all(mid <= np.maximum(a, y2) + 1e-15) and np.all(mid >= np.minimum(a, y2) - 1e-15)


def test_gate_end_points_through_forward():
    w, x = _small(6, 10, 4, 2, 16, 8, 3, seed=8)
    plain, _ = O.forward(w, x, use_gate=False)
    x1 = dict(x, gate=np.ones_like(x["gate"]))
    out1, _ = O.forward(w, x1)
    assert np.array_equal(out1, plain)
    x0 = dict(x, gate=np.zeros_like(x["gate"]))
    out0, _ = O.forward(w, x0)
    assert np.array_equal(out0[0], x["y2"][0].astype(np.float64))


def test_route_dense_heads_follow_dense_path():
    w, x = _small(8, 14, 4, 2, 16, 8, 3, seed=9)
    x["route"] = np.array([[1, 0, 0, 1]], np.uint8)
    out, idx = O.forward(w, x, use_gate=False)
    dense = O.dense_causal_attention(x["q"][0], x["k"][0], x["v"][0])
    np.testing.assert_allclose(out[0][:, [1, 2]], dense[:, [1, 2]], atol=1e-12)
    sparse_only, _ = O.forward(w, x, use_gate=False, use_route=False)
    np.testing.assert_allclose(out[0][:, [0, 3]], sparse_only[0][:, [0, 3]], atol=0)
    # all heads dense: the indexer is skipped and the index rows are -1
    x["route"] = np.zeros((1, 4), np.uint8)
    out, idx = O.forward(w, x, use_gate=False)
    assert np.all(idx == -1)
    np.testing.assert_allclose(out[0], dense, atol=1e-12)


def test_forward_golden():
    g = _golden()["forward"]
    p = P(batch=1, **{k: v for k, v in g["dims"].items() if k != "batch" and k != "idx_dim"})
    x = {k: np.array(g[k], np.float64) for k in ("q_idx", "k_idx", "q", "k", "v", "gate", "y2")}
    x["route"] = np.array(g["route"], np.uint8)
    out, idx = O.forward(p, x)
    assert idx.tolist() == g["idx"]
    np.testing.assert_allclose(out, g["out"], atol=1e-14)


def test_gqa_mapping_groups_are_contiguous():
    """Hq=4, Hkv=2: heads 0,1 read KV head 0 and heads 2,3 read KV head 1."""
    w, x = _small(3, 3, 4, 2, 8, 4, 8, seed=10)
    x["v"][0, :, 0, :] = 1.0
    x["v"][0, :, 1, :] = 2.0
    out, _ = O.forward(w, x, use_gate=False)
    np.testing.assert_allclose(out[0, :, :2], 1.0, atol=1e-14)
    np.testing.assert_allclose(out[0, :, 2:], 2.0, atol=1e-14)


# --------------------------------------------------------------------------- generator
def test_synth_is_seeded_and_typed():
    w = synth.WORKLOADS["tiny_prefill_fp32"]
    a = synth.make_inputs(w)
    b = synth.make_inputs(w)
    for key in a:
        assert np.array_equal(a[key], b[key])
    assert a["q_idx"].min() >= -8 and a["q_idx"].max() <= 8
    assert np.all(a["q_idx"] == np.round(a["q_idx"]))
    w2 = synth.WORKLOADS["decode_b8_ctx128k"].replace(kv_len=2048)
    c = synth.make_inputs(w2)
    for key in ("q", "k", "v"):
        synth.to_bf16_bits(c[key])    # raises unless bf16-exact
    assert c["route"].shape == (8, 32) and np.all(c["route"] == 1)
    sub = synth.make_inputs(w2, parts=("k",))
    assert np.array_equal(sub["k"], c["k"])


def test_synth_bf16_rounding_ties_to_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e38], np.float32)
    r = synth.round_to_bf16(x)
    assert r[0] == 1.0 and r[1] == 1.0 and r[2] == 1.0 + 2 ** -6 and r[3] == -2.5


def test_synth_planted_rows():
    w = synth.WORKLOADS["decode_ctx1m_mqa"].replace(kv_len=1 << 16)
    x = synth.make_inputs(w, parts=("k_idx",))
    pos = x["planted"]
    assert len(np.unique(pos)) == 16
    assert np.max(np.abs(x["k_idx"][0, pos])) > 4 and np.max(np.abs(np.delete(x["k_idx"][0], pos, 0))) <= 4


# --------------------------------------------------------------------------- per-head selection
def _per_head(n_q, kv_len, h_q, h_kv, ih, k, seed):
    w = synth.Workload("ph", 1, n_q, kv_len, h_q, h_kv, 16, 8, k, "fp32", "fp32", (-3, 3),
                       seed=seed, idx_heads=ih)
    return w, synth.make_inputs(w)


@pytest.mark.parametrize("n_q,kv_len,h_q,h_kv,ih,k", [(5, 9, 4, 2, 4, 3), (3, 8, 4, 1, 2, 4),
                                                      (6, 6, 8, 2, 8, 2), (1, 9, 4, 4, 4, 5)])
def test_per_head_selection_matches_per_head_masked_sdpa(n_q, kv_len, h_q, h_kv, ih, k):
    """Per-head top-k ([GDSA] §四.1 pseudo-code: indices [batch, heads, top_k]):
    each indexer head's set is the brute-force top-k of its own exact integer
    scores, and query head h attends over set h // (Hq / H), i.e. SDPA with a
    per-head mask of that set."""
    w, x = _per_head(n_q, kv_len, h_q, h_kv, ih, k, seed=8)
    assert x["q_idx"].shape == (1, n_q, ih, 8)
    out, idx = O.forward(w, x, use_gate=False)
    assert idx.shape == (1, n_q, ih, k)
    want = np.zeros_like(out[0])
    for h in range(h_q):
        mask = np.zeros((n_q, kv_len), bool)
        for n in range(n_q):
            vis = O.visible_count(n, n_q, kv_len)
            s = x["k_idx"][0, :vis].astype(np.int64) @ x["q_idx"][0, n, h // (h_q // ih)].astype(np.int64)
            sel = _brute_force_top_k(list(s), k)
            assert idx[0, n, h // (h_q // ih)].tolist() == sel + [-1] * (k - len(sel))
            mask[n, sel] = True
        hk = h // (h_q // h_kv)
        want[:, h] = _sdpa(x["q"][0][:, h:h + 1], x["k"][0][:, hk:hk + 1], x["v"][0][:, hk:hk + 1],
                           mask)[:, 0]
    np.testing.assert_allclose(out[0], want, rtol=0, atol=1e-12)


def test_per_head_with_equal_queries_is_the_shared_selection():
    """Every indexer head given the same query selects the shared set, and the
    outputs equal those of the shared selection."""
    w1, x1 = _small(7, 20, 8, 2, 16, 8, 5, seed=9)
    wh = w1.replace(idx_heads=4)
    xh = dict(x1, q_idx=np.repeat(x1["q_idx"][:, :, None, :], 4, axis=2))
    o1, i1 = O.forward(w1, x1)
    oh, ih = O.forward(wh, xh)
    assert np.array_equal(ih, np.repeat(i1[:, :, None, :], 4, axis=2))
    assert np.array_equal(oh, o1)


# --------------------------------------------------------------------------- route producer
def test_router_golden():
    """Hand-derived example: mean pooling, a unit cut by the ReLU, the bias,
    and a tie that keeps full attention ([EA] §2.2)."""
    g = _golden()["router"]
    k = np.array(g["k_current"], dtype=np.float64)
    logits, route = O.route_heads(k, np.array(g["w1"], float), np.array(g["b1"], float),
                                  np.array(g["w2"], float), np.array(g["b2"], float))
    np.testing.assert_array_equal(logits, np.array(g["logits"], float))
    np.testing.assert_array_equal(route, np.array(g["route"], np.uint8))


def _router_case(seed=3, n=5, h_kv=2, d=8, hidden=16, h_q=6):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((n, h_kv, d))
    r = {"w1": rng.standard_normal((h_kv * d, hidden)), "b1": rng.standard_normal(hidden),
         "w2": rng.standard_normal((hidden, h_q, 2)), "b2": rng.standard_normal((h_q, 2))}
    return k, r


def test_router_matches_torch_linear_layers():
    """The same MLP built from torch's linear layers in float64 on the mean key."""
    k, r = _router_case()
    logits, route = O.route_heads(k, r["w1"], r["b1"], r["w2"], r["b2"])
    x = torch.from_numpy(k.reshape(k.shape[0], -1)).mean(dim=0)
    hid = torch.nn.functional.relu(torch.nn.functional.linear(
        x, torch.from_numpy(r["w1"]).T, torch.from_numpy(r["b1"])))
    want = torch.nn.functional.linear(hid, torch.from_numpy(r["w2"].reshape(16, -1)).T,
                                      torch.from_numpy(r["b2"].reshape(-1))).reshape(-1, 2)
    np.testing.assert_allclose(logits, want.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(route, torch.argmax(want, dim=1).numpy().astype(np.uint8))


def test_router_invariances():
    k, r = _router_case(seed=4)
    logits, route = O.route_heads(k, r["w1"], r["b1"], r["w2"], r["b2"])
    # the order of the current tokens does not matter (pooling), their values do
    l2, r2 = O.route_heads(k[::-1], r["w1"], r["b1"], r["w2"], r["b2"])
    np.testing.assert_allclose(l2, logits, rtol=1e-12, atol=1e-12)
    l3, _ = O.route_heads(k[:-1], r["w1"], r["b1"], r["w2"], r["b2"])
    assert not np.allclose(l3, logits)
    # swapping the full and sparse columns flips every decision
    l4, r4 = O.route_heads(k, r["w1"], r["b1"], r["w2"][:, :, ::-1], r["b2"][:, ::-1])
    assert np.all(logits[:, 0] != logits[:, 1])
    np.testing.assert_array_equal(r4, 1 - route)
    # a positive scale of the output layer keeps every decision
    _, r5 = O.route_heads(k, r["w1"], r["b1"], r["w2"] * 3.0, r["b2"] * 3.0)
    np.testing.assert_array_equal(r5, route)
    # a large negative first-layer bias silences every unit: the decision is b2's
    _, r6 = O.route_heads(k, r["w1"], r["b1"] - 1e6, r["w2"], r["b2"])
    np.testing.assert_array_equal(r6, (r["b2"][:, 1] > r["b2"][:, 0]).astype(np.uint8))


def test_router_reads_only_the_current_tokens():
    """route_batch pools keys L - N .. L - 1 of each sequence: changing the
    earlier context leaves the route unchanged, changing a current key does not."""
    w = synth.Workload("r", 2, 3, 10, 4, 2, 8, 16, 4, "fp32", "fp32", (-4, 4), seed=9)
    x = synth.make_inputs(w)
    r = synth.make_router(w, hidden=16)
    logits, route = O.route_batch(w, x["k"], r)
    k2 = x["k"].copy()
    k2[:, :7] = 100.0
    l2, _ = O.route_batch(w, k2, r)
    np.testing.assert_array_equal(l2, logits)
    k2[1, 9, 0, 0] += 1.0
    l3, _ = O.route_batch(w, k2, r)
    np.testing.assert_array_equal(l3[0], logits[0])
    assert not np.allclose(l3[1], logits[1])


def test_router_size_matches_the_stated_parameter_count():
    """[EA] §2.2 puts the router near 0.27 M parameters per layer: with the
    keys of 8 KV heads of 128 dims, 256 hidden units and two logits for each
    of 32 query heads the MLP has 0.279 M."""
    w = synth.WORKLOADS["elastic_prefill_64k"]
    r = synth.make_router(w)
    count = sum(v.size for v in r.values())
    assert count == 1024 * 256 + 256 + 256 * 64 + 64
    assert abs(count - 0.27e6) / 0.27e6 < 0.05
