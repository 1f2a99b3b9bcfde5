"""Host-side checks of the C ABI (CPU only: no kernel is launched).

The library must load and export every function include/dsa.h declares, and
every invalid-argument class must be rejected with its documented status
before anything touches the GPU.
"""
import ctypes

import pytest

from top_sparse_attention_indexer_amd import binding as B


def _p(**kw):
    base = dict(batch=2, n_q=4, kv_len=64, h_q=8, h_kv=2, head_dim=128, idx_dim=64, top_k=16,
                qkv_dtype="bf16", idx_dtype="bf16")
    base.update(kw)
    return B.problem(**base)


FAKE = 1 << 40        # a 16-byte aligned non-null address; never dereferenced
MISALIGNED = FAKE + 4


def test_library_exports_every_declared_symbol():
    lib = B.lib()
    declared = B.header_symbols()
    assert {"dsa_workspace_size", "dsa_indexer_scores", "dsa_topk", "dsa_sparse_attn",
            "dsa_fused_forward", "dsa_exec_status", "dsa_set_wait_limit",
            "dsa_last_error"} <= set(declared)
    # the binding marshals exactly what the header declares
    assert set(declared) == set(B._SIGNATURES)
    for name in declared:
        assert hasattr(lib, name), name


def _status(fn, *args):
    return fn(*args)


def test_workspace_size_and_problem_validation():
    lib = B.lib()
    n = ctypes.c_size_t(0)
    assert lib.dsa_workspace_size(ctypes.byref(_p()), ctypes.byref(n)) == B.DSA_OK and n.value > 0
    bad = [
        (_p(n_q=65), B.DSA_ERR_INVALID_ARG, "exceeds kv_len"),
        (_p(h_q=6, h_kv=4), B.DSA_ERR_INVALID_ARG, "multiple"),
        (_p(top_k=0), B.DSA_ERR_INVALID_ARG, "top_k"),
        (_p(kv_len=0, n_q=0), B.DSA_ERR_INVALID_ARG, "kv_len"),
        (_p(batch=-1), B.DSA_ERR_INVALID_ARG, ">= 0"),
        (_p(h_kv=0), B.DSA_ERR_INVALID_ARG, "head counts"),
        (_p(head_dim=96), B.DSA_ERR_UNSUPPORTED, "head_dim"),
        (_p(idx_dim=48), B.DSA_ERR_UNSUPPORTED, "idx_dim"),
        (_p(qkv_dtype=7), B.DSA_ERR_UNSUPPORTED, "qkv_dtype"),
        (_p(idx_dtype=3), B.DSA_ERR_UNSUPPORTED, "idx_dtype"),
        (_p(softmax_scale=float("nan")), B.DSA_ERR_INVALID_ARG, "finite"),
        (_p(idx_heads=-1), B.DSA_ERR_INVALID_ARG, "idx_heads"),
        (_p(h_q=8, idx_heads=3), B.DSA_ERR_INVALID_ARG, "multiple of idx_heads"),
    ]
    for prob, status, msg in bad:
        assert lib.dsa_workspace_size(ctypes.byref(prob), ctypes.byref(n)) == status
        assert msg in lib.dsa_last_error().decode()
    assert lib.dsa_workspace_size(None, ctypes.byref(n)) == B.DSA_ERR_INVALID_ARG


def test_workspace_scales_sensibly():
    # decode: scores of every row plus small scratch
    dec = B.problem(8, 1, 131072, 32, 8, 128, 64, 2048)
    assert 8 * 131072 * 4 <= B.dsa_workspace_size(dec) < 64 << 20
    # long prefill: chunked, well below the full score matrix (34 GB here):
    # per-range attention partials capped at 6 GiB per launch, candidate
    # lists at 1 GiB, plus the launch's index rows
    pre = B.problem(2, 65536, 65536, 32, 8, 128, 64, 2048)
    assert B.dsa_workspace_size(pre) < (8 << 30)
    # empty problems need nothing
    assert B.dsa_workspace_size(B.problem(0, 4, 16, 4, 1, 64, 32, 8)) == 0
    assert B.dsa_workspace_size(B.problem(3, 0, 16, 4, 1, 64, 32, 8)) == 0


def test_null_and_misaligned_pointers_are_rejected_before_launch():
    lib = B.lib()
    p = ctypes.byref(_p())
    ws_n = B.dsa_workspace_size(_p())
    # indexer
    assert lib.dsa_indexer_scores(p, None, FAKE, FAKE, None) == B.DSA_ERR_INVALID_ARG
    assert "q_idx" in lib.dsa_last_error().decode()
    assert lib.dsa_indexer_scores(p, FAKE, MISALIGNED, FAKE, None) == B.DSA_ERR_INVALID_ARG
    assert "aligned" in lib.dsa_last_error().decode()
    # top-k: workspace missing / too small
    assert lib.dsa_topk(p, FAKE, FAKE, None, 0, None) == B.DSA_ERR_WORKSPACE
    assert lib.dsa_topk(p, FAKE, FAKE, FAKE, 16, None) == B.DSA_ERR_WORKSPACE
    assert lib.dsa_topk(p, FAKE, None, FAKE, ws_n, None) == B.DSA_ERR_INVALID_ARG
    # attention: gate without y2, missing out
    args = [FAKE, FAKE, FAKE, FAKE]
    assert lib.dsa_sparse_attn(p, *args, FAKE, None, None, FAKE, FAKE, ws_n, None) == B.DSA_ERR_INVALID_ARG
    assert "y2" in lib.dsa_last_error().decode()
    assert lib.dsa_sparse_attn(p, *args, None, None, None, None, FAKE, ws_n, None) == B.DSA_ERR_INVALID_ARG
    # fused: every required pointer
    full = [FAKE] * 9     # q_idx, k_idx, q, k, v, gate, y2, route, out
    for i, name in [(0, "q_idx"), (1, "k_idx"), (2, "q"), (3, "k"), (4, "v"), (8, "out")]:
        a = list(full)
        a[i] = None
        st = lib.dsa_fused_forward(p, *a, None, FAKE, ws_n, None)
        assert st == B.DSA_ERR_INVALID_ARG and name in lib.dsa_last_error().decode()
    a = list(full)
    a[6] = None           # gate given, y2 missing
    assert lib.dsa_fused_forward(p, *a, None, FAKE, ws_n, None) == B.DSA_ERR_INVALID_ARG
    assert lib.dsa_fused_forward(p, *full, MISALIGNED, FAKE, ws_n, None) == B.DSA_ERR_INVALID_ARG
    assert lib.dsa_fused_forward(p, *full, None, FAKE, 16, None) == B.DSA_ERR_WORKSPACE
    assert lib.dsa_fused_forward(p, *full, None, None, ws_n, None) == B.DSA_ERR_WORKSPACE
    assert lib.dsa_fused_forward(p, *full, None, MISALIGNED, ws_n, None) == B.DSA_ERR_INVALID_ARG


def test_empty_problems_are_no_ops():
    lib = B.lib()
    for prob in (B.problem(0, 4, 16, 4, 1, 64, 32, 8), B.problem(2, 0, 16, 4, 1, 64, 32, 8)):
        p = ctypes.byref(prob)
        assert lib.dsa_indexer_scores(p, None, None, None, None) == B.DSA_OK
        assert lib.dsa_topk(p, None, None, None, 0, None) == B.DSA_OK
        assert lib.dsa_sparse_attn(p, *([None] * 9), 0, None) == B.DSA_OK
        assert lib.dsa_fused_forward(p, *([None] * 11), 0, None) == B.DSA_OK
        assert lib.dsa_last_error().decode() == ""


def test_binding_raises_dsa_error():
    with pytest.raises(B.DsaError) as ei:
        B.dsa_workspace_size(_p(top_k=-3))
    assert ei.value.status == B.DSA_ERR_INVALID_ARG


def test_exec_status_without_a_decode_launch():
    """dsa_exec_status needs a workspace; one that no decode launch used has
    nothing to report (and needs no device to say so)."""
    lib = B.lib()
    assert lib.dsa_exec_status(None, None) == B.DSA_ERR_INVALID_ARG
    assert "null" in lib.dsa_last_error().decode()
    assert lib.dsa_exec_status(FAKE, None) == B.DSA_OK


def test_router_arguments_are_checked_before_launch():
    lib = B.lib()
    p = ctypes.byref(_p())
    good = B.DsaRouter(16, FAKE, FAKE, FAKE, FAKE)
    n = ctypes.c_size_t(0)
    assert lib.dsa_route_workspace_size(p, ctypes.byref(good), ctypes.byref(n)) == B.DSA_OK
    # the routed forward needs at least what the forward needs
    assert n.value >= B.dsa_workspace_size(_p()) > 0
    bad = [(None, "router is null"),
           (ctypes.byref(B.DsaRouter(0, FAKE, FAKE, FAKE, FAKE)), "hidden"),
           (ctypes.byref(B.DsaRouter(70000, FAKE, FAKE, FAKE, FAKE)), "hidden"),
           (ctypes.byref(B.DsaRouter(16, None, FAKE, FAKE, FAKE)), "w1"),
           (ctypes.byref(B.DsaRouter(16, FAKE, FAKE, MISALIGNED, FAKE)), "w2")]
    for r, msg in bad:
        assert lib.dsa_route_workspace_size(p, r, ctypes.byref(n)) == B.DSA_ERR_INVALID_ARG
        assert msg in lib.dsa_last_error().decode()
        assert lib.dsa_route_heads(p, r, FAKE, FAKE, None, FAKE, 1 << 30, None) == B.DSA_ERR_INVALID_ARG
    g = ctypes.byref(good)
    assert lib.dsa_route_heads(p, g, None, FAKE, None, FAKE, 1 << 30, None) == B.DSA_ERR_INVALID_ARG
    assert lib.dsa_route_heads(p, g, FAKE, None, None, FAKE, 1 << 30, None) == B.DSA_ERR_INVALID_ARG
    assert lib.dsa_route_heads(p, g, FAKE, FAKE, MISALIGNED, FAKE, 1 << 30, None) == B.DSA_ERR_INVALID_ARG
    assert lib.dsa_route_heads(p, g, FAKE, FAKE, None, FAKE, 16, None) == B.DSA_ERR_WORKSPACE
    # routed forward: route_out required, every forward check before the router runs
    full = [FAKE] * 7     # q_idx, k_idx, q, k, v, gate, y2
    assert lib.dsa_fused_forward_routed(p, g, *full, None, FAKE, None, FAKE, 1 << 30,
                                        None) == B.DSA_ERR_INVALID_ARG
    assert "route_out" in lib.dsa_last_error().decode()
    a = list(full)
    a[2] = None
    assert lib.dsa_fused_forward_routed(p, g, *a, FAKE, FAKE, None, FAKE, 1 << 30,
                                        None) == B.DSA_ERR_INVALID_ARG
    assert lib.dsa_fused_forward_routed(p, g, *full, FAKE, FAKE, None, FAKE, 16,
                                        None) == B.DSA_ERR_WORKSPACE
    # empty problems: no-ops
    e = ctypes.byref(B.problem(0, 4, 16, 4, 1, 64, 32, 8))
    assert lib.dsa_route_heads(e, g, None, None, None, None, 0, None) == B.DSA_OK
