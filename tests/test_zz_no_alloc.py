"""The entry point that allocates nothing (dsa_fused_forward_noalloc) against
dsa_fused_forward with a caller workspace: same index rows bit for bit, same
outputs within the float tolerance, on two calls in a row (the second on a
smaller problem), for decode and a short prefill; an oversized problem is
rejected before anything is enqueued."""
import numpy as np
import pytest
import torch

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


def _w(B_, N, L, Hq, Hkv, d, didx, K, dt="bf16", route_p=None, seed=11):
    rng = (-4, 4) if dt == "bf16" else (-8, 8)
    return synth.Workload("noalloc", B_, N, L, Hq, Hkv, d, didx, K, dt, dt, rng,
                          route_sparse_p=route_p, seed=seed)


def _both(w, announce):
    x = synth.make_inputs(w)
    dev = to_device(w, x)
    p = B.problem_for(w)
    args = (dev["q_idx"], dev["k_idx"], dev["q"], dev["k"], dev["v"], dev["gate"], dev["y2"],
            dev["route"])
    shape_o = (w.batch, w.n_q, w.h_q, w.head_dim)
    shape_i = (w.batch, w.n_q, w.top_k)
    out_a = torch.empty(shape_o, dtype=torch.float32, device="cuda")
    idx_a = torch.full(shape_i, -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(1, B.dsa_workspace_size(p)), dtype=torch.uint8, device="cuda")
    B.dsa_fused_forward(p, *args, out_a, idx_a, ws)
    out_b = torch.empty(shape_o, dtype=torch.float32, device="cuda")
    idx_b = torch.full(shape_i, -7, dtype=torch.int32, device="cuda")
    announce(f"fused_forward_noalloc {w}")
    B.dsa_fused_forward_noalloc(p, *args, out_b, idx_b)
    torch.cuda.synchronize()
    assert torch.equal(idx_a, idx_b)
    assert torch.max(torch.abs(out_a - out_b)).item() <= TOL[w.qkv_dtype]


@pytest.mark.parametrize("kind", ["decode", "prefill"])
def test_noalloc_matches_workspace_entry_point(kind, announce):
    if kind == "decode":
        first = synth.WORKLOADS["decode_b8_ctx128k"].replace(kv_len=60000)
        second = _w(3, 1, 9000, 16, 4, 128, 64, 700, seed=3)
    else:
        first = _w(1, 300, 2000, 8, 2, 128, 64, 256, route_p=0.5, seed=5)
        second = _w(1, 100, 700, 4, 1, 64, 32, 64, seed=6)
    _both(first, announce)
    _both(second, announce)      # smaller, right after: the array keeps the last contents


def test_noalloc_rejects_oversized_problems():
    w = synth.WORKLOADS["elastic_prefill_64k"]
    p = B.problem_for(w)
    fake = 1 << 40
    with pytest.raises(B.DsaError) as ei:
        B.dsa_fused_forward_noalloc(p, *([fake] * 9), None, None)
    assert ei.value.status == B.DSA_ERR_WORKSPACE
    assert "no-allocation" in str(ei.value)
