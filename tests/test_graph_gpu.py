"""The fused forward captured into a HIP graph and replayed.

A captured call replays the same kernel arguments every time, so nothing a
launch needs to be fresh may travel as an argument (the single-launch
decode's epoch is advanced on the device under capture).  Each replay is
compared bit-exactly with the eager result of the same call, with eager work
(including eager forwards on the same workspace) between the replays.
"""
import pytest
import torch

from top_sparse_attention_indexer_amd import binding as B
from top_sparse_attention_indexer_amd import synth
from top_sparse_attention_indexer_amd.tensors import to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    yield
    torch.cuda.synchronize()


def _w(B_, N, L, Hq, Hkv, d, didx, K, route_p=None, seed=51):
    return synth.Workload("graph", B_, N, L, Hq, Hkv, d, didx, K, "bf16", "bf16", (-4, 4),
                          route_sparse_p=route_p, seed=seed)


CASES = [
    # single-launch decode (device epoch under capture)
    ("decode", _w(4, 1, 20000, 8, 2, 128, 64, 512), False),
    ("decode_noalloc", _w(2, 2, 9000, 8, 2, 128, 64, 300), True),
    # prefill: on-chip indexer, key-range attention with both routes
    ("prefill", _w(1, 300, 9000, 8, 2, 128, 64, 256, route_p=0.6), False),
]


@pytest.mark.parametrize("name,w,noalloc", CASES, ids=[c[0] for c in CASES])
def test_graph_replay_matches_eager(name, w, noalloc, announce):
    x = synth.make_inputs(w)
    dev = to_device(w, x)
    p = B.problem_for(w)
    out = torch.empty((w.batch, w.n_q, w.h_q, w.head_dim), dtype=torch.float32, device="cuda")
    idx = torch.empty((w.batch, w.n_q, w.top_k), dtype=torch.int32, device="cuda")
    ws = None if noalloc else torch.empty(max(1, B.dsa_workspace_size(p)), dtype=torch.uint8,
                                          device="cuda")

    def forward():
        if noalloc:
            B.dsa_fused_forward_noalloc(p, dev["q_idx"], dev["k_idx"], dev["q"], dev["k"], dev["v"],
                                        dev["gate"], dev["y2"], dev["route"], out, idx)
        else:
            B.dsa_fused_forward(p, dev["q_idx"], dev["k_idx"], dev["q"], dev["k"], dev["v"],
                                dev["gate"], dev["y2"], dev["route"], out, idx, ws)

    s = torch.cuda.Stream()
    announce(f"graph capture {name} {w}")
    with torch.cuda.stream(s):
        forward()                        # set-up and warm-up on the capture stream
        forward()
    torch.cuda.synchronize()
    out_ref, idx_ref = out.clone(), idx.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        forward()
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))
        idx.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, idx_ref), f"replay {rep}: index rows differ"
        assert torch.equal(out, out_ref), f"replay {rep}: outputs differ"
        if ws is not None:
            B.dsa_exec_status(ws, s)     # raises if a wait gave up
        # an eager forward on the same workspace between replays
        with torch.cuda.stream(s):
            out.fill_(0.0)
            forward()
        torch.cuda.synchronize()
        assert torch.equal(out, out_ref), f"eager call after replay {rep} differs"
