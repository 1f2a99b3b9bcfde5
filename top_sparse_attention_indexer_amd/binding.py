"""ctypes binding of libdsa.so (the C ABI of include/dsa.h).

Argument marshalling only: torch tensors supply device pointers and the
current HIP stream; every step of the computation runs in the library's
kernels.  There is no fallback: if the library is missing, loading fails.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libdsa.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "dsa.h")

DSA_OK, DSA_ERR_INVALID_ARG, DSA_ERR_UNSUPPORTED, DSA_ERR_WORKSPACE, DSA_ERR_HIP, DSA_ERR_EXEC = range(6)
DSA_FP32, DSA_BF16 = 0, 1
STATUS_NAMES = {0: "DSA_OK", 1: "DSA_ERR_INVALID_ARG", 2: "DSA_ERR_UNSUPPORTED",
                3: "DSA_ERR_WORKSPACE", 4: "DSA_ERR_HIP", 5: "DSA_ERR_EXEC"}


class DsaProblem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q", ctypes.c_int32), ("kv_len", ctypes.c_int32),
                ("h_q", ctypes.c_int32), ("h_kv", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("idx_dim", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("qkv_dtype", ctypes.c_int32), ("idx_dtype", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("idx_heads", ctypes.c_int32)]


class DsaRouter(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("w1", ctypes.c_void_p), ("b1", ctypes.c_void_p),
                ("w2", ctypes.c_void_p), ("b2", ctypes.c_void_p)]


class DsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None
_vp = ctypes.c_void_p
_PP = ctypes.POINTER(DsaProblem)
_RP = ctypes.POINTER(DsaRouter)
_SIGNATURES = {
    "dsa_workspace_size": (ctypes.c_int, [_PP, ctypes.POINTER(ctypes.c_size_t)]),
    "dsa_indexer_scores": (ctypes.c_int, [_PP, _vp, _vp, _vp, _vp]),
    "dsa_topk": (ctypes.c_int, [_PP, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "dsa_sparse_attn": (ctypes.c_int, [_PP, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                       ctypes.c_size_t, _vp]),
    "dsa_fused_forward": (ctypes.c_int, [_PP, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                         _vp, ctypes.c_size_t, _vp]),
    "dsa_fused_forward_noalloc": (ctypes.c_int, [_PP, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                                 _vp, _vp]),
    "dsa_route_workspace_size": (ctypes.c_int, [_PP, _RP, ctypes.POINTER(ctypes.c_size_t)]),
    "dsa_route_heads": (ctypes.c_int, [_PP, _RP, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "dsa_fused_forward_routed": (ctypes.c_int, [_PP, _RP, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                                _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "dsa_exec_status": (ctypes.c_int, [_vp, _vp]),
    "dsa_set_wait_limit": (None, [ctypes.c_uint32]),
    "dsa_profile_start": (ctypes.c_int, [ctypes.c_int32]),
    "dsa_profile_stop": (ctypes.c_int, [ctypes.POINTER(ctypes.c_double),
                                        ctypes.POINTER(ctypes.c_int32), ctypes.c_int32,
                                        ctypes.POINTER(ctypes.c_int64)]),
    "dsa_last_error": (ctypes.c_char_p, []),
}


def header_symbols(path: str = HEADER):
    """Function names declared in include/dsa.h."""
    text = open(path, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z_]+)\s*\(", text)))


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m top_sparse_attention_indexer_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def problem(batch, n_q, kv_len, h_q, h_kv, head_dim, idx_dim, top_k,
            qkv_dtype="bf16", idx_dtype="bf16", softmax_scale=0.0, idx_heads=1) -> DsaProblem:
    dt = {"fp32": DSA_FP32, "bf16": DSA_BF16, DSA_FP32: DSA_FP32, DSA_BF16: DSA_BF16}
    return DsaProblem(batch, n_q, kv_len, h_q, h_kv, head_dim, idx_dim, top_k,
                      dt.get(qkv_dtype, qkv_dtype), dt.get(idx_dtype, idx_dtype), softmax_scale,
                      idx_heads)


def problem_for(w, softmax_scale: float = 0.0) -> DsaProblem:
    """Problem of any object carrying the workload attributes."""
    return problem(w.batch, w.n_q, w.kv_len, w.h_q, w.h_kv, w.head_dim, w.idx_dim, w.top_k,
                   w.qkv_dtype, w.idx_dtype, softmax_scale, getattr(w, "idx_heads", 1))


def _check(status: int):
    if status != DSA_OK:
        raise DsaError(status, lib().dsa_last_error().decode())


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _nbytes(ws) -> int:
    return 0 if ws is None else ws.numel() * ws.element_size()


def dsa_workspace_size(p: DsaProblem) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().dsa_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def dsa_indexer_scores(p, q_idx, k_idx, scores, stream=None):
    _check(lib().dsa_indexer_scores(ctypes.byref(p), _ptr(q_idx), _ptr(k_idx), _ptr(scores),
                                    _stream(stream)))


def dsa_topk(p, scores, topk_idx, ws=None, stream=None):
    _check(lib().dsa_topk(ctypes.byref(p), _ptr(scores), _ptr(topk_idx), _ptr(ws), _nbytes(ws),
                          _stream(stream)))


def dsa_sparse_attn(p, q, k, v, topk_idx, gate, y2, route, out, ws=None, stream=None):
    _check(lib().dsa_sparse_attn(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(topk_idx),
                                 _ptr(gate), _ptr(y2), _ptr(route), _ptr(out), _ptr(ws),
                                 _nbytes(ws), _stream(stream)))


def dsa_fused_forward(p, q_idx, k_idx, q, k, v, gate, y2, route, out, topk_idx_out=None,
                      ws=None, stream=None):
    _check(lib().dsa_fused_forward(ctypes.byref(p), _ptr(q_idx), _ptr(k_idx), _ptr(q), _ptr(k),
                                   _ptr(v), _ptr(gate), _ptr(y2), _ptr(route), _ptr(out),
                                   _ptr(topk_idx_out), _ptr(ws), _nbytes(ws), _stream(stream)))


def dsa_fused_forward_noalloc(p, q_idx, k_idx, q, k, v, gate, y2, route, out,
                              topk_idx_out=None, stream=None):
    _check(lib().dsa_fused_forward_noalloc(ctypes.byref(p), _ptr(q_idx), _ptr(k_idx), _ptr(q),
                                           _ptr(k), _ptr(v), _ptr(gate), _ptr(y2), _ptr(route),
                                           _ptr(out), _ptr(topk_idx_out), _stream(stream)))


def router(w1, b1, w2, b2) -> DsaRouter:
    """Router weights (device float32 tensors): w1 [Hkv*d, hidden], b1 [hidden],
    w2 [hidden, Hq, 2], b2 [Hq, 2].  The caller keeps the tensors alive."""
    return DsaRouter(int(w1.shape[1]), _ptr(w1), _ptr(b1), _ptr(w2), _ptr(b2))


def dsa_route_workspace_size(p: DsaProblem, r: DsaRouter) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().dsa_route_workspace_size(ctypes.byref(p), ctypes.byref(r), ctypes.byref(n)))
    return n.value


def dsa_route_heads(p, r, k, route, logits=None, ws=None, stream=None):
    _check(lib().dsa_route_heads(ctypes.byref(p), ctypes.byref(r), _ptr(k), _ptr(route),
                                 _ptr(logits), _ptr(ws), _nbytes(ws), _stream(stream)))


def dsa_fused_forward_routed(p, r, q_idx, k_idx, q, k, v, gate, y2, route_out, out,
                             topk_idx_out=None, ws=None, stream=None):
    _check(lib().dsa_fused_forward_routed(ctypes.byref(p), ctypes.byref(r), _ptr(q_idx),
                                          _ptr(k_idx), _ptr(q), _ptr(k), _ptr(v), _ptr(gate),
                                          _ptr(y2), _ptr(route_out), _ptr(out),
                                          _ptr(topk_idx_out), _ptr(ws), _nbytes(ws),
                                          _stream(stream)))


def dsa_exec_status(ws, stream=None):
    """Raises DsaError(DSA_ERR_EXEC) if the last fused forward on ``ws`` gave up."""
    _check(lib().dsa_exec_status(_ptr(ws), _stream(stream)))


def dsa_set_wait_limit(polls: int):
    lib().dsa_set_wait_limit(int(polls))


STAGES = ("indexer", "topk", "attention", "merge", "decode", "prep", "route")


def dsa_profile_start(max_launches: int = 65536):
    _check(lib().dsa_profile_start(int(max_launches)))


def dsa_profile_stop():
    """{stage: (milliseconds, launches)} summed since dsa_profile_start, and the
    count of launches that were not timed."""
    n = len(STAGES)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int32 * n)()
    dropped = ctypes.c_int64(0)
    _check(lib().dsa_profile_stop(ms, cnt, n, ctypes.byref(dropped)))
    return {STAGES[i]: (ms[i], cnt[i]) for i in range(n)}, dropped.value


def dsa_last_error() -> str:
    return lib().dsa_last_error().decode()
