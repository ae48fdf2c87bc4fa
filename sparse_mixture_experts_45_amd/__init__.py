"""Sparse Mixture-of-Experts layer forward for MI355X (gfx950).

Thin Python binding of ``libmoe_hip.so`` (declared in ``include/moe.h``).  The
functions below carry the C names and only marshal arguments: torch tensors
supply device memory and the current HIP stream; every step of the layer runs
in the library's HIP kernels.  There is no fallback: if the library is not
built, or a tensor is not on the GPU, the call raises.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import torch

__all__ = [
    "MOE_F32", "MOE_BF16", "MOE_ACT_GELU", "MOE_ACT_RELU", "MOE_ROUTE_TOKEN",
    "MOE_ROUTE_EXPERT", "MoeError", "moe_config",
    "moe_weights", "moe_stats", "config", "library", "moe_workspace_bytes", "moe_route",
    "moe_dispatch", "moe_expert_ffn", "moe_combine", "moe_forward", "moe_status_string",
    "workspace", "LIB_PATH", "moe_grads", "moe_train_workspace_bytes", "moe_forward_train",
    "moe_backward", "train_workspace", "moe_forward_noalloc", "MOE_NOALLOC_SCRATCH_BYTES",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_hip.so")

MOE_F32, MOE_BF16 = 0, 1
MOE_ACT_GELU, MOE_ACT_RELU = 0, 1
MOE_ROUTE_TOKEN, MOE_ROUTE_EXPERT = 0, 1
_STATUS = {0: "MOE_OK", -1: "MOE_ERR_INVALID_ARG", -2: "MOE_ERR_UNSUPPORTED",
           -3: "MOE_ERR_WORKSPACE", -4: "MOE_ERR_HIP", -5: "MOE_ERR_SCRATCH"}
MOE_NOALLOC_SCRATCH_BYTES = 128 << 20  # include/moe.h


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__("%s returned %s (%s)" % (fn, _STATUS.get(status, status),
                                                  moe_status_string(status)))


class moe_config(C.Structure):
    _fields_ = [("T", C.c_int64), ("d_model", C.c_int32), ("d_ff", C.c_int32),
                ("n_experts", C.c_int32), ("top_k", C.c_int32), ("act", C.c_int32),
                ("dtype", C.c_int32), ("capacity", C.c_int32), ("renormalize", C.c_int32),
                ("shared_d_ff", C.c_int32), ("routing", C.c_int32)]


class moe_weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("Wg", "bg", "W1", "b1", "W2", "b2",
                                          "Ws1", "bs1", "Ws2", "bs2")]


class moe_grads(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("dx", "dWg", "dbg", "dW1", "db1", "dW2", "db2",
                                          "dWs1", "dbs1", "dWs2", "dbs2")]


class moe_stats(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("topk_idx", "topk_w", "counts", "kept",
                                          "mean_prob", "balance", "cv2", "ec_idx",
                                          "ec_w")]


_lib = None


def library() -> C.CDLL:
    """Load libmoe_hip.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libmoe_hip.so is not built; run "
                               "`python -m sparse_mixture_experts_45_amd.build`")
        lib = C.CDLL(LIB_PATH)
        P, S = C.c_void_p, C.c_size_t
        CP = C.POINTER(moe_config)
        lib.moe_workspace_bytes.argtypes = [CP]
        lib.moe_workspace_bytes.restype = S
        lib.moe_route.argtypes = [CP, P, P, P, P, P, P, P, P, P, S, P]
        lib.moe_dispatch.argtypes = [CP, P, P, P, P, P, P, P, P, S, P]
        lib.moe_expert_ffn.argtypes = [CP, P, C.POINTER(moe_weights), P, P, P, P, P, P, S, P]
        lib.moe_combine.argtypes = [CP, P, P, P, P, P]
        lib.moe_forward.argtypes = [CP, C.POINTER(moe_weights), P, P, C.POINTER(moe_stats),
                                    P, S, P]
        lib.moe_train_workspace_bytes.argtypes = [CP]
        lib.moe_train_workspace_bytes.restype = S
        lib.moe_forward_train.argtypes = lib.moe_forward.argtypes
        lib.moe_forward_noalloc.argtypes = [CP, C.POINTER(moe_weights), P, P,
                                            C.POINTER(moe_stats), P]
        lib.moe_backward.argtypes = [CP, C.POINTER(moe_weights), P, P, C.c_float,
                                     C.POINTER(moe_grads), P, S, P]
        for f in ("moe_route", "moe_dispatch", "moe_expert_ffn", "moe_combine", "moe_forward",
                  "moe_forward_train", "moe_backward", "moe_forward_noalloc"):
            getattr(lib, f).restype = C.c_int
        lib.moe_status_string.argtypes = [C.c_int]
        lib.moe_status_string.restype = C.c_char_p
        _lib = lib
    return _lib


def moe_status_string(status: int) -> str:
    return library().moe_status_string(int(status)).decode()


def config(T: int, d_model: int, d_ff: int, n_experts: int, top_k: int, *, act: str = "gelu",
           dtype=torch.bfloat16, capacity: int = -1, renormalize: bool = True,
           shared_d_ff: int = 0, routing: str = "token") -> moe_config:
    dt = {torch.float32: MOE_F32, torch.bfloat16: MOE_BF16}[dtype]
    a = {"gelu": MOE_ACT_GELU, "relu": MOE_ACT_RELU}[act]
    r = {"token": MOE_ROUTE_TOKEN, "expert": MOE_ROUTE_EXPERT}[routing]
    return moe_config(int(T), int(d_model), int(d_ff), int(n_experts), int(top_k), a, dt,
                      int(capacity), int(bool(renormalize)), int(shared_d_ff), r)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _ws(ws: Optional[torch.Tensor]):
    if ws is None:
        raise ValueError("a workspace tensor is required (see workspace())")
    return _ptr(ws), ws.numel() * ws.element_size()


def _check(fn: str, rc: int):
    if rc != 0:
        raise MoeError(fn, rc)


def moe_workspace_bytes(cfg: moe_config) -> int:
    return int(library().moe_workspace_bytes(C.byref(cfg)))


def workspace(cfg: moe_config, device="cuda") -> torch.Tensor:
    """A uint8 device tensor of moe_workspace_bytes(cfg) bytes (torch's allocator
    returns 256-byte aligned blocks)."""
    n = moe_workspace_bytes(cfg)
    if n == 0:
        raise MoeError("moe_workspace_bytes", -1)
    return torch.empty(n, dtype=torch.uint8, device=device)


def moe_route(cfg, x, Wg, bg, topk_idx, topk_w, probs=None, mean_prob=None, balance=None,
              ws=None, stream=None):
    wp, wn = _ws(ws)
    _check("moe_route", library().moe_route(
        C.byref(cfg), _ptr(x), _ptr(Wg), _ptr(bg), _ptr(topk_idx), _ptr(topk_w), _ptr(probs),
        _ptr(mean_prob), _ptr(balance), wp, wn, _stream(stream)))


def moe_dispatch(cfg, topk_idx, counts, kept, offsets, row_token, row_slot, inv, ws=None,
                 stream=None):
    wp, wn = _ws(ws)
    _check("moe_dispatch", library().moe_dispatch(
        C.byref(cfg), _ptr(topk_idx), _ptr(counts), _ptr(kept), _ptr(offsets), _ptr(row_token),
        _ptr(row_slot), _ptr(inv), wp, wn, _stream(stream)))


def _weights(w: dict) -> moe_weights:
    return moe_weights(*[_ptr(w.get(n)) for n in ("Wg", "bg", "W1", "b1", "W2", "b2",
                                                  "Ws1", "bs1", "Ws2", "bs2")])


def moe_expert_ffn(cfg, x, weights: dict, offsets, row_token, row_slot, topk_w, y_rows,
                   ws=None, stream=None):
    wp, wn = _ws(ws)
    w = _weights(weights)
    _check("moe_expert_ffn", library().moe_expert_ffn(
        C.byref(cfg), _ptr(x), C.byref(w), _ptr(offsets), _ptr(row_token), _ptr(row_slot),
        _ptr(topk_w), _ptr(y_rows), wp, wn, _stream(stream)))


def moe_combine(cfg, y_rows, inv, offsets, y, stream=None):
    _check("moe_combine", library().moe_combine(
        C.byref(cfg), _ptr(y_rows), _ptr(inv), _ptr(offsets), _ptr(y), _stream(stream)))


def moe_forward(cfg, weights: dict, x, y, stats: Optional[dict] = None, ws=None, stream=None):
    wp, wn = _ws(ws)
    w = _weights(weights)
    st = moe_stats(*[_ptr((stats or {}).get(n)) for n in
                      ("topk_idx", "topk_w", "counts", "kept", "mean_prob", "balance", "cv2",
                       "ec_idx", "ec_w")])
    _check("moe_forward", library().moe_forward(
        C.byref(cfg), C.byref(w), _ptr(x), _ptr(y), C.byref(st), wp, wn, _stream(stream)))


def moe_forward_noalloc(cfg, weights: dict, x, y, stats: Optional[dict] = None, stream=None):
    """moe_forward with the library's static per-GPU scratch as workspace (no
    device allocation by the library or here)."""
    w = _weights(weights)
    st = moe_stats(*[_ptr((stats or {}).get(n)) for n in
                      ("topk_idx", "topk_w", "counts", "kept", "mean_prob", "balance", "cv2",
                       "ec_idx", "ec_w")])
    _check("moe_forward_noalloc", library().moe_forward_noalloc(
        C.byref(cfg), C.byref(w), _ptr(x), _ptr(y), C.byref(st), _stream(stream)))


def moe_train_workspace_bytes(cfg: moe_config) -> int:
    return int(library().moe_train_workspace_bytes(C.byref(cfg)))


def train_workspace(cfg: moe_config, device="cuda") -> torch.Tensor:
    """A uint8 device tensor of moe_train_workspace_bytes(cfg) bytes."""
    n = moe_train_workspace_bytes(cfg)
    if n == 0:
        raise MoeError("moe_train_workspace_bytes", -1)
    return torch.empty(n, dtype=torch.uint8, device=device)


def _stats(stats: Optional[dict]) -> moe_stats:
    return moe_stats(*[_ptr((stats or {}).get(n)) for n in
                       ("topk_idx", "topk_w", "counts", "kept", "mean_prob", "balance", "cv2",
                        "ec_idx", "ec_w")])


def moe_forward_train(cfg, weights: dict, x, y, stats: Optional[dict] = None, ws=None,
                      stream=None):
    wp, wn = _ws(ws)
    w = _weights(weights)
    st = _stats(stats)
    _check("moe_forward_train", library().moe_forward_train(
        C.byref(cfg), C.byref(w), _ptr(x), _ptr(y), C.byref(st), wp, wn, _stream(stream)))


def moe_backward(cfg, weights: dict, x, dy, grads: dict, aux_coef: float = 0.0, ws=None,
                 stream=None):
    """grads: tensors keyed dx, dWg, dbg, dW1, db1, dW2, db2, dWs1, dbs1, dWs2, dbs2
    (missing keys are not computed)."""
    wp, wn = _ws(ws)
    w = _weights(weights)
    g = moe_grads(*[_ptr(grads.get(n)) for n, _ in moe_grads._fields_])
    _check("moe_backward", library().moe_backward(
        C.byref(cfg), C.byref(w), _ptr(x), _ptr(dy), float(aux_coef), C.byref(g), wp, wn,
        _stream(stream)))
