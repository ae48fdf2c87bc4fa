"""fp64 CPU oracle of the sparse-MoE layer, forward and backward (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg use this
package; the product path never imports it.  The arithmetic lives in
``moe_oracle.c`` (plain loops, fp64, OpenMP across independent tokens) and
this module only marshals numpy arrays to it.  ``build()`` compiles it with
gcc (no fast-math: sums are never reassociated).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

ACT = {"gelu": 0, "relu": 1}
DTYPE = {"f32": 0, "bf16": 1}


class _Cfg(C.Structure):
    _fields_ = [("T", C.c_int64), ("d", C.c_int32), ("F", C.c_int32), ("E", C.c_int32),
                ("k", C.c_int32), ("act", C.c_int32), ("dtype", C.c_int32),
                ("capacity", C.c_int32), ("renormalize", C.c_int32), ("Fs", C.c_int32)]


class _Weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("Wg", "bg", "W1", "b1", "W2", "b2", "Ws1", "bs1",
                                          "Ws2", "bs2")]


class _Grads(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("dx", "dWg", "dbg", "dW1", "db1", "dW2", "db2",
                                          "dWs1", "dbs1", "dWs2", "dbs2")]


def build() -> str:
    """Compile liboracle.so from moe_oracle.c (always recompiles)."""
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
           "-Wall", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = C.CDLL(_LIB)
        P = C.c_void_p
        lib.orc_route.argtypes = [C.POINTER(_Cfg), P, P, P, P, P, P, P, P, P, P, P]
        lib.orc_dispatch.argtypes = [C.POINTER(_Cfg), P, P, P, P, P, P]
        lib.orc_experts.argtypes = [C.POINTER(_Cfg)] + [P] * 13 + [C.c_int64, P]
        lib.orc_expert_row.argtypes = [C.POINTER(_Cfg)] + [P] * 9 + [C.c_int64, C.c_int32,
                                                                     C.c_double, P]
        for f in (lib.orc_route, lib.orc_dispatch, lib.orc_experts, lib.orc_expert_row):
            f.restype = C.c_int
        lib.orc_threads.argtypes = []
        lib.orc_threads.restype = C.c_int
        lib.orc_cv2.argtypes = [P, C.c_int32]
        lib.orc_cv2.restype = C.c_double
        lib.orc_ec_select.argtypes = [C.POINTER(_Cfg), P, P, P, C.c_int64, P, P]
        lib.orc_ec_select.restype = C.c_int
        W, G = C.POINTER(_Weights), C.POINTER(_Grads)
        lib.orc_backward.argtypes = [C.POINTER(_Cfg), P, W, P, C.c_double, P, P, P, P, G]
        lib.orc_backward_tokens.argtypes = [C.POINTER(_Cfg), P, W, P, C.c_double, P, P, P, P,
                                            P, C.c_int64, P, P, P]
        lib.orc_backward_expert_entries.argtypes = [C.POINTER(_Cfg), P, W, P, P, P, P,
                                                    C.c_int32, C.c_int32, P, C.c_int32, P,
                                                    P, P, P, P]
        for f in (lib.orc_backward, lib.orc_backward_tokens, lib.orc_backward_expert_entries):
            f.restype = C.c_int
        _lib = lib
    return _lib


def threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().orc_threads())


def _cfg(shape, T: Optional[int] = None) -> _Cfg:
    return _Cfg(shape.T if T is None else T, shape.d, shape.F, shape.E, shape.k,
                ACT[shape.act], DTYPE[shape.dtype], shape.capacity, shape.renormalize,
                shape.Fs)


def _p(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def route(shape, inp, *, with_probs: bool = True) -> dict:
    """Routing, capacity and statistics for every token of ``inp``."""
    lib = _load()
    T, E, k = shape.T, shape.E, shape.k
    r = dict(topk_idx=np.zeros((T, k), np.int32), topk_w=np.zeros((T, k), np.float64),
             probs=np.zeros((T, E), np.float64) if with_probs else None,
             counts=np.zeros(E, np.int32), kept=np.zeros(E, np.int32),
             keep=np.zeros((T, k), np.int32), mean_prob=np.zeros(E, np.float64),
             balance=np.zeros(1, np.float64))
    c = _cfg(shape)
    rc = lib.orc_route(C.byref(c), _p(inp["x"]), _p(inp["Wg"]), _p(inp["bg"]),
                       _p(r["topk_idx"]), _p(r["topk_w"]), _p(r["probs"]), _p(r["counts"]),
                       _p(r["kept"]), _p(r["keep"]), _p(r["mean_prob"]), _p(r["balance"]))
    if rc != 0:
        raise ValueError("orc_route failed")
    r["balance"] = float(r["balance"][0])
    r["cv2"] = cv2(r["counts"])
    return r


def cv2(counts) -> float:
    """Squared coefficient of variation of per-expert counts (unbiased variance / mean^2)."""
    lib = _load()
    c = np.ascontiguousarray(counts, dtype=np.int32)
    return float(lib.orc_cv2(_p(c), C.c_int32(len(c))))


def dispatch(shape, topk_idx: np.ndarray, keep: np.ndarray) -> dict:
    """Expert-major, token-ascending grouping implied by the routing."""
    lib = _load()
    T, E, k = shape.T, shape.E, shape.k
    nrows = T * k + (T if shape.Fs else 0)
    d = dict(offsets=np.zeros(E + 2, np.int32), row_token=np.full(max(nrows, 1), -1, np.int32),
             row_slot=np.full(max(nrows, 1), -1, np.int32), inv=np.zeros((T, k), np.int32))
    c = _cfg(shape)
    ti = np.ascontiguousarray(topk_idx, np.int32)
    kp = np.ascontiguousarray(keep, np.int32)
    if lib.orc_dispatch(C.byref(c), _p(ti), _p(kp), _p(d["offsets"]), _p(d["row_token"]),
                        _p(d["row_slot"]), _p(d["inv"])) != 0:
        raise ValueError("orc_dispatch failed")
    n = int(d["offsets"][E + 1])
    d["row_token"], d["row_slot"] = d["row_token"][:n], d["row_slot"][:n]
    return d


def experts(shape, inp, rt: dict, tokens: Optional[Sequence[int]] = None) -> np.ndarray:
    """Layer output rows y[len(tokens), d] in fp64 (all tokens when None)."""
    lib = _load()
    toks = np.arange(shape.T, dtype=np.int64) if tokens is None else \
        np.ascontiguousarray(tokens, dtype=np.int64)
    y = np.zeros((len(toks), shape.d), np.float64)
    c = _cfg(shape)
    tw = np.ascontiguousarray(rt["topk_w"], np.float64)
    rc = lib.orc_experts(C.byref(c), _p(inp["x"]), _p(inp["W1"]), _p(inp["b1"]), _p(inp["W2"]),
                         _p(inp["b2"]), _p(inp.get("Ws1")), _p(inp.get("bs1")),
                         _p(inp.get("Ws2")), _p(inp.get("bs2")),
                         _p(np.ascontiguousarray(rt["topk_idx"], np.int32)), _p(tw),
                         _p(np.ascontiguousarray(rt["keep"], np.int32)), _p(toks),
                         len(toks), _p(y))
    if rc != 0:
        raise ValueError("orc_experts failed")
    return y


def expert_row(shape, inp, t: int, e: int, g: float) -> np.ndarray:
    """g * E_e(x_t) for one token (e = -1: the shared expert)."""
    lib = _load()
    out = np.zeros(shape.d, np.float64)
    c = _cfg(shape)
    rc = lib.orc_expert_row(C.byref(c), _p(inp["x"]), _p(inp["W1"]), _p(inp["b1"]),
                            _p(inp["W2"]), _p(inp["b2"]), _p(inp.get("Ws1")),
                            _p(inp.get("bs1")), _p(inp.get("Ws2")), _p(inp.get("bs2")),
                            int(t), int(e), float(g), _p(out))
    if rc != 0:
        raise ValueError("orc_expert_row failed")
    return out


def forward(shape, inp, tokens=None) -> dict:
    """Whole layer: routing for all tokens, outputs for ``tokens`` (all if None)."""
    rt = route(shape, inp)
    rt["y"] = experts(shape, inp, rt, tokens)
    return rt


def ec_capacity(shape) -> int:
    """Tokens each expert takes under expert-choice routing: the capacity when one is
    set, else floor(T * k / E) (k read as the capacity factor); at most T."""
    c = shape.capacity if shape.capacity >= 0 else (shape.T * shape.k) // shape.E
    return min(c, shape.T)


def ec_route(shape, inp) -> dict:
    """Expert-choice routing: sel[T, E] (1 where expert e took token t), the fp64
    router probabilities p[T, E], per-expert counts and the load statistics."""
    lib = _load()
    T, E = shape.T, shape.E
    Ce = ec_capacity(shape)
    r = dict(sel=np.zeros((T, E), np.int32), p=np.zeros((T, E), np.float64), C=Ce)
    if lib.orc_ec_select(C.byref(_cfg(shape)), _p(inp["x"]), _p(inp["Wg"]), _p(inp["bg"]),
                         Ce, _p(r["sel"]), _p(r["p"])) != 0:
        raise ValueError("orc_ec_select failed")
    r["counts"] = r["sel"].sum(axis=0).astype(np.int32)
    r["kept"] = r["counts"].copy()
    # load statistics of the same softmax (orc_route's definition)
    st = route(shape, inp, with_probs=False)
    r["mean_prob"], r["balance"] = st["mean_prob"], st["balance"]
    r["cv2"] = cv2(r["counts"])
    return r


def ec_experts(shape, inp, r: dict, tokens=None) -> np.ndarray:
    """Expert-choice outputs from a selection ``r`` (ec_route's): y[t] = sum over the
    experts that took t, in expert order, of p[t, e] E_e(x_t), plus the shared
    expert; for ``tokens`` (all if None)."""
    E = shape.E
    # the token's candidate slots are all E experts in order; untaken ones are
    # masked off, so the sum runs over the taking experts in expert order
    slots = dict(topk_idx=np.tile(np.arange(E, dtype=np.int32), (shape.T, 1)),
                 topk_w=r["p"], keep=r["sel"])
    return experts(shape.with_(k=E), inp, slots, tokens)


def ec_forward(shape, inp, tokens=None) -> dict:
    """Expert-choice layer: selection, statistics and outputs for ``tokens``."""
    r = ec_route(shape, inp)
    r["y"] = ec_experts(shape, inp, r, tokens)
    return r


def combine(shape, y_rows: np.ndarray, inv: np.ndarray, offsets: np.ndarray) -> np.ndarray:
    """Gather-combine of expert rows in fp64: y[t] = sum_i y_rows[inv[t,i]] (+ shared row).

    Plain loops over slots in ascending order, then the shared row (rows start
    at offsets[E]).  Small numpy helper; tokens independent."""
    T, k, E = shape.T, shape.k, shape.E
    y = np.zeros((T, shape.d), np.float64)
    yr = y_rows.astype(np.float64)
    for i in range(k):
        r = inv[:, i]
        m = r >= 0
        y[m] += yr[r[m]]
    if shape.Fs:
        base = int(offsets[E])
        y += yr[base:base + T]
    return y


# ---------------------------------------------------------------------------
# Backward pass (token choice): gradients of L = sum_t <dy_t, y_t> + alpha * balance
# with the top-k selection and the capacity drops held fixed.


def _weights(inp) -> _Weights:
    return _Weights(*[_p(inp.get(n)) for n in ("Wg", "bg", "W1", "b1", "W2", "b2", "Ws1",
                                                "bs1", "Ws2", "bs2")])


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def backward(shape, inp, dy, alpha: float = 0.0, rt: Optional[dict] = None) -> dict:
    """Every gradient, fp64, summed over tokens in token order (small shapes):
    dx [T, d], dWg [E, d], dbg [E], dW1 [E, F, d], db1 [E, F], dW2 [E, d, F],
    db2 [E, d], and with a shared expert dWs1 [Fs, d], dbs1 [Fs], dWs2 [d, Fs],
    dbs2 [d].  dy [T, d] (any float dtype, widened exactly)."""
    rt = route(shape, inp, with_probs=False) if rt is None else rt
    T, d, E, F, Fs = shape.T, shape.d, shape.E, shape.F, shape.Fs
    z = np.zeros
    g = dict(dx=z((T, d)), dWg=z((E, d)), dbg=z(E), dW1=z((E, F, d)), db1=z((E, F)),
             dW2=z((E, d, F)), db2=z((E, d)))
    if Fs:
        g.update(dWs1=z((Fs, d)), dbs1=z(Fs), dWs2=z((d, Fs)), dbs2=z(d))
    gr = _Grads(*[_p(g.get(n[0])) for n in _Grads._fields_])
    w = _weights(inp)
    dy64 = _f64(dy)
    rc = _load().orc_backward(C.byref(_cfg(shape)), _p(inp["x"]), C.byref(w), _p(dy64),
                              float(alpha), _p(np.ascontiguousarray(rt["topk_idx"], np.int32)),
                              _p(_f64(rt["topk_w"])),
                              _p(np.ascontiguousarray(rt["keep"], np.int32)),
                              _p(_f64(rt["mean_prob"])), C.byref(gr))
    if rc != 0:
        raise ValueError("orc_backward failed")
    return g


def backward_tokens(shape, inp, dy, tokens, alpha: float = 0.0, rt: Optional[dict] = None):
    """dx [n, d], router-score gradient dl [n, E] and gate gradient dg [n, k] of
    the listed tokens."""
    rt = route(shape, inp, with_probs=False) if rt is None else rt
    toks = np.ascontiguousarray(tokens, dtype=np.int64)
    n = len(toks)
    out = dict(dx=np.zeros((n, shape.d)), dl=np.zeros((n, shape.E)), dg=np.zeros((n, shape.k)))
    w = _weights(inp)
    dy64 = _f64(dy)
    rc = _load().orc_backward_tokens(
        C.byref(_cfg(shape)), _p(inp["x"]), C.byref(w), _p(dy64), float(alpha),
        _p(np.ascontiguousarray(rt["topk_idx"], np.int32)), _p(_f64(rt["topk_w"])),
        _p(np.ascontiguousarray(rt["keep"], np.int32)), _p(_f64(rt["mean_prob"])), _p(toks), n,
        _p(out["dx"]), _p(out["dl"]), _p(out["dg"]))
    if rc != 0:
        raise ValueError("orc_backward_tokens failed")
    return out


def backward_expert_entries(shape, inp, dy, e: int, f_list, j_list, rt: Optional[dict] = None):
    """Entries of expert e's weight gradients (e = -1: the shared expert):
    dW1 [nf, nj] = dW1[e][f_list][:, j_list], db1 [nf], dW2 [nj, nf] =
    dW2[e][j_list][:, f_list], db2 [nj]."""
    rt = route(shape, inp, with_probs=False) if rt is None else rt
    fl = np.ascontiguousarray(f_list, np.int32)
    jl = np.ascontiguousarray(j_list, np.int32)
    out = dict(dW1=np.zeros((len(fl), len(jl))), db1=np.zeros(len(fl)),
               dW2=np.zeros((len(jl), len(fl))), db2=np.zeros(len(jl)))
    w = _weights(inp)
    dy64 = _f64(dy)
    rc = _load().orc_backward_expert_entries(
        C.byref(_cfg(shape)), _p(inp["x"]), C.byref(w), _p(dy64),
        _p(np.ascontiguousarray(rt["topk_idx"], np.int32)), _p(_f64(rt["topk_w"])),
        _p(np.ascontiguousarray(rt["keep"], np.int32)), int(e), len(fl), _p(fl), len(jl),
        _p(jl), _p(out["dW1"]), _p(out["db1"]), _p(out["dW2"]), _p(out["db2"]))
    if rc != 0:
        raise ValueError("orc_backward_expert_entries failed")
    return out


def ec_slots(shape, r: dict) -> tuple:
    """Expert choice as k = E slots: (shape with k = E and no renormalisation,
    routing dict with every expert a slot, gates p, the selection as keep)."""
    E = shape.E
    s = shape.with_(k=E, renormalize=0)
    rt = dict(topk_idx=np.tile(np.arange(E, dtype=np.int32), (shape.T, 1)),
              topk_w=np.ascontiguousarray(r["p"], np.float64),
              keep=np.ascontiguousarray(r["sel"], np.int32),
              mean_prob=np.ascontiguousarray(r["mean_prob"], np.float64))
    return s, rt


def ec_backward(shape, inp, dy, alpha: float = 0.0, r: Optional[dict] = None) -> dict:
    """Every gradient of the expert-choice layer (selection fixed), fp64."""
    r = ec_route(shape, inp) if r is None else r
    s, rt = ec_slots(shape, r)
    return backward(s, inp, dy, alpha, rt=rt)
