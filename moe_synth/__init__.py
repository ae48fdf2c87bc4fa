"""Seeded synthetic inputs for the sparse-MoE layer forward.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It only draws and stores numbers: it holds none of the layer's
arithmetic.  The one calculation it does is the input-conditioning filter
that redraws token rows whose top-(k+1) router scores sit closer together
than a fixed margin, so that any correct fp32 evaluation of the router picks
the same experts in the same slot order (for expert-choice routing: token
rows at a near-tie on some expert's top-C boundary of router probabilities).

Workloads are the five layer shapes named after what they are:

* ``tiny_f32``            T=64,   d=64,   d_ff=256,   E=8,   k=2, GELU, fp32
* ``page1_b4s512``        T=2048, d=768,  d_ff=3072,  E=8,   k=2, GELU, bf16
  (the batch 4 x seq 512 x d_model 768 example of "Mixture of Experts (MoE)
  and Mixtral", section "Output:")
* ``mixtral_t4096``       T=4096, d=4096, d_ff=14336, E=8,   k=2, GELU, bf16
* ``switch_e64_top1_cap`` T=8192, d=1024, d_ff=4096,  E=64,  k=1, ReLU, bf16,
  capacity floor(1.25*T/E)=160, router bias = log of a Zipf(1.1) law
* ``deepseek_e256_top8``  T=512,  d=7168, d_ff=2048,  E=256, k=8, GELU, bf16,
  plus one always-on shared expert with d_ff=2048
* ``expert_choice_t8192_e64`` T=8192, d=1024, d_ff=4096, E=64, GELU, bf16,
  expert-choice routing: each expert takes its top 256 tokens (k = 2 read as
  the capacity factor)

Distributions: x ~ N(0,1); router and expert weights ~ N(0, 1/fan_in)
(std = fan_in**-0.5); biases ~ N(0, 0.01) read as variance 0.01 (std 0.1).
bf16 tensors are fp32 draws rounded to bf16 with round-to-nearest-even and
are returned as uint16 bit patterns; the router weight and bias stay fp32.

Every tensor has its own counter-keyed stream
``SeedSequence([seed, tag, index])`` so experts can be drawn in parallel and
independently of each other.
"""
from __future__ import annotations

import concurrent.futures as _cf
import math
import os
from dataclasses import dataclass, replace
from typing import Optional

import numpy as np

__all__ = [
    "LayerShape", "WORKLOADS", "WORKLOAD_ORDER", "workload", "make_inputs",
    "f32_to_bf16_bits", "bf16_bits_to_f32", "random_rows", "MARGIN", "EC_MARGIN",
    "ec_tokens_per_expert",
]

MARGIN = 1e-3

# stream tags (fixed forever: changing one changes every generated tensor)
_TAG_X, _TAG_X_REDRAW, _TAG_WG, _TAG_BG = 1, 2, 3, 4
_TAG_W1, _TAG_B1, _TAG_W2, _TAG_B2 = 5, 6, 7, 8
_TAG_WS1, _TAG_BS1, _TAG_WS2, _TAG_BS2 = 9, 10, 11, 12
_TAG_ROWS = 13
_TAG_X_REDRAW_EC = 14


@dataclass(frozen=True)
class LayerShape:
    name: str
    T: int
    d: int
    F: int
    E: int
    k: int
    act: str = "gelu"          # "gelu" (exact erf form) or "relu"
    dtype: str = "bf16"        # "f32" or "bf16": x, y, expert weights and biases
    capacity: int = -1         # <0: unlimited; else max rows per routed expert
    Fs: int = 0                # d_ff of the always-on shared expert (0: none)
    router_bias: str = "none"  # "none" | "normal" | "zipf1.1"
    renormalize: int = 1
    expert_bias: bool = True
    routing: str = "token"     # "token": each token takes its top-k experts;
                               # "expert": each expert takes its top-C tokens

    def with_(self, **kw) -> "LayerShape":
        return replace(self, **kw)

    @property
    def active_flop(self) -> float:
        """Expert FLOPs of one layer call if no row is dropped (2 FLOP/MAC)."""
        per_row = 4.0 * self.d * self.F
        f = self.T * self.k * per_row
        if self.Fs:
            f += self.T * 4.0 * self.d * self.Fs
        return f


WORKLOADS = {
    "tiny_f32": LayerShape("tiny_f32", T=64, d=64, F=256, E=8, k=2,
                           dtype="f32", router_bias="normal"),
    "page1_b4s512": LayerShape("page1_b4s512", T=2048, d=768, F=3072, E=8, k=2),
    "mixtral_t4096": LayerShape("mixtral_t4096", T=4096, d=4096, F=14336, E=8, k=2),
    "switch_e64_top1_cap": LayerShape("switch_e64_top1_cap", T=8192, d=1024, F=4096,
                                      E=64, k=1, act="relu", capacity=160,
                                      router_bias="zipf1.1"),
    "deepseek_e256_top8": LayerShape("deepseek_e256_top8", T=512, d=7168, F=2048,
                                     E=256, k=8, Fs=2048),
    # one expert-parallel rank's share of the DeepSeek-shaped layer on 8 GPUs
    # with 512 tokens each: its 32 experts receive the 4096 rows routed to
    # them (about 128 each) and stream 1.9 GB of weights; a top-1 router over
    # the 32 local experts stands in for the remote routing and the exchange
    "deepseek_ep8_rank": LayerShape("deepseek_ep8_rank", T=4096, d=7168, F=2048, E=32, k=1),
    # expert-choice routing on the Switch-style shape: each of the 64 experts
    # takes its top floor(T*k/E) = 256 tokens (capacity factor k = 2)
    "expert_choice_t8192_e64": LayerShape("expert_choice_t8192_e64", T=8192, d=1024,
                                          F=4096, E=64, k=2, routing="expert"),
}
WORKLOAD_ORDER = ["tiny_f32", "page1_b4s512", "mixtral_t4096",
                  "switch_e64_top1_cap", "deepseek_e256_top8", "deepseek_ep8_rank"]


def workload(name_or_index) -> LayerShape:
    if isinstance(name_or_index, int):
        return WORKLOADS[WORKLOAD_ORDER[name_or_index]]
    return WORKLOADS[name_or_index]


# --------------------------------------------------------------------- bf16
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


# ------------------------------------------------------------------ streams
def _rng(seed: int, tag: int, index: int = 0, attempt: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([int(seed), tag, int(index), int(attempt)])))


def _normal(seed, tag, index, shape, std, dtype, out=None):
    g = _rng(seed, tag, index)
    z = g.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        z *= np.float32(std)
    if dtype == "bf16":
        if out is not None:
            out[...] = f32_to_bf16_bits(z)
            return out
        return f32_to_bf16_bits(z)
    if out is not None:
        out[...] = z
        return out
    return z


def random_rows(seed: int, shape, dtype="f32") -> np.ndarray:
    """Plain N(0,1) tensor for stage-level tests (e.g. expert rows to combine)."""
    return _normal(seed, _TAG_ROWS, 0, shape, 1.0, dtype)


def _to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _margin_ok(xr64: np.ndarray, Wg64: np.ndarray, bg64, k: int, E: int, margin: float):
    """True per row when the top-(k+1) sorted router scores are pairwise >= margin apart.

    Only the gaps among the k+1 highest scores are checked (all of them when
    k == E)."""
    s = xr64 @ Wg64.T
    if bg64 is not None:
        s = s + bg64
    m = min(k + 1, E)
    if m < 2:
        return np.ones(s.shape[0], dtype=bool)
    top = -np.sort(-s, axis=1)[:, :m]
    gaps = top[:, :-1] - top[:, 1:]
    return np.all(gaps >= margin, axis=1)


def ec_tokens_per_expert(shape: LayerShape) -> int:
    """Tokens each expert takes under expert-choice routing: the capacity when one
    is given, else floor(T*k/E) (k read as the capacity factor); at most T."""
    c = shape.capacity if shape.capacity >= 0 else (shape.T * shape.k) // shape.E
    return min(c, shape.T)


EC_MARGIN = 1e-6


def _ec_boundary_ties(x64, Wg64, bg64, C: int, margin: float):
    """Token rows at a near-tie on some expert's top-C boundary: for every expert,
    the fp64 router probabilities of the C-th and (C+1)-th largest tokens closer
    than `margin` (absolute; an fp32 evaluation is far more precise)."""
    T = x64.shape[0]
    if C <= 0 or C >= T:
        return np.zeros(0, dtype=np.int64)
    s = x64 @ Wg64.T
    if bg64 is not None:
        s = s + bg64
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=1, keepdims=True)
    bad = set()
    for e in range(p.shape[1]):
        col = p[:, e]
        order = np.argsort(-col, kind="stable")
        a, b = order[C - 1], order[C]
        if col[a] - col[b] < margin:
            bad.update((int(a), int(b)))
    return np.array(sorted(bad), dtype=np.int64)


def make_inputs(shape: LayerShape, seed: int, *, margin: float = MARGIN,
                threads: Optional[int] = None) -> dict:
    """Draw every input of one layer call.

    Returns a dict with numpy arrays: ``x [T,d]``, ``Wg [E,d]`` (f32),
    ``bg [E]`` (f32 or None), ``W1 [E,F,d]``, ``b1 [E,F]``, ``W2 [E,d,F]``,
    ``b2 [E,d]`` and, when ``Fs`` > 0, ``Ws1 [Fs,d]``, ``bs1``, ``Ws2 [d,Fs]``,
    ``bs2``.  bf16 tensors are uint16 bit patterns.  ``redrawn`` counts the
    token rows replaced by the margin filter.
    """
    s = shape
    dt = s.dtype
    nthr = threads or _threads()
    np_dt = np.uint16 if dt == "bf16" else np.float32
    out = {"shape": s, "seed": seed}

    Wg = _normal(seed, _TAG_WG, 0, (s.E, s.d), 1.0 / math.sqrt(s.d), "f32")
    if s.router_bias == "none":
        bg = None
    elif s.router_bias == "normal":
        bg = _normal(seed, _TAG_BG, 0, (s.E,), 0.1, "f32")
    elif s.router_bias == "zipf1.1":
        # b_g[e] = ln p_e with p_e proportional to (e+1)^-1.1
        w = np.arange(1, s.E + 1, dtype=np.float64) ** -1.1
        bg = np.log(w / w.sum()).astype(np.float32)
    else:
        raise ValueError(s.router_bias)
    out["Wg"], out["bg"] = Wg, bg

    x = _normal(seed, _TAG_X, 0, (s.T, s.d), 1.0, dt)
    redrawn = 0
    if margin > 0 and s.T > 0 and s.routing == "expert":
        # expert choice: redraw the token rows that sit at a near-tie on some
        # expert's top-C boundary until no boundary is that close
        Wg64 = Wg.astype(np.float64)
        bg64 = None if bg is None else bg.astype(np.float64)
        C = ec_tokens_per_expert(s)
        attempt = np.zeros(s.T, dtype=np.int64)
        for _ in range(1000):
            bad = _ec_boundary_ties(_to_f64(x, dt), Wg64, bg64, C, EC_MARGIN)
            if bad.size == 0:
                break
            for t in bad:
                attempt[t] += 1
                row = _rng(seed, _TAG_X_REDRAW_EC, t, attempt[t]).standard_normal(
                    (s.d,), dtype=np.float32)
                x[t] = f32_to_bf16_bits(row) if dt == "bf16" else row
                redrawn += 1
        else:  # pragma: no cover
            raise RuntimeError("expert-choice margin filter did not settle")
    elif margin > 0 and s.T > 0:
        Wg64 = Wg.astype(np.float64)
        bg64 = None if bg is None else bg.astype(np.float64)
        ok = _margin_ok(_to_f64(x, dt), Wg64, bg64, s.k, s.E, margin)
        for t in np.nonzero(~ok)[0]:
            for attempt in range(1, 1000):
                row = _rng(seed, _TAG_X_REDRAW, t, attempt).standard_normal(
                    (1, s.d), dtype=np.float32)
                if dt == "bf16":
                    row = f32_to_bf16_bits(row)
                if _margin_ok(_to_f64(row, dt), Wg64, bg64, s.k, s.E, margin)[0]:
                    x[t] = row[0]
                    redrawn += 1
                    break
            else:  # pragma: no cover
                raise RuntimeError("margin filter could not redraw row %d" % t)
    out["x"], out["redrawn"] = x, redrawn

    W1 = np.empty((s.E, s.F, s.d), dtype=np_dt)
    W2 = np.empty((s.E, s.d, s.F), dtype=np_dt)
    b1 = np.empty((s.E, s.F), dtype=np_dt) if s.expert_bias else None
    b2 = np.empty((s.E, s.d), dtype=np_dt) if s.expert_bias else None
    sd1, sd2 = 1.0 / math.sqrt(s.d), 1.0 / math.sqrt(s.F)

    def one(e):
        _normal(seed, _TAG_W1, e, (s.F, s.d), sd1, dt, out=W1[e])
        _normal(seed, _TAG_W2, e, (s.d, s.F), sd2, dt, out=W2[e])
        if s.expert_bias:
            _normal(seed, _TAG_B1, e, (s.F,), 0.1, dt, out=b1[e])
            _normal(seed, _TAG_B2, e, (s.d,), 0.1, dt, out=b2[e])

    if s.E * s.F * s.d >= (1 << 22) and nthr > 1:
        with _cf.ThreadPoolExecutor(nthr) as ex:
            list(ex.map(one, range(s.E)))
    else:
        for e in range(s.E):
            one(e)
    out.update(W1=W1, b1=b1, W2=W2, b2=b2)

    if s.Fs:
        out["Ws1"] = _normal(seed, _TAG_WS1, 0, (s.Fs, s.d), 1.0 / math.sqrt(s.d), dt)
        out["Ws2"] = _normal(seed, _TAG_WS2, 0, (s.d, s.Fs), 1.0 / math.sqrt(s.Fs), dt)
        out["bs1"] = _normal(seed, _TAG_BS1, 0, (s.Fs,), 0.1, dt) if s.expert_bias else None
        out["bs2"] = _normal(seed, _TAG_BS2, 0, (s.d,), 0.1, dt) if s.expert_bias else None
    else:
        out.update(Ws1=None, bs1=None, Ws2=None, bs2=None)
    return out


def to_device(inp: dict, device="cuda") -> dict:
    """Copy the arrays of ``make_inputs`` to torch tensors on ``device``.

    bf16 bit patterns become torch.bfloat16 tensors with the same bits; fp32
    stays fp32; None stays None."""
    import torch

    out = {}
    for key in ("x", "Wg", "bg", "W1", "b1", "W2", "b2", "Ws1", "bs1", "Ws2", "bs2"):
        a = inp.get(key)
        if a is None:
            out[key] = None
        elif a.dtype == np.uint16:
            out[key] = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
        else:
            out[key] = torch.from_numpy(np.ascontiguousarray(a)).to(device)
    return out
