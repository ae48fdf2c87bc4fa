"""Pins of the oracle's backward pass (CPU only).

The loss is L = sum_t <dy_t, y_t> + alpha * balance, with the top-k selection
and the capacity drops held fixed.  Nothing here re-types the oracle's chain
rule: the expected gradients come from torch's autograd (fp64) through the
layer written as torch CPU library calls, from central finite differences of
the (separately pinned) forward oracle, from the zero-sum invariant of a
softmax gradient, from the closed form of the balance term's gradient, and
from linearity in dy.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

import oracle
from moe_synth import LayerShape, bf16_bits_to_f32, make_inputs

PARAMS = ("x", "Wg", "bg", "W1", "b1", "W2", "b2", "Ws1", "bs1", "Ws2", "bs2")
GRAD = {"x": "dx", "Wg": "dWg", "bg": "dbg", "W1": "dW1", "b1": "db1", "W2": "dW2",
        "b2": "db2", "Ws1": "dWs1", "bs1": "dbs1", "Ws2": "dWs2", "bs2": "dbs2"}


def small(**kw):
    base = dict(name="b", T=36, d=24, F=40, E=6, k=2, dtype="f32", router_bias="normal")
    base.update(kw)
    return LayerShape(**base)


def as64(a, shape, name):
    if a is None:
        return None
    router = name in ("Wg", "bg")
    v = bf16_bits_to_f32(a) if (shape.dtype == "bf16" and not router) else a
    return torch.from_numpy(np.asarray(v, np.float64).copy())


def dy_of(shape, seed=5):
    return np.random.default_rng(seed).standard_normal((shape.T, shape.d))


def torch_grads(shape, inp, rt, dy, alpha):
    """Autograd of the layer as torch library calls with the oracle's selection
    (topk_idx, keep) held fixed: F.linear router, softmax, gather of the chosen
    probabilities, optional renormalisation, per-expert F.linear / act / F.linear
    on the rows that chose it, gate-weighted sum, shared expert, plus
    alpha * torch.var(mean probability) (unbiased)."""
    P = {n: as64(inp.get(n), shape, n) for n in PARAMS}
    for v in P.values():
        if v is not None:
            v.requires_grad_(True)
    x = P["x"]
    probs = torch.softmax(Fn.linear(x, P["Wg"], P["bg"]), dim=-1)
    idx = torch.from_numpy(rt["topk_idx"].astype(np.int64))
    keep = torch.from_numpy(rt["keep"].astype(bool))
    g = probs.gather(1, idx)
    if shape.renormalize:
        g = g / g.sum(dim=-1, keepdim=True)
    act = Fn.gelu if shape.act == "gelu" else torch.relu
    y = torch.zeros_like(x)
    for e in range(shape.E):
        hit = (idx == e) & keep
        rows = hit.any(dim=-1).nonzero().flatten()
        if rows.numel() == 0:
            continue
        b1 = None if P["b1"] is None else P["b1"][e]
        b2 = None if P["b2"] is None else P["b2"][e]
        out = Fn.linear(act(Fn.linear(x[rows], P["W1"][e], b1)), P["W2"][e], b2)
        gate = (g[rows] * hit[rows]).sum(dim=-1, keepdim=True)
        y = y.index_add(0, rows, gate * out)
    if shape.Fs:
        y = y + Fn.linear(act(Fn.linear(x, P["Ws1"], P["bs1"])), P["Ws2"], P["bs2"])
    L = (torch.from_numpy(dy) * y).sum()
    if alpha:
        L = L + alpha * torch.var(probs.mean(dim=0))
    L.backward()
    return {GRAD[n]: v.grad.numpy() for n, v in P.items() if v is not None}


def assert_close(got, want, rel=1e-9, what=""):
    scale = max(float(np.abs(want).max()), 1e-30)
    err = float(np.abs(got - want).max())
    assert err <= rel * scale, (what, err, scale)


CASES = [
    small(Fs=16, capacity=10, router_bias="zipf1.1"),
    small(dtype="bf16", act="relu", renormalize=0, E=5, k=3),
    small(E=4, k=4),
    small(E=1, k=1, T=20),
    small(d=16, F=32, E=8, k=2, Fs=24, act="relu", expert_bias=False, router_bias="none"),
]


@pytest.mark.parametrize("shape", CASES, ids=lambda s: "%s_E%d_k%d_Fs%d_cap%d_%s" % (
    s.dtype, s.E, s.k, s.Fs, s.capacity, s.act))
@pytest.mark.parametrize("alpha", [0.0, 0.7])
def test_backward_matches_torch_autograd(shape, alpha):
    if shape.E == 1 and alpha:
        pytest.skip("balance is undefined for one expert")
    inp = make_inputs(shape, 21)
    rt = oracle.route(shape, inp, with_probs=False)
    dy = dy_of(shape)
    got = oracle.backward(shape, inp, dy, alpha, rt=rt)
    want = torch_grads(shape, inp, rt, dy, alpha)
    for key, w in want.items():
        assert_close(got[key], w, what=key)
    if shape.capacity >= 0:
        assert (rt["keep"] == 0).any()   # some pairs were dropped


def _loss(shape, inp, dy, alpha):
    r = oracle.forward(shape, inp)
    L = float(np.sum(dy * r["y"]))
    return L + (alpha * r["balance"] if alpha else 0.0), r


GROUPS = [("x",), ("Wg", "bg"), ("W1", "b1"), ("W2", "b2"), ("Ws1", "bs1", "Ws2", "bs2")]


@pytest.mark.parametrize("group", GROUPS, ids=lambda g: "+".join(g))
def test_backward_matches_central_differences(group):
    """Directional derivative of the forward oracle's loss along a random
    direction of one parameter group.  Inputs are stored in fp32, so the step
    actually taken is the difference of the two rounded points; the selection
    must be the same at both points."""
    shape = small(Fs=16, capacity=12, T=30)
    alpha = 0.9
    inp = make_inputs(shape, 8)
    dy = dy_of(shape, 9)
    rt = oracle.route(shape, inp, with_probs=False)
    grads = oracle.backward(shape, inp, dy, alpha, rt=rt)
    rng = np.random.default_rng(17)
    eps = 1e-4
    plus, minus, an = dict(inp), dict(inp), 0.0
    for name in group:
        a = inp[name]
        v = rng.standard_normal(a.shape)
        ap = (a.astype(np.float64) + eps * v).astype(np.float32)
        am = (a.astype(np.float64) - eps * v).astype(np.float32)
        plus[name], minus[name] = ap, am
        step = (ap.astype(np.float64) - am.astype(np.float64)) / (2 * eps)
        an += float(np.sum(grads[GRAD[name]] * step))
    Lp, rp = _loss(shape, plus, dy, alpha)
    Lm, rm = _loss(shape, minus, dy, alpha)
    for r in (rp, rm):
        assert np.array_equal(r["topk_idx"], rt["topk_idx"])
        assert np.array_equal(r["keep"], rt["keep"])
    fd = (Lp - Lm) / (2 * eps)
    assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (fd, an)


def test_router_gradient_sums_to_zero_over_experts():
    """A softmax's gradient sums to zero over its outputs, so summed over
    experts the router weight and bias gradients vanish."""
    shape = small(E=7, k=3, Fs=8)
    inp = make_inputs(shape, 4)
    g = oracle.backward(shape, inp, dy_of(shape), alpha=0.4)
    scale = float(np.abs(g["dWg"]).max())
    assert float(np.abs(g["dWg"].sum(axis=0)).max()) <= 1e-12 * scale
    assert abs(float(g["dbg"].sum())) <= 1e-12 * float(np.abs(g["dbg"]).max())
    d = oracle.backward_tokens(shape, inp, dy_of(shape), np.arange(shape.T), alpha=0.4)
    assert float(np.abs(d["dl"].sum(axis=1)).max()) <= 1e-13


def test_balance_term_closed_form():
    """With dy = 0 only the balance term acts: d balance / d p[t, e] =
    2 (m_e - mean m) / ((E - 1) T), then the softmax Jacobian p (dp - <p, dp>),
    then dWg = dl^T x and dbg = sum_t dl; every expert-weight gradient is zero."""
    shape = small(E=5, k=2, Fs=8)
    inp = make_inputs(shape, 6)
    alpha = 1.3
    r = oracle.route(shape, inp)
    p, m = r["probs"], r["mean_prob"]
    E, T = shape.E, shape.T
    dp = np.broadcast_to(alpha * 2 * (m - m.mean()) / ((E - 1) * T), p.shape)
    dl = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
    g = oracle.backward(shape, inp, np.zeros((T, shape.d)), alpha)
    x = inp["x"].astype(np.float64)
    assert_close(g["dWg"], dl.T @ x, 1e-12, "dWg")
    assert_close(g["dbg"], dl.sum(axis=0), 1e-12, "dbg")
    assert_close(g["dx"], dl @ inp["Wg"].astype(np.float64), 1e-12, "dx")
    for key in ("dW1", "db1", "dW2", "db2", "dWs1", "dbs1", "dWs2", "dbs2"):
        assert not np.any(g[key]), key


def test_linear_in_upstream_gradient():
    shape = small(E=4, k=2, capacity=8)
    inp = make_inputs(shape, 12)
    a, b = dy_of(shape, 1), dy_of(shape, 2)
    ga = oracle.backward(shape, inp, a)
    gb = oracle.backward(shape, inp, b)
    gab = oracle.backward(shape, inp, 2.0 * a - b)
    for key in ga:
        assert_close(gab[key], 2.0 * ga[key] - gb[key], 1e-11, key)


def test_sampled_entry_points_agree_with_the_full_backward():
    """backward_tokens and backward_expert_entries (used for large shapes)
    against the full backward on a small one."""
    shape = small(Fs=16, capacity=10, k=3)
    inp = make_inputs(shape, 3)
    dy = dy_of(shape, 4)
    g = oracle.backward(shape, inp, dy, alpha=0.2)
    toks = [0, 5, 35]
    t = oracle.backward_tokens(shape, inp, dy, toks, alpha=0.2)
    assert np.allclose(t["dx"], g["dx"][toks], rtol=0, atol=1e-13)
    fl, jl = [0, 7, 39], [1, 23]
    for e in (0, 3, -1):
        W1, b1, W2, b2 = (("dWs1", "dbs1", "dWs2", "dbs2") if e < 0 else
                          ("dW1", "db1", "dW2", "db2"))
        G1 = g[W1] if e < 0 else g[W1][e]
        G2 = g[W2] if e < 0 else g[W2][e]
        B1 = g[b1] if e < 0 else g[b1][e]
        B2 = g[b2] if e < 0 else g[b2][e]
        fl_ = [f for f in fl if f < shape.Fs] if e < 0 else fl
        s = oracle.backward_expert_entries(shape, inp, dy, e, fl_, jl)
        assert np.allclose(s["dW1"], G1[np.ix_(fl_, jl)], rtol=0, atol=1e-12)
        assert np.allclose(s["dW2"], G2[np.ix_(jl, fl_)], rtol=0, atol=1e-12)
        assert np.allclose(s["db1"], B1[fl_], rtol=0, atol=1e-12)
        assert np.allclose(s["db2"], B2[jl], rtol=0, atol=1e-12)


def torch_ec_grads(shape, inp, sel, dy, alpha):
    """Autograd of the expert-choice layer as torch library calls with the
    oracle's selection held fixed: y = sum_e sel[:, e] p[:, e] E_e(x) (+ shared)."""
    P = {n: as64(inp.get(n), shape, n) for n in PARAMS}
    for v in P.values():
        if v is not None:
            v.requires_grad_(True)
    x = P["x"]
    probs = torch.softmax(Fn.linear(x, P["Wg"], P["bg"]), dim=-1)
    act = Fn.gelu if shape.act == "gelu" else torch.relu
    y = torch.zeros_like(x)
    selt = torch.from_numpy(sel.astype(bool))
    for e in range(shape.E):
        rows = selt[:, e].nonzero().flatten()
        if rows.numel() == 0:
            continue
        b1 = None if P["b1"] is None else P["b1"][e]
        b2 = None if P["b2"] is None else P["b2"][e]
        out = Fn.linear(act(Fn.linear(x[rows], P["W1"][e], b1)), P["W2"][e], b2)
        y = y.index_add(0, rows, probs[rows, e:e + 1] * out)
    if shape.Fs:
        y = y + Fn.linear(act(Fn.linear(x, P["Ws1"], P["bs1"])), P["Ws2"], P["bs2"])
    L = (torch.from_numpy(dy) * y).sum()
    if alpha:
        L = L + alpha * torch.var(probs.mean(dim=0))
    L.backward()
    return {GRAD[n]: v.grad.numpy() for n, v in P.items() if v is not None}


@pytest.mark.parametrize("shape", [
    small(routing="expert", Fs=16),
    small(routing="expert", dtype="bf16", act="relu", E=5, k=2, capacity=9),
    small(routing="expert", E=70, k=3, T=50, router_bias="none"),
], ids=["f32_shared", "bf16_capacity", "e70"])
def test_ec_backward_matches_torch_autograd(shape):
    inp = make_inputs(shape, 23)
    r = oracle.ec_route(shape, inp)
    dy = dy_of(shape)
    got = oracle.ec_backward(shape, inp, dy, 0.6, r=r)
    want = torch_ec_grads(shape, inp, r["sel"], dy, 0.6)
    for key, w in want.items():
        assert_close(got[key], w, what=key)
