"""Pins of the fp64 CPU oracle against what the pages and the mathematics fix.

Every test here runs on the CPU.  None of them re-types the oracle's own
loops: the expected values come from the worked example printed on the
roadtointelligence page, closed forms, and special cases that reduce to torch
CPU library routines (nn.Linear layout via F.linear, the erf GELU of F.gelu,
torch.topk, torch.std).
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

import oracle
from moe_synth import LayerShape, bf16_bits_to_f32, f32_to_bf16_bits, make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def small(**kw):
    base = dict(name="t", T=40, d=24, F=40, E=6, k=2, dtype="f32", router_bias="normal")
    base.update(kw)
    return LayerShape(**base)


def widen(a, dtype):
    if a is None:
        return None
    return torch.from_numpy(bf16_bits_to_f32(a) if dtype == "bf16" else a).double()


def torch_reference(shape, inp):
    """The layer as torch CPU library calls, fp64: F.linear router, softmax,
    torch.topk, optional renormalise, per-expert F.linear/act/F.linear MLP on
    the tokens that picked it, gate-weighted sum, plus the shared expert."""
    dt = shape.dtype
    x = widen(inp["x"], dt)
    Wg = torch.from_numpy(inp["Wg"]).double()
    bg = None if inp["bg"] is None else torch.from_numpy(inp["bg"]).double()
    probs = torch.softmax(Fn.linear(x, Wg, bg), dim=-1)
    w, idx = torch.topk(probs, shape.k, dim=-1)
    if shape.renormalize:
        w = w / w.sum(dim=-1, keepdim=True)
    act = (lambda z: Fn.gelu(z)) if shape.act == "gelu" else torch.relu
    y = torch.zeros_like(x)
    W1, W2 = widen(inp["W1"], dt), widen(inp["W2"], dt)
    b1 = widen(inp["b1"], dt)
    b2 = widen(inp["b2"], dt)
    for e in range(shape.E):
        hit = (idx == e)
        rows = hit.any(dim=-1).nonzero().flatten()
        if rows.numel() == 0:
            continue
        out = Fn.linear(act(Fn.linear(x[rows], W1[e], None if b1 is None else b1[e])),
                        W2[e], None if b2 is None else b2[e])
        gate = (w[rows] * hit[rows]).sum(dim=-1, keepdim=True)
        y[rows] += gate * out
    if shape.Fs:
        bs1 = widen(inp["bs1"], dt)
        bs2 = widen(inp["bs2"], dt)
        y += Fn.linear(act(Fn.linear(x, widen(inp["Ws1"], dt), bs1)), widen(inp["Ws2"], dt), bs2)
    return y.numpy(), idx.numpy(), w.numpy(), probs.numpy()


# ------------------------------------------------------------ worked example
def worked_example_inputs(scores, E, k):
    shape = LayerShape("worked", T=1, d=E, F=4, E=E, k=k, dtype="f32", router_bias="none")
    inp = make_inputs(shape, 0, margin=0)
    inp["x"] = np.array([scores], np.float32)
    inp["Wg"] = np.eye(E, dtype=np.float32)  # identity router: logits are the scores
    return shape, inp


def test_worked_example_gates():
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    shape, inp = worked_example_inputs(g["scores"], g["n_experts"], g["top_k"])
    r = oracle.route(shape, inp)
    expect_idx = [e - 1 for e in g["selected_experts_one_based"]]
    assert r["topk_idx"][0].tolist() == expect_idx
    w = r["topk_w"][0]
    assert [round(v, g["printed_decimals"]) for v in w] == g["printed_weights_2dp"]
    # closed form: softmax over the two kept scores (2.0 and 1.9, as stored in fp32)
    e20, e19 = math.exp(2.0), math.exp(float(np.float32(1.9)))
    assert abs(w[0] - e20 / (e20 + e19)) < 1e-14
    assert abs(w[1] - e19 / (e20 + e19)) < 1e-14
    assert abs(w.sum() - 1.0) < 1e-15
    # the full softmax over all eight scores
    s = np.array(g["scores"], np.float32).astype(np.float64)
    p = np.exp(s) / np.exp(s).sum()
    assert np.allclose(r["probs"][0], p, rtol=0, atol=1e-15)


def test_worked_example_without_renormalisation():
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    shape, inp = worked_example_inputs(g["scores"], g["n_experts"], g["top_k"])
    shape = shape.with_(renormalize=0)
    r = oracle.route(shape, inp)
    s = np.array(g["scores"], np.float32).astype(np.float64)
    p = np.exp(s) / np.exp(s).sum()
    assert r["topk_idx"][0].tolist() == [2, 6]
    assert np.allclose(r["topk_w"][0], [p[2], p[6]], rtol=0, atol=1e-15)


def test_worked_example_combine_closed_form():
    """With W2 = 0 each expert returns its bias b2, so y = g0 b2[2] + g1 b2[6]."""
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    shape, inp = worked_example_inputs(g["scores"], g["n_experts"], g["top_k"])
    inp["W2"] = np.zeros_like(inp["W2"])
    y = oracle.forward(shape, inp)["y"][0]
    e20, e19 = math.exp(2.0), math.exp(float(np.float32(1.9)))
    b2 = inp["b2"].astype(np.float64)
    expect = e20 / (e20 + e19) * b2[2] + e19 / (e20 + e19) * b2[6]
    assert np.allclose(y, expect, rtol=0, atol=1e-15)


# -------------------------------------------------------------- invariants
@pytest.mark.parametrize("k", [1, 2, 3, 6])
def test_gates_sum_to_one_and_k_distinct(k):
    shape = small(k=k)
    inp = make_inputs(shape, 3)
    r = oracle.route(shape, inp)
    assert np.allclose(r["topk_w"].sum(axis=1), 1.0, atol=1e-14)
    for row in r["topk_idx"]:
        assert len(set(row.tolist())) == k and row.min() >= 0 and row.max() < shape.E
    assert r["counts"].sum() == shape.T * k
    if k == 1:
        assert np.all(r["topk_w"] == 1.0)


def test_mixtral_form_equals_softmax_topk_renormalise():
    """softmax over the top-k scores (others at -inf) equals renormalised top-k of
    the full softmax (roadtointelligence router formula vs the botmartz code)."""
    shape = small(k=3, E=7)
    inp = make_inputs(shape, 5)
    r = oracle.route(shape, inp)
    s = inp["x"].astype(np.float64) @ inp["Wg"].astype(np.float64).T + inp["bg"]
    for t in range(shape.T):
        masked = np.full(shape.E, -np.inf)
        masked[r["topk_idx"][t]] = s[t, r["topk_idx"][t]]
        g = np.exp(masked - masked.max())
        g /= g.sum()
        assert np.allclose(g[r["topk_idx"][t]], r["topk_w"][t], rtol=0, atol=1e-12)


def test_selection_descending_and_lowest_index_on_ties():
    shape = small(T=3, d=4, E=4, k=2, router_bias="none")
    inp = make_inputs(shape, 1, margin=0)
    inp["Wg"] = np.eye(4, dtype=np.float32)
    inp["x"] = np.array([[0.0, 0.0, 0.0, 0.0], [1.0, 3.0, 3.0, 2.0], [-1.0, 0.5, 0.5, 0.5]],
                        np.float32)
    r = oracle.route(shape, inp)
    assert r["topk_idx"].tolist() == [[0, 1], [1, 2], [1, 2]]
    assert np.allclose(r["topk_w"], 0.5)


# ------------------------------------------------------ library special cases
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("act,renorm", [("gelu", 1), ("relu", 0), ("relu", 1)])
def test_matches_torch_library_layer(dtype, act, renorm):
    shape = small(dtype=dtype, act=act, renormalize=renorm, T=50, d=32, F=48, E=5, k=2)
    inp = make_inputs(shape, 11)
    y_ref, idx, w, probs = torch_reference(shape, inp)
    r = oracle.forward(shape, inp)
    assert np.array_equal(r["topk_idx"], idx)
    assert np.allclose(r["topk_w"], w, rtol=0, atol=1e-14)
    assert np.allclose(r["probs"], probs, rtol=0, atol=1e-14)
    assert np.allclose(r["y"], y_ref, rtol=1e-12, atol=1e-12)


def test_matches_torch_with_shared_expert():
    shape = small(Fs=20, T=30, E=6, k=3)
    inp = make_inputs(shape, 2)
    y_ref, idx, w, _ = torch_reference(shape, inp)
    r = oracle.forward(shape, inp)
    assert np.array_equal(r["topk_idx"], idx)
    assert np.allclose(r["y"], y_ref, rtol=1e-12, atol=1e-12)


def test_single_expert_is_plain_mlp():
    """E = 1, k = 1: the layer is the textbook two-layer MLP F.linear/gelu/F.linear."""
    shape = small(E=1, k=1, T=17, d=16, F=36)
    inp = make_inputs(shape, 4)
    x = torch.from_numpy(inp["x"]).double()
    h = Fn.gelu(Fn.linear(x, torch.from_numpy(inp["W1"][0]).double(),
                          torch.from_numpy(inp["b1"][0]).double()))
    y = Fn.linear(h, torch.from_numpy(inp["W2"][0]).double(),
                  torch.from_numpy(inp["b2"][0]).double()).numpy()
    assert np.allclose(oracle.forward(shape, inp)["y"], y, rtol=1e-13, atol=1e-13)


def test_all_experts_is_dense_soft_mixture():
    """k = E: every expert runs and y = sum_e p_e E_e(x) with the full softmax."""
    shape = small(E=4, k=4)
    inp = make_inputs(shape, 6)
    r = oracle.forward(shape, inp)
    y = np.zeros((shape.T, shape.d))
    for e in range(shape.E):
        for t in range(shape.T):
            y[t] += r["probs"][t, e] * oracle.expert_row(shape, inp, t, e, 1.0)
    assert np.allclose(r["y"], y, rtol=1e-12, atol=1e-13)


def test_dense_masked_brute_force():
    """Evaluate every expert on every token in numpy fp64 and mask to the top-k:
    the other experts contribute exactly nothing."""
    shape = small(T=30, d=20, F=28, E=6, k=2)
    inp = make_inputs(shape, 8)
    r = oracle.forward(shape, inp)
    x = inp["x"].astype(np.float64)
    gelu = np.vectorize(lambda z: 0.5 * z * (1.0 + math.erf(z / math.sqrt(2.0))))
    allout = np.stack([gelu(x @ inp["W1"][e].T.astype(np.float64) + inp["b1"][e])
                       @ inp["W2"][e].T.astype(np.float64) + inp["b2"][e]
                       for e in range(shape.E)], axis=1)          # [T, E, d]
    mask = np.zeros((shape.T, shape.E))
    for t in range(shape.T):
        mask[t, r["topk_idx"][t]] = r["topk_w"][t]
    y = np.einsum("te,ted->td", mask, allout)
    assert np.allclose(r["y"], y, rtol=1e-12, atol=1e-12)


def test_linear_in_output_projection():
    shape = small()
    inp = make_inputs(shape, 9)
    y1 = oracle.forward(shape, inp)["y"]
    inp2 = dict(inp, W2=inp["W2"] * np.float32(2.0), b2=inp["b2"] * np.float32(2.0))
    y2 = oracle.forward(shape, inp2)["y"]
    assert np.array_equal(y2, 2.0 * y1)


def test_token_permutation_equivariance():
    shape = small(T=32)
    inp = make_inputs(shape, 12)
    y = oracle.forward(shape, inp)["y"]
    perm = np.random.default_rng(0).permutation(shape.T)
    y2 = oracle.forward(shape, dict(inp, x=np.ascontiguousarray(inp["x"][perm])))["y"]
    assert np.allclose(y2, y[perm], rtol=0, atol=1e-13)


# ---------------------------------------------------------------- capacity
def test_capacity_at_least_tokens_is_unlimited():
    shape = small(T=30)
    inp = make_inputs(shape, 13)
    a = oracle.forward(shape, inp)
    b = oracle.forward(shape.with_(capacity=shape.T), inp)
    assert np.array_equal(a["y"], b["y"]) and np.all(b["keep"] == 1)


def test_capacity_zero_leaves_only_shared_expert():
    shape = small(T=20, Fs=12, capacity=0)
    inp = make_inputs(shape, 14)
    r = oracle.forward(shape, inp)
    assert r["kept"].sum() == 0 and np.all(r["keep"] == 0)
    shared = np.stack([oracle.expert_row(shape, inp, t, -1, 1.0) for t in range(shape.T)])
    assert np.array_equal(r["y"], shared)
    r0 = oracle.forward(shape.with_(Fs=0), inp)
    assert np.all(r0["y"] == 0.0)


@pytest.mark.parametrize("k", [1, 2])
def test_capacity_keeps_first_tokens_in_index_order(k):
    """A bias forcing every token onto experts 0..k-1 keeps exactly tokens 0..C-1."""
    C_ = 7
    shape = small(T=25, E=5, k=k, capacity=C_, router_bias="none")
    inp = make_inputs(shape, 15, margin=0)
    inp["bg"] = np.array([50.0, 40.0, 0.0, 0.0, 0.0], np.float32)
    r = oracle.forward(shape, inp)
    assert np.all(r["topk_idx"] == np.arange(k))
    assert r["counts"][:k].tolist() == [shape.T] * k
    assert r["kept"][:k].tolist() == [C_] * k
    assert np.all(r["keep"][:C_] == 1) and np.all(r["keep"][C_:] == 0)
    assert np.all(r["y"][C_:] == 0.0)
    unl = oracle.forward(shape.with_(capacity=-1), inp)
    assert np.array_equal(r["y"][:C_], unl["y"][:C_])   # survivors are not renormalised again


def test_capacity_conservation_on_skewed_router():
    shape = small(T=200, E=8, k=2, capacity=30, router_bias="zipf1.1")
    inp = make_inputs(shape, 16)
    r = oracle.route(shape, inp)
    assert r["counts"].sum() == shape.T * shape.k
    assert np.array_equal(r["kept"], np.minimum(r["counts"], shape.capacity))
    assert r["keep"].sum() == r["kept"].sum()
    dropped = shape.T * shape.k - r["keep"].sum()
    assert dropped > 0
    for e in range(shape.E):
        toks = [t for t in range(shape.T) for i in range(shape.k) if r["topk_idx"][t, i] == e]
        kept_t = [t for t in range(shape.T) for i in range(shape.k)
                  if r["topk_idx"][t, i] == e and r["keep"][t, i]]
        assert kept_t == toks[:shape.capacity]


def test_dispatch_grouping():
    shape = small(T=60, E=5, k=2, capacity=20, Fs=8, router_bias="zipf1.1")
    inp = make_inputs(shape, 17)
    r = oracle.route(shape, inp)
    d = oracle.dispatch(shape, r["topk_idx"], r["keep"])
    off = d["offsets"]
    assert off[0] == 0 and np.array_equal(np.diff(off[:shape.E + 1]), r["kept"])
    assert off[shape.E + 1] - off[shape.E] == shape.T
    for e in range(shape.E):
        toks = d["row_token"][off[e]:off[e + 1]]
        assert np.all(np.diff(toks) > 0)
        for rr in range(off[e], off[e + 1]):
            t, i = d["row_token"][rr], d["row_slot"][rr]
            assert r["topk_idx"][t, i] == e and d["inv"][t, i] == rr
    assert np.array_equal(d["inv"] >= 0, r["keep"] == 1)
    assert np.array_equal(d["row_token"][off[shape.E]:], np.arange(shape.T))


def _torch_expert_rows(shape, inp, toks, e):
    """E_e(x_t) for the listed tokens as torch CPU library calls, fp64
    (e = -1: the shared expert)."""
    dt = shape.dtype
    x = widen(inp["x"], dt)[toks]
    act = (lambda z: Fn.gelu(z)) if shape.act == "gelu" else torch.relu
    if e < 0:
        W1, b1, W2, b2 = (widen(inp[n], dt) for n in ("Ws1", "bs1", "Ws2", "bs2"))
    else:
        W1, W2 = widen(inp["W1"], dt)[e], widen(inp["W2"], dt)[e]
        b1 = None if inp["b1"] is None else widen(inp["b1"], dt)[e]
        b2 = None if inp["b2"] is None else widen(inp["b2"], dt)[e]
    return Fn.linear(act(Fn.linear(x, W1, b1)), W2, b2).numpy()


@pytest.mark.parametrize("k,Fs", [(2, 8), (3, 0), (1, 8)])
def test_combine_over_grouped_rows(k, Fs):
    """The output equation y_t = sum_i g_i E_{e_i}(x_t) (+ S(x_t)) assembled by the
    gather combine: expert rows computed with torch library calls, each scaled by
    its gate and placed at the row the dispatch grouping gives it (dropped slots
    get none, shared rows start at offsets[E]), summed by oracle.combine.  The
    sum must equal the same equation written per token with the keep mask."""
    shape = small(T=48, E=5, k=k, capacity=14, Fs=Fs, router_bias="zipf1.1")
    inp = make_inputs(shape, 19)
    r = oracle.route(shape, inp)
    d = oracle.dispatch(shape, r["topk_idx"], r["keep"])
    T, E = shape.T, shape.E
    assert (r["keep"] == 0).any(), "the case must drop some slots"
    off = d["offsets"]
    nrows = int(off[E + 1])
    y_rows = np.full((nrows, shape.d), np.nan)
    for e in range(E):
        rows = np.arange(off[e], off[e + 1])
        if rows.size == 0:
            continue
        toks, slots = d["row_token"][rows], d["row_slot"][rows]
        gates = r["topk_w"][toks, slots][:, None]
        y_rows[rows] = gates * _torch_expert_rows(shape, inp, toks, e)
    if Fs:
        y_rows[off[E]:off[E] + T] = _torch_expert_rows(shape, inp, np.arange(T), -1)
    assert not np.isnan(y_rows).any()
    got = oracle.combine(shape, y_rows, d["inv"], off)
    # the same equation per token: kept slots only, gates not renormalised again
    want = np.zeros((T, shape.d))
    for t in range(T):
        for i in range(k):
            if r["keep"][t, i]:
                e = int(r["topk_idx"][t, i])
                want[t] += r["topk_w"][t, i] * _torch_expert_rows(shape, inp, [t], e)[0]
    if Fs:
        want += _torch_expert_rows(shape, inp, np.arange(T), -1)
    assert np.allclose(got, want, rtol=0, atol=1e-12)
    # and the oracle's own per-token layer output
    assert np.allclose(got, oracle.experts(shape, inp, r), rtol=0, atol=1e-12)


# -------------------------------------------------------------- statistics
def test_balance_is_torch_std_squared():
    shape = small(T=64, E=8, router_bias="zipf1.1")
    inp = make_inputs(shape, 18)
    r = oracle.route(shape, inp)
    mp = torch.from_numpy(r["probs"]).mean(dim=0)
    assert np.allclose(r["mean_prob"], mp.numpy(), rtol=0, atol=1e-15)
    assert abs(r["balance"] - float(torch.std(mp) ** 2)) < 1e-15
    assert abs(r["mean_prob"].sum() - 1.0) < 1e-13


def test_uniform_router_gives_zero_balance():
    shape = small(T=10, E=4, k=2, router_bias="none")
    inp = make_inputs(shape, 19, margin=0)
    inp["Wg"] = np.zeros_like(inp["Wg"])
    r = oracle.route(shape, inp)
    assert np.all(r["mean_prob"] == 0.25) and r["balance"] == 0.0
    assert np.all(r["topk_idx"] == [0, 1])


@pytest.mark.parametrize("k,expect", [(1, 5.0), (2, 1.875)])
def test_cv2_of_forced_routing(k, expect):
    """All T tokens forced onto experts 0..k-1 of E = 5: counts are T on k experts and 0
    elsewhere, so cv^2 = unbiased variance / mean^2 is E (k = 1) or 30/16 (k = 2) exactly."""
    shape = small(T=25, E=5, k=k, router_bias="none")
    inp = make_inputs(shape, 15, margin=0)
    inp["bg"] = np.array([50.0, 40.0, 0.0, 0.0, 0.0], np.float32)
    r = oracle.route(shape, inp)
    assert r["counts"].tolist() == [shape.T] * k + [0] * (shape.E - k)
    assert r["cv2"] == expect


def test_cv2_is_zero_when_every_expert_is_chosen():
    shape = small(T=13, E=4, k=4)
    r = oracle.route(shape, make_inputs(shape, 21))
    assert r["counts"].tolist() == [13] * 4 and r["cv2"] == 0.0


def test_cv2_undefined_cases():
    assert np.isnan(oracle.cv2([7]))          # one expert: no variance
    assert np.isnan(oracle.cv2([0, 0, 0]))    # no pairs: zero mean
    assert oracle.cv2([1, 2, 3]) == 0.25      # variance 1 (ddof 1), mean 2


def test_one_token_statistics_by_hand():
    """T = 1: mean_prob is the token's softmax; balance its unbiased variance."""
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    shape, inp = worked_example_inputs(g["scores"], 8, 2)
    r = oracle.route(shape, inp)
    s = np.array(g["scores"], np.float32).astype(np.float64)
    p = np.exp(s) / np.exp(s).sum()
    assert np.allclose(r["mean_prob"], p, atol=1e-15)
    assert abs(r["balance"] - np.var(p, ddof=1)) < 1e-15


def test_empty_batch():
    shape = small(T=0)
    inp = make_inputs(shape, 20)
    r = oracle.forward(shape, inp)
    assert r["y"].shape == (0, shape.d) and r["counts"].sum() == 0
    assert np.all(np.isnan(r["mean_prob"]))


# -------------------------------------------------------------- activation
def test_gelu_and_relu_special_values():
    """GELU is the erf form (F.gelu default); GELU(0) = 0; ReLU is exact."""
    shape = LayerShape("g", T=5, d=8, F=8, E=1, k=1, dtype="f32", expert_bias=False)
    inp = make_inputs(shape, 0, margin=0)
    inp["x"] = np.zeros((5, 8), np.float32)
    inp["x"][:, 0] = [0.0, 1.0, -1.0, 3.5, -0.25]
    inp["W1"] = np.eye(8, dtype=np.float32)[None]
    inp["W2"] = np.eye(8, dtype=np.float32)[None]
    y = oracle.forward(shape, inp)["y"][:, 0]
    z = torch.tensor([0.0, 1.0, -1.0, 3.5, -0.25], dtype=torch.float64)
    assert y[0] == 0.0
    assert np.allclose(y, Fn.gelu(z).numpy(), rtol=0, atol=1e-15)
    yr = oracle.forward(shape.with_(act="relu"), inp)["y"][:, 0]
    assert yr.tolist() == [0.0, 1.0, 0.0, 3.5, 0.0]


# ---------------------------------------------------------- expert choice
def test_ec_each_expert_takes_exactly_C_tokens():
    """Perfect load balance by construction: every expert takes min(C, T) tokens."""
    for cap, expect in [(-1, (40 * 2) // 6), (5, 5), (100, 40), (0, 0)]:
        shape = small(routing="expert", capacity=cap)
        r = oracle.ec_route(shape, make_inputs(shape, 30))
        assert r["C"] == expect
        assert r["counts"].tolist() == [expect] * shape.E
        if expect:
            assert r["cv2"] == 0.0
        else:
            assert np.isnan(r["cv2"])


def test_ec_uniform_probabilities_take_the_lowest_tokens():
    """W_g = 0, no bias: every probability is 1/E, so each expert's top-C is the
    first C tokens (lower token index first among equals)."""
    shape = small(T=20, E=4, k=1, routing="expert", router_bias="none", capacity=6)
    inp = make_inputs(shape, 31, margin=0)
    inp["Wg"] = np.zeros_like(inp["Wg"])
    r = oracle.ec_route(shape, inp)
    assert np.all(r["p"] == 0.25)
    assert np.all(r["sel"][:6] == 1) and np.all(r["sel"][6:] == 0)


def test_ec_with_every_token_is_the_dense_soft_mixture():
    """C = T: every expert takes every token, so y = sum_e p_e E_e(x), the layer that
    token-choice routing gives with k = E and no renormalisation."""
    shape = small(T=24, E=5, k=2, routing="expert", capacity=24, Fs=8)
    inp = make_inputs(shape, 32, margin=0)
    r = oracle.ec_forward(shape, inp)
    assert np.all(r["sel"] == 1)
    tc = oracle.forward(shape.with_(routing="token", k=shape.E, renormalize=0, capacity=-1), inp)
    assert np.allclose(r["y"], tc["y"], rtol=1e-12, atol=1e-13)


def test_ec_dense_masked_brute_force():
    """numpy fp64: every expert on every token, masked to the pairs the experts took
    and weighted by the router probability; the selection re-derived from a stable
    sort of the fp32-rounded probabilities."""
    shape = small(T=30, d=20, F=28, E=6, k=2, routing="expert", capacity=7)
    inp = make_inputs(shape, 33)
    r = oracle.ec_forward(shape, inp)
    x = inp["x"].astype(np.float64)
    s_ = x @ inp["Wg"].T.astype(np.float64) + inp["bg"].astype(np.float64)
    p = np.exp(s_ - s_.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    assert np.allclose(r["p"], p, rtol=0, atol=1e-15)
    for e in range(shape.E):
        take = np.argsort(-p[:, e].astype(np.float32), kind="stable")[:7]
        assert sorted(np.nonzero(r["sel"][:, e])[0].tolist()) == sorted(take.tolist())
    gelu = np.vectorize(lambda z: 0.5 * z * (1.0 + math.erf(z / math.sqrt(2.0))))
    allout = np.stack([gelu(x @ inp["W1"][e].T.astype(np.float64) + inp["b1"][e])
                       @ inp["W2"][e].T.astype(np.float64) + inp["b2"][e]
                       for e in range(shape.E)], axis=1)          # [T, E, d]
    y = np.einsum("te,ted->td", r["sel"] * p, allout)
    assert np.allclose(r["y"], y, rtol=1e-12, atol=1e-12)
    # a token nobody took gets exactly zero
    none = np.nonzero(r["sel"].sum(axis=1) == 0)[0]
    assert len(none) > 0 and np.all(r["y"][none] == 0.0)


def test_ec_one_expert_is_the_plain_mlp():
    """E = 1 and C = T: p = 1, so the layer is the textbook two-layer MLP."""
    shape = small(T=9, E=1, k=1, routing="expert", capacity=9)
    inp = make_inputs(shape, 34, margin=0)
    r = oracle.ec_forward(shape, inp)
    x = torch.from_numpy(inp["x"]).double()
    ref = Fn.linear(Fn.gelu(Fn.linear(x, widen(inp["W1"][0], "f32"), widen(inp["b1"][0], "f32"))),
                    widen(inp["W2"][0], "f32"), widen(inp["b2"][0], "f32"))
    assert np.allclose(r["y"], ref.numpy(), rtol=1e-12, atol=1e-13)
