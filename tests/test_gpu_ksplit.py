"""K split of a last, partly filled round of GEMM tiles (the LDS-DMA tiers that
take one tile per block).  When a launch's tiles leave the final round of
resident blocks at most half full, each tile of that round is cut into S parts
along K; each part parks its fp32 partial tile and the last to arrive adds the
S partials in part order before the epilogue.

The shapes below are chosen so that the up- or the down-projection (or both)
split, with S = 2, 3 and 4, with and without a shared expert, under token and
expert choice; `planned_splits` restates the launch plan so each case asserts
that it covers what it is meant to.  Each case is checked against the oracle
(the forward output in full; the backward's dx on sampled tokens and entries
of the weight and bias gradients), and twice in a row for bit equality: the
partial sums are added in a fixed order.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_mixture_experts_45_amd as moe
from moe_synth import LayerShape, make_inputs
from gpu_common import (check_ec_selection, check_routing, check_y, cfg_of, device_inputs,
                        gpu_forward, gpu_forward_ec, say)
from test_gpu_backward import check, dy_device, gpu_backward, make_dy

pytestmark = pytest.mark.gpu

# tiers of the LDS-DMA GEMM that split: rows and columns per tile, blocks per CU
TIERS = {"large": (256, 256, 1), "tall": (192, 256, 1), "mid": (128, 128, 2)}
SPLIT_MAX, SPLIT_MIN_STEPS, BK = 4, 32, 64


def tier_of(shape):
    """The tile tier the library picks for this shape (bf16, K multiple of 64)."""
    if shape.routing == "expert":
        C = oracle.ec_capacity(shape)
        rows = shape.E * C
        whole = C >= 256 and (-(-C // 256) * 256 - C) * 8 <= C
    else:
        rows = shape.T * shape.k if shape.capacity < 0 else min(shape.T * shape.k,
                                                                 shape.E * shape.capacity)
        whole = False
    avg = rows // shape.E
    fills = (shape.routing != "expert" and shape.capacity < 0 and avg >= 128 and
             shape.E * -(-max(avg, 1) // 256) *
             min(-(-max(shape.F, shape.Fs) // 256), -(-shape.d // 256)) >= 128)
    if fills and avg + 2.0 * avg ** 0.5 <= 192:
        return "tall"
    if avg >= 768 or whole or fills:
        return "large"
    return "mid" if avg >= 256 else None


def split_plan(total, slots, smax):
    if smax < 2 or total <= 0 or total % slots == 0:
        return 1
    s = min(smax, slots // (total % slots))
    return s if s >= 2 else 1


HEAVY_ROWS = 64  # the forward's 256-row tiles take a group's last <= 64 rows


def row_tiles(rows, BM, extra):
    """Row tiles of one group: ceil(rows / BM), less one when the last would hold
    at most `extra` rows (they join the previous tile)."""
    m = -(-int(rows) // BM)
    return m - 1 if extra and m >= 2 and rows - (m - 1) * BM <= extra else m


def planned_splits(shape, kept, forward=True):
    """S of the up- and the down-projection launch, from the kept rows per expert."""
    tier = tier_of(shape)
    BM, BN, per_cu = TIERS[tier]
    extra = HEAVY_ROWS if forward and tier == "large" else 0
    slots = torch.cuda.get_device_properties(0).multi_processor_count * per_cu
    rt = sum(row_tiles(r, BM, extra) for r in kept) + (row_tiles(shape.T, BM, extra)
                                                       if shape.Fs else 0)
    out = []
    for N, K, Ks in ((max(shape.F, shape.Fs), shape.d, shape.d), (shape.d, shape.F, shape.Fs)):
        kt = (min(K, Ks) if shape.Fs else K) // BK
        out.append(split_plan(rt * -(-N // BN), slots, min(SPLIT_MAX, kt // SPLIT_MIN_STEPS)))
    return tuple(out)


def L(name, **kw):
    base = dict(name=name, dtype="bf16", router_bias="normal")
    base.update(kw)
    return LayerShape(**base)


# (shape, the (up, down) splits it is built for)
CASES = [
    (L("mid_up4", T=256, d=8192, F=256, E=2, k=2), (4, 1)),
    (L("mid_down3", T=256, d=256, F=6144, E=2, k=2, act="relu"), (1, 3)),
    (L("large_up2", T=768, d=4096, F=512, E=2, k=2), (2, 1)),
    (L("large_down4_shared", T=768, d=256, F=8192, E=2, k=2, Fs=8192), (1, 4)),
    (L("large_ec_up2", T=1024, d=4096, F=512, E=4, k=1, routing="expert"), (2, 1)),
    # 800 rows per expert (k = E): 3 x 256 + 32, so each expert's last tile is
    # a heavy one of 288 rows, and it is split along K (up-projection; then the
    # down-projection with a heavy shared-expert tile too)
    (L("large_up2_heavy", T=800, d=4096, F=512, E=2, k=2), (2, 1)),
    (L("large_down4_heavy_shared", T=800, d=256, F=8192, E=2, k=2, Fs=8192), (1, 4)),
]


# 192-row tiles: about 128 rows for each of 32 experts, no capacity limit and
# no router bias (seeds 22 and 23 keep every expert below 192 rows, so each
# expert is one row tile)
TALL = [
    (L("tall_up2", T=4096, d=4096, F=1024, E=32, k=1, router_bias="none"), (2, 1)),
    (L("tall_down2", T=4096, d=1024, F=4096, E=32, k=1, act="relu", router_bias="none"),
     (1, 2)),
    # a shared expert narrower than the routed ones: 22 more row tiles, no
    # split, and the input-gradient pass skips the tiles past its width
    (L("tall_shared", T=4096, d=1024, F=1024, E=32, k=1, Fs=512, router_bias="none"), (1, 1)),
]


@pytest.mark.parametrize("shape,splits", CASES, ids=[c[0].name for c in CASES])
def test_split_forward(shape, splits):
    say("case", shape, "splits", splits)
    inp = make_inputs(shape, 21)
    dev = device_inputs(inp)
    if shape.routing == "expert":
        C = oracle.ec_capacity(shape)
        ref = oracle.ec_forward(shape, inp)
        g = gpu_forward_ec(shape, dev, C)
        check_ec_selection(shape, g, ref)
    else:
        ref = oracle.forward(shape, inp)
        g = gpu_forward(shape, dev)
        check_routing(shape, g, ref)
    assert planned_splits(shape, g["kept"]) == splits
    check_y(shape, g["y"], ref["y"])
    # the same call again: bit-identical output
    g2 = gpu_forward_ec(shape, dev, C) if shape.routing == "expert" else gpu_forward(shape, dev)
    assert torch.equal(g["y_raw"].view(torch.int16), g2["y_raw"].view(torch.int16))


@pytest.mark.parametrize("shape,splits", TALL, ids=[c[0].name for c in TALL])
def test_split_forward_tall(shape, splits):
    """The 192-row tier; outputs on sampled tokens (every 16th, and the last
    32), which the oracle computes one by one."""
    say("case", shape, "splits", splits)
    inp = make_inputs(shape, 23)
    dev = device_inputs(inp)
    ref = oracle.route(shape, inp)
    g = gpu_forward(shape, dev)
    check_routing(shape, g, ref)
    assert tier_of(shape) == "tall"
    assert planned_splits(shape, g["kept"]) == splits
    toks = np.unique(np.concatenate([np.arange(0, shape.T, 16), np.arange(shape.T - 32, shape.T)]))
    check_y(shape, g["y"][toks], oracle.experts(shape, inp, ref, toks))
    g2 = gpu_forward(shape, dev)
    assert torch.equal(g["y_raw"].view(torch.int16), g2["y_raw"].view(torch.int16))


BWD = CASES[:4] + TALL  # the training forward uses no heavy tiles


@pytest.mark.parametrize("shape,splits", BWD, ids=[c[0].name for c in BWD])
def test_split_backward(shape, splits):
    """The input-gradient pass runs the same GEMMs with K = d for dz and K =
    d_ff for dz W1, so it splits where the forward does.  dx on sampled tokens
    and entries of both experts' weight and bias gradients against the oracle
    (computed one by one), then a second run bit for bit."""
    say("case", shape)
    inp = make_inputs(shape, 22)
    dy_raw, dy64 = make_dy(shape, 5)
    alpha = 0.2
    dev = device_inputs(inp)
    names = ["dx", "dW1", "db1", "dW2", "db2"]
    got, _ = gpu_backward(shape, dev, dy_device(shape, dy_raw), alpha, names)
    rt = oracle.route(shape, inp, with_probs=False)
    toks = np.linspace(0, shape.T - 1, 24).astype(np.int64)
    bt = oracle.backward_tokens(shape, inp, dy64, toks, alpha, rt=rt)
    check(shape, got["dx"][toks], bt["dx"], "dx")
    rng = np.random.default_rng(2)
    for e in range(shape.E) if shape.E <= 4 else (0, shape.E // 2, shape.E - 1):
        fl = np.sort(rng.choice(shape.F, 16, replace=False))
        jl = np.sort(rng.choice(shape.d, 16, replace=False))
        ent = oracle.backward_expert_entries(shape, inp, dy64, e, fl, jl, rt=rt)
        check(shape, got["dW1"][e][np.ix_(fl, jl)], ent["dW1"], "dW1[%d]" % e)
        check(shape, got["dW2"][e][np.ix_(jl, fl)], ent["dW2"], "dW2[%d]" % e)
        check(shape, got["db1"][e][fl], ent["db1"], "db1[%d]" % e)
        check(shape, got["db2"][e][jl], ent["db2"], "db2[%d]" % e)
    again, _ = gpu_backward(shape, dev, dy_device(shape, dy_raw), alpha, names)
    for n in got:
        assert np.array_equal(got[n], again[n]), n
