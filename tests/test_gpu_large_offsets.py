"""A layer whose expert hidden activations H [T k, d_ff] span more than 4 GiB.

The LDS-DMA GEMM addresses its A operand with 32-bit byte offsets; a contiguous
A (H in the down-projection, dz in the input-gradient pass, the transposed
activations of the weight gradients) takes a 64-bit base per row tile so those
offsets stay inside one tile.  With T = 262144, k = 2 and d_ff = 8320, H holds
8.7 GB: the rows of the last experts sit beyond byte 2^32 of it.  The output is
checked against the oracle on tokens whose rows lie there (and a spread of
others); the backward's dx on the same tokens and entries of the last expert's
weight gradients, including hidden units whose transposed rows lie past 4 GiB.
"""
import numpy as np
import pytest
import torch

import oracle
from moe_synth import LayerShape, make_inputs
from gpu_common import check_routing, check_y, device_inputs, gpu_forward, say
from test_gpu_backward import check, dy_device, gpu_backward, make_dy

pytestmark = pytest.mark.gpu

SHAPE = LayerShape("h_over_4gib", T=262144, d=64, F=8320, E=8, k=2, dtype="bf16",
                   router_bias="normal")
ROW_4GIB = (1 << 32) // (SHAPE.F * 2)  # first H row that starts past byte 2^32


def tokens_past_4gib(ref, n):
    d = oracle.dispatch(SHAPE, ref["topk_idx"], ref["keep"])
    rt = d["row_token"]
    assert len(rt) > ROW_4GIB + n
    far = rt[np.linspace(ROW_4GIB, len(rt) - 1, n).astype(np.int64)]
    spread = np.linspace(0, SHAPE.T - 1, 8).astype(np.int64)
    return np.unique(np.concatenate([far, spread]))


def test_forward_h_over_4gib():
    say("case", SHAPE)
    inp = make_inputs(SHAPE, 31)
    ref = oracle.route(SHAPE, inp)
    dev = device_inputs(inp)
    g = gpu_forward(SHAPE, dev)
    check_routing(SHAPE, g, ref)
    toks = tokens_past_4gib(ref, 24)
    check_y(SHAPE, g["y"][toks], oracle.experts(SHAPE, inp, ref, toks))
    del dev, g
    torch.cuda.empty_cache()


def test_backward_h_over_4gib():
    say("case", SHAPE, "backward")
    inp = make_inputs(SHAPE, 32)
    dy_raw, dy64 = make_dy(SHAPE, 7)
    alpha = 0.1
    dev = device_inputs(inp)
    names = ["dx", "dW1", "db1", "dW2", "db2"]
    got, _ = gpu_backward(SHAPE, dev, dy_device(SHAPE, dy_raw), alpha, names)
    rt = oracle.route(SHAPE, inp, with_probs=False)
    toks = tokens_past_4gib(rt, 16)
    bt = oracle.backward_tokens(SHAPE, inp, dy64, toks, alpha, rt=rt)
    check(SHAPE, got["dx"][toks], bt["dx"], "dx")
    # the last expert's rows are the last of H; hidden units >= 4096 are the
    # transposed-activation rows past 4 GiB
    rng = np.random.default_rng(3)
    e = SHAPE.E - 1
    fl = np.sort(np.concatenate([rng.choice(4096, 4, replace=False),
                                 4096 + rng.choice(SHAPE.F - 4096, 12, replace=False)]))
    jl = np.sort(rng.choice(SHAPE.d, 12, replace=False))
    ent = oracle.backward_expert_entries(SHAPE, inp, dy64, e, fl, jl, rt=rt)
    check(SHAPE, got["dW1"][e][np.ix_(fl, jl)], ent["dW1"], "dW1")
    check(SHAPE, got["dW2"][e][np.ix_(jl, fl)], ent["dW2"], "dW2")
    check(SHAPE, got["db1"][e][fl], ent["db1"], "db1")
    check(SHAPE, got["db2"][e][jl], ent["db2"], "db2")
    del dev
    torch.cuda.empty_cache()
