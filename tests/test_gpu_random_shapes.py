"""GPU parity on seeded random layer shapes.

Each case draws its shape from a seeded generator: tokens, model and hidden
widths (half of them multiples of 64, which take the LDS-DMA tiers, the rest
multiples of 8), experts, top-k, dtype, activation, renormalisation, a
capacity limit, a shared expert, the router bias and the routing mode.  The
output is compared with the oracle in full, routing and statistics exactly as
in the hand-picked cases; every fourth case also runs the backward and checks
dx and every weight gradient against the oracle's.
"""
import numpy as np
import pytest
import torch

import oracle
from moe_synth import LayerShape, make_inputs
from gpu_common import (check_ec_selection, check_routing, check_y, device_inputs, gpu_forward,
                        gpu_forward_ec, say)
from test_gpu_backward import check, dy_device, gpu_backward, make_dy

pytestmark = pytest.mark.gpu

N_CASES = 24


def draw_shape(i):
    rng = np.random.default_rng(1000 + i)
    step = 64 if i % 2 == 0 else 8
    d = int(step * rng.integers(1, 512 // step + 1))
    F = int(step * rng.integers(1, 640 // step + 1))
    E = int(rng.choice([1, 2, 3, 5, 8, 13, 32, 40]))
    routing = "expert" if rng.random() < 0.2 and E > 1 else "token"
    k = int(rng.integers(1, min(E, 6) + 1))
    T = int(rng.integers(1, 600))
    cap = -1
    if routing == "token" and rng.random() < 0.3:
        cap = int(rng.integers(0, max(2, T * k // E) + 1))
    Fs = int(step * rng.integers(1, 320 // step + 1)) if rng.random() < 0.3 else 0
    return LayerShape("random%02d" % i, T=T, d=d, F=F, E=E, k=k,
                      dtype="f32" if rng.random() < 0.25 else "bf16",
                      act="relu" if rng.random() < 0.4 else "gelu",
                      renormalize=0 if rng.random() < 0.2 else 1,
                      capacity=cap, Fs=Fs, routing=routing,
                      router_bias=str(rng.choice(["none", "normal"])))


CASES = [draw_shape(i) for i in range(N_CASES)]


@pytest.mark.parametrize("shape", CASES, ids=[s.name for s in CASES])
def test_random_shape(shape):
    say("case", shape)
    inp = make_inputs(shape, 40)
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
    check_y(shape, g["y"], ref["y"])
    if int(shape.name[-2:]) % 4 != 0 or shape.routing == "expert":
        return
    dy_raw, dy64 = make_dy(shape, 9)
    alpha = 0.3 if shape.E > 1 else 0.0
    names = ["dx", "dW1", "db1", "dW2", "db2"] + (["dWs1", "dbs1", "dWs2", "dbs2"]
                                                    if shape.Fs else [])
    got, _ = gpu_backward(shape, dev, dy_device(shape, dy_raw), alpha, names)
    want = oracle.backward(shape, inp, dy64, alpha)
    for n in names:
        check(shape, got[n], want[n], n)
    del dev
    torch.cuda.empty_cache()
