"""GPU parity on seeded random layer shapes large enough for the 256-, 192- and
128-row tiers of the grouped GEMM.

The shapes are drawn so that rows per expert land where the library takes
those tiers: at least 768 on average (256-row tiles, whose forward merges a
group's last rows into its previous tile when they are at most 64, and whose
last round of tiles may be split along K), 128-165 with many experts and wide
enough layers (192-row tiles), or 256-767 (128-row tiles).  Widths are
multiples of 64 (the LDS-DMA tiers), partly not multiples of the tile width,
and a shared expert is present in some cases.  Routing, counts and statistics
are checked for every token; outputs on the tokens behind both ends of every
32-row block of every expert (so every row tile of every tile height, heavy
and split ones included, has rows checked at both ends) plus a spread sample,
each token row by row against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from moe_synth import LayerShape, make_inputs
from gpu_common import check_routing, check_y, device_inputs, gpu_forward, say
from test_gpu_workloads import sample_tokens

pytestmark = pytest.mark.gpu


def draw_large(i):
    rng = np.random.default_rng(2000 + i)
    kind = ("large", "large", "large", "large", "tall", "tall", "mid", "mid")[i]
    if kind == "large":
        E = int(rng.choice([2, 3, 4, 6, 8]))
        k = int(rng.integers(1, min(E, 2) + 1))
        avg = int(rng.integers(768, 1500))
        d = int(64 * rng.integers(4, 11))
        F = int(64 * rng.integers(4, 17))
    elif kind == "tall":
        E = int(rng.choice([32, 64]))
        k = int(rng.integers(1, 3))
        avg = int(rng.integers(128, 160))
        lo = 13 if E == 32 else 5  # E * min(F, d) / 256 tiles >= 128
        d = int(64 * rng.integers(lo, lo + 4))
        F = int(64 * rng.integers(lo, lo + 4))
    else:
        E = int(rng.choice([4, 8, 16]))
        k = int(rng.integers(1, 3))
        avg = int(rng.integers(256, 700))
        d = int(64 * rng.integers(2, 9))
        F = int(64 * rng.integers(2, 13))
    T = int(avg * E // k)
    Fs = int(64 * rng.integers(2, 9)) if rng.random() < 0.4 else 0
    return LayerShape("rand_%s%d" % (kind, i), T=T, d=d, F=F, E=E, k=k, dtype="bf16",
                      act="relu" if rng.random() < 0.4 else "gelu",
                      renormalize=0 if rng.random() < 0.2 else 1, capacity=-1, Fs=Fs,
                      routing="token", router_bias=str(rng.choice(["none", "normal"])))


CASES = [draw_large(i) for i in range(8)]


@pytest.mark.parametrize("shape", CASES, ids=[s.name for s in CASES])
def test_random_large_shape(shape):
    say("case", shape)
    inp = make_inputs(shape, 41)
    ref = oracle.route(shape, inp)
    dev = device_inputs(inp)
    g = gpu_forward(shape, dev)
    check_routing(shape, g, ref)
    toks = sample_tokens(shape, ref, 32)
    y_ref = oracle.experts(shape, inp, ref, toks)
    r = check_y(shape, g["y"][toks], y_ref)
    say("  rel-L2 on %d tokens: %.3g" % (len(toks), r))
    del dev
    torch.cuda.empty_cache()
