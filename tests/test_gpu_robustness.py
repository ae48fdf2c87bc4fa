"""GPU robustness: randomly drawn small shapes against the oracle, guard-banded
output buffers (no write outside the arrays the ABI describes), and HIP-graph
capture with several replays checked against eager runs."""
import numpy as np
import pytest
import torch

import oracle
import sparse_mixture_experts_45_amd as moe
from moe_synth import LayerShape, make_inputs
from gpu_common import cfg_of, check_routing, check_y, device_inputs, gpu_forward, say

pytestmark = pytest.mark.gpu


def draw_shapes(n, seed):
    """Seeded draws over the configuration space (multiples of 8 for d, d_ff)."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.integers(1, 41))
        k = int(rng.integers(1, min(E, 8) + 1))
        T = int(rng.integers(1, 700))
        kw = dict(name="draw%d" % i, T=T, d=8 * int(rng.integers(1, 41)),
                  F=8 * int(rng.integers(1, 49)), E=E, k=k,
                  dtype=str(rng.choice(["f32", "bf16"])), act=str(rng.choice(["gelu", "relu"])),
                  renormalize=int(rng.integers(0, 2)),
                  router_bias=str(rng.choice(["none", "normal", "zipf1.1"])),
                  capacity=int(rng.integers(0, T * k // E + 2)) if rng.random() < 0.4 else -1,
                  Fs=8 * int(rng.integers(1, 25)) if rng.random() < 0.3 else 0)
        out.append(LayerShape(**kw))
    return out


@pytest.mark.parametrize("shape", draw_shapes(24, 2024), ids=lambda s: s.name)
def test_drawn_shapes(shape):
    say("case", shape)
    inp = make_inputs(shape, 5)
    ref = oracle.forward(shape, inp)
    g = gpu_forward(shape, device_inputs(inp))
    check_routing(shape, g, ref)
    check_y(shape, g["y"], ref["y"])


@pytest.mark.parametrize("shape", draw_shapes(12, 77), ids=lambda s: s.name)
def test_drawn_shapes_backward(shape):
    """Every gradient of sum <dy, y> + 0.3 balance against the oracle's (balance
    term off for one expert, where it is undefined)."""
    from test_gpu_backward import check, dy_device, gpu_backward, make_dy
    say("case", shape)
    alpha = 0.3 if shape.E > 1 else 0.0
    inp = make_inputs(shape, 6)
    dy_raw, dy64 = make_dy(shape, 9)
    want = oracle.backward(shape, inp, dy64, alpha)
    got, _ = gpu_backward(shape, device_inputs(inp), dy_device(shape, dy_raw), alpha)
    for n in got:
        check(shape, got[n], want[n], n)


GUARD = 4096  # bytes of canary before and after each output


def guarded(shape_, dtype):
    """An output tensor inside a larger byte buffer filled with 0xA5."""
    n = int(np.prod(shape_)) * torch.tensor([], dtype=dtype).element_size()
    buf = torch.full((GUARD + n + GUARD,), 0xA5, dtype=torch.uint8, device="cuda")
    view = buf[GUARD:GUARD + n].view(dtype).view(*shape_)
    return buf, view


def untouched(buf):
    b = buf.cpu().numpy()
    return bool(np.all(b[:GUARD] == 0xA5) and np.all(b[-GUARD:] == 0xA5))


@pytest.mark.parametrize("routing", ["token", "expert"])
def test_outputs_stay_inside_their_buffers(routing):
    shape = LayerShape("guard", T=333, d=136, F=200, E=9, k=3, dtype="bf16", Fs=64,
                       capacity=70 if routing == "token" else -1, router_bias="normal",
                       routing=routing)
    inp = make_inputs(shape, 3)
    dev = device_inputs(inp)
    c = cfg_of(shape)
    T, d, E, k = shape.T, shape.d, shape.E, shape.k
    bufs = {}
    yb, y = guarded((T, d), torch.bfloat16)
    bufs["y"] = yb
    st = {}
    for name, sh, dt in (("counts", (E,), torch.int32), ("kept", (E,), torch.int32),
                         ("mean_prob", (E,), torch.float32), ("balance", (1,), torch.float32),
                         ("cv2", (1,), torch.float32)):
        bufs[name], st[name] = guarded(sh, dt)
    if routing == "token":
        bufs["topk_idx"], st["topk_idx"] = guarded((T, k), torch.int32)
        bufs["topk_w"], st["topk_w"] = guarded((T, k), torch.float32)
        fwd = moe.moe_forward_train
        ws = moe.train_workspace(c)
    else:
        C = oracle.ec_capacity(shape)
        bufs["ec_idx"], st["ec_idx"] = guarded((E, C), torch.int32)
        bufs["ec_w"], st["ec_w"] = guarded((E, C), torch.float32)
        fwd = moe.moe_forward
        ws = moe.workspace(c)
    fwd(c, dev, dev["x"], y, st, ws)
    if routing == "token":
        g = {}
        F, Fs = shape.F, shape.Fs
        for name, sh, dt in (("dx", (T, d), torch.bfloat16), ("dWg", (E, d), torch.float32),
                             ("dbg", (E,), torch.float32), ("dW1", (E, F, d), torch.bfloat16),
                             ("db1", (E, F), torch.bfloat16), ("dW2", (E, d, F), torch.bfloat16),
                             ("db2", (E, d), torch.bfloat16), ("dWs1", (Fs, d), torch.bfloat16),
                             ("dbs1", (Fs,), torch.bfloat16), ("dWs2", (d, Fs), torch.bfloat16),
                             ("dbs2", (d,), torch.bfloat16)):
            bufs[name], g[name] = guarded(sh, dt)
        dy = torch.randn((T, d), device="cuda").to(torch.bfloat16)
        moe.moe_backward(c, dev, dev["x"], dy, g, aux_coef=0.1, ws=ws)
    torch.cuda.synchronize()
    bad = [n for n, b in bufs.items() if not untouched(b)]
    assert not bad, bad


def _replays(capture, eager_out, other):
    """Capture `capture` (which writes into the tensors of eager_out's keys),
    replay it three times with other eager work in between, and compare each
    replay with the eager result bit for bit."""
    outs = capture.__outs__
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        capture()  # warm-up on the capture stream
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        capture()
    torch.cuda.synchronize()
    for r in range(3):
        for t in outs.values():
            t.view(torch.uint8).fill_(0x5A)
        other()
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        for n, t in outs.items():
            assert torch.equal(t.view(torch.uint8), eager_out[n].view(torch.uint8)), (r, n)


def test_graph_replays_match_eager():
    """moe_forward (token and expert choice) and a training step, captured in
    HIP graphs and replayed three times, each with unrelated eager layer calls
    and synchronisations in between."""
    for routing in ("token", "expert"):
        shape = LayerShape("graph", T=400, d=192, F=256, E=8, k=2, dtype="bf16", Fs=64,
                           capacity=120 if routing == "token" else -1, routing=routing)
        inp = make_inputs(shape, 8)
        dev = device_inputs(inp)
        c = cfg_of(shape)
        ws = moe.workspace(c)
        y = torch.empty((shape.T, shape.d), dtype=torch.bfloat16, device="cuda")
        moe.moe_forward(c, dev, dev["x"], y, None, ws)
        torch.cuda.synchronize()
        eager = {"y": y.clone()}
        other_shape = LayerShape("other", T=300, d=128, F=192, E=4, k=2, dtype="bf16")
        oinp = device_inputs(make_inputs(other_shape, 1))

        def other():
            gpu_forward(other_shape, oinp)
            torch.ones(1 << 20, device="cuda").sum()

        def capture():
            moe.moe_forward(c, dev, dev["x"], y, None, ws)
        capture.__outs__ = {"y": y}
        _replays(capture, eager, other)

    # training step: forward_train + backward
    shape = LayerShape("graph_train", T=300, d=128, F=192, E=6, k=2, dtype="bf16", Fs=64,
                       capacity=110)
    inp = make_inputs(shape, 4)
    dev = device_inputs(inp)
    c = cfg_of(shape)
    ws = moe.train_workspace(c)
    T, d, F, E, Fs = shape.T, shape.d, shape.F, shape.E, shape.Fs
    y = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    dy = torch.randn((T, d), device="cuda").to(torch.bfloat16)
    bf = torch.bfloat16
    grads = dict(dx=torch.empty((T, d), dtype=bf, device="cuda"),
                 dWg=torch.empty((E, d), device="cuda"), dbg=torch.empty(E, device="cuda"),
                 dW1=torch.empty((E, F, d), dtype=bf, device="cuda"),
                 db1=torch.empty((E, F), dtype=bf, device="cuda"),
                 dW2=torch.empty((E, d, F), dtype=bf, device="cuda"),
                 db2=torch.empty((E, d), dtype=bf, device="cuda"),
                 dWs1=torch.empty((Fs, d), dtype=bf, device="cuda"),
                 dbs2=torch.empty(d, dtype=bf, device="cuda"))

    def step():
        moe.moe_forward_train(c, dev, dev["x"], y, None, ws)
        moe.moe_backward(c, dev, dev["x"], dy, grads, aux_coef=0.05, ws=ws)
    step()
    torch.cuda.synchronize()
    eager = {n: t.clone() for n, t in grads.items()}
    eager["y"] = y.clone()
    other_shape = LayerShape("other", T=200, d=64, F=64, E=4, k=2, dtype="bf16")
    oinp = device_inputs(make_inputs(other_shape, 2))
    step.__outs__ = dict(grads, y=y)
    _replays(step, eager, lambda: gpu_forward(other_shape, oinp))


def test_graph_of_several_calls():
    """Several moe_forward calls captured back to back in one HIP graph (as the
    benchmark replays them), on the 256-row tier with heavy tiles and a K split
    of the last round: the calls share one workspace, so each call's tile list
    must leave the split counters ready for the next.  Each replay equals the
    eager result bit for bit, and the oracle within tolerance."""
    shape = LayerShape("graph_heavy", T=800, d=256, F=8192, E=2, k=2, dtype="bf16", Fs=8192,
                       router_bias="normal")
    say("case", shape)
    inp = make_inputs(shape, 21)
    dev = device_inputs(inp)
    c = cfg_of(shape)
    ws = moe.workspace(c)
    y = torch.empty((shape.T, shape.d), dtype=torch.bfloat16, device="cuda")
    moe.moe_forward(c, dev, dev["x"], y, None, ws)
    torch.cuda.synchronize()
    check_y(shape, y.float().cpu().numpy().astype(np.float64), oracle.forward(shape, inp)["y"])
    eager = {"y": y.clone()}
    other_shape = LayerShape("other", T=200, d=64, F=64, E=4, k=2, dtype="bf16")
    oinp = device_inputs(make_inputs(other_shape, 2))

    def capture():
        for _ in range(3):
            moe.moe_forward(c, dev, dev["x"], y, None, ws)
    capture.__outs__ = {"y": y}
    _replays(capture, eager, lambda: gpu_forward(other_shape, oinp))
