#!/usr/bin/env python3
"""Benchmark of the sparse-MoE layer forward on one MI355X.

One step = one moe_forward call (router, softmax/top-k/renormalise, dispatch
with the capacity limit, grouped expert GEMMs with fused epilogues, shared
expert, combine) over one batch of synthetic tokens already resident in HBM.
Prints one JSON line.

Measurement legs:
  * value: tokens per second over exactly --steps timed moe_forward calls,
    bracketed by device synchronisation.
  * roofline: the expert grouped GEMM (one moe_expert_ffn call: the up- and
    down-projection kernels) timed with HIP events on the stream it runs on,
    over --steps calls, against the bf16 MFMA peak (or HBM peak when the
    workload is weight-bandwidth bound).
  * cpu_baseline: the fp64 oracle on a bounded sample of the same batch, on
    the host cores (rank 0, one GPU only).
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 matrix
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
RIDGE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)


def parse():
    p = argparse.ArgumentParser(description=__doc__)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="page1_b4s512")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target CPU time of the oracle sample")
    p.add_argument("--graph", type=int, default=1,
                   help="1: replay moe_forward from a captured HIP graph")
    return p.parse_args()


def algorithmic(shape, kept_rows, hit_experts):
    """Active FLOPs and algorithmic HBM bytes of one expert-FFN call."""
    elt = 2 if shape.dtype == "bf16" else 4
    flop = 4.0 * kept_rows * shape.d * shape.F
    wbytes = hit_experts * (2.0 * shape.d * shape.F + shape.F + shape.d) * elt
    if shape.Fs:
        flop += 4.0 * shape.T * shape.d * shape.Fs
        wbytes += (2.0 * shape.d * shape.Fs + shape.Fs + shape.d) * elt
    # activations: read x rows once, write y rows once (fp32 expert rows)
    nrows = kept_rows + (shape.T if shape.Fs else 0)
    abytes = shape.T * shape.d * elt + nrows * shape.d * 4
    return flop, wbytes + abytes


def cpu_baseline(shape, inp, seconds):
    import oracle
    t0 = time.perf_counter()
    rt = oracle.route(shape, inp, with_probs=False)
    t_route = time.perf_counter() - t0
    # calibrate on a few tokens, then size the sample to ~`seconds`
    n0 = min(shape.T, 8)
    t1 = time.perf_counter()
    oracle.experts(shape, inp, rt, np.arange(n0))
    per_tok = (time.perf_counter() - t1) / max(n0, 1)
    n = int(min(shape.T, max(n0, seconds / max(per_tok, 1e-9))))
    toks = np.arange(n)
    t2 = time.perf_counter()
    oracle.experts(shape, inp, rt, toks)
    t_exp = time.perf_counter() - t2
    # whole-batch routing cost is prorated to the sample's share of tokens
    dt = t_exp + t_route * n / max(shape.T, 1)
    return {"value": round(n / dt, 3), "unit": "tokens/s", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": "fp64 oracle: routing of all %d tokens (prorated) + expert MLPs and "
                      "combine of the first %d tokens of the %s batch, %.1f s" %
                      (shape.T, n, shape.name, dt)}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the MoE layer here is the data-parallel "
              "replica of one GPU; multi-GPU runs are not part of this build "
              "(requested --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import sparse_mixture_experts_45_amd as moe
    from moe_synth import make_inputs, to_device, workload

    shape = workload(args.workload)
    inp = make_inputs(shape, args.seed)
    dev = to_device(inp, "cuda")
    tdt = torch.bfloat16 if shape.dtype == "bf16" else torch.float32
    cfg = moe.config(shape.T, shape.d, shape.F, shape.E, shape.k, act=shape.act, dtype=tdt,
                     capacity=shape.capacity, renormalize=bool(shape.renormalize),
                     shared_d_ff=shape.Fs)
    ws = moe.workspace(cfg)
    T, k, E = shape.T, shape.k, shape.E
    x = dev["x"]
    y = torch.empty((T, shape.d), dtype=tdt, device="cuda")
    st = dict(counts=torch.empty(E, dtype=torch.int32, device="cuda"),
              kept=torch.empty(E, dtype=torch.int32, device="cuda"))
    stream = torch.cuda.Stream()

    def step():
        moe.moe_forward(cfg, dev, x, y, st, ws, stream=stream)

    torch.cuda.synchronize()
    graph = None
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step()
    torch.cuda.synchronize()
    if args.graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            step()
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            for _ in range(2):
                graph.replay()
        torch.cuda.synchronize()

    # ---- timed region: exactly K steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        for _ in range(args.steps):
            if graph is not None:
                graph.replay()
            else:
                step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps

    kept = st["kept"].cpu().numpy()
    kept_rows = int(kept.sum())
    hit = int((kept > 0).sum())

    # ---- expert grouped GEMM (one moe_expert_ffn call) timed with HIP events
    topk_idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    topk_w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    nrows = T * k + (T if shape.Fs else 0)
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    kept_t = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 2, dtype=torch.int32, device="cuda")
    row_token = torch.empty(nrows, dtype=torch.int32, device="cuda")
    row_slot = torch.empty(nrows, dtype=torch.int32, device="cuda")
    inv = torch.empty((T, k), dtype=torch.int32, device="cuda")
    y_rows = torch.empty((nrows, shape.d), dtype=torch.float32, device="cuda")
    with torch.cuda.stream(stream):
        moe.moe_route(cfg, x, dev["Wg"], dev["bg"], topk_idx, topk_w, None, None, None, ws,
                      stream=stream)
        moe.moe_dispatch(cfg, topk_idx, counts, kept_t, offsets, row_token, row_slot, inv, ws,
                         stream=stream)
        for _ in range(3):
            moe.moe_expert_ffn(cfg, x, dev, offsets, row_token, row_slot, topk_w, y_rows, ws,
                               stream=stream)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for a, b in evs:
            a.record(stream)
            moe.moe_expert_ffn(cfg, x, dev, offsets, row_token, row_slot, topk_w, y_rows, ws,
                               stream=stream)
            b.record(stream)
    torch.cuda.synchronize()
    ffn_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))

    flop, nbytes = algorithmic(shape, kept_rows, hit)
    ai = flop / nbytes
    if ai >= RIDGE:
        peak = PEAK_BF16_TFLOPS if shape.dtype == "bf16" else PEAK_F32_TFLOPS
        achieved = flop / (ffn_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": None}
    else:
        achieved = nbytes / (ffn_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None}
    roof.update(kernel="expert grouped GEMM: up-projection + down-projection launches of one "
                       "moe_expert_ffn call", kernel_ms=round(ffn_ms, 4),
                algorithmic_flop=flop, algorithmic_bytes=nbytes)

    value = T * args.steps / elapsed
    out = {
        "metric": "MoE layer tokens/s; expert GEMM % of bf16 MFMA peak (% HBM peak at small T)",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if shape.dtype == "bf16" else "f32",
        "data": "synthetic (seeded; random-init weights)",
        "config": {"workload": shape.name, "tokens": T, "d_model": shape.d, "d_ff": shape.F,
                   "n_experts": E, "top_k": k, "capacity": shape.capacity,
                   "shared_d_ff": shape.Fs, "act": shape.act, "hip_graph": bool(graph),
                   "kept_rows": kept_rows, "experts_hit": hit},
        "layer_tflops": round(flop / (ms_per_step * 1e-3) / 1e12, 2),
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(shape, inp, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
