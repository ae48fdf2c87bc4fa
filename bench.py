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
    workload is weight-bandwidth bound).  The default workload is the
    Mixtral-shaped layer (T=4096, d=4096, d_ff=14336, 8 experts, top-2), where
    the expert GEMM is bound by the matrix cores.
  * roofline_hbm: the same measurement on a second, weight-streaming workload
    (default: the DeepSeek-shaped layer, T=512, 256 experts top-8 plus a
    shared expert, 15 GB of bf16 expert weights) against the HBM peak, with
    that layer's own forward time.
  * cpu_baseline: the fp64 oracle on a bounded sample of the same batch, on
    the host cores (rank 0, one GPU only).
"""
import argparse
import hashlib
import json
import math
import os
import sqlite3
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
    p.add_argument("--workload", default="mixtral_t4096")
    p.add_argument("--hbm-workload", default="deepseek_e256_top8",
                   help="second workload whose expert FFN is timed against the HBM peak "
                        "(roofline_hbm); 'none' to skip")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target CPU time of the oracle sample")
    p.add_argument("--graph", type=int, default=1,
                   help="1: replay moe_forward from a captured HIP graph")
    p.add_argument("--traffic-probe", action="store_true",
                   help="run under rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE: a plain device "
                        "copy of known size, then moe_expert_ffn calls")
    p.add_argument("--traffic-summarize", nargs=2, metavar=("FETCH_DB", "WRITE_DB"),
                   help="turn the two probe databases into the stored traffic summary")
    p.add_argument("--pmc-summarize", nargs=2, metavar=("RESULTS_DB", "PROBE_LOG"),
                   help="turn a rocprofv3 --pmc (+ --kernel-trace) run of --traffic-probe into the "
                        "stored matrix-core utilisation summary")
    p.add_argument("--trace-summarize", nargs=2, metavar=("RESULTS_DB", "BENCH_JSON"),
                   help="turn a rocprofv3 --kernel-trace --stats run of this bench (its "
                        "results database and the JSON line it printed) into the stored "
                        "kernel-trace summary")
    p.add_argument("--backward", action="store_true",
                   help="time a training step (moe_forward_train + moe_backward with every "
                        "gradient and the balance term) instead of the forward")
    return p.parse_args()


# ---------------------------------------------------------------------------
# HBM traffic of the expert GEMM from rocprofv3 counters.  FETCH_SIZE and
# WRITE_SIZE (KiB per dispatch) are taken in two runs of the probe, each
# scaled by what the same counter reads for a device-to-device copy of
# COPY_BYTES; the summary records a hash of the GEMM kernel's sources and is
# used only while they are unchanged.
COPY_BYTES = 256 << 20


# sources of the grouped-GEMM kernels whose traffic is stored (the kernel file and
# every header it includes)
FFN_REPS = 8  # moe_expert_ffn calls per timed replay of the roofline measurement

GEMM_SOURCES = ["sparse_mixture_experts_45_amd/csrc/gemm.hip",
                "sparse_mixture_experts_45_amd/csrc/kernels.h",
                "sparse_mixture_experts_45_amd/csrc/common.h",
                "sparse_mixture_experts_45_amd/csrc/block_ops.h",
                "include/moe.h"]


def source_hash():
    h = hashlib.sha256()
    for rel in GEMM_SOURCES:
        h.update(rel.encode())
        with open(os.path.join(ROOT, rel), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_path(workload):
    return os.path.join(ROOT, "profiles", "traffic_expert_gemm_%s.md" % workload)


def stored_traffic(workload):
    """Bytes per moe_expert_ffn call (up + down GEMM), or None if absent or stale."""
    path = traffic_path(workload)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    try:
        rec = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    except (IndexError, ValueError):
        return None
    if rec.get("source_hash") != source_hash():
        return None
    return rec["traffic_bytes_per_call"]


def layer_config(moe, torch, shape):
    tdt = torch.bfloat16 if shape.dtype == "bf16" else torch.float32
    return moe.config(shape.T, shape.d, shape.F, shape.E, shape.k, act=shape.act, dtype=tdt,
                      capacity=shape.capacity, renormalize=bool(shape.renormalize),
                      shared_d_ff=shape.Fs, routing=shape.routing)


def ffn_call(moe, torch, shape, dev, stream=None):
    """Arguments of one moe_expert_ffn call over the rows this layer groups:
    moe_route + moe_dispatch under token choice; under expert choice, the
    selection moe_forward reports (ec_idx: E x C tokens, ascending per expert;
    ec_w: their gates) as rows e*C + j, as moe_forward itself groups them."""
    T, k, E = shape.T, shape.k, shape.E
    i32 = dict(dtype=torch.int32, device="cuda")
    cfg = layer_config(moe, torch, shape)
    ws = moe.workspace(cfg)
    if shape.routing == "expert":
        C = min(shape.capacity if shape.capacity >= 0 else T * k // E, T)
        y = torch.empty((T, shape.d), dtype=dev["x"].dtype, device="cuda")
        ec_idx = torch.empty((E, C), **i32)
        ec_w = torch.empty((E, C), dtype=torch.float32, device="cuda")
        moe.moe_forward(cfg, dev, dev["x"], y, dict(ec_idx=ec_idx, ec_w=ec_w), ws, stream=stream)
        nrows = E * C + (T if shape.Fs else 0)
        row_token = torch.empty(nrows, **i32)
        row_token[:E * C] = ec_idx.view(-1)
        if shape.Fs:
            row_token[E * C:] = torch.arange(T, **i32)
        offsets = torch.arange(E + 2, **i32) * C
        offsets[E + 1] = nrows
        row_slot, topk_w = None, ec_w.view(-1)
    else:
        nrows = T * k + (T if shape.Fs else 0)
        topk_idx, inv = torch.empty((T, k), **i32), torch.empty((T, k), **i32)
        topk_w = torch.empty((T, k), dtype=torch.float32, device="cuda")
        counts, kept = torch.empty(E, **i32), torch.empty(E, **i32)
        offsets = torch.empty(E + 2, **i32)
        row_token, row_slot = torch.empty(nrows, **i32), torch.empty(nrows, **i32)
        moe.moe_route(cfg, dev["x"], dev["Wg"], dev["bg"], topk_idx, topk_w, None, None, None,
                      ws, stream=stream)
        moe.moe_dispatch(cfg, topk_idx, counts, kept, offsets, row_token, row_slot, inv, ws,
                         stream=stream)
    y_rows = torch.empty((max(nrows, 1), shape.d), dtype=torch.float32, device="cuda")
    return (cfg, dev["x"], dev, offsets, row_token, row_slot, topk_w, y_rows, ws)


def traffic_probe(args):
    import torch
    import sparse_mixture_experts_45_amd as moe
    from moe_synth import make_inputs, to_device, workload

    a = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    del a, b
    shape = workload(args.workload)
    dev = to_device(make_inputs(shape, args.seed), "cuda")
    fargs = ffn_call(moe, torch, shape, dev)
    for _ in range(5):
        moe.moe_expert_ffn(*fargs)
    torch.cuda.synchronize()
    # the grouping of these calls (token choice: what moe_dispatch wrote)
    offsets = fargs[3].cpu().numpy()
    kept = np.diff(offsets[:shape.E + 1])
    print(json.dumps({"probe": "expert FFN", "workload": shape.name,
                      "kept_rows": int(kept.sum()), "experts_hit": int((kept > 0).sum())}),
          flush=True)


# epilogue mode of a grouped-GEMM kernel: its last integer template argument
# (a trailing bool says whether B is read [K, N])
GEMM_MODE_UP, GEMM_MODE_DOWN = 0, 1


def _template_args(kernel_name):
    return [x.strip() for x in kernel_name.split("<", 1)[1].split(">", 1)[0].split(",")]


def gemm_mode(kernel_name):
    """Epilogue mode of a grouped-GEMM kernel: the LDS-DMA kernel's ninth template
    argument (<BM, BN, BK, NS, WM, WN, OCC, PERSIST, MODE, BT, XR>), else the
    register-staged kernel's last integer one (<T, BM, BN, BK, WM, WN, MODE, BT>)."""
    args = _template_args(kernel_name)
    if "grouped_gemm_dma_kernel" in kernel_name:
        return int(args[8])
    return int([x for x in args if x.lstrip("-").isdigit()][-1])


def gemm_bt(kernel_name):
    """Whether a grouped-GEMM kernel reads B stored [K, N] (the input-gradient pass)."""
    return "true" in _template_args(kernel_name)


def _counter_rows(db, counter):
    con = sqlite3.connect(db)
    rows = con.execute("select dispatch_id, kernel_name, value from counters_collection "
                       "where counter_name = ? order by dispatch_id", (counter,)).fetchall()
    con.close()
    return rows


def traffic_summarize(args):
    fetch_db, write_db = args.traffic_summarize
    rec = {"workload": args.workload, "source_hash": source_hash(), "copy_bytes": COPY_BYTES}
    kib = {}
    for counter, db in (("FETCH_SIZE", fetch_db), ("WRITE_SIZE", write_db)):
        rows = _counter_rows(db, counter)
        copies = [v for _, n, v in rows if "copyBuffer" in n][:3]
        if len(copies) < 3:
            sys.exit("no calibration copies in %s" % db)
        factor = (COPY_BYTES / 1024.0) / float(np.mean(copies))
        rec[counter.lower() + "_copy_kib"] = float(np.mean(copies))
        rec[counter.lower() + "_factor"] = round(factor, 4)
        for tag, mode in (("up", GEMM_MODE_UP), ("down", GEMM_MODE_DOWN)):
            vals = [v for _, n, v in rows
                    if "grouped_gemm" in n and gemm_mode(n) == mode and not gemm_bt(n)]
            if not vals:
                sys.exit("no %s GEMM dispatches in %s" % (tag, db))
            kib[(tag, counter)] = (float(np.mean(vals)), len(vals), factor)
    total = 0.0
    rec["kernels"] = {}
    for tag in ("up", "down"):
        f_kib, n, f_fac = kib[(tag, "FETCH_SIZE")]
        w_kib, _, w_fac = kib[(tag, "WRITE_SIZE")]
        fb, wb = f_kib * 1024 * f_fac, w_kib * 1024 * w_fac
        rec["kernels"][tag] = {"fetch_kib": round(f_kib, 1), "write_kib": round(w_kib, 1),
                               "fetch_bytes": round(fb), "write_bytes": round(wb),
                               "dispatches": n}
        total += fb + wb
    rec["traffic_bytes_per_call"] = round(total)
    wl = args.workload
    # the profiler runs that wrote the two databases: output directory and
    # file prefix read back from their paths
    runs = []
    for db in (fetch_db, write_db):
        rel = os.path.relpath(os.path.abspath(db), ROOT)
        runs.append((rel, os.path.dirname(rel), os.path.basename(rel)[:-len("_results.db")]))
    cmds = [
        "cd /tmp && export TMPDIR=/tmp   # then, from the repository root:",
        "rocprofv3 --pmc FETCH_SIZE -d %s -o %s -- "
        "python3 bench.py --traffic-probe --workload %s" % (runs[0][1], runs[0][2], wl),
        "rocprofv3 --pmc WRITE_SIZE -d %s -o %s -- "
        "python3 bench.py --traffic-probe --workload %s" % (runs[1][1], runs[1][2], wl),
        "python3 bench.py --workload %s --traffic-summarize %s %s" % (wl, runs[0][0], runs[1][0]),
    ]
    lines = [
        "# HBM traffic of the expert grouped GEMM: %s" % wl, "",
        "FETCH_SIZE and WRITE_SIZE per dispatch (rocprofv3 `--pmc`, one counter per run), each "
        "scaled by what the same counter reads for a device-to-device copy of %d MiB "
        "(the first three `__amd_rocclr_copyBuffer` dispatches of the probe)." % (COPY_BYTES >> 20),
        "", "Commands (committed files only):", "", "```"] + cmds + ["```", "",
        "| kernel | dispatches | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | fetch bytes (scaled) | "
        "write bytes (scaled) |", "|---|---|---|---|---|---|"]
    for tag in ("up", "down"):
        r = rec["kernels"][tag]
        lines.append("| %s-projection | %d | %.1f | %.1f | %.0f | %.0f |" % (
            tag, r["dispatches"], r["fetch_kib"], r["write_kib"], r["fetch_bytes"],
            r["write_bytes"]))
    lines += ["", "Calibration: copy FETCH_SIZE %.1f KiB (factor %.4f), WRITE_SIZE %.1f KiB "
              "(factor %.4f) for %d KiB moved." % (rec["fetch_size_copy_kib"],
                                                   rec["fetch_size_factor"],
                                                   rec["write_size_copy_kib"],
                                                   rec["write_size_factor"], COPY_BYTES >> 10),
              "", "Traffic per moe_expert_ffn call (up + down): %.1f MB." % (total / 1e6),
              "", "```json", json.dumps(rec, indent=1), "```", ""]
    with open(traffic_path(wl), "w") as fh:
        fh.write("\n".join(lines))
    print(json.dumps(rec))


def trace_path(workload):
    return os.path.join(ROOT, "profiles", "kernel_trace_%s.md" % workload)


def _kernel_durations(db):
    """{kernel name: [durations in ns]} of every dispatch in a rocprofv3 database."""
    con = sqlite3.connect(db)
    rows = con.execute("select name, duration from kernels").fetchall()
    con.close()
    out = {}
    for name, dur in rows:
        out.setdefault(name, []).append(float(dur))
    return out


def trace_summarize(args):
    """Kernel-trace summary of one profiled bench run: every kernel's call count
    and durations from the rocprofv3 database, and the expert FFN per call
    (row-tile list + up GEMM + down GEMM averages) turned into the roofline
    fraction with the algorithmic work of the workload the run reported."""
    db, bench_json = args.trace_summarize
    line = [ln for ln in open(bench_json) if ln.lstrip().startswith("{")][-1]
    run = json.loads(line)
    if "backward" in run:
        return trace_summarize_backward(db, bench_json, run)
    from moe_synth import workload
    shape = workload(run["config"]["workload"])
    kept_rows, hit = run["config"]["kept_rows"], run["config"]["experts_hit"]
    durs = _kernel_durations(db)
    total = sum(sum(v) for v in durs.values())
    names = sorted(durs, key=lambda n: -sum(durs[n]))
    gemm = lambda mode: [n for n in names  # noqa: E731
                         if "grouped_gemm" in n and gemm_mode(n) == mode and not gemm_bt(n)]
    up, dn = gemm(GEMM_MODE_UP), gemm(GEMM_MODE_DOWN)
    tl = [n for n in names if "build_tiles_kernel" in n]
    if len(up) != 1 or len(dn) != 1:
        sys.exit("expected one up- and one down-projection GEMM kernel in %s" % db)
    avg = lambda n: float(np.mean(durs[n])) / 1e3  # noqa: E731  (us)
    t_tl = avg(tl[0]) if tl else 0.0
    ffn_us = avg(up[0]) + avg(dn[0]) + t_tl
    flop, nbytes = algorithmic(shape, kept_rows, hit)
    rel_db = os.path.relpath(os.path.abspath(db), ROOT)
    rel_json = os.path.relpath(os.path.abspath(bench_json), ROOT)
    s = shape
    tflops = flop / (ffn_us * 1e-6) / 1e12
    gbs = nbytes / (ffn_us * 1e-6) / 1e9
    lines = [
        "# Kernel trace: bench.py forward, %s (T=%d, d=%d, d_ff=%d, E=%d, top-%d, %s, %s%s%s)"
        % (s.name, s.T, s.d, s.F, s.E, s.k, "GELU" if s.act == "gelu" else "ReLU",
           s.dtype, ", capacity %d" % s.capacity if s.capacity >= 0 else "",
           ", shared expert d_ff %d" % s.Fs if s.Fs else ""), "",
        "Commands (from the repository root, on one MI355X; `cd /tmp && export TMPDIR=/tmp` "
        "first for the profiler's scratch files):", "", "```",
        "rocprofv3 --kernel-trace --stats -d %s -o %s -- python3 bench.py --workload %s "
        "--hbm-workload none --no-cpu-baseline --steps 20 --warmup 5 > %s"
        % (os.path.dirname(rel_db), os.path.basename(rel_db)[:-len("_results.db")], s.name,
           rel_json),
        "python3 bench.py --trace-summarize %s %s" % (rel_db, rel_json),
        "```", "",
        "| kernel | calls | avg (us) | min (us) | max (us) | share |",
        "|---|---|---|---|---|---|"]
    for n in names:
        v = durs[n]
        lines.append("| `%s` | %d | %.2f | %.2f | %.2f | %.1f %% |" % (
            n, len(v), avg(n), min(v) / 1e3, max(v) / 1e3, 100.0 * sum(v) / total))
    lines += ["", "Expert FFN per call (averages): row-tile list %.2f + up-projection %.2f + "
              "down-projection %.2f = %.2f us." % (t_tl, avg(up[0]), avg(dn[0]), ffn_us),
              "",
              "Algorithmic work of the call (%d kept routed rows, %d experts hit): %.4g FLOP, "
              "%.4g bytes." % (kept_rows, hit, flop, nbytes), "",
              "From the trace: %.1f TFLOP/s = %.4f of the 2500 TFLOP/s bf16 peak; %.1f GB/s = "
              "%.4f of the 8000 GB/s HBM peak." % (tflops, tflops / PEAK_BF16_TFLOPS, gbs,
                                                    gbs / PEAK_HBM_GBS), "",
              "The profiled run's own bench line (HIP events around graph replays, under the "
              "profiler): expert FFN %.4f ms, roofline fraction %.4f (%s bound); layer %.4f ms "
              "per call, %.1f tokens/s." % (run["roofline"]["kernel_ms"], run["roofline"]["frac"],
                                            run["roofline"]["bound"], run["ms_per_step"],
                                            run["value"]),
              ""]
    with open(trace_path(s.name), "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))


def trace_summarize_backward(db, bench_json, run):
    """Kernel-trace summary of one profiled `--backward` run: every kernel's
    call count and durations, and the run's own training-step line."""
    wl = run["config"]["workload"]
    durs = _kernel_durations(db)
    total = sum(sum(v) for v in durs.values())
    names = sorted(durs, key=lambda n: -sum(durs[n]))
    rel_db = os.path.relpath(os.path.abspath(db), ROOT)
    rel_json = os.path.relpath(os.path.abspath(bench_json), ROOT)
    b = run["backward"]
    lines = [
        "# Kernel trace: training step (moe_forward_train + moe_backward), %s" % wl, "",
        "Commands (from the repository root, on one MI355X; `cd /tmp && export TMPDIR=/tmp` "
        "first for the profiler's scratch files):", "", "```",
        "rocprofv3 --kernel-trace --stats -d %s -o %s -- python3 bench.py --backward --workload %s "
        "--steps %d --warmup %d > %s" % (os.path.dirname(rel_db),
                                         os.path.basename(rel_db)[:-len("_results.db")], wl,
                                         run["steps"], run["warmup"], rel_json),
        "python3 bench.py --trace-summarize %s %s" % (rel_db, rel_json),
        "```", "",
        "| kernel | calls | avg (us) | min (us) | max (us) | share |",
        "|---|---|---|---|---|---|"]
    for n in names:
        v = durs[n]
        lines.append("| `%s` | %d | %.2f | %.2f | %.2f | %.1f %% |" % (
            n, len(v), float(np.mean(v)) / 1e3, min(v) / 1e3, max(v) / 1e3,
            100.0 * sum(v) / total))
    lines += ["", "The profiled run's own bench line (under the profiler): training step %.4f ms, "
              "backward %.4f ms (HIP events), backward GEMM work %.4g FLOP = %.1f TFLOP/s, %.4f "
              "of the bf16 peak." % (run["ms_per_step"], b["ms"], b["gemm_flop"],
                                     b["achieved_tflops"], b["frac"]), ""]
    with open(os.path.join(ROOT, "profiles", "kernel_trace_backward_%s.md" % wl), "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))


PMC_COUNTERS = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA", "SQ_WAIT_ANY", "SQ_WAVE_CYCLES",
                "SQ_BUSY_CU_CYCLES", "SQ_INSTS_LDS", "SQ_WAIT_INST_LDS", "SQ_LDS_BANK_CONFLICT",
                "GRBM_GUI_ACTIVE"]
N_SIMD = 1024        # 256 CUs x 4 SIMDs
N_XCD = 8
MFMA_CYCLES = 32     # v_mfma_f32_32x32x16_bf16: 32 cycles of one SIMD's matrix core
MFMA_FLOP = 32 * 32 * 16 * 2


def pmc_path(workload):
    return os.path.join(ROOT, "profiles", "pmc_expert_gemm_%s.md" % workload)


def pmc_summarize(args):
    """Matrix-core utilisation of the up and down GEMMs of one workload from a
    rocprofv3 --pmc run (with --kernel-trace for durations) of --traffic-probe:
    per-dispatch averages of the counters, the engine clock they imply and the
    MFMA busy fraction at that clock and at the 2.4 GHz the peak assumes."""
    db, log = args.pmc_summarize
    probe = json.loads([ln for ln in open(log) if ln.startswith('{"probe"')][-1])
    from moe_synth import workload
    shape = workload(probe["workload"])
    con = sqlite3.connect(db)
    rows = con.execute("select dispatch_id, kernel_name, counter_name, value from "
                       "counters_collection").fetchall()
    durs = dict(con.execute("select dispatch_id, duration from kernels").fetchall())
    con.close()
    per = {}
    for did, name, cname, val in rows:
        if "grouped_gemm" not in name or gemm_bt(name):
            continue
        tag = {GEMM_MODE_UP: "up", GEMM_MODE_DOWN: "down"}.get(gemm_mode(name))
        if tag is None:
            continue
        d = per.setdefault(tag, {"name": name, "disp": {}})
        d["disp"].setdefault(did, {})[cname] = d["disp"].get(did, {}).get(cname, 0.0) + float(val)
    kept = probe["kept_rows"]
    # MFMA instructions the kept rows need, per GEMM: rows x N x K / (32 x 32 x 16)
    need = {"up": kept * shape.F * shape.d / 16384.0, "down": kept * shape.d * shape.F / 16384.0}
    if shape.Fs:
        need = {k: v + shape.T * shape.Fs * shape.d / 16384.0 for k, v in need.items()}
    rel_db = os.path.relpath(os.path.abspath(db), ROOT)
    rel_log = os.path.relpath(os.path.abspath(log), ROOT)
    wl = shape.name
    lines = ["# Matrix-core utilisation of the expert GEMMs: %s" % wl, "",
             "One `rocprofv3 --pmc` pass (with `--kernel-trace` for durations) over `bench.py "
             "--traffic-probe` (a 256 MiB copy, then five `moe_expert_ffn` calls); per-dispatch "
             "averages.  Commands (from the repository root, on one MI355X; "
             "`cd /tmp && export TMPDIR=/tmp` first):", "", "```",
             "rocprofv3 --kernel-trace --pmc %s -d %s -o %s -- python3 bench.py --traffic-probe "
             "--workload %s > %s" % (" ".join(PMC_COUNTERS), os.path.dirname(rel_db),
                                     os.path.basename(rel_db)[:-len("_results.db")], wl, rel_log),
             "python3 bench.py --pmc-summarize %s %s" % (rel_db, rel_log), "```", "",
             "| counter | up-projection | down-projection |", "|---|---|---|"]
    avg = {}
    for tag in ("up", "down"):
        if tag not in per:
            sys.exit("no %s-projection dispatches with counters in %s" % (tag, db))
        disp = per[tag]["disp"]
        avg[tag] = {c: float(np.mean([v.get(c, 0.0) for v in disp.values()])) for c in PMC_COUNTERS}
        avg[tag]["us"] = float(np.mean([durs[i] for i in disp if i in durs])) / 1e3
        avg[tag]["n"] = len(disp)
    for c in PMC_COUNTERS:
        lines.append("| `%s` | %.4g | %.4g |" % (c, avg["up"][c], avg["down"][c]))
    lines.append("| duration (us, under the profiler) | %.1f | %.1f |" % (avg["up"]["us"],
                                                                         avg["down"]["us"]))
    lines += ["", "Kernels: `%s` (up), `%s` (down)." % (per["up"]["name"], per["down"]["name"]),
              "", "Derived (per dispatch):"]
    for tag in ("up", "down"):
        a = avg[tag]
        cyc = a["GRBM_GUI_ACTIVE"] / N_XCD          # engine cycles over the kernel
        clk = cyc / a["us"] if a["us"] else 0.0     # MHz
        busy = a["SQ_VALU_MFMA_BUSY_CYCLES"] / (N_SIMD * cyc) if cyc else 0.0
        busy24 = (a["SQ_INSTS_MFMA"] * MFMA_CYCLES / N_SIMD) / (a["us"] * 2400.0)
        lines.append(
            "- %s: %.3g MFMA instructions (%.3g for the kept rows: %.1f %% on padding rows); "
            "%.1f cycles per MFMA; engine clock %.0f MHz (`GRBM_GUI_ACTIVE` / %d XCDs / "
            "duration); matrix cores busy %.1f %% of the cycles at that clock, %.1f %% of a "
            "2.4 GHz kernel duration; waves waiting %.1f %% of their cycles (`SQ_WAIT_ANY` / "
            "`SQ_WAVE_CYCLES`); executed %.0f TFLOP/s, useful %.0f TFLOP/s; LDS bank "
            "conflicts %.3g." % (
                tag, a["SQ_INSTS_MFMA"], need[tag],
                100.0 * (a["SQ_INSTS_MFMA"] - need[tag]) / max(a["SQ_INSTS_MFMA"], 1.0),
                a["SQ_VALU_MFMA_BUSY_CYCLES"] / max(a["SQ_INSTS_MFMA"], 1.0), clk, N_XCD,
                100.0 * busy, 100.0 * busy24,
                100.0 * a["SQ_WAIT_ANY"] / max(a["SQ_WAVE_CYCLES"], 1.0),
                a["SQ_INSTS_MFMA"] * MFMA_FLOP / (a["us"] * 1e-6) / 1e12,
                need[tag] * MFMA_FLOP / (a["us"] * 1e-6) / 1e12, a["SQ_LDS_BANK_CONFLICT"]))
    lines += ["", "Grouping of the probed calls: %d kept routed rows, %d experts hit." % (
        kept, probe["experts_hit"]), ""]
    with open(pmc_path(wl), "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))


def algorithmic(shape, kept_rows, hit_experts):
    """Active FLOPs and algorithmic HBM bytes of one expert-FFN call."""
    elt = 2 if shape.dtype == "bf16" else 4
    flop = 4.0 * kept_rows * shape.d * shape.F
    wbytes = hit_experts * (2.0 * shape.d * shape.F + shape.F + shape.d) * elt
    if shape.Fs:
        flop += 4.0 * shape.T * shape.d * shape.Fs
        wbytes += (2.0 * shape.d * shape.Fs + shape.Fs + shape.d) * elt
    # activations: x read once and the layer output y written once, both in the
    # layer dtype (the grouped rows, H and the fp32 expert rows are
    # intermediates of this implementation, not algorithmic bytes)
    abytes = 2 * shape.T * shape.d * elt
    return flop, wbytes + abytes


def cpu_baseline(shape, inp, seconds):
    """The fp64 oracle on the host cores over a bounded sample of the batch: routing of
    the whole batch (timed once, prorated to the tokens processed), then expert MLPs
    and combine over consecutive chunks of tokens in batch order (wrapping around
    the batch), until about `seconds` of work."""
    import oracle
    t0 = time.perf_counter()
    if shape.routing == "expert":
        sel = oracle.ec_route(shape, inp)
        experts = lambda toks: oracle.ec_experts(shape, inp, sel, toks)  # noqa: E731
    else:
        rt = oracle.route(shape, inp, with_probs=False)
        experts = lambda toks: oracle.experts(shape, inp, rt, toks)  # noqa: E731
    t_route = time.perf_counter() - t0
    T = max(shape.T, 1)
    # chunks of about a tenth of the budget, sized from the tokens already timed
    n, t_exp, done = min(shape.T, 8), 0.0, 0
    while True:
        toks = (done + np.arange(n)) % T
        t2 = time.perf_counter()
        experts(toks)
        t_exp += time.perf_counter() - t2
        done += n
        dt = t_exp + t_route * done / T
        if dt >= seconds or shape.T == 0:
            break
        per_tok = dt / done
        n = int(max(1, min(shape.T, (seconds - dt) / per_tok, 0.1 * seconds / per_tok + 1)))
    if done >= shape.T:
        what = "%d tokens = %.2f passes over the %d-token %s batch" % (done, done / T, shape.T,
                                                                      shape.name)
    else:
        what = "the first %d tokens of the %d-token %s batch" % (done, shape.T, shape.name)
    return {"value": round(done / dt, 3), "unit": "tokens/s", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": "fp64 oracle: routing (timed on the whole batch, prorated) + expert "
                      "MLPs and combine of %s, %.1f s" % (what, dt)}


def bench_backward(args):
    """Training step of the layer: moe_forward_train then moe_backward (all
    gradients, balance coefficient 0.01), replayed from one HIP graph; the
    backward alone is timed with events on its stream."""
    import torch
    import sparse_mixture_experts_45_amd as moe
    from moe_synth import make_inputs, to_device, workload

    shape = workload(args.workload)
    dev = to_device(make_inputs(shape, args.seed), "cuda")
    cfg = layer_config(moe, torch, shape)
    ws = moe.train_workspace(cfg)
    T, d, F, E, Fs = shape.T, shape.d, shape.F, shape.E, shape.Fs
    tdt = dev["x"].dtype
    gen = torch.Generator(device="cuda").manual_seed(args.seed + 1)
    dy = torch.randn((T, d), generator=gen, device="cuda").to(tdt)
    y = torch.empty((T, d), dtype=tdt, device="cuda")
    z = lambda *sh, dt=tdt: torch.empty(sh, dtype=dt, device="cuda")  # noqa: E731
    grads = dict(dx=z(T, d), dWg=z(E, d, dt=torch.float32), dbg=z(E, dt=torch.float32),
                 dW1=z(E, F, d), db1=z(E, F), dW2=z(E, d, F), db2=z(E, d))
    if Fs:
        grads.update(dWs1=z(Fs, d), dbs1=z(Fs), dWs2=z(d, Fs), dbs2=z(d))
    kept = torch.empty(E, dtype=torch.int32, device="cuda")
    stream = torch.cuda.Stream()

    def fwd():
        moe.moe_forward_train(cfg, dev, dev["x"], y, dict(kept=kept), ws, stream=stream)

    def bwd():
        moe.moe_backward(cfg, dev, dev["x"], dy, grads, aux_coef=0.01, ws=ws, stream=stream)

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            fwd()
            bwd()
    torch.cuda.synchronize()
    g_step = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_step, stream=stream):
        fwd()
        bwd()
    g_bwd = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_bwd, stream=stream):
        bwd()
    torch.cuda.synchronize()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        for _ in range(args.steps):
            g_step.replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    with torch.cuda.stream(stream):
        for a, b in evs:
            fwd()  # the backward reads what this forward leaves in the workspace
            a.record(stream)
            g_bwd.replay()
            b.record(stream)
    torch.cuda.synchronize()
    bwd_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    kept_rows = int(kept.sum())
    # backward GEMM work: input-gradient pass and weight-gradient pass, each 4 d F
    # per kept row (+ 4 d Fs per token for the shared expert)
    flop = 8.0 * kept_rows * d * F + (8.0 * T * d * Fs if Fs else 0.0)
    peak = PEAK_BF16_TFLOPS if shape.dtype == "bf16" else PEAK_F32_TFLOPS
    ach = flop / (bwd_ms * 1e-3) / 1e12
    out = {
        "metric": "MoE layer training step (forward + backward) tokens/s",
        "value": round(T * args.steps / elapsed, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / args.steps, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if shape.dtype == "bf16" else "f32",
        "data": "synthetic (seeded; random-init weights; dy ~ N(0, 1))",
        "config": {"workload": shape.name, "tokens": T, "d_model": d, "d_ff": F,
                   "n_experts": E, "top_k": shape.k, "capacity": shape.capacity,
                   "shared_d_ff": Fs, "routing": shape.routing, "aux_coef": 0.01,
                   "hip_graph": True, "kept_rows": kept_rows},
        "backward": {"ms": round(bwd_ms, 4), "gemm_flop": flop, "achieved_tflops": round(ach, 1),
                     "peak_tflops": peak, "frac": round(ach / peak, 4)},
    }
    print(json.dumps(out), flush=True)


def calls_per_graph(steps):
    """Layer calls captured in one HIP graph: the largest of 10, 5, 4, 2, 1 that
    divides `steps` (replays of a one-call graph left ~0.1 ms between replays
    on the Mixtral-shaped layer that several calls per replay do not)."""
    return next(n for n in (10, 5, 4, 2, 1) if steps % n == 0)


def time_layer(moe, torch, shape, dev, steps, warmup, use_graph):
    """moe_forward over `steps` calls (replayed from a HIP graph of
    calls_per_graph(steps) calls when use_graph), bracketed by device
    synchronisation.  Returns (seconds, kept [E] counts)."""
    tdt = torch.bfloat16 if shape.dtype == "bf16" else torch.float32
    cfg = layer_config(moe, torch, shape)
    ws = moe.workspace(cfg)
    T, E = shape.T, shape.E
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
        for _ in range(warmup):
            step()
    torch.cuda.synchronize()
    per = calls_per_graph(steps)
    if use_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for _ in range(per):
                step()
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            for _ in range(2):
                graph.replay()
        torch.cuda.synchronize()

    # ---- timed region: exactly `steps` layer calls
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        if graph is not None:
            for _ in range(steps // per):
                graph.replay()
        else:
            for _ in range(steps):
                step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kept = st["kept"].cpu().numpy()
    del graph, ws
    return elapsed, kept


def ffn_roofline(moe, torch, shape, dev, kept, steps, use_graph):
    """The expert FFN (one moe_expert_ffn call: row-tile list, up-projection GEMM,
    down-projection GEMM) timed with HIP events on the stream it is launched on:
    FFN_REPS back-to-back calls per graph replay, `steps` replays.  Returns the
    roofline object against the bf16 MFMA peak or the HBM peak, whichever bounds
    the call's algorithmic work."""
    kept_rows = int(kept.sum())
    hit = int((kept > 0).sum())
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        fargs = ffn_call(moe, torch, shape, dev, stream=stream)
        for _ in range(3):
            moe.moe_expert_ffn(*fargs, stream=stream)
    torch.cuda.synchronize()
    # FFN_REPS moe_expert_ffn calls (tile list, up GEMM, down GEMM each)
    # replayed from one graph: the events bracket the kernels without host
    # launch gaps, and the graph's own launch latency is paid once per
    # FFN_REPS calls, as in a model whose layers share one graph
    ffn_graph = None
    if use_graph:
        ffn_graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(ffn_graph, stream=stream):
            for _ in range(FFN_REPS):
                moe.moe_expert_ffn(*fargs, stream=stream)
        torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    with torch.cuda.stream(stream):
        for a, b in evs:
            a.record(stream)
            if ffn_graph is not None:
                ffn_graph.replay()
            else:
                for _ in range(FFN_REPS):
                    moe.moe_expert_ffn(*fargs, stream=stream)
            b.record(stream)
    torch.cuda.synchronize()
    ffn_ms = float(np.mean([a.elapsed_time(b) for a, b in evs])) / FFN_REPS
    del ffn_graph, fargs

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
    traffic = stored_traffic(shape.name)
    roof["traffic"] = None if traffic is None else float(traffic)
    roof.update(kernel="expert FFN: one moe_expert_ffn call (row-tile list, up-projection "
                       "GEMM, down-projection GEMM), timed as %d back-to-back calls"
                       % FFN_REPS, kernel_ms=round(ffn_ms, 4),
                algorithmic_flop=flop, algorithmic_bytes=nbytes,
                achieved_tflops=round(flop / (ffn_ms * 1e-3) / 1e12, 2),
                achieved_gbs=round(nbytes / (ffn_ms * 1e-3) / 1e9, 1))
    return roof


def main():
    args = parse()
    if args.traffic_summarize:
        traffic_summarize(args)
        return
    if args.trace_summarize:
        trace_summarize(args)
        return
    if args.pmc_summarize:
        pmc_summarize(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the MoE layer here is the data-parallel "
              "replica of one GPU; this library has no multi-GPU path "
              "(requested --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    if args.traffic_probe:
        traffic_probe(args)
        return
    if args.backward:
        bench_backward(args)
        return

    import torch
    import sparse_mixture_experts_45_amd as moe
    from moe_synth import make_inputs, to_device, workload

    shape = workload(args.workload)
    inp = make_inputs(shape, args.seed)
    dev = to_device(inp, "cuda")
    T, k, E = shape.T, shape.k, shape.E
    elapsed, kept = time_layer(moe, torch, shape, dev, args.steps, args.warmup, args.graph)
    ms_per_step = elapsed * 1e3 / args.steps
    kept_rows = int(kept.sum())
    hit = int((kept > 0).sum())
    roof = ffn_roofline(moe, torch, shape, dev, kept, args.steps, args.graph)
    flop, _ = algorithmic(shape, kept_rows, hit)

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
                   "shared_d_ff": shape.Fs, "act": shape.act, "routing": shape.routing,
                   "hip_graph": bool(args.graph),
                   "calls_per_graph": calls_per_graph(args.steps) if args.graph else 0,
                   "kept_rows": kept_rows, "experts_hit": hit},
        "layer_tflops": round(flop / (ms_per_step * 1e-3) / 1e12, 2),
        "roofline": roof,
    }
    del dev
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(shape, inp, args.cpu_seconds)
    del inp
    if args.hbm_workload and args.hbm_workload != "none" and args.hbm_workload != shape.name:
        # the weight-streaming workload, measured the same way on its own inputs
        s2 = workload(args.hbm_workload)
        dev2 = to_device(make_inputs(s2, args.seed), "cuda")
        el2, kept2 = time_layer(moe, torch, s2, dev2, args.steps, args.warmup, args.graph)
        r2 = ffn_roofline(moe, torch, s2, dev2, kept2, args.steps, args.graph)
        r2.update(workload=s2.name, layer_ms=round(el2 * 1e3 / args.steps, 4),
                  layer_tokens_per_s=round(s2.T * args.steps / el2, 1),
                  kept_rows=int(kept2.sum()), experts_hit=int((kept2 > 0).sum()))
        out["roofline_hbm"] = r2
        del dev2
        torch.cuda.empty_cache()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
