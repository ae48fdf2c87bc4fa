"""Host-side logic of bench.py (CPU only): the one-GPU guard, the algorithmic
work figures the roofline divides by, the kernel-mode parsing of the traffic
summarizer, and the stored traffic summaries."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from moe_synth import WORKLOADS, workload  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_work_page1():
    """page-1 shape: 4096 kept rows of d=768, d_ff=3072, 8 experts hit:
    FLOP = 4 * rows * d * d_ff; bytes = bf16 W1, b1, W2, b2 of 8 experts + bf16 x
    read once + bf16 y written once (no intermediates)."""
    s = workload("page1_b4s512")
    flop, nbytes = bench.algorithmic(s, 4096, 8)
    assert flop == 4.0 * 4096 * 768 * 3072
    w = 8 * (2 * 768 * 3072 + 3072 + 768) * 2
    assert nbytes == w + 2 * 2048 * 768 * 2


def test_algorithmic_work_shared_expert():
    s = workload("deepseek_e256_top8")
    flop, nbytes = bench.algorithmic(s, 4096, 256)
    assert flop == 4.0 * 4096 * 7168 * 2048 + 4.0 * 512 * 7168 * 2048
    w = 257 * (2 * 7168 * 2048 + 2048 + 7168) * 2
    assert nbytes == w + 2 * 512 * 7168 * 2


@pytest.mark.parametrize("steps,per", [(50, 10), (20, 10), (15, 5), (8, 4), (6, 2), (7, 1), (1, 1)])
def test_calls_per_graph_divides_the_steps(steps, per):
    assert bench.calls_per_graph(steps) == per and steps % per == 0


def test_default_workloads():
    """The default bench line is the Mixtral-shaped layer (matrix-core bound) with
    the DeepSeek-shaped layer (weight streaming) as its second roofline."""
    old = sys.argv
    sys.argv = ["bench.py"]
    try:
        a = bench.parse()
    finally:
        sys.argv = old
    assert a.workload == "mixtral_t4096"
    assert a.hbm_workload == "deepseek_e256_top8"
    s = workload(a.workload)
    flop, nbytes = bench.algorithmic(s, s.T * s.k, s.E)
    assert flop / nbytes > bench.RIDGE
    s2 = workload(a.hbm_workload)
    flop2, nbytes2 = bench.algorithmic(s2, s2.T * s2.k, s2.E)
    assert flop2 / nbytes2 < bench.RIDGE


@pytest.mark.parametrize("name,mode,bt", [
    ("moe::grouped_gemm_dma_kernel<128, 128, 64, 2, 2, 4, 2, 0, 0, false, 0>", 0, False),
    ("void moe::grouped_gemm_dma_kernel<256, 256, 64, 2, 2, 4, 2, 0, 1, true, 0>(moe::GemmArgs)",
     1, True),
    ("void moe::grouped_gemm_dma_kernel<256, 256, 64, 2, 2, 4, 2, 0, 1, false, 1>(moe::GemmArgs)",
     1, False),
    ("moe::grouped_gemm_kernel<float, 64, 64, 32, 2, 2, 3, false>", 3, False),
])
def test_gemm_mode_of_kernel_name(name, mode, bt):
    assert bench.gemm_mode(name) == mode
    assert bench.gemm_bt(name) == bt


def test_stored_traffic_summaries_parse():
    """Every token-choice and expert-choice bf16 workload has a summary whose
    JSON record carries the per-call byte total and the per-kernel counters."""
    for name, s in WORKLOADS.items():
        if s.dtype != "bf16":
            continue
        path = bench.traffic_path(name)
        assert os.path.exists(path), path
        text = open(path).read()
        rec = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
        assert rec["workload"] == name
        assert rec["traffic_bytes_per_call"] > 0
        assert set(rec["kernels"]) == {"up", "down"}
        assert len(rec["source_hash"]) == 16
