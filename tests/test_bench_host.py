"""Host-side checks of bench.py (no GPU): the one-GPU guard, that the committed
counter summaries were taken on the current kernel sources (so the JSON line's
traffic field is filled), and the CPU oracle baseline leg on a tiny workload."""
import os
import subprocess
import sys

import pytest

import bench
from quantized_scaled_dot_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("workload,kernel,sources", [
    ("video-dit-32k", "attn_fwd_kernel", bench.KERNEL_SOURCES),
    ("video-dit-32k-qk4", "attn_fwd_kernel", bench.KERNEL_SOURCES),
    ("video-dit-32k-qk4-qsmooth", "attn_fwd_kernel", bench.KERNEL_SOURCES),
    ("decode-32k-gqa", "decode_chunk_kernel", bench.DECODE_SOURCES),
])
def test_counter_summaries_match_the_current_kernel_source(workload, kernel, sources):
    t = bench.measured_traffic(workload, kernel, sources)
    assert t is not None and t > 0, f"profiles/{kernel}.{workload}.pmc.txt was taken on another kernel source"


@pytest.mark.parametrize("workload", ["video-dit-32k", "llm-prefill-4k-causal"])
def test_quantize_pass_summaries_match_the_current_source(workload):
    path = os.path.join(ROOT, "profiles", f"quantize_passes.{workload}.pmc.txt")
    sha = [l.split(":", 1)[1].strip() for l in open(path) if l.startswith("kernel_source_sha256_16:")]
    srcs = ("quantized_scaled_dot_amd/csrc/quant.hip", "quantized_scaled_dot_amd/csrc/common.h")
    assert sha == [bench.kernel_source_sha(srcs)]


def test_cpu_baseline_leg_on_a_tiny_workload():
    w = synth.WORKLOADS["tiny-f16-256"]
    Q, K, V = synth.make_inputs(w)
    r = bench.cpu_baseline(w, Q, K, V, budget_s=0.5)
    assert r["kind"] == "oracle" and r["unit"] == "TOPS"
    assert r["value"] > 0 and r["cores"] >= 1
    assert "random query rows" in r["sample"]
