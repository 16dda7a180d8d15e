"""Host-side checks of bench.py (no GPU): the one-GPU guard, that the JSON line's
traffic field comes from a counter summary only while that summary's kernel
source hash is current (null otherwise), and the CPU oracle baseline leg on a
tiny workload."""
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


SUMMARIES = [
    ("video-dit-32k", "attn_fwd_kernel", bench.KERNEL_SOURCES),
    ("video-dit-32k-qk4", "attn_fwd_kernel", bench.KERNEL_SOURCES),
    ("video-dit-32k-qk4-qsmooth", "attn_fwd_kernel", bench.KERNEL_SOURCES),
    ("decode-32k-gqa", "decode_chunk_kernel", bench.DECODE_SOURCES),
]


def _fields(path):
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    return vals


@pytest.mark.parametrize("workload,kernel,sources", SUMMARIES)
def test_counter_summaries_fill_traffic_only_for_their_own_kernel_source(workload, kernel, sources):
    """A summary names the source hash it was taken on and positive HBM bytes; bench.py reports
    those bytes only while the kernel source still has that hash (else traffic is null)."""
    path = os.path.join(ROOT, "profiles", f"{kernel}.{workload}.pmc.txt")
    vals = _fields(path)
    assert float(vals["hbm_bytes_per_launch"]) > 0
    current = vals["kernel_source_sha256_16"] == bench.kernel_source_sha(sources)
    t = bench.measured_traffic(workload, kernel, sources)
    assert (t == float(vals["hbm_bytes_per_launch"])) if current else (t is None)


def test_traffic_is_null_for_a_stale_summary(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "attn_fwd_kernel.x.pmc.txt").write_text("kernel_source_sha256_16: 0000000000000000\n"
                                                     "hbm_bytes_per_launch: 123\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    for p in bench.KERNEL_SOURCES:
        (tmp_path / p).parent.mkdir(parents=True, exist_ok=True)
        (tmp_path / p).write_text("source")
    assert bench.measured_traffic("x") is None
    (prof / "attn_fwd_kernel.x.pmc.txt").write_text(f"kernel_source_sha256_16: {bench.kernel_source_sha()}\n"
                                                     "hbm_bytes_per_launch: 123\n")
    assert bench.measured_traffic("x") == 123.0


@pytest.mark.parametrize("workload", ["video-dit-32k", "llm-prefill-4k-causal"])
def test_quantize_pass_summaries_name_their_source(workload):
    path = os.path.join(ROOT, "profiles", f"quantize_passes.{workload}.pmc.txt")
    sha = [l.split(":", 1)[1].strip() for l in open(path) if l.startswith("kernel_source_sha256_16:")]
    assert len(sha) == 1 and len(sha[0]) == 16


def test_cpu_baseline_leg_on_a_tiny_workload():
    w = synth.WORKLOADS["tiny-f16-256"]
    Q, K, V = synth.make_inputs(w)
    r = bench.cpu_baseline(w, Q, K, V, budget_s=0.5)
    assert r["kind"] == "oracle" and r["unit"] == "TOPS"
    assert r["value"] > 0 and r["cores"] >= 1
    assert "random query rows" in r["sample"]


def test_shader_clock_is_read_from_amd_smi_and_rocm_smi_json():
    amd = [{"gpu": 0, "clock": {"gfx_0": {"clk": {"value": 2087, "unit": "MHz"}, "min_clk": {"value": 500},
                                          "max_clk": {"value": 2400}, "clk_locked": "N/A", "deep_sleep": "DISABLED"},
                                "mem_0": {"clk": {"value": 1900, "unit": "MHz"}}}}]
    assert [v for _, v in bench._mhz_values(amd)] == [2087.0]
    rocm = {"card0": {"sclk clock speed:": "(2100Mhz)", "sclk clock level:": "1", "mclk clock speed:": "(1900Mhz)"}}
    assert [v for _, v in bench._mhz_values(rocm)] == [2100.0]
