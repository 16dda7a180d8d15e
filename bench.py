"""Benchmark of the quantized attention forward on one MI355X.

One step = the whole hot path on one batch of synthetic input: quantize Q and K
(K smoothing, INT8 per block) and V (FP8, per-channel scales) in one library
call (sage_quantize_qkv, three launches), then the fused attention kernel.
Inputs are resident in HBM before timing starts.

Metric: attention TOPS = 4*B*H*N^2*d / t (halved for causal) with t the
wall-clock time of one step.  The JSON line also carries the attention
kernel's own rate against the dense INT8/FP8 matrix-core peak (roofline, on
the mean of the per-step HIP-event timings; attn_kernel_ms is their median,
with the mean and p95 beside it), the peak allocated device memory, the shader
clock read with
amd-smi while the attention kernel runs back to back, and
the CPU oracle timed on a bounded sample of the same workload, and the
quantize passes' achieved HBM bandwidth (algorithmic bytes: 2 read + 1 written
per element of Q, K and V; the statistics passes read K and V a second time).

Decode workloads (few new queries against a long cache): the cache is
quantized once before timing (it is built at prefill); a step is quantize_q
plus the split-KV decode (chunk kernel + merge).  Its roofline is HBM: the
algorithmic bytes are the K/V codes and scales read once per query row group,
the Q codes and scales and O.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from quantized_scaled_dot_amd import synth  # noqa: E402

MFMA_PEAK_TOPS = 5000.0          # MI355X dense INT8 = dense FP8 = 5.0 P op/s
FP4_PEAK_TOPS = 10100.0          # MI355X dense FP4 (MXFP4) 10.1 P op/s
# 4-bit QK^T: half the counted ops on FP4, half (P~V) on FP8 -> 1 / (0.5/10.1 + 0.5/5.0) P op/s
QK4_PEAK_TOPS = 1.0 / (0.5 / FP4_PEAK_TOPS + 0.5 / MFMA_PEAK_TOPS)
# with Q smoothing the block mean against the INT8 K adds 2d INT8 ops (INT8 rate = FP8 rate) per
# (query, key) pair beyond the 4d counted: 4d counted ops need 2d FP4 + 4d INT8/FP8 matrix work
# -> 4 / (2/10.1 + 4/5.0) P op/s
QK4S_PEAK_TOPS = 4.0 / (2.0 / FP4_PEAK_TOPS + 4.0 / MFMA_PEAK_TOPS)
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, 8 TB/s
DEFAULT_WORKLOAD = "video-dit-32k"
METRIC = "attention TOPS (4·B·H·N²·d/t) at 1 MI355X; % of INT8/FP8 MFMA peak"
KERNEL_SOURCES = ("quantized_scaled_dot_amd/csrc/attn.hip", "quantized_scaled_dot_amd/csrc/common.h")
DECODE_SOURCES = ("quantized_scaled_dot_amd/csrc/decode.hip", "quantized_scaled_dot_amd/csrc/common.h")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _mhz_values(obj, path=""):
    """Every (key path, MHz) pair of an amd-smi / rocm-smi JSON document whose path names the
    graphics (shader) clock."""
    out = []
    if isinstance(obj, dict):
        for k, v in obj.items():
            out += _mhz_values(v, f"{path}/{k}".lower())
    elif isinstance(obj, list):
        for i, v in enumerate(obj):
            out += _mhz_values(v, f"{path}/{i}")
    else:
        comps = path.split("/")
        skip = any(x in c for c in comps for x in ("min", "max", "locked", "level", "sleep"))
        named = any("sclk" in c for c in comps) or (any("gfx" in c for c in comps) and any("clk" in c for c in comps))
        digits = "".join(ch if (ch.isdigit() or ch == ".") else " " for ch in str(obj)).split()
        if digits and named and not skip:
            try:
                out.append((path, float(digits[0])))
            except ValueError:
                pass
    return out


def read_sclk_mhz():
    """Current shader clock of GPU 0 in MHz (amd-smi, else rocm-smi), or None."""
    import subprocess
    for cmd in (["amd-smi", "metric", "-g", "0", "-c", "--json"], ["rocm-smi", "-d", "0", "--showclocks", "--json"]):
        try:
            r = subprocess.run(cmd, capture_output=True, text=True, timeout=20)
            vals = [v for p, v in _mhz_values(json.loads(r.stdout)) if 100 <= v <= 5000]
        except Exception:   # tool missing, not JSON, no such field: try the next one
            continue
        if vals:
            return max(vals)   # several XCD entries: the graphics clock is the same for all
    return None


def under_profiler():
    """True when a profiler's library is preloaded into this process (its children inherit it, so
    the clock reader, itself a script, would start with the profiler attached)."""
    return any(k.startswith(("ROCPROF", "ROCP_")) for k in os.environ) or "rocprof" in os.environ.get("LD_PRELOAD", "")


def sample_sclk(run, seconds=1.5):
    """Keep the GPU busy with run() (enqueue-only, on the bench stream) for about `seconds` while
    another thread reads the shader clock; returns {"samples", "median", "min", "max"} in MHz or None
    (also None under a profiler, where the reader is not started)."""
    if under_profiler():
        return None
    import threading
    samples, stop = [], threading.Event()

    def reader():
        while not stop.is_set():
            v = read_sclk_mhz()
            if v is None:
                return
            samples.append(v)

    th = threading.Thread(target=reader, daemon=True)
    t0 = time.perf_counter()
    th.start()
    while time.perf_counter() - t0 < seconds:
        run()
        torch.cuda.synchronize()
    stop.set()
    th.join(timeout=30)
    if not samples:
        return None
    return {"samples": len(samples), "median_mhz": float(np.median(samples)), "min_mhz": min(samples),
            "max_mhz": max(samples)}


def kernel_source_sha(sources=KERNEL_SOURCES):
    h = hashlib.sha256()
    for p in sources:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, kernel="attn_fwd_kernel", sources=KERNEL_SOURCES):
    """HBM bytes per launch of ``kernel`` from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}.{workload}.pmc.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_sha(sources):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, Q, K, V, budget_s=20.0):
    """The oracle as it stands, on the host cores: full quantization of Q, K, V,
    then attention for a bounded sample of query rows; extrapolated to the step."""
    from oracle import oracle as orc

    qb, kb, vb = synth.bits(Q), synth.bits(K), synth.bits(V)
    t0 = time.perf_counter()
    if w.qk4:
        qk = orc.quantize_qk4(qb, kb, w.dtype_code, smooth_q=w.smooth_q)
    else:
        qk = orc.quantize_qk(qb, kb, w.dtype_code, w.blk_q, w.blk_k)
    vc, vs = orc.quantize_v4(vb, w.dtype_code) if w.pv4 else orc.quantize_v(vb, w.dtype_code)
    t_quant = time.perf_counter() - t0

    def attend(rows):
        if w.pv4:
            return orc.attn_rows_fp4(qk, vc, vs, w.causal, w.sm_scale, rows=rows)
        if w.qk4:
            return orc.attn_rows_qk4(qk, vc, vs, w.causal, w.sm_scale, rows=rows)
        return orc.attn_rows(qk, vc, vs, w.blk_q, w.blk_k, w.causal, w.sm_scale, rows=rows)

    rng = np.random.default_rng(0)
    total_rows = w.B * w.H * w.N
    # calibrate with a small batch, then size the sample to the budget
    rows = rng.choice(total_rows, 64, replace=False).astype(np.int64)
    t0 = time.perf_counter()
    attend(rows)
    per_row = (time.perf_counter() - t0) / len(rows)
    n = int(max(64, min(total_rows, (budget_s - t_quant) / max(per_row, 1e-9))))
    rows = rng.choice(total_rows, n, replace=False).astype(np.int64)
    t0 = time.perf_counter()
    attend(rows)
    t_rows = time.perf_counter() - t0
    t_step = t_quant + t_rows * total_rows / n
    return {"value": round(w.ops / t_step / 1e12, 6), "unit": "TOPS", "cores": orc.num_threads(), "kind": "oracle",
            "sample": f"oracle quantization of all of Q, K, V ({t_quant:.1f} s) plus attention for {n} random query "
                      f"rows of {total_rows} ({t_rows:.1f} s), extrapolated linearly to the full step "
                      f"({t_step:.0f} s)"}


MFMA_PROBE_WG, MFMA_PROBE_ITERS = 512, 20000   # about 10 ms: 2 workgroups per CU, 2^20 ops a wave per iteration


def mfma_sustained(sage, stream, attn_tops, reps=3):
    """Sustained dense INT8/FP8 matrix rate from the library's probe (the attention kernel's
    matrix instructions per KV tile at its occupancy, and nothing else), timed with HIP events on
    the stream it runs on; the attention kernel's fraction of it; and the clock that rate implies
    at the published 5.0 P op/s for 2.4 GHz."""
    ops = 4.0 * 2 ** 20 * MFMA_PROBE_WG * MFMA_PROBE_ITERS
    ms = []
    for i in range(reps + 1):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        st = sage.sage_probe_mfma_peak(MFMA_PROBE_WG, MFMA_PROBE_ITERS, None, stream.cuda_stream)
        b.record(stream)
        if st != sage.SAGE_OK:
            raise RuntimeError(sage.sage_status_string(st))
        torch.cuda.synchronize()
        if i:   # the first launch warms up
            ms.append(a.elapsed_time(b))
    t = float(np.median(ms))
    tops = ops / (t * 1e-3) / 1e12
    return {"tops": round(tops, 1), "attn_frac": round(attn_tops / tops, 4),
            "implied_clock_ghz": round(2.4 * tops / MFMA_PEAK_TOPS, 3), "probe_ms": round(t, 3)}


HBM_PROBE_BYTES = 1 << 30   # 1 GiB, four times the last-level cache


def hbm_sustained(sage, stream, dev, reps=3):
    """Sustained HBM read bandwidth from the library's streaming-read probe (1 GiB read once per
    launch, HIP events on the probe's stream), the measured ceiling of the HBM-bound passes."""
    buf = torch.empty(HBM_PROBE_BYTES, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    sink = torch.empty(1024 * 256, dtype=torch.int32, device=dev)
    ms = []
    for i in range(reps + 1):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        st = sage.sage_probe_hbm_read(buf.data_ptr(), HBM_PROBE_BYTES, sink.data_ptr(), stream.cuda_stream)
        b.record(stream)
        if st != sage.SAGE_OK:
            raise RuntimeError(sage.sage_status_string(st))
        torch.cuda.synchronize()
        if i:   # the first launch warms up
            ms.append(a.elapsed_time(b))
    t = float(np.median(ms))
    del buf, sink
    return {"gbs": round(HBM_PROBE_BYTES / (t * 1e-3) / 1e9, 1), "probe_ms": round(t, 4), "bytes": HBM_PROBE_BYTES}


def decode_rows(w):
    return w.B * w.H * w.N


def cpu_baseline_decode(w, Q, K, V, kv_chunk, budget_s=20.0):
    """The oracle on the host cores for a decode step: quantize the new queries,
    then the split-KV attention of a bounded sample of query rows against the
    quantized cache (quantized once beforehand, as on the GPU)."""
    from oracle import oracle as orc

    qk = orc.quantize_qk(synth.bits(Q), synth.bits(K), w.dtype_code, w.blk_q, w.blk_k)
    vc, vs = orc.quantize_v(synth.bits(V), w.dtype_code)
    t0 = time.perf_counter()
    orc.quantize_q(synth.bits(Q), w.dtype_code, w.blk_q)
    t_quant = time.perf_counter() - t0
    total_rows = decode_rows(w)
    rng = np.random.default_rng(0)
    rows = rng.choice(total_rows, min(16, total_rows), replace=False).astype(np.int64)
    t0 = time.perf_counter()
    orc.attn_rows_split(qk, vc, vs, w.blk_q, w.blk_k, w.causal, w.sm_scale, kv_chunk, rows=rows)
    per_row = (time.perf_counter() - t0) / len(rows)
    n = int(max(16, min(total_rows, budget_s / max(per_row, 1e-9))))
    rows = rng.choice(total_rows, n, replace=False).astype(np.int64)
    t0 = time.perf_counter()
    orc.attn_rows_split(qk, vc, vs, w.blk_q, w.blk_k, w.causal, w.sm_scale, kv_chunk, rows=rows)
    t_rows = time.perf_counter() - t0
    t_step = t_quant + t_rows * total_rows / n
    return {"value": round(w.ops / t_step / 1e12, 6), "unit": "TOPS", "cores": orc.num_threads(), "kind": "oracle",
            "sample": f"oracle quantization of the {w.B * w.H * w.N} new queries ({t_quant:.3f} s) plus split-KV "
                      f"attention (chunks of {kv_chunk} keys) for {n} random query rows of {total_rows} "
                      f"({t_rows:.1f} s), extrapolated linearly to the full step ({t_step:.2f} s); the cache is "
                      f"quantized beforehand and not timed"}


def bench_decode(args, w, Q, K, V, Qd, Kd, Vd, sage, dev):
    B, H, N, d, Hkv, Nkv = w.B, w.H, w.N, w.d, w.Hkv, w.Nkv
    kc = sage.quantize_k(Kd, w.blk_k)
    vq = sage.quantize_v(Vd)
    chunk = sage.sage_decode_kv_chunk(B, H, Hkv, N, Nkv, d)
    ws = torch.empty(max(sage.sage_attn_decode_workspace_bytes(B, H, Hkv, N, Nkv, d, chunk), 16), dtype=torch.uint8,
                     device=dev)
    out = torch.empty((B, H, N, d), dtype=w.torch_dtype, device=dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        q = sage.quantize_q(Qd, w.blk_q)
        if ev is not None:
            ev[0].record(stream)
        sage.attn_decode(q, kc, vq, causal=w.causal, sm_scale=w.sm_scale, out=out, kv_chunk=chunk, workspace=ws)
        if ev is not None:
            ev[1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(2)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t = time.perf_counter() - t0
    dec_ms = [e[0].elapsed_time(e[1]) for e in evs]
    ms_step = t * 1e3 / args.steps
    peak_mem = torch.cuda.max_memory_allocated(dev)
    dec_mean = float(np.mean(dec_ms))
    dec_avg = float(np.median(dec_ms))   # the p50 is the headline decode time
    value = w.ops / (ms_step * 1e-3) / 1e12
    # algorithmic bytes of one decode call: every K/V code and scale once per group of 32 query rows
    # of a K/V head, the Q codes and scales, O
    groups = -(-(H // Hkv) * N // 32)
    nkt = -(-Nkv // 64)
    kv_bytes = B * Hkv * groups * (2 * nkt * 64 * d + nkt * 64 // w.blk_k * 4 + d * 4)
    q_bytes = B * H * N * d + B * H * -(-N // w.blk_q) * 4
    o_bytes = B * H * N * d * torch.tensor([], dtype=w.torch_dtype).element_size()
    alg = kv_bytes + q_bytes + o_bytes
    gbs = alg / (dec_mean * 1e-3) / 1e9   # roofline: the average launch duration
    log(f"[bench] decode step {ms_step:.3f} ms; decode call p50 {dec_avg:.4f} ms mean {dec_mean:.4f} "
        f"p95 {np.percentile(dec_ms, 95):.4f}: {gbs:.0f} GB/s of {alg / 1e6:.1f} MB algorithmic "
        f"({100 * gbs / HBM_PEAK_GBS:.1f}% of 8 TB/s); split {chunk} keys; peak allocated "
        f"{peak_mem / 2 ** 20:.0f} MiB")
    q_keep = sage.quantize_q(Qd, w.blk_q)
    sclk = sample_sclk(lambda: sage.attn_decode(q_keep, kc, vq, causal=w.causal, sm_scale=w.sm_scale, out=out,
                                                kv_chunk=chunk, workspace=ws))
    log(f"[bench] shader clock while the decode kernels run: {sclk}")
    hbm = hbm_sustained(sage, stream, dev)
    log(f"[bench] HBM read probe: {hbm['gbs']:.0f} GB/s sustained; decode at {100 * gbs / hbm['gbs']:.1f}% of it")
    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] CPU oracle baseline (~{args.cpu_budget:.0f} s)...")
        cpu = cpu_baseline_decode(w, Q, K, V, chunk, budget_s=args.cpu_budget)
        log(f"[bench] CPU oracle: {cpu}")
    line = {
        "metric": METRIC, "value": round(value, 4), "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int8+fp8 (fp32 softmax)", "data": "synthetic",
        "config": {"workload": w.name, "B": B, "H": H, "N": N, "Hkv": Hkv, "Nkv": Nkv, "d": d, "causal": w.causal,
                   "in_dtype": w.dtype, "blk_q": w.blk_q, "blk_k": w.blk_k, "kv_chunk": chunk,
                   "parallelism": "none (1 GPU)"},
        "decode_ms": round(dec_avg, 5),
        "decode_ms_p50": round(dec_avg, 5),
        "decode_ms_mean": round(dec_mean, 5),
        "decode_ms_p95": round(float(np.percentile(dec_ms, 95)), 5),
        "peak_allocated_bytes": int(peak_mem),
        "sclk_during_decode": sclk,
        "roofline": {"bound": "hbm", "kernel": "decode_chunk_kernel + decode_merge_kernel", "achieved": round(gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(w.name, "decode_chunk_kernel", DECODE_SOURCES),
                     "frac_of_hbm_read_probe": round(gbs / hbm["gbs"], 4)},
        "hbm_read_sustained": hbm,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=list(synth.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle work for the CPU baseline")
    ap.add_argument("--pmc-calibration", action="store_true",
                    help="run one plain 256 MiB device copy first (scale reference for HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the path shards over (batch, head) with no "
              "communication, and this benchmark runs and reports the single-GPU share.", file=sys.stderr)
        sys.exit(2)

    from quantized_scaled_dot_amd import sage

    w = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    log(f"[bench] workload {w.name}: B={w.B} H={w.H} N={w.N} Hkv={w.Hkv} Nkv={w.Nkv} d={w.d} {w.dtype} "
        f"causal={w.causal}")
    Q, K, V = synth.make_inputs(w)
    Qd, Kd, Vd = Q.to(dev), K.to(dev), V.to(dev)
    if args.pmc_calibration:
        src = torch.empty(64 << 20, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] calibration copy: 268435456 bytes read, 268435456 bytes written")

    if w.decode:
        bench_decode(args, w, Q, K, V, Qd, Kd, Vd, sage, dev)
        return
    B, H, N, d, Hkv, Nkv = w.B, w.H, w.N, w.d, w.Hkv, w.Nkv
    ws_qk = torch.empty(max(sage.sage_quantize_qk_workspace_bytes(B, Hkv, Nkv, d), 16), dtype=torch.uint8, device=dev)
    ws_v = torch.empty(max(sage.sage_quantize_v_workspace_bytes(B, Hkv, Nkv, d), 16), dtype=torch.uint8, device=dev)
    ws_qkv = torch.empty(max(sage.sage_quantize_qkv_workspace_bytes(B, Hkv, Nkv, d), 16), dtype=torch.uint8, device=dev)
    out = torch.empty((B, H, N, d), dtype=w.torch_dtype, device=dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[2].record(stream)
        if w.qk4:
            q = sage.quantize_qk4(Qd, Kd, workspace=ws_qk, smooth_q=w.smooth_q)
            v = sage.quantize_v4(Vd) if w.pv4 else sage.quantize_v(Vd, workspace=ws_v)
        else:   # quantize_qk + quantize_v in one call (three launches)
            q, v = sage.quantize_qkv(Qd, Kd, Vd, w.blk_q, w.blk_k, workspace=ws_qkv)
        if ev is not None:
            ev[0].record(stream)
        if w.pv4:
            sage.attn_fwd_fp4(q, v, causal=w.causal, sm_scale=w.sm_scale, out=out)
        elif w.qk4:
            sage.attn_fwd_qk4(q, v, causal=w.causal, sm_scale=w.sm_scale, out=out)
        else:
            sage.attn_fwd(q, v, causal=w.causal, sm_scale=w.sm_scale, out=out)
        if ev is not None:
            ev[1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t = time.perf_counter() - t0
    attn_ms = [e[0].elapsed_time(e[1]) for e in evs]
    quant_ms = [e[2].elapsed_time(e[0]) for e in evs]
    ms_step = t * 1e3 / args.steps
    peak_mem = torch.cuda.max_memory_allocated(dev)
    attn_avg = float(np.mean(attn_ms))
    attn_p50 = float(np.median(attn_ms))
    attn_p95 = float(np.percentile(attn_ms, 95))
    value = w.ops / (ms_step * 1e-3) / 1e12
    attn_tops = w.ops / (attn_avg * 1e-3) / 1e12       # roofline: the average launch duration
    attn_tops_p50 = w.ops / (attn_p50 * 1e-3) / 1e12
    peak = (FP4_PEAK_TOPS if w.pv4 else QK4S_PEAK_TOPS if w.smooth_q else QK4_PEAK_TOPS) if w.qk4 else MFMA_PEAK_TOPS
    log(f"[bench] step {ms_step:.3f} ms ({value:.1f} TOPS); attention kernel p50 {attn_p50:.3f} ms "
        f"mean {attn_avg:.3f} p95 {attn_p95:.3f} ({attn_tops_p50:.1f} TOPS at p50, {attn_tops:.1f} at the mean: "
        f"{100 * attn_tops / peak:.1f}% of peak {peak:.0f}); peak allocated {peak_mem / 2 ** 20:.0f} MiB")

    q_el, kv_el = B * H * N * d, B * Hkv * Nkv * d
    if w.qk4:   # Q and K: 2-byte inputs, half-byte codes plus a byte per 32; V as below (FP4 V: like Q and K)
        quant_alg = (q_el + kv_el) * (2 + 0.5 + 1 / 32) + (kv_el * (2 + 0.5 + 1 / 32) if w.pv4 else 3 * kv_el)
        if w.smooth_q:   # K also in INT8 (a byte per value; one exponent byte per 64 keys)
            quant_alg += kv_el * (1 + 1 / (64 * d))
    else:
        quant_alg = 3 * (q_el + 2 * kv_el)  # Q, K, V: read 2-byte inputs, write 1-byte codes
    quant_act = quant_alg + (2 if w.pv4 else 2 * 2) * kv_el   # the K-sum (and V-max) passes read K (and V) once more
    if w.smooth_q:
        quant_act += 2 * q_el + 2 * kv_el   # the block-mean pass reads Q, the INT8 K pass K once more
    quant_avg = float(np.mean(quant_ms))
    quant_gbs = quant_alg / (quant_avg * 1e-3) / 1e9
    log(f"[bench] quantize passes avg {quant_avg:.3f} ms: {quant_gbs:.0f} GB/s algorithmic "
        f"({100 * quant_gbs / HBM_PEAK_GBS:.1f}% of 8 TB/s), {quant_act / (quant_avg * 1e-3) / 1e9:.0f} GB/s moved")

    def attn_only():
        if w.pv4:
            sage.attn_fwd_fp4(q_keep[0], q_keep[1], causal=w.causal, sm_scale=w.sm_scale, out=out)
        elif w.qk4:
            sage.attn_fwd_qk4(q_keep[0], q_keep[1], causal=w.causal, sm_scale=w.sm_scale, out=out)
        else:
            sage.attn_fwd(q_keep[0], q_keep[1], causal=w.causal, sm_scale=w.sm_scale, out=out)

    q_keep = ((sage.quantize_qk4(Qd, Kd, workspace=ws_qk, smooth_q=w.smooth_q),
               sage.quantize_v4(Vd) if w.pv4 else sage.quantize_v(Vd, workspace=ws_v))
              if w.qk4 else sage.quantize_qkv(Qd, Kd, Vd, w.blk_q, w.blk_k, workspace=ws_qkv))
    sclk = sample_sclk(attn_only)
    log(f"[bench] shader clock while the attention kernel runs: {sclk}")

    hbm = hbm_sustained(sage, stream, dev)
    log(f"[bench] HBM read probe: {hbm['gbs']:.0f} GB/s sustained; quantize passes at "
        f"{100 * quant_gbs / hbm['gbs']:.1f}% of it (algorithmic bytes)")

    sustained = None
    if not w.qk4:
        sustained = mfma_sustained(sage, stream, attn_tops)
        log(f"[bench] matrix-core probe: {sustained['tops']:.1f} TOPS sustained (implied clock "
            f"{sustained['implied_clock_ghz']:.2f} GHz); attention kernel at {100 * sustained['attn_frac']:.1f}% of it")

    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] CPU oracle baseline (~{args.cpu_budget:.0f} s)...")
        cpu = cpu_baseline(w, Q, K, V, budget_s=args.cpu_budget)
        log(f"[bench] CPU oracle: {cpu}")

    line = {
        "metric": METRIC, "value": round(value, 3), "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": ("fp4 (fp32 softmax)" if w.pv4 else "int8+fp4+fp8 (fp32 softmax)" if w.smooth_q
                                           else "fp4+fp8 (fp32 softmax)") if w.qk4 else "int8+fp8 (fp32 softmax)",
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "H": H, "N": N, "Hkv": Hkv, "Nkv": Nkv, "d": d, "causal": w.causal,
                   "in_dtype": w.dtype,
                   "blk_q": w.blk_q, "blk_k": w.blk_k, "kv_tile": sage.sage_kv_tile(), "parallelism": "none (1 GPU)"},
        "attn_kernel_ms": round(attn_p50, 4),
        "attn_kernel_ms_p50": round(attn_p50, 4),
        "attn_kernel_ms_mean": round(attn_avg, 4),
        "attn_kernel_ms_p95": round(attn_p95, 4),
        "attn_tops": round(attn_tops_p50, 3),
        "attn_tops_mean": round(attn_tops, 3),
        "peak_allocated_bytes": int(peak_mem),
        "sclk_during_attention": sclk,
        "frac_of_mfma_peak_step": round(value / peak, 4),
        "roofline": {"bound": "mfma", "kernel": "attn_fwd_kernel", "achieved": round(attn_tops, 3),
                     "peak": round(peak, 1), "unit": "TFLOP/s", "frac": round(attn_tops / peak, 4),
                     "traffic": measured_traffic(w.name)},
        "quantize": {"ms": round(quant_avg, 4), "bound": "hbm", "algorithmic_bytes": quant_alg,
                     "bytes_moved": quant_act, "achieved": round(quant_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(quant_gbs / HBM_PEAK_GBS, 4), "frac_of_hbm_read_probe": round(quant_gbs / hbm["gbs"], 4)},
        "mfma_sustained": sustained,
        "hbm_read_sustained": hbm,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
