"""Build libsage.so (the gfx950 HIP kernels and their C ABI) in-tree with hipcc.

Each source is compiled to an object with the common flags plus its own (the
attention source once per part of its kernel instances), in parallel, then the
objects are linked into one shared library.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libsage.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # every fp32 operation rounds on its own: only explicit fma() calls fuse
    "-ffp-contract=off",
    # packed-fp32 VALU instructions stay disabled
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mcode-object-version=5",
    "-I", os.path.join(ROOT, "include"),
]
# The attention kernel never produces or tests NaNs (inputs are finite by
# contract); not honouring them lets floor+convert fuse into v_cvt_flr_i32_f32.
# The host-side argument checks in api.hip do rely on NaN semantics.
SOURCES = {"quant.hip": [], "attn.hip": ["-fno-honor-nans"], "decode.hip": ["-fno-honor-nans"], "api.hip": [],
           "peak.hip": []}
# the attention kernel instances are split into this many compile units (SAGE_ATTN_PART in attn.hip)
ATTN_PARTS = 8
NOISE = "is not a recognized feature for this target"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if NOISE not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if verbose and err.strip():
        print(err, file=sys.stderr)


def _jobs():
    jobs = []
    for src, flags in SOURCES.items():
        if src == "attn.hip":
            for p in range(ATTN_PARTS):
                jobs.append((src, [*flags, f"-DSAGE_ATTN_PART={p}"], f"attn_p{p}.o"))
        else:
            jobs.append((src, flags, src.replace(".hip", ".o")))
    return jobs


def build(verbose: bool = False, extra=(), workers: int = 0) -> str:
    os.makedirs(OBJ, exist_ok=True)
    jobs = _jobs()
    cmds = [[HIPCC, *COMMON, *flags, *extra, "-c", os.path.join(CSRC, src), "-o", os.path.join(OBJ, obj)]
            for src, flags, obj in jobs]
    workers = workers or min(len(cmds), os.cpu_count() or 1, 16)
    with ThreadPoolExecutor(max_workers=workers) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    objs = [os.path.join(OBJ, obj) for _, _, obj in jobs]
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", LIB + ".tmp"], verbose)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True, extra=sys.argv[1:]))
