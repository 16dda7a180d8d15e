"""Build libsage.so (the gfx950 HIP kernels and their C ABI) in-tree with hipcc."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsage.so")
SOURCES = ["quant.hip", "attn.hip", "api.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # every fp32 operation rounds on its own: only explicit fma() calls fuse
    "-ffp-contract=off",
    # packed-fp32 VALU instructions stay disabled
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mcode-object-version=5",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False, extra=()) -> str:
    cmd = [HIPCC, *FLAGS, *extra, *[os.path.join(CSRC, s) for s in SOURCES], "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True, extra=sys.argv[1:]))
