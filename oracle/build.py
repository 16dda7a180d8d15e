"""Build the CPU oracle shared library (test infrastructure only).

Compiles ``sage_oracle.c`` with gcc: ``-O2 -fopenmp -ffp-contract=off`` and no
``-ffast-math``, so every fp32 operation is a single IEEE round-to-nearest-even
step and the only fused multiply-adds are the explicit ``fmaf`` calls.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "sage_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False, src: str = SRC, out: str = LIB, extra=()) -> str:
    """Compile ``src`` into the shared library ``out`` (atomically replaced); ``extra``
    flags are appended (the sanitizer build of the tests uses them)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-Wall", "-Wextra", *extra, "-o", out + ".tmp", src, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
