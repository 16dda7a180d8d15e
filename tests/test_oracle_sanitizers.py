"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The oracle's C source is built with ``-fsanitize=address,undefined`` (plus
float-to-integer conversion overflow, which ``undefined`` leaves out in gcc) and
no recovery, and the whole pin suite runs against that build in a subprocess
with the ASan runtime preloaded: any out-of-bounds access, use after free,
signed overflow, misaligned access or overflowing conversion aborts the run.
A copy of the source with the K mean's fixed-point clamp raised back to 2^20
(whose sum overflows int64 at the length limit with saturated channels) must
be caught, so that a clean run is known to mean something.
"""
import os
import subprocess
import sys
import tempfile

import pytest

from oracle import build as obuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined,float-cast-overflow",
       "-fno-sanitize-recover=all"]


def _asan_runtime():
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def _run_pins(lib, select=None):
    env = dict(os.environ, SAGE_ORACLE_LIB=lib, OMP_NUM_THREADS="4", LD_PRELOAD=_asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    # -s: the sanitizer's report goes straight to the captured stderr of this subprocess
    cmd = [sys.executable, "-m", "pytest", PINS, "-x", "-q", "-s", "-p", "no:cacheprovider", "-m", "not gpu"]
    if select:
        cmd += ["-k", select]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    return r.returncode, r.stdout + r.stderr


pytestmark = pytest.mark.skipif(_asan_runtime() is None, reason="gcc's AddressSanitizer runtime is not installed")


@pytest.fixture(scope="module")
def tmp():
    with tempfile.TemporaryDirectory() as d:
        yield d


def test_pin_suite_runs_clean_under_asan_and_ubsan(tmp):
    lib = obuild.build(out=os.path.join(tmp, "liboracle_san.so"), extra=SAN)
    rc, out = _run_pins(lib)
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-3000:]
    assert rc == 0, out[-3000:]


def test_the_sanitizer_build_catches_an_overflowing_k_mean_clamp(tmp):
    with open(obuild.SRC) as f:
        src = f.read()
    old = "static const double KMEAN_CLAMP = 524288.0;"
    assert src.count(old) == 1
    path = os.path.join(tmp, "clamp20.c")
    with open(path, "w") as f:
        f.write(src.replace(old, "static const double KMEAN_CLAMP = 1048576.0;"))
    lib = obuild.build(src=path, out=os.path.join(tmp, "libclamp20_san.so"), extra=SAN)
    rc, out = _run_pins(lib, select="length_limit")
    assert rc != 0 and "signed integer overflow" in out, out[-3000:]
