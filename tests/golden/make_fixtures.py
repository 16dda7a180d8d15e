"""Writes tests/golden/*.txt from the oracle alone (test infrastructure).

The pages print no worked numeric example of the method (they hold abstracts, a
product card and a blog summary), so no fixture can carry the pages' own values.
These files are snapshots of the oracle on small seeded inputs: a change to the
oracle's arithmetic shows up as a diff here and has to be made on purpose (run
this script and commit the result).  They are not pins; the pins are in
tests/test_oracle_pins.py.  The HIP path is compared with them on the GPU.

Usage: python tests/golden/make_fixtures.py
"""
import hashlib
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from oracle import oracle as orc  # noqa: E402
from quantized_scaled_dot_amd import synth  # noqa: E402

# (fixture name, workload, overrides, sampled flat query rows)
CASES = [
    ("tiny-causal-f16", "tiny-f16-256", dict(causal=True), [0, 1, 63, 64, 200, 255, 256, 511]),
    ("tiny-gqa-ragged-bf16", "llm-prefill-4k-causal",
     dict(B=1, H=4, Hkv_=2, N=100, Nkv_=150, d=64, blk_q=32, blk_k=16), [0, 1, 50, 99, 100, 250, 399]),
]


def workload(name, base, kw):
    return synth.WORKLOADS[base].with_(name=name, **kw)


def compute(w, rows):
    """The oracle's quantization and attention rows for workload w (seed of the workload)."""
    Q, K, V = synth.make_inputs(w)
    qb, kb, vb = synth.bits(Q), synth.bits(K), synth.bits(V)
    qk = orc.quantize_qk(qb, kb, w.dtype_code, w.blk_q, w.blk_k)
    vc, vs = orc.quantize_v(vb, w.dtype_code)
    O = orc.attn_rows(qk, vc, vs, w.blk_q, w.blk_k, w.causal, w.sm_scale, rows=np.asarray(rows, np.int64))
    return {"q_codes": qk["q_codes"], "k_codes": qk["k_codes"], "v_codes": vc, "q_scale": qk["q_scale"],
            "k_scale": qk["k_scale"], "k_mean": qk["k_mean"], "v_scale": vs, "O": O}


def digest(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def hexf(a):
    return " ".join(float(x).hex() for x in np.asarray(a, np.float32).ravel())


def render(name, w, rows, r):
    out = [f"# oracle snapshot '{name}': workload {w.name} B={w.B} Hq={w.H} Hkv={w.Hkv} Nq={w.N} Nkv={w.Nkv} "
           f"d={w.d} {w.dtype} causal={w.causal} blk_q={w.blk_q} blk_k={w.blk_k} seed={w.seed}",
           "# written by tests/golden/make_fixtures.py from oracle.quantize_qk, quantize_v and attn_rows;",
           "# code arrays as sha256 of their bytes, fp32 values as exact hex floats",
           f"rows {' '.join(str(int(x)) for x in rows)}"]
    for key in ("q_codes", "k_codes", "v_codes"):
        out.append(f"{key} {r[key].shape} {digest(r[key])}".replace(", ", ","))
    for key in ("q_scale", "k_scale", "k_mean", "v_scale"):
        out.append(f"{key} {hexf(r[key])}")
    for i, row in enumerate(r["O"]):
        out.append(f"O[{int(rows[i])}] {hexf(row)}")
    return "\n".join(out) + "\n"


def main():
    for name, base, kw, rows in CASES:
        w = workload(name, base, kw)
        path = os.path.join(HERE, name + ".txt")
        with open(path, "w") as f:
            f.write(render(name, w, rows, compute(w, rows)))
        print("wrote", path)


if __name__ == "__main__":
    main()
