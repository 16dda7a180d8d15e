"""Mutation check of the oracle's pins (CPU only).

Each mutant below is a copy of the oracle's C source with one plausible
mistake planted in it: a wrong rounding or tie rule, an off-by-one exponent,
a dropped term, a flipped sign, a wrong index, a missing rescale.  Every copy
is compiled with the oracle's own flags and the pin suite
(``test_oracle_pins.py``) is run against it in a subprocess; the pins must fail
on every mutant.  A mutant that survives names a property of the method that
no pin fixes.  The unmodified source, built the same way, must pass, so a
failure is the mutant's and not the harness's.

Not mutated: choices the pages leave open, where either option meets every
property they fix, so no pin can or should tell them apart.  Two of them:
truncating rather than rounding each element to the 2^-24 grid of the
fixed-point K mean (both give the mean to 2^-24 per element), and flushing an
INT8 block to zero below a maximum of 2^-120 rather than only at zero (a guard
that keeps 127/max finite; the scores of such a block are below any error
bound).  Each is one reading, and the HIP path matches it bit for bit.

The mistakes are planted in the oracle only, never in the HIP path.
"""
import concurrent.futures as cf
import os
import subprocess
import sys
import tempfile

import pytest

from oracle import build as obuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (name, text in the oracle source, replacement, occurrences replaced).
# Each text must occur exactly `count` times, so that a change to the oracle
# that moves a site shows up here instead of silently testing nothing.
MUTANTS = [
    # FP8 e4m3 codec
    ("e4m3 ties away from zero", "double r = rint(ldexp(a, 3 - k));",
     "double r = floor(ldexp(a, 3 - k) + 0.5);", 1),
    ("e4m3 saturates late", "if (a >= 448.0) return sign | 0x7E;", "if (a >= 480.0) return sign | 0x7E;", 1),
    ("e4m3 subnormal step 2^-8", "double r = rint(a * 512.0);", "double r = rint(a * 256.0);", 1),
    ("e4m3 decode exponent bias", "else v = ldexp(8.0 + m, e - 10);", "else v = ldexp(8.0 + m, e - 11);", 1),
    # exp2 of the softmax
    ("exp instead of exp2", "return (float)exp2((double)t);", "return (float)exp((double)t);", 1),
    # E2M1 and its blocks
    ("e2m1 ties to the odd code", "(dk == db && (k & 1) == 0)", "(dk == db && (k & 1) == 1)", 1),
    ("mx4 block exponent off by one", "int e = (int)floor(log2((double)a)) - 2;",
     "int e = (int)floor(log2((double)a)) - 1;", 1),
    ("int8 power-of-two exponent one too large", "e = ilogb((double)a) - 6;", "e = ilogb((double)a) - 5;", 1),
    ("int8 power-of-two exponent not raised past 127", "if (ldexp((double)a, -e) > 127.0) e += 1;", "", 1),
    ("int8 power-of-two codes truncated", "double y = nearbyint(ldexp((double)x[k], -e));",
     "double y = trunc(ldexp((double)x[k], -e));", 1),
    # K smoothing
    ("k mean clamp 2^20 overflows int64 at the length limit", "KMEAN_CLAMP = 524288.0;",
     "KMEAN_CLAMP = 1048576.0;", 1),
    ("k mean divides by N+1", "mu[c] = (float)(((double)s * 0x1p-24) / (double)N);",
     "mu[c] = (float)(((double)s * 0x1p-24) / (double)(N + 1));", 1),
    ("k mean added, not subtracted", "buf[(size_t)t * d + c] = load_in(Kh, idx, dtype) - mu[c];",
     "buf[(size_t)t * d + c] = load_in(Kh, idx, dtype) + mu[c];", 1),
    ("4-bit K not smoothed", "- mu[32 * b + k];\n        quant_block_mx4(",
     ";\n        quant_block_mx4(", 1),
    ("INT8 K of the mean term not smoothed", "load_in(K, ((size_t)bh * N + n0 + i) * d + c, dtype) - mu[c];",
     "load_in(K, ((size_t)bh * N + n0 + i) * d + c, dtype);", 1),
    # INT8 block quantizer
    ("int8 scale over 128", "float dl = a / 127.0f;", "float dl = a / 128.0f;", 1),
    ("int8 codes truncated", "float y = rintf(x[k] * r);", "float y = truncf(x[k] * r);", 1),
    # V per-channel FP8 quantizer
    ("v scale over 447", "dl = a / 448.0f; r = 448.0f / a;", "dl = a / 447.0f; r = 448.0f / a;", 1),
    ("v scale of channel 0 everywhere", "(double)v_scale[(size_t)bk * d + c]",
     "(double)v_scale[(size_t)bk * d]", 2),
    # Q smoothing
    ("q block mean over 32 in a ragged block", "qm[c] = (float)(sum / n);", "qm[c] = (float)(sum / 32);", 1),
    ("q mean added, not subtracted", "load_in(Q, r * d + 32 * b + k, dtype) - qm[32 * b + k];",
     "load_in(Q, r * d + 32 * b + k, dtype) + qm[32 * b + k];", 1),
    # scores
    ("int8 dot drops the last channel", "for (int c = 0; c < d; c++) s += (int32_t)x->q[c] * (int32_t)k[c];",
     "for (int c = 0; c < d - 1; c++) s += (int32_t)x->q[c] * (int32_t)k[c];", 1),
    ("4-bit block scale off by one", "s += ldexp(blk, (int)x->q4s[b] + (int)ks[b] - 254);",
     "s += ldexp(blk, (int)x->q4s[b] + (int)ks[b] - 253);", 1),
    ("q-mean term scale off by one", "s += ldexp((double)dot, x->qms + (int)x->k8s[j / 64] - 254);",
     "s += ldexp((double)dot, x->qms + (int)x->k8s[j / 64] - 255);", 1),
    ("q-mean term dropped", "s += ldexp((double)dot, x->qms + (int)x->k8s[j / 64] - 254);",
     "s += 0.0 * ldexp((double)dot, x->qms + (int)x->k8s[j / 64] - 254);", 1),
    ("q-mean term with the K block of the previous key", "(int)x->k8s[j / 64]", "(int)x->k8s[j > 0 ? (j - 1) / 64 : 0]",
     1),
    ("q-mean term drops the last channel", "for (int c = 0; c < d; c++) dot += (int64_t)x->qm[c] * (int64_t)k8[c];",
     "for (int c = 0; c < d - 1; c++) dot += (int64_t)x->qm[c] * (int64_t)k8[c];", 1),
    ("k block scale of the previous key", "c2[jj] = (x->dq * x->ks[j / x->blk_k]) * x->s2;",
     "c2[jj] = (x->dq * x->ks[(j > 0 ? j - 1 : 0) / x->blk_k]) * x->s2;", 1),
    ("q block scale of the previous row", "x->dq = q_scale[(size_t)bh * nbq + i / blk_q];",
     "x->dq = q_scale[(size_t)bh * nbq + (i > 0 ? i - 1 : 0) / blk_q];", 1),
    ("softmax scale without log2 e", "x->s2 = sm_scale * LOG2E_F;", "x->s2 = sm_scale;", 1),
    # heads and masks
    ("grouped heads interleaved", "return (bh / Hq) * Hkv + (bh % Hq) / (Hq / Hkv);",
     "return (bh / Hq) * Hkv + (bh % Hq) % Hkv;", 1),
    ("causal mask aligned top-left", "x->last = causal ? i + ((int64_t)Nkv - Nq) : (int64_t)Nkv - 1;",
     "x->last = causal ? i : (int64_t)Nkv - 1;", 1),
    ("causal mask ignored inside a tile", "if (x->last - j0 + 1 < nvis) nvis = (int)(x->last - j0 + 1);",
     "", 1),
    # online softmax
    ("alpha with the sign flipped", "float alpha = first ? 0.0f : oracle_exp2f(m - mnew);",
     "float alpha = first ? 0.0f : oracle_exp2f(mnew - m);", 1),
    ("row sum not rescaled", "l = fmaf(alpha, l, rowsum);", "l = l + rowsum;", 1),
    ("accumulator not rescaled", "oacc[c] = fmaf(alpha, oacc[c], (float)oblk[c]);",
     "oacc[c] = oacc[c] + (float)oblk[c];", 1),
    ("P~ without the 2^8 headroom", "float mm = mnew - 8.0f;", "float mm = mnew;", 1),
    ("INT8 row sum over the fp32 P~, not the FP8 codes", "if (!x->q4) rowsum = (float)code_sum;",
     "if (!x->q4) { rowsum = 0.0f; for (int jj = 0; jj < nvis; jj++) rowsum += pt[jj]; }", 1),
    ("INT8 row sum of the first half of the keys", "if (!x->q4) rowsum = (float)code_sum;",
     "if (!x->q4) { double h = 0; for (int jj = 0; jj < nvis / 2; jj++) h += x->vdec[ph[jj]]; rowsum = (float)h; }",
     1),
    ("INT8 exponent offset without the score bias", "const float K = fmaf(SCORE_BIAS, c2[jj], mm);",
     "const float K = mm;", 1),
    ("INT8 exponent argument without the score bias", "fmaf(SCORE_BIAS + S[jj], c2[jj], -K)",
     "fmaf(S[jj], c2[jj], -K)", 1),
    # split-KV merge
    ("split merge weight inverted", "const float w = oracle_exp2f(mc[c] - mstar);",
     "const float w = oracle_exp2f(mstar - mc[c]);", 1),
    # second batch: subtler slips
    ("K read transposed", "s += (int32_t)x->q[c] * (int32_t)k[c];",
     "s += (int32_t)x->q[c] * (int32_t)x->k[(size_t)c * x->Nkv + j];", 1),
    ("V of the first head for every head", "x->v = v_codes + (size_t)bk * Nkv * d;", "x->v = v_codes;", 1),
    ("running max never raised", "float mnew = first ? mt : (mt > m ? mt : m);",
     "float mnew = first ? mt : m;", 1),
    ("normalizer off by 0.1%", "(double)v_scale[(size_t)bk * d + c]) / (double)l);",
     "(double)v_scale[(size_t)bk * d + c]) / ((double)l * 1.001));", 2),
    ("e2m1 decode drops the sign", "return (c & 8) ? -m : m;", "return m;", 1),
    ("e2m1 without the magnitude 6", "for (int k = 1; k < 8; k++) {", "for (int k = 1; k < 7; k++) {", 1),
    ("P~ not quantized to FP8", "acc += x->vdec[ph[jj]] * x->vdec[",
     "acc += (double)pt[jj] * x->vdec[", 1),
    # third batch: split merge, block edge cases, Q-smoothing blocks
    ("split merge: row sums not weighted", "L = fmaf(w, lc[c], L);", "L = L + lc[c];", 1),
    ("split merge: chunks without a visible key kept", "      if (!vis[c]) continue;\n", "", 1),
    ("all-zero MX blocks get scale byte 127", "    *scale = 0;\n", "    *scale = 127;\n", 1),
    # FP4 P~V
    ("FP4 P~ block exponent one too large", "float fe = floorf(amax) - 2.0f;", "float fe = floorf(amax) - 1.0f;", 1),
    ("FP4 P~ blocks of 64 keys", "for (int b0 = 0; b0 < nvis; b0 += 32) {\n        const int b1 = b0 + 32 < nvis ? b0 + 32 : nvis;",
     "for (int b0 = 0; b0 < nvis; b0 += 64) {\n        const int b1 = b0 + 64 < nvis ? b0 + 64 : nvis;", 1),
    ("FP4 P~ not quantized", "pd[jj] = ldexp(oracle_e2m1_decode(ph[jj]), e);", "pd[jj] = p;", 1),
    ("FP4 row sum of the unquantized P~", "          code_sum += pd[jj];\n", "          code_sum += p;\n", 1),
    ("FP4 V scale of the previous key's block", "(int)x->v4s[(size_t)(j / 32) * d + c] - 127",
     "(int)x->v4s[(size_t)((j > 0 ? j - 1 : 0) / 32) * d + c] - 127", 1),
    ("FP4 V scale off by one", "(int)x->v4s[(size_t)(j / 32) * d + c] - 127", "(int)x->v4s[(size_t)(j / 32) * d + c] - 126", 1),
    ("Q-smoothing blocks of 16 rows", "const int n0 = 32 * blk, n = (N - n0 < 32) ? N - n0 : 32;\n      float* qm",
     "const int n0 = 16 * blk, n = (N - n0 < 16) ? N - n0 : 16;\n      float* qm", 1),
]

PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")


def _mutate(src, old, new, count):
    n = src.count(old)
    if n != count:
        raise AssertionError(f"site {old!r} occurs {n} times in the oracle, expected {count}")
    return src.replace(old, new)


def _run_pins(lib):
    env = dict(os.environ, SAGE_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    cmd = [sys.executable, "-m", "pytest", PINS, "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu"]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr).strip().splitlines()[-3:]
    return r.returncode, "\n".join(tail)


def _build_and_run(tmp, idx, src):
    path = os.path.join(tmp, f"m{idx}.c")
    with open(path, "w") as f:
        f.write(src)
    lib = os.path.join(tmp, f"libm{idx}.so")
    try:
        obuild.build(src=path, out=lib)
    except subprocess.CalledProcessError as e:
        return ("compile", str(e))
    return _run_pins(lib)


@pytest.fixture(scope="module")
def outcomes():
    with open(obuild.SRC) as f:
        src = f.read()
    sources = [src] + [_mutate(src, old, new, n) for _, old, new, n in MUTANTS]
    with tempfile.TemporaryDirectory() as tmp, cf.ThreadPoolExecutor(4) as pool:
        futs = [pool.submit(_build_and_run, tmp, i, s) for i, s in enumerate(sources)]
        res = [f.result() for f in futs]
    return res


def test_unmodified_oracle_passes_the_pins(outcomes):
    rc, tail = outcomes[0]
    assert rc == 0, f"the pins fail on the unmodified oracle built in isolation:\n{tail}"


@pytest.mark.parametrize("k", range(len(MUTANTS)), ids=[m[0] for m in MUTANTS])
def test_pins_kill_the_mutant(outcomes, k):
    rc, tail = outcomes[k + 1]
    assert rc != "compile", f"mutant did not compile: {tail}"
    assert rc != 0, f"mutant '{MUTANTS[k][0]}' survives the pin suite:\n{tail}"
