"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.

Bar: bit-exact K means, INT8 Q/K codes and scales, FP8 V codes and scales
and int32 QK^T tiles; fp32 O within max-abs 2e-3 of the oracle (only the
single heads at the 2^19-token length limit take max(2e-3, INNER_REL * A) per
element, for the FP8 instruction's inner sum window; see INNER_REL); cosine
similarity to fp64 exact attention >= 0.995.  FP8 codes of P~: the kernel's
exp2 is the hardware fp32 exp2 (within one ulp; the oracle rounds the exact
value once), so a code may differ by one e4m3 step where P~ lies within an ulp
of a rounding tie: at most P_FLIP_FRAC of the visible codes, all others equal.
"""
import os

import numpy as np
import pytest
import torch

from oracle import oracle as orc
from quantized_scaled_dot_amd import synth

pytestmark = pytest.mark.gpu

O_TOL = 2e-3
P_FLIP_FRAC = 1e-4
S_SENTINEL = np.iinfo(np.int32).min
P_SENTINEL = 0x7F


def _sage():
    from quantized_scaled_dot_amd import sage
    return sage


def run_gpu(w, Q, K, V, out_dtype=torch.float32, dump_tiles=(), check_runtime=True, layout="bhnd"):
    """Q [B,H,N,d], K/V [B,Hkv,Nkv,d] through the C ABI; with layout="bnhd" the
    device inputs are [B,N,H,d] copies and O comes back [B,N,H,d].  res["O"]
    is always [B,H,N,d]."""
    sage = _sage()
    if check_runtime:
        assert len(sage.loaded_hip_runtimes()) == 1, sage.loaded_hip_runtimes()
    dev = torch.device("cuda:0")
    tok = layout == "bnhd"
    Qd, Kd, Vd = ((t.transpose(1, 2) if tok else t).contiguous().to(dev) for t in (Q, K, V))
    qk = sage.quantize_qk(Qd, Kd, w.blk_q, w.blk_k, layout=layout)
    vq = sage.quantize_v(Vd, layout=layout)
    dump = None
    if dump_tiles:
        sel = torch.tensor(list(dump_tiles), dtype=torch.int32, device=dev)
        s_d = torch.full((len(dump_tiles), 128, w.Nkv), S_SENTINEL, dtype=torch.int32, device=dev)
        p_d = torch.full((len(dump_tiles), 128, w.Nkv), P_SENTINEL, dtype=torch.uint8, device=dev)
        dump = (sel, s_d, p_d)
    O = sage.attn_fwd(qk, vq, causal=w.causal, sm_scale=w.sm_scale, out_dtype=out_dtype, layout=layout, dump=dump)
    torch.cuda.synchronize()
    assert O.shape == ((w.B, w.N, w.H, w.d) if tok else (w.B, w.H, w.N, w.d))
    res = {k: (v.cpu().numpy() if torch.is_tensor(v) else v) for k, v in qk.items()}
    res["v_codes"] = sage.v_codes_to_natural(vq[0]).cpu().numpy()
    res["v_codes_tiled"] = vq[0]
    res["v_scale"] = vq[1].cpu().numpy()
    res["O"] = (O.transpose(1, 2) if tok else O).float().cpu().numpy()
    res["O_dev"] = O
    res["qk_dev"], res["vq_dev"] = qk, vq
    if dump:
        res["s_dump"], res["p_dump"] = dump[1].cpu().numpy(), dump[2].cpu().numpy()
    return res


def run_oracle_quant(w, Q, K, V):
    qk = orc.quantize_qk(synth.bits(Q), synth.bits(K), w.dtype_code, w.blk_q, w.blk_k)
    vc, vs = orc.quantize_v(synth.bits(V), w.dtype_code)
    return qk, vc, vs


def check_quant_bit_exact(g, qk, vc, vs):
    """Codes and scales bit-exact on the real tokens and blocks; the padding
    of the device buffers (Q rows to a multiple of 128, K/V rows to a multiple
    of 64, their extra blocks) is all zero."""
    def split(got, n, axis=2):
        return np.split(got, [n], axis=axis)

    assert np.array_equal(g["k_mean"].view(np.uint32), qk["k_mean"].view(np.uint32)), "k_mean"
    for key in ("q_scale", "k_scale"):
        real, pad = split(g[key], qk[key].shape[2])
        assert np.array_equal(real.view(np.uint32), qk[key].view(np.uint32)), key
        assert not pad.any(), f"{key} padding"
    for key, ref in (("q_codes", qk["q_codes"]), ("k_codes", qk["k_codes"]), ("v_codes", vc)):
        real, pad = split(g[key], ref.shape[2])
        if not np.array_equal(real, ref):
            bad = np.argwhere(real != ref)
            raise AssertionError(f"{key}: {len(bad)} mismatches, first at {bad[0]}")
        assert not pad.any(), f"{key} padding"
    assert np.array_equal(g["v_scale"].view(np.uint32), vs.view(np.uint32))


def check_dump(w, g, qk, tiles):
    """Yields (flat query rows, their P~ dump rows, visibility) of each dumped
    tile; rows past N (padding of the last query tile) are left out."""
    nqt = -(-w.N // 128)
    for k, tid in enumerate(tiles):
        bh, qt = divmod(tid, nqt)
        nr = min(128, w.N - qt * 128)
        rows = bh * w.N + qt * 128 + np.arange(nr)
        s_ref = orc.qk_int32(qk["q_codes"], qk["k_codes"], rows)
        s_got = g["s_dump"][k][:nr]
        written = s_got != S_SENTINEL
        i = qt * 128 + np.arange(nr)[:, None]
        j = np.arange(w.Nkv)[None, :]
        visible = (j <= i + (w.Nkv - w.N)) if w.causal else np.ones_like(written)
        assert written[visible].all(), "a visible score was not computed"
        assert np.array_equal(s_got[written], s_ref[written]), "int32 QK^T mismatch"
        yield rows, g["p_dump"][k][:nr], visible


def check_p_codes(p_got, p_ref, visible, flip_frac=P_FLIP_FRAC):
    """Every visible P~ code written; codes equal except for rare one-step flips."""
    written = p_got != P_SENTINEL
    assert written[visible].all(), "a visible P~ code was not written"
    got, ref = p_got[written].astype(np.int16), p_ref[written].astype(np.int16)
    diff = np.abs(got - ref)
    assert diff.max(initial=0) <= 1, f"FP8 P~ code off by {diff.max()} steps"
    n_flip = int((diff == 1).sum())
    assert n_flip <= flip_frac * got.size + 1, f"{n_flip} of {got.size} P~ codes differ by one step"
    return n_flip


def cosine(a, b):
    a = a.astype(np.float64).ravel()
    b = b.astype(np.float64).ravel()
    return float(a @ b / np.sqrt((a @ a) * (b @ b)))


# The FP8 matrix instruction sums each group of 8 products of its 64-key block inside a window
# of about 13 bits below the group's largest product (measured; the oracle sums the block
# exactly).  An element of O can then differ from the oracle by up to 7 * 2^-13 of
# A = sum_j P^_j |V^_jc| delta_c / sum_j P^_j, the P^-weighted mean of |V| in that channel
# (observed: 2^-12.9 of A on an outlier channel with |O| = 24).  The bar is the larger of the
# absolute 2e-3 and 2^-11 * A, so only elements whose weighted |V| exceeds 4 (outlier
# channels) are allowed more than 2e-3.  It is used only for the single heads at the 2^19-token
# length limit (outside the five stated workloads, which are held to the plain 2e-3): there a
# 2^19-key row with x8 V outlier channels differed from the oracle by 3.06e-3 at |O| = 23.6 with
# every P~ code equal, a known exceedance of 2e-3 that this bar records.
INNER_REL = 2.0 ** -11


def weighted_abs_v(P_rows, rows, vc, vs, w):
    """A[i, c] of the flat query rows `rows` (over B*Hq*Nq) from their FP8 P~ codes
    P_rows [len(rows), Nkv] and the V codes / scales of their K/V heads."""
    vcf, vsf = vc.reshape(-1, w.Nkv, w.d), vs.reshape(-1, w.d)
    g = w.H // w.Hkv
    bks = np.array([(r // w.N // w.H) * w.Hkv + (r // w.N % w.H) // g for r in rows])
    out = np.empty((len(rows), w.d))
    for bk in np.unique(bks):
        sel = np.flatnonzero(bks == bk)
        p = orc.e4m3_decode(P_rows[sel])
        out[sel] = (p @ np.abs(orc.e4m3_decode(vcf[bk]))) * vsf[bk] / p.sum(axis=1, keepdims=True)
    return out


def check_o_inner(O_rows, O_ref, A, name=""):
    """Element-wise bar max(O_TOL, INNER_REL * A) (see INNER_REL)."""
    err = np.abs(O_rows.astype(np.float64) - O_ref)
    bar = np.maximum(O_TOL, INNER_REL * A)
    worst = np.unravel_index(int(np.argmax(err / bar)), err.shape)
    print(f"{name}: max |O - oracle| {err.max():.3g}; worst element {worst}: error {err[worst]:.3g}, "
          f"bar {bar[worst]:.3g}, A {A[worst]:.3g}")
    assert (err <= bar).all(), f"|O - oracle| {err[worst]:.3g} above the bar {bar[worst]:.3g}"


# ------------------------------------------------------------------ small cases: every row
SMALL = {
    "tiny-f16-256": dict(),
    "causal-bf16-d128-N1024": dict(base="llm-prefill-4k-causal", B=1, H=2, N=1024),
    "vit-f16-d64-N512": dict(base="vit-2k-f16", B=2, H=2, N=512),
    "outliers-causal-N2048": dict(base="long-prefill-128k-causal", H=2, N=2048),
    "blkq64-causal-f16-N384": dict(base="llm-prefill-4k-causal", B=1, H=3, N=384, blk_q=64, dtype="float16"),
    "min-N128-causal-d64-bf16": dict(base="vit-2k-f16", B=2, H=1, N=128, causal=True, dtype="bfloat16"),
    "noncausal-bf16-d128-blkq64": dict(base="video-dit-32k", H=2, N=768, blk_q=64),
}


def small_workload(name):
    kw = dict(SMALL[name])
    base = kw.pop("base", name)
    return synth.WORKLOADS[base].with_(name=name, **kw)


@pytest.mark.parametrize("name", list(SMALL))
def test_small_full_parity(name):
    w = small_workload(name)
    Q, K, V = synth.make_inputs(w)
    nqt = -(-w.N // 128)
    tiles = sorted({0, nqt - 1, (w.B * w.H - 1) * nqt + nqt // 2})
    g = run_gpu(w, Q, K, V, dump_tiles=tiles)
    qk, vc, vs = run_oracle_quant(w, Q, K, V)
    check_quant_bit_exact(g, qk, vc, vs)
    O_ref, P_ref = orc.attn_rows(qk, vc, vs, w.blk_q, w.blk_k, w.causal, w.sm_scale, want_p=True)
    for rows, p_got, visible in check_dump(w, g, qk, tiles):
        check_p_codes(p_got, P_ref[rows], visible)
    O = g["O"].reshape(-1, w.d)
    err = np.abs(O - O_ref)
    assert err.max() <= O_TOL, f"max |O - oracle| = {err.max():.3g} at row {np.unravel_index(err.argmax(), err.shape)}"
    ex = orc.exact_attention(Q.float().numpy(), K.float().numpy(), V.float().numpy(), w.causal, w.sm_scale)
    assert cosine(O, ex) >= 0.995


# grouped K/V heads (Hkv < H), fewer queries than keys (the queries are the
# last N of Nkv positions; causal visibility j <= i + Nkv - N), and the
# token-major [B, N, H, d] layout.  B*Hkv = 8 and 16 take the kernel's
# per-XCD K/V-head order, the others the plain order.
SMALL_EX = {
    "gqa4-causal-bf16-d128": dict(base="llm-prefill-4k-causal", B=2, H=8, Hkv_=2, N=512),
    "gqa2-xcd-f16-d64": dict(base="vit-2k-f16", B=1, H=16, Hkv_=8, N=256),
    "gqa4-xcd-causal-d128": dict(base="llm-prefill-4k-causal", B=2, H=16, Hkv_=4, N=384),
    "chunk256-of-1024-causal-blkq64": dict(base="llm-prefill-4k-causal", B=1, H=2, N=256, Nkv_=1024, blk_q=64),
    "q384-of-k128-noncausal-f16": dict(base="tiny-f16-256", B=1, H=2, N=384, Nkv_=128),
    "mqa-chunk128-of-640-causal-d64": dict(base="vit-2k-f16", B=2, H=4, Hkv_=1, N=128, Nkv_=640, causal=True),
    "gqa8-xcd-chunk-noncausal-d128": dict(base="video-dit-32k", B=2, H=64, Hkv_=8, N=128, Nkv_=512),
    # lengths that are not multiples of 128: partial last Q block / query tile,
    # partial last KV tile, causal offsets that are not tile multiples
    "ragged-causal-N200-d128": dict(base="llm-prefill-4k-causal", B=1, H=2, N=200),
    "ragged-f16-d64-N77-blkq64": dict(base="vit-2k-f16", B=2, H=2, N=77, blk_q=64),
    "ragged-gqa-causal-130-of-1000": dict(base="llm-prefill-4k-causal", B=1, H=8, Hkv_=2, N=130, Nkv_=1000,
                                          blk_q=64),
    "ragged-one-key-tail-d64": dict(base="vit-2k-f16", B=1, H=2, N=256, Nkv_=65),
    "ragged-single-token-causal": dict(base="llm-prefill-4k-causal", B=1, H=1, N=1),
    "ragged-causal-300-of-384": dict(base="llm-prefill-4k-causal", B=1, H=2, N=300, Nkv_=384),
    "ragged-mqa-256-of-333": dict(base="video-dit-32k", B=1, H=4, Hkv_=1, N=256, Nkv_=333),
    "ragged-xcd-causal-d64-N190": dict(base="vit-2k-f16", B=1, H=16, Hkv_=8, N=190, causal=True,
                                       dtype="bfloat16"),
    # finer quantization granularity: one Q scale per wave (32 rows), K scales
    # per 16 or 32 keys (two runs of 16 keys per lane and tile)
    "fine-q32-k16-causal-d128": dict(base="llm-prefill-4k-causal", B=1, H=2, N=512, blk_q=32, blk_k=16),
    "fine-k32-noncausal-d64": dict(base="vit-2k-f16", B=1, H=2, N=384, blk_k=32),
    "fine-q32-k16-ragged-gqa-d64": dict(base="vit-2k-f16", B=1, H=4, Hkv_=2, N=200, Nkv_=333, causal=True,
                                        blk_q=32, blk_k=16),
    "fine-k32-outliers-causal": dict(base="long-prefill-128k-causal", H=2, N=1024, blk_k=32),
}


def small_ex_workload(name):
    kw = dict(SMALL_EX[name])
    base = kw.pop("base")
    return synth.WORKLOADS[base].with_(name=name, **kw)


@pytest.mark.parametrize("layout", ["bhnd", "bnhd"])
@pytest.mark.parametrize("name", list(SMALL_EX))
def test_small_grouped_and_unequal_parity(name, layout):
    w = small_ex_workload(name)
    Q, K, V = synth.make_inputs(w)
    assert Q.shape == (w.B, w.H, w.N, w.d) and K.shape == (w.B, w.Hkv, w.Nkv, w.d)
    nqt = -(-w.N // 128)
    tiles = sorted({0, nqt - 1, (w.B * w.H - 1) * nqt + nqt // 2, (w.B * w.H // 2) * nqt})
    g = run_gpu(w, Q, K, V, dump_tiles=tiles, layout=layout)
    qk, vc, vs = run_oracle_quant(w, Q, K, V)
    check_quant_bit_exact(g, qk, vc, vs)
    O_ref, P_ref = orc.attn_rows(qk, vc, vs, w.blk_q, w.blk_k, w.causal, w.sm_scale, want_p=True)
    for rows, p_got, visible in check_dump(w, g, qk, tiles):
        check_p_codes(p_got, P_ref[rows], visible)
    O = g["O"].reshape(-1, w.d)
    err = np.abs(O - O_ref)
    assert err.max() <= O_TOL, f"max |O - oracle| = {err.max():.3g} at row {np.unravel_index(err.argmax(), err.shape)}"
    ex = orc.exact_attention(Q.float().numpy(), K.float().numpy(), V.float().numpy(), w.causal, w.sm_scale)
    assert cosine(O, ex) >= 0.995


# A seeded sweep over the shape space of the C ABI: head size, input dtype, grouped heads, lengths
# that are not tile multiples (queries at the end of the keys), the causal mask, block sizes, the
# two layouts, sm_scale, the K channel bias and V outlier channels; every other case quantizes with
# the fused call.  Each case is printed with its parameters.  The sweep reaches beyond the
# benchmark shapes (sm_scale up to 0.3, x8 V outlier channels in short heads), where a few
# outlier-channel elements of O exceed 2e-3 by the FP8 matrix instruction's inner-sum window: the
# instruction sums each group of 8 products in a window of about 13 bits below the group's
# largest, so an element moves by at most 7 * 2^-13 of A (the P~-weighted mean of |V^| * delta_V
# of its channel, see weighted_abs_v).  The bar is max(2e-3, 7 * 2^-13 * A) element by element:
# plain 2e-3 wherever A < 2.3, i.e. on every ordinary channel.  (First case of the sweep: error
# 4.97e-3 at |O| = 14.8 on an outlier channel with A = 11.3, every code and scale bit-exact.)
INNER_MAX = 7 * 2.0 ** -13
def _random_cases(n=48, seed=2026):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        d = int(rng.choice([64, 128]))
        Hkv = int(rng.integers(1, 4))
        g = int(rng.choice([1, 2, 4]))
        causal = bool(rng.integers(0, 2))
        Nkv = int(rng.integers(1, 700))
        Nq = int(rng.integers(1, Nkv + 1)) if causal or rng.random() < 0.5 else int(rng.integers(1, 700))
        cases.append(dict(
            name=f"rnd{i:02d}", B=int(rng.integers(1, 3)), H=Hkv * g, Hkv_=Hkv, N=Nq, Nkv_=Nkv, d=d,
            dtype=str(rng.choice(["float16", "bfloat16"])), causal=causal,
            blk_q=int(rng.choice([32, 64, 128])), blk_k=int(rng.choice([16, 32, 64])),
            bias_var=float(rng.choice([0.0, 2.0, 4.0])),
            sm_scale=float(np.float32(rng.uniform(0.05, 0.3))),
            v_outlier_channels=int(rng.choice([0, 0, d // 10])), v_outlier_scale=8.0, seed=int(rng.integers(0, 1 << 30)),
            layout=str(rng.choice(["bhnd", "bnhd"])), fused=bool(i % 2)))
    return cases


RANDOM_CASES = {c["name"]: c for c in _random_cases()}


@pytest.mark.parametrize("name", list(RANDOM_CASES))
def test_seeded_random_shapes_against_the_oracle(name):
    kw = dict(RANDOM_CASES[name])
    layout, fused = kw.pop("layout"), kw.pop("fused")
    w = synth.Workload(**kw)
    print(f"{name}: {kw} layout={layout} fused={fused}", flush=True)
    sage = _sage()
    Q, K, V = synth.make_inputs(w)
    dev = torch.device("cuda:0")
    tok = layout == "bnhd"
    Qd, Kd, Vd = ((t.transpose(1, 2) if tok else t).contiguous().to(dev) for t in (Q, K, V))
    if fused:
        qk, vq = sage.quantize_qkv(Qd, Kd, Vd, w.blk_q, w.blk_k, layout=layout)
    else:
        qk = sage.quantize_qk(Qd, Kd, w.blk_q, w.blk_k, layout=layout)
        vq = sage.quantize_v(Vd, layout=layout)
    O = sage.attn_fwd(qk, vq, causal=w.causal, sm_scale=w.sm_scale, out_dtype=torch.float32, layout=layout)
    torch.cuda.synchronize()
    g = {k: (v.cpu().numpy() if torch.is_tensor(v) else v) for k, v in qk.items()}
    g["v_codes"] = sage.v_codes_to_natural(vq[0]).cpu().numpy()
    g["v_scale"] = vq[1].cpu().numpy()
    qk_ref, vc, vs = run_oracle_quant(w, Q, K, V)
    check_quant_bit_exact(g, qk_ref, vc, vs)
    O = (O.transpose(1, 2) if tok else O).cpu().numpy().reshape(-1, w.d)
    O_ref, P_ref = orc.attn_rows(qk_ref, vc, vs, w.blk_q, w.blk_k, w.causal, w.sm_scale, want_p=True)
    rows = np.arange(w.B * w.H * w.N)
    A = weighted_abs_v(P_ref, rows, vc, vs, w)
    err = np.abs(O.astype(np.float64) - O_ref)
    bar = np.maximum(O_TOL, INNER_MAX * A)
    worst = np.unravel_index(int(np.argmax(err / bar)), err.shape)
    print(f"{name}: max |O - oracle| {err.max():.3g}; {(err > O_TOL).sum()} elements above 2e-3; worst against "
          f"the bar: error {err[worst]:.3g}, bar {bar[worst]:.3g}, A {A[worst]:.3g}", flush=True)
    assert (err <= bar).all(), f"|O - oracle| {err[worst]:.3g} above the bar {bar[worst]:.3g} at {worst}"
    ex = orc.exact_attention(Q.float().numpy(), K.float().numpy(), V.float().numpy(), w.causal, w.sm_scale)
    assert cosine(O, ex) >= 0.995


# INT8 at d = 128 on whole 256-row query tiles runs in 8-wave workgroups of 256 rows: always
# without the causal mask, and with it where a query row sees 16384 keys or more on average
# (Nkv - Nq/2).  The dump instance always runs 128-row workgroups.  The per-row arithmetic is
# the same (a wave skips the same tiles wholly after its rows), so O must be bit-identical to the
# 128-row kernel's, and within 2e-3 of the oracle.
WIDE = {
    "wide-noncausal-N768-blkq64": dict(base="video-dit-32k", B=1, H=2, N=768, blk_q=64),
    "wide-gqa-chunk-512-of-1024": dict(base="video-dit-32k", B=2, H=8, Hkv_=2, N=512, Nkv_=1024),
    "wide-fine-k16-N512": dict(base="video-dit-32k", B=1, H=3, N=512, blk_q=32, blk_k=16),
    "wide-mqa-N256-xcd": dict(base="video-dit-32k", B=1, H=64, Hkv_=8, N=256),
    "wide-causal-chunk-256-of-16512": dict(base="long-prefill-128k-causal", B=1, H=2, N=256, Nkv_=16512),
    "wide-causal-gqa-512-of-16640": dict(base="long-prefill-128k-causal", B=1, H=2, Hkv_=1, N=512, Nkv_=16640),
}


@pytest.mark.parametrize("layout", ["bhnd", "bnhd"])
@pytest.mark.parametrize("name", list(WIDE))
def test_wide_workgroups_equal_the_128_row_kernel(name, layout):
    kw = dict(WIDE[name])
    w = synth.WORKLOADS[kw.pop("base")].with_(name=name, **kw)
    Q, K, V = synth.make_inputs(w)
    assert w.d == 128 and w.N % 256 == 0 and w.Nkv % 128 == 0 and (not w.causal or w.Nkv - w.N // 2 >= 16384)
    nqt = -(-w.N // 128)
    g = run_gpu(w, Q, K, V, dump_tiles=(0,), layout=layout)     # the 128-row instance
    sage = _sage()
    tok = layout == "bnhd"
    for dt in (torch.float32, w.torch_dtype):
        o = sage.attn_fwd(g["qk_dev"], g["vq_dev"], causal=w.causal, sm_scale=w.sm_scale, out_dtype=dt, layout=layout)
        torch.cuda.synchronize()
        o = (o.transpose(1, 2) if tok else o).cpu()
        ref = torch.from_numpy(g["O"]).to(dt)
        assert torch.equal(o.view(torch.int16 if dt != torch.float32 else torch.int32),
                           ref.view(torch.int16 if dt != torch.float32 else torch.int32)), f"{dt}: differs"
    qk, vc, vs = run_oracle_quant(w, Q, K, V)
    O_ref = orc.attn_rows(qk, vc, vs, w.blk_q, w.blk_k, w.causal, w.sm_scale)
    assert np.abs(g["O"].reshape(-1, w.d) - O_ref).max() <= O_TOL
    assert nqt >= 2


QKV_CASES = ["gqa4-causal-bf16-d128", "gqa2-xcd-f16-d64", "ragged-gqa-causal-130-of-1000", "ragged-f16-d64-N77-blkq64",
             "fine-q32-k16-ragged-gqa-d64", "fine-k32-outliers-causal", "ragged-single-token-causal"]


# the small shapes in both layouts, the full-size workloads in the head-major one
QKV_FULL = ["llm-prefill-4k-causal", "video-dit-32k", "vit-2k-f16", "long-prefill-128k-causal"]


@pytest.mark.parametrize("name,layout", [(n, l) for n in QKV_CASES for l in ("bhnd", "bnhd")] +
                         [(n, "bhnd") for n in QKV_FULL])
def test_fused_qkv_quantize_equals_the_two_calls(name, layout):
    """sage_quantize_qkv gives the codes, scales and K means of sage_quantize_qk + sage_quantize_v
    bit for bit (including the zero padding), on grouped, ragged and finer-block shapes and four
    full-size workloads (d = 64 and 128; 32768 and 131072 keys take the streaming loads in its
    first pass, 4096 and 2048 the cached ones)."""
    if name in synth.WORKLOADS:
        w = synth.WORKLOADS[name]
    else:
        w = small_ex_workload(name)
    sage = _sage()
    Q, K, V = synth.make_inputs(w)
    dev = torch.device("cuda:0")
    tok = layout == "bnhd"
    Qd, Kd, Vd = ((t.transpose(1, 2) if tok else t).contiguous().to(dev) for t in (Q, K, V))
    qk = sage.quantize_qk(Qd, Kd, w.blk_q, w.blk_k, layout=layout)
    vq = sage.quantize_v(Vd, layout=layout)
    qk2, vq2 = sage.quantize_qkv(Qd, Kd, Vd, w.blk_q, w.blk_k, layout=layout)
    torch.cuda.synchronize()
    for key in ("q_codes", "q_scale", "k_codes", "k_scale", "k_mean"):
        a, b = qk[key].cpu(), qk2[key].cpu()
        assert a.shape == b.shape and torch.equal(a.view(torch.uint8), b.view(torch.uint8)), key
    for a, b in zip(vq, vq2):
        assert torch.equal(a.cpu().view(torch.uint8), b.cpu().view(torch.uint8))
    if name not in synth.WORKLOADS:   # and the oracle's, on the small shapes
        g = {k: (v.cpu().numpy() if torch.is_tensor(v) else v) for k, v in qk2.items()}
        g["v_codes"] = sage.v_codes_to_natural(vq2[0]).cpu().numpy()
        g["v_scale"] = vq2[1].cpu().numpy()
        check_quant_bit_exact(g, *run_oracle_quant(w, Q, K, V))


@pytest.mark.parametrize("name", ["gqa4-xcd-causal-d128", "chunk256-of-1024-causal-blkq64"])
def test_token_major_layout_is_bit_identical(name):
    """The layout only changes addressing: codes, scales and O bits agree."""
    w = small_ex_workload(name)
    Q, K, V = synth.make_inputs(w)
    a = run_gpu(w, Q, K, V, out_dtype=torch.bfloat16)
    b = run_gpu(w, Q, K, V, out_dtype=torch.bfloat16, layout="bnhd")
    for key in ("q_codes", "k_codes", "v_codes", "k_mean", "q_scale", "k_scale", "v_scale", "O"):
        assert np.array_equal(a[key], b[key]), key


def test_square_problem_through_the_extended_entry_points():
    """H = Hkv, N = Nkv, [B,H,N,d]: the _ex entry points give the plain ones' bits."""
    sage = _sage()
    w = small_workload("causal-bf16-d128-N1024")
    Q, K, V = synth.make_inputs(w)
    g = run_gpu(w, Q, K, V)
    dev = torch.device("cuda:0")
    Qd, Kd, Vd = (t.to(dev) for t in (Q, K, V))
    B, H, N, d = Q.shape
    st = torch.cuda.current_stream().cuda_stream
    codes = dict(q=torch.empty_like(Qd, dtype=torch.int8), k=torch.empty_like(Kd, dtype=torch.int8),
                 qs=torch.empty((B, H, N // w.blk_q), dtype=torch.float32, device=dev),
                 ks=torch.empty((B, H, N // 64), dtype=torch.float32, device=dev),
                 km=torch.empty((B, H, d), dtype=torch.float32, device=dev),
                 v=torch.empty((B, H, N // 64, d, 64), dtype=torch.uint8, device=dev),
                 vs=torch.empty((B, H, d), dtype=torch.float32, device=dev))
    ws = torch.empty(1 << 22, dtype=torch.uint8, device=dev)
    p = {k: t.data_ptr() for k, t in codes.items()}
    assert sage.sage_quantize_qk_ex(Qd.data_ptr(), Kd.data_ptr(), w.dtype_code, sage.SAGE_LAYOUT_BHND, B, H, H, N, N,
                                    d, w.blk_q, 64, p["q"], p["qs"], p["k"], p["ks"], p["km"], ws.data_ptr(),
                                    ws.numel(), st) == 0
    assert sage.sage_quantize_v_ex(Vd.data_ptr(), w.dtype_code, sage.SAGE_LAYOUT_BHND, B, H, N, d, p["v"], p["vs"],
                                   ws.data_ptr(), ws.numel(), st) == 0
    O = torch.empty((B, H, N, d), dtype=torch.float32, device=dev)
    assert sage.sage_attn_fwd_ex(p["q"], p["qs"], p["k"], p["ks"], p["v"], p["vs"], O.data_ptr(), sage.SAGE_F32,
                                 sage.SAGE_LAYOUT_BHND, B, H, H, N, N, d, w.blk_q, 64, int(w.causal), w.sm_scale,
                                 st) == 0
    torch.cuda.synchronize()
    assert np.array_equal(codes["q"].cpu().numpy(), g["q_codes"])
    assert np.array_equal(codes["k"].cpu().numpy(), g["k_codes"])
    assert np.array_equal(codes["km"].cpu().numpy(), g["k_mean"])
    assert torch.equal(codes["v"].cpu(), g["v_codes_tiled"].cpu())
    assert np.array_equal(O.cpu().numpy(), g["O"])


def test_output_dtypes_round_the_fp32_result():
    w = small_workload("causal-bf16-d128-N1024")
    Q, K, V = synth.make_inputs(w)
    g = run_gpu(w, Q, K, V)
    sage = _sage()
    ref = torch.from_numpy(g["O"])
    for dt in (torch.bfloat16, torch.float16):
        o = sage.attn_fwd(g["qk_dev"], g["vq_dev"], causal=w.causal, sm_scale=w.sm_scale, out_dtype=dt)
        torch.cuda.synchronize()
        got, exp = o.cpu(), ref.to(dt)
        bad = (got.view(torch.int16) != exp.view(torch.int16)).nonzero()
        if len(bad):
            i = tuple(bad[0].tolist())
            raise AssertionError(f"{dt}: {len(bad)} mismatches; first {i}: fp32 {ref[i].item()!r} "
                                 f"got {got[i].item()!r} expected {exp[i].item()!r}")


def test_repeat_runs_are_bit_identical():
    w = small_workload("outliers-causal-N2048")
    Q, K, V = synth.make_inputs(w)
    g1 = run_gpu(w, Q, K, V)
    g2 = run_gpu(w, Q, K, V)
    for key in ("q_codes", "k_codes", "v_codes", "k_mean", "q_scale", "k_scale", "v_scale", "O"):
        assert np.array_equal(g1[key], g2[key]), key


def test_drop_in_attention_matches_separate_calls():
    sage = _sage()
    w = small_workload("vit-f16-d64-N512")
    Q, K, V = synth.make_inputs(w)
    g = run_gpu(w, Q, K, V, out_dtype=torch.float16)
    o = sage.attention(Q.cuda(), K.cuda(), V.cuda(), causal=w.causal, sm_scale=w.sm_scale, blk_q=w.blk_q)
    torch.cuda.synchronize()
    assert o.dtype == torch.float16 and torch.equal(o.cpu(), g["O_dev"].cpu())


# ------------------------------------------------------------------ edge cases
def _edge_inputs(w, kind):
    Q, K, V = synth.make_inputs(w)
    if kind == "zero-q":
        Q = torch.zeros_like(Q)
    elif kind == "constant-k":
        K = torch.ones_like(K) * 3
    elif kind == "zero-v-channel":
        V = V.clone()
        V[..., 5] = 0
    elif kind == "large":
        Q, K, V = Q * 64, K * 64, V * 1000
    elif kind == "tiny":
        Q, K, V = Q * 2 ** -10, K * 2 ** -10, V * 2 ** -10
    elif kind == "zero-q-block":
        Q = Q.clone()
        Q[:, :, 128:256] = 0
    return Q, K, V


@pytest.mark.parametrize("kind", ["zero-q", "constant-k", "zero-v-channel", "large", "tiny", "zero-q-block"])
def test_edge_cases(kind):
    w = small_workload("blkq64-causal-f16-N384") if kind != "large" else small_workload("causal-bf16-d128-N1024")
    Q, K, V = _edge_inputs(w, kind)
    g = run_gpu(w, Q, K, V, dump_tiles=(1,))
    qk, vc, vs = run_oracle_quant(w, Q, K, V)
    check_quant_bit_exact(g, qk, vc, vs)
    O_ref, P_ref = orc.attn_rows(qk, vc, vs, w.blk_q, w.blk_k, w.causal, w.sm_scale, want_p=True)
    for rows, p_got, visible in check_dump(w, g, qk, (1,)):
        check_p_codes(p_got, P_ref[rows], visible)
    O = g["O"].reshape(-1, w.d)
    tol = O_TOL * (1000 if kind == "large" else 1)  # V scaled by 1000: same relative bar
    assert np.abs(O - O_ref).max() <= tol
    assert np.isfinite(O).all()


# ------------------------------------------------------------------ full-size workloads, sampled rows
def _sample_rows(w, rng, n_rand=24):
    BH, N = w.B * w.H, w.N
    first = np.arange(16)                                   # early causal rows: few keys, big weights
    last = (BH - 1) * N + N - 1 - np.arange(8)
    rand = rng.integers(0, BH * N, n_rand)
    return np.unique(np.concatenate([first, last, rand])).astype(np.int64)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_full_size_workload(name):
    w = synth.WORKLOADS[name]
    Q, K, V = synth.make_inputs(w)
    if w.pv4:
        g = run_gpu_fp4(w, Q, K, V)
        r, v4 = check_fp4_quant(w, g, Q, K, V)
        rows = _sample_rows(w, np.random.default_rng(123))
        O_ref = orc.attn_rows_fp4(r, *v4, w.causal, w.sm_scale, rows=rows)
        O = g["O"].reshape(-1, w.d)
        assert np.abs(O[rows] - O_ref).max() <= O_TOL
        ex = orc.exact_attention(Q.float().numpy(), K.float().numpy(), V.float().numpy(), w.causal, w.sm_scale,
                                 rows=rows)
        assert cosine(O[rows], ex) >= FP4_COS
        return
    if w.qk4:
        g = run_gpu_qk4(w, Q, K, V)
        r = orc.quantize_qk4(synth.bits(Q), synth.bits(K), w.dtype_code, smooth_q=w.smooth_q)
        vc, vs = orc.quantize_v(synth.bits(V), w.dtype_code)
        check_qk4_quant(w, g, r)
        rows = _sample_rows(w, np.random.default_rng(123))
        O_ref = orc.attn_rows_qk4(r, vc, vs, w.causal, w.sm_scale, rows=rows)
        O = g["O"].reshape(-1, w.d)
        assert np.abs(O[rows] - O_ref).max() <= O_TOL
        ex = orc.exact_attention(Q.float().numpy(), K.float().numpy(), V.float().numpy(), w.causal, w.sm_scale,
                                 rows=rows)
        assert cosine(O[rows], ex) >= QK4_COS
        return
    if w.decode:
        # the split the library picks for this shape, on both sides
        g = run_gpu_decode(w, Q, K, V, 0)
        qk, vc, vs = run_oracle_quant(w, Q, K, V)
        check_quant_bit_exact(g, qk, vc, vs)
        rows = np.unique(np.concatenate([np.arange(8), w.B * w.H * w.N - 1 - np.arange(8),
                                         np.random.default_rng(7).integers(0, w.B * w.H * w.N, 48)]))
        O_ref = orc.attn_rows_split(qk, vc, vs, w.blk_q, w.blk_k, w.causal, w.sm_scale, kv_chunk=g["kv_chunk"],
                                    rows=rows)
        O = g["O"].reshape(-1, w.d)
        assert np.abs(O[rows] - O_ref).max() <= O_TOL
        ex = orc.exact_attention(Q.float().numpy(), K.float().numpy(), V.float().numpy(), w.causal, w.sm_scale,
                                 rows=rows)
        assert cosine(O[rows], ex) >= 0.995
        return
    nqt = -(-w.N // 128)
    tiles = (0, w.B * w.H * nqt - 1)
    g = run_gpu(w, Q, K, V, dump_tiles=tiles)
    qk, vc, vs = run_oracle_quant(w, Q, K, V)
    check_quant_bit_exact(g, qk, vc, vs)
    # The kernel instance that serves users (and that bench.py times) has no dump stores: run it on
    # the same device codes, in fp32 and in the input dtype, and check it against the oracle.
    sage = _sage()
    O_prod = sage.attn_fwd(g["qk_dev"], g["vq_dev"], causal=w.causal, sm_scale=w.sm_scale, out_dtype=torch.float32)
    O_user = sage.attn_fwd(g["qk_dev"], g["vq_dev"], causal=w.causal, sm_scale=w.sm_scale, out_dtype=w.torch_dtype)
    torch.cuda.synchronize()
    O = O_prod.cpu().numpy().reshape(-1, w.d)
    assert np.array_equal(O.view(np.uint32), g["O"].reshape(-1, w.d).view(np.uint32)), \
        "the instance without dump stores gives other O bits than the dump instance"
    assert torch.equal(O_user.cpu().view(torch.int16), O_prod.cpu().to(w.torch_dtype).view(torch.int16)), \
        f"{w.dtype} output is not the round-to-nearest-even cast of the fp32 O"
    del O_prod, O_user
    rows = _sample_rows(w, np.random.default_rng(123))
    dumps = list(check_dump(w, g, qk, tiles))
    dump_rows = np.concatenate([r for r, _, _ in dumps])
    # one whole head where the oracle finishes it in seconds (N * Nkv * d <= 2^31: the tiny, 4k
    # causal, ViT, ragged and finer-block workloads)
    head_rows = np.arange(0)
    if w.N * w.Nkv * w.d <= 2 ** 31:
        bh = (w.B * w.H) // 2
        head_rows = bh * w.N + np.arange(w.N)
    O_ref, P_ref = orc.attn_rows(qk, vc, vs, w.blk_q, w.blk_k, w.causal, w.sm_scale,
                                 rows=np.concatenate([rows, dump_rows, head_rows]), want_p=True)
    at = len(rows)
    for r, p_got, visible in dumps:
        check_p_codes(p_got, P_ref[at: at + len(r)], visible)
        at += len(r)
    all_rows = np.concatenate([rows, dump_rows, head_rows])
    err = np.abs(O[all_rows].astype(np.float64) - O_ref)
    worst = np.unravel_index(int(err.argmax()), err.shape)
    print(f"{name}: {len(all_rows)} rows ({len(dump_rows)} of the dumped tiles, {len(head_rows)} of one whole "
          f"head): max |O - oracle| {err.max():.3g} at row {all_rows[worst[0]]}, channel {worst[1]}")
    assert err.max() <= O_TOL, f"max |O - oracle| = {err.max():.3g} at row {all_rows[worst[0]]}"
    ex = orc.exact_attention(Q.float().numpy(), K.float().numpy(), V.float().numpy(), w.causal, w.sm_scale, rows=rows)
    assert cosine(O[rows], ex) >= 0.995


# ------------------------------------------------------------------ the longest supported sequence
MAX_LEN = {
    # one head at the length limit of the C ABI (2^19 tokens): causal d = 128 with V outliers, and a
    # ragged non-causal d = 64 length just below it; the 4-bit scores at the limit; and decode of four
    # queries of two grouped heads against a cache at the limit
    "max-len-causal-d128": dict(base="long-prefill-128k-causal", H=1, N=1 << 19),
    "max-len-ragged-d64": dict(base="vit-2k-f16", B=1, H=1, N=(1 << 19) - 37),
    "max-len-qk4": dict(base="video-dit-32k-qk4", H=1, N=1 << 19),
    "max-len-fp4": dict(base="video-dit-32k-fp4", H=1, N=1 << 19),
    "max-len-decode": dict(base="decode-128k-gqa-4q", B=1, H=2, Hkv_=1, Nkv_=1 << 19),
}


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", list(MAX_LEN))
def test_maximum_length(name):
    kw = dict(MAX_LEN[name])
    w = synth.WORKLOADS[kw.pop("base")].with_(name=name, **kw)
    Q, K, V = synth.make_inputs(w)
    if w.pv4:
        g = run_gpu_fp4(w, Q, K, V)
        r, v4 = check_fp4_quant(w, g, Q, K, V)
        rows = _sample_rows(w, np.random.default_rng(5), n_rand=16)
        O_ref = orc.attn_rows_fp4(r, *v4, w.causal, w.sm_scale, rows=rows)
        O = g["O"].reshape(-1, w.d)
        assert np.abs(O[rows] - O_ref).max() <= O_TOL
        ex = orc.exact_attention(Q.float().numpy(), K.float().numpy(), V.float().numpy(), w.causal, w.sm_scale,
                                 rows=rows)
        assert cosine(O[rows], ex) >= FP4_COS
        return
    if w.qk4:
        g = run_gpu_qk4(w, Q, K, V)
        r = orc.quantize_qk4(synth.bits(Q), synth.bits(K), w.dtype_code, smooth_q=w.smooth_q)
        vc, vs = orc.quantize_v(synth.bits(V), w.dtype_code)
        check_qk4_quant(w, g, r)
        rows = _sample_rows(w, np.random.default_rng(5), n_rand=16)
        O_ref = orc.attn_rows_qk4(r, vc, vs, w.causal, w.sm_scale, rows=rows)
        O = g["O"].reshape(-1, w.d)
        assert np.abs(O[rows] - O_ref).max() <= O_TOL
        ex = orc.exact_attention(Q.float().numpy(), K.float().numpy(), V.float().numpy(), w.causal, w.sm_scale,
                                 rows=rows)
        assert cosine(O[rows], ex) >= QK4_COS
        return
    if w.decode:
        g = run_gpu_decode(w, Q, K, V, 0)
        qk, vc, vs = run_oracle_quant(w, Q, K, V)
        check_quant_bit_exact(g, qk, vc, vs)
        rows = np.arange(w.B * w.H * w.N)
        O_ref = orc.attn_rows_split(qk, vc, vs, w.blk_q, w.blk_k, w.causal, w.sm_scale, kv_chunk=g["kv_chunk"],
                                    rows=rows)
        assert np.abs(g["O"].reshape(-1, w.d) - O_ref).max() <= O_TOL
        ex = orc.exact_attention(Q.float().numpy(), K.float().numpy(), V.float().numpy(), w.causal, w.sm_scale,
                                 rows=rows)
        assert cosine(g["O"].reshape(-1, w.d), ex) >= 0.995
        return
    g = run_gpu(w, Q, K, V)
    qk, vc, vs = run_oracle_quant(w, Q, K, V)
    check_quant_bit_exact(g, qk, vc, vs)
    rows = _sample_rows(w, np.random.default_rng(5), n_rand=16)
    O_ref, P_ref = orc.attn_rows(qk, vc, vs, w.blk_q, w.blk_k, w.causal, w.sm_scale, rows=rows, want_p=True)
    O = g["O"].reshape(-1, w.d)
    check_o_inner(O[rows], O_ref, weighted_abs_v(P_ref, rows, vc, vs, w), name)
    ex = orc.exact_attention(Q.float().numpy(), K.float().numpy(), V.float().numpy(), w.causal, w.sm_scale, rows=rows)
    assert cosine(O[rows], ex) >= 0.995


@pytest.mark.timeout(300)
def test_k_mean_at_the_length_limit_with_saturated_channels():
    """2^19 tokens with channels far past the fixed-point clamp on every token: the int64 channel
    sums reach +-2^62 without overflowing; K mean, codes and scales equal the oracle's bit for bit."""
    w = synth.WORKLOADS["vit-2k-f16"].with_(name="kmean-saturated", B=1, H=1, N=1 << 19, dtype="bfloat16")
    Q, K, V = synth.make_inputs(w)
    K = K.clone()
    K[..., 0] = 2.0 ** 100
    K[..., 1] = -3.0e38
    K[..., 2] = 2.0 ** 19
    sage = _sage()
    qk = sage.quantize_qk(Q.cuda(), K.cuda(), w.blk_q, w.blk_k)
    torch.cuda.synchronize()
    ref = orc.quantize_qk(synth.bits(Q), synth.bits(K), w.dtype_code, w.blk_q, w.blk_k)
    km = qk["k_mean"].cpu().numpy()
    assert km[0, 0, :3].tolist() == [2.0 ** 19, -(2.0 ** 19), 2.0 ** 19]
    assert np.array_equal(km.view(np.uint32), ref["k_mean"].view(np.uint32))
    for key in ("k_codes", "q_codes"):
        assert np.array_equal(qk[key].cpu().numpy()[:, :, :w.N], ref[key]), key
    for key in ("k_scale", "q_scale"):
        got = qk[key].cpu().numpy()[:, :, :ref[key].shape[2]]
        assert np.array_equal(got.view(np.uint32), ref[key].view(np.uint32)), key


@pytest.mark.timeout(600)
def test_offsets_beyond_2gib():
    """33 copies of one 2^19-token head: each input tensor spans 2.2 GB, so the last heads sit past
    every 32-bit byte offset.  Every head's codes, scales and O must equal head 0's bit for bit,
    and head 0 matches the oracle."""
    H = 33
    w1 = synth.WORKLOADS["vit-2k-f16"].with_(name="one-head", B=1, H=1, N=1 << 19, causal=True)
    w = w1.with_(name="offsets-beyond-2gib", H=H)
    Q1, K1, V1 = synth.make_inputs(w1)
    Q, K, V = (t.repeat(1, H, 1, 1) for t in (Q1, K1, V1))
    assert Q.numel() * Q.element_size() > (1 << 31)
    g = run_gpu(w, Q, K, V)
    for key in ("q_codes", "q_scale", "k_codes", "k_scale", "k_mean", "v_codes", "v_scale", "O"):
        a = g[key]
        assert all(np.array_equal(a[:, h], a[:, 0]) for h in range(1, H)), key
    one = {k: (v[:, :1] if isinstance(v, np.ndarray) else v) for k, v in g.items()}
    qk, vc, vs = run_oracle_quant(w1, Q1, K1, V1)
    check_quant_bit_exact(one, qk, vc, vs)
    rows = _sample_rows(w1, np.random.default_rng(9), n_rand=8)
    O_ref = orc.attn_rows(qk, vc, vs, w1.blk_q, w1.blk_k, w1.causal, w1.sm_scale, rows=rows)
    assert np.abs(one["O"].reshape(-1, w1.d)[rows] - O_ref).max() <= O_TOL


# ------------------------------------------------------------------ committed oracle snapshots (tests/golden)
def _fixtures():
    import importlib.util
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "make_fixtures.py")
    spec = importlib.util.spec_from_file_location("make_fixtures", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


FIX = _fixtures()


@pytest.mark.parametrize("case", FIX.CASES, ids=[c[0] for c in FIX.CASES])
def test_hip_path_matches_the_committed_oracle_snapshot(case):
    """The snapshot was written by the oracle alone; the HIP path must give the same code bytes
    (over the real rows; the padding is zero), the same scales and K means bit for bit, and the
    sampled O rows within the O bar."""
    name, base, kw, rows = case
    w = FIX.workload(name, base, kw)
    fx = {}
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", name + ".txt")) as f:
        for line in f:
            if not line.startswith("#"):
                key, rest = line.rstrip("\n").split(" ", 1)
                fx[key] = rest
    Q, K, V = synth.make_inputs(w)
    g = run_gpu(w, Q, K, V)
    for key, n in (("q_codes", w.N), ("k_codes", w.Nkv), ("v_codes", w.Nkv)):
        real, pad = np.split(g[key], [n], axis=2)
        assert FIX.digest(real) == fx[key].split()[-1], key
        assert not pad.any(), f"{key} padding"
    for key, n in (("q_scale", -(-w.N // w.blk_q)), ("k_scale", -(-w.Nkv // w.blk_k))):
        assert FIX.hexf(g[key][:, :, :n]) == fx[key], key
    for key in ("k_mean", "v_scale"):
        assert FIX.hexf(g[key]) == fx[key], key
    O = g["O"].reshape(-1, w.d)
    for r in rows:
        ref = np.array([float.fromhex(x) for x in fx[f"O[{r}]"].split()])
        assert np.abs(O[r] - ref).max() <= O_TOL, r


# ------------------------------------------------------------------ decode (split-KV) over a quantized cache
DECODE = {
    # name: (workload overrides, kv_chunk, layout)
    "gqa4-one-query-ragged-1000": (dict(base="llm-prefill-4k-causal", B=2, H=8, Hkv_=2, N=1, Nkv_=1000), 128, "bhnd"),
    "gqa8-four-queries-noncausal": (dict(base="video-dit-32k", B=1, H=16, Hkv_=2, N=4, Nkv_=4096), 256, "bhnd"),
    "gqa2-two-row-groups-fine-d64": (dict(base="vit-2k-f16", B=1, H=4, Hkv_=2, N=20, Nkv_=333, causal=True, blk_q=32,
                                          blk_k=16), 64, "bnhd"),
    "mha-tiny-cache-default-split": (dict(base="vit-2k-f16", B=3, H=4, N=1, Nkv_=70, causal=True), 0, "bhnd"),
    "late-chunk-invisible-to-early-rows": (dict(base="llm-prefill-4k-causal", B=1, H=1, N=40, Nkv_=130), 64, "bhnd"),
    "outliers-gqa-k32": (dict(base="long-prefill-128k-causal", H=8, Hkv_=2, N=2, Nkv_=3000, blk_k=32), 512, "bnhd"),
}


def decode_workload(name):
    kw, chunk, layout = DECODE[name]
    kw = dict(kw)
    return synth.WORKLOADS[kw.pop("base")].with_(name=name, **kw), chunk, layout


def run_gpu_decode(w, Q, K, V, kv_chunk, layout="bhnd", out_dtype=torch.float32):
    """Queries and cache quantized separately (quantize_q, quantize_k,
    quantize_v), then the split-KV decode; res["O"] is [B,H,N,d]."""
    sage = _sage()
    dev = torch.device("cuda:0")
    tok = layout == "bnhd"
    Qd, Kd, Vd = ((t.transpose(1, 2) if tok else t).contiguous().to(dev) for t in (Q, K, V))
    q = sage.quantize_q(Qd, w.blk_q, layout=layout)
    kc = sage.quantize_k(Kd, w.blk_k, layout=layout)
    vq = sage.quantize_v(Vd, layout=layout)
    if kv_chunk == 0:
        kv_chunk = sage.sage_decode_kv_chunk(w.B, w.H, w.Hkv, w.N, w.Nkv, w.d)
    O = sage.attn_decode(q, kc, vq, causal=w.causal, sm_scale=w.sm_scale, out_dtype=out_dtype, layout=layout,
                         kv_chunk=kv_chunk)
    torch.cuda.synchronize()
    res = {k: v.cpu().numpy() for k, v in list(q.items()) + list(kc.items()) if torch.is_tensor(v)}
    res["v_codes"] = sage.v_codes_to_natural(vq[0]).cpu().numpy()
    res["v_scale"] = vq[1].cpu().numpy()
    res["O"] = (O.transpose(1, 2) if tok else O).float().cpu().numpy()
    res["kv_chunk"] = kv_chunk
    res["dev"] = (q, kc, vq)
    return res


@pytest.mark.parametrize("name", list(DECODE))
def test_decode_against_the_split_oracle(name):
    w, chunk, layout = decode_workload(name)
    Q, K, V = synth.make_inputs(w)
    g = run_gpu_decode(w, Q, K, V, chunk, layout)
    qk, vc, vs = run_oracle_quant(w, Q, K, V)
    check_quant_bit_exact(g, qk, vc, vs)
    O_ref = orc.attn_rows_split(qk, vc, vs, w.blk_q, w.blk_k, w.causal, w.sm_scale, kv_chunk=g["kv_chunk"])
    O = g["O"].reshape(-1, w.d)
    err = np.abs(O - O_ref)
    assert err.max() <= O_TOL, f"max |O - oracle| = {err.max():.3g} at row {np.unravel_index(err.argmax(), err.shape)}"
    ex = orc.exact_attention(Q.float().numpy(), K.float().numpy(), V.float().numpy(), w.causal, w.sm_scale)
    assert cosine(O, ex) >= 0.995


@pytest.mark.parametrize("name", ["gqa4-one-query-ragged-1000", "gqa2-two-row-groups-fine-d64"])
def test_decode_with_one_split_is_the_attention_kernel(name):
    """kv_chunk covering the whole cache: per row the decode wave computes what
    the attention kernel computes (same tiles, same order), and the merge of one
    split is exact, so O agrees bit for bit."""
    sage = _sage()
    w, _, layout = decode_workload(name)
    Q, K, V = synth.make_inputs(w)
    g = run_gpu_decode(w, Q, K, V, -(-w.Nkv // 64) * 64, layout)
    q, kc, vq = g["dev"]
    qk = dict(q_codes=q["q_codes"], q_scale=q["q_scale"], k_codes=kc["k_codes"], k_scale=kc["k_scale"],
              blk_q=w.blk_q, blk_k=w.blk_k, Nq=w.N, Nkv=w.Nkv)
    O = sage.attn_fwd(qk, vq, causal=w.causal, sm_scale=w.sm_scale, layout=layout)
    torch.cuda.synchronize()
    O = (O.transpose(1, 2) if layout == "bnhd" else O).cpu().numpy()
    assert np.array_equal(O.view(np.uint32), g["O"].view(np.uint32))


def test_separate_quantize_calls_equal_the_fused_one():
    sage = _sage()
    w = small_ex_workload("chunk256-of-1024-causal-blkq64")
    Q, K, V = synth.make_inputs(w)
    Qd, Kd = Q.cuda(), K.cuda()
    both = sage.quantize_qk(Qd, Kd, w.blk_q, w.blk_k)
    q = sage.quantize_q(Qd, w.blk_q)
    kc = sage.quantize_k(Kd, w.blk_k)
    torch.cuda.synchronize()
    for key in ("q_codes", "q_scale"):
        assert torch.equal(both[key], q[key]), key
    for key in ("k_codes", "k_scale", "k_mean"):
        assert torch.equal(both[key], kc[key]), key


def test_decode_output_dtypes_round_the_fp32_result():
    w, chunk, layout = decode_workload("gqa8-four-queries-noncausal")
    Q, K, V = synth.make_inputs(w)
    g = run_gpu_decode(w, Q, K, V, chunk, layout)
    sage = _sage()
    q, kc, vq = g["dev"]
    for dt in (torch.bfloat16, torch.float16):
        o = sage.attn_decode(q, kc, vq, causal=w.causal, sm_scale=w.sm_scale, out_dtype=dt, kv_chunk=chunk)
        torch.cuda.synchronize()
        assert torch.equal(o.cpu().view(torch.int16), torch.from_numpy(g["O"]).to(dt).view(torch.int16))


# ------------------------------------------------------------------ 4-bit QK^T (E2M1, 32-channel power-of-two blocks)
QK4 = {
    "qk4-noncausal-bf16-d128": (dict(base="video-dit-32k", H=2, N=768), "bhnd"),
    "qk4-causal-gqa-d128": (dict(base="llm-prefill-4k-causal", B=1, H=8, Hkv_=2, N=512), "bnhd"),
    "qk4-ragged-chunk-causal-d64": (dict(base="vit-2k-f16", B=1, H=4, Hkv_=2, N=200, Nkv_=333, causal=True), "bhnd"),
    "qk4-outliers-causal": (dict(base="long-prefill-128k-causal", H=2, N=1024), "bhnd"),
    # Q smoothing (with a channel bias in Q where stated)
    "qk4s-noncausal-bf16-d128-qbias": (dict(base="video-dit-32k", H=2, N=768, smooth_q=True, q_bias_var=4.0), "bhnd"),
    "qk4s-causal-gqa-d128-qbias": (dict(base="llm-prefill-4k-causal", B=1, H=8, Hkv_=2, N=512, smooth_q=True,
                                        q_bias_var=4.0), "bnhd"),
    "qk4s-ragged-chunk-causal-d64-qbias": (dict(base="vit-2k-f16", B=1, H=4, Hkv_=2, N=200, Nkv_=333, causal=True,
                                                smooth_q=True, q_bias_var=2.0), "bhnd"),
    "qk4s-ragged-noncausal-d128-qbias": (dict(base="llm-prefill-4k-causal", B=2, H=4, N=300, causal=False,
                                              smooth_q=True, q_bias_var=4.0), "bnhd"),
    "qk4s-no-bias-d128": (dict(base="video-dit-32k", H=2, N=640, smooth_q=True), "bhnd"),
}
QK4_COS = 0.98   # 4-bit scores: about three bits fewer than INT8
FP4_COS = 0.96   # FP4 P~V as well: one mantissa bit for P~ and V (oracle on the video shape: 0.969)


def unpack4(codes):
    """[..., d/2] packed bytes -> [..., d] E2M1 codes (even channel in the low nibble)."""
    c = np.asarray(codes, np.uint8)
    return np.stack([c & 15, c >> 4], axis=-1).reshape(*c.shape[:-1], 2 * c.shape[-1])


def run_gpu_qk4(w, Q, K, V, layout="bhnd", dump_tiles=(), out_dtype=torch.float32, smooth_q=None):
    sage = _sage()
    dev = torch.device("cuda:0")
    tok = layout == "bnhd"
    Qd, Kd, Vd = ((t.transpose(1, 2) if tok else t).contiguous().to(dev) for t in (Q, K, V))
    qk4 = sage.quantize_qk4(Qd, Kd, layout=layout, smooth_q=w.smooth_q if smooth_q is None else smooth_q)
    vq = sage.quantize_v(Vd, layout=layout)
    dump = None
    if dump_tiles:
        sel = torch.tensor(list(dump_tiles), dtype=torch.int32, device=dev)
        s_d = torch.full((len(dump_tiles), 128, w.Nkv), S_SENTINEL, dtype=torch.int32, device=dev)
        p_d = torch.full((len(dump_tiles), 128, w.Nkv), P_SENTINEL, dtype=torch.uint8, device=dev)
        dump = (sel, s_d, p_d)
    O = sage.attn_fwd_qk4(qk4, vq, causal=w.causal, sm_scale=w.sm_scale, out_dtype=out_dtype, layout=layout, dump=dump)
    torch.cuda.synchronize()
    res = {k: v.cpu().numpy() for k, v in qk4.items() if torch.is_tensor(v)}
    res["v_codes"] = sage.v_codes_to_natural(vq[0]).cpu().numpy()
    res["v_scale"] = vq[1].cpu().numpy()
    res["O"] = (O.transpose(1, 2) if tok else O).float().cpu().numpy()
    if dump:
        res["s_dump"], res["p_dump"] = dump[1].cpu().numpy(), dump[2].cpu().numpy()
    return res


def check_qk4_quant(w, g, r):
    for key, n in (("q4", w.N), ("k4", w.Nkv)):
        codes, scale = unpack4(g[key + "_codes"]), g[key + "_scale"]
        assert np.array_equal(codes[:, :, :n], r[key + "_codes"]), key + " codes"
        assert np.array_equal(scale[:, :, :n], r[key + "_scale"]), key + " scales"
        assert not codes[:, :, n:].any() and not scale[:, :, n:].any(), key + " padding"
    assert np.array_equal(g["k_mean"].view(np.uint32), r["k_mean"].view(np.uint32))
    if "qm_codes" in r:   # Q smoothing: block means (fp32 bits), their INT8 codes and exponents, INT8 K
        nb = r["q_mean"].shape[2]
        assert np.array_equal(g["q_mean"][:, :, :nb].view(np.uint32), r["q_mean"].view(np.uint32)), "q_mean"
        assert np.array_equal(g["qm_codes"][:, :, :nb], r["qm_codes"]), "qm codes"
        assert np.array_equal(g["qm_scale"][:, :, :nb], r["qm_scale"]), "qm exponents"
        assert not g["q_mean"][:, :, nb:].any() and not g["qm_codes"][:, :, nb:].any(), "qm padding"
        assert (g["qm_scale"][:, :, nb:] == 127 - 63).all(), "qm padding exponents (all-zero blocks)"
        assert np.array_equal(g["k8_codes"][:, :, :w.Nkv], r["k8_codes"]), "k8 codes"
        assert np.array_equal(g["k8_scale"], r["k8_scale"]), "k8 exponents"
        assert not g["k8_codes"][:, :, w.Nkv:].any(), "k8 padding"


def qm_terms(r, w, rows):
    """The Q-smoothing term of flat query rows ``rows`` against every key, from the
    oracle's INT8 codes and exponents (exact in fp64): [len(rows), Nkv]."""
    nbq = r["qm_codes"].shape[2]
    qm = r["qm_codes"].reshape(w.B * w.H, nbq, w.d).astype(np.float64)
    k8 = r["k8_codes"].reshape(w.B * w.Hkv, w.Nkv, w.d).astype(np.float64)
    eq = r["qm_scale"].reshape(w.B * w.H, nbq).astype(np.int64) - 127
    ek = np.repeat(r["k8_scale"].reshape(w.B * w.Hkv, -1).astype(np.int64) - 127, 64, axis=1)[:, :w.Nkv]
    g = w.H // w.Hkv
    out = np.empty((len(rows), w.Nkv))
    for k, row in enumerate(rows):
        bh, i = divmod(int(row), w.N)
        out[k] = (k8[bh // g] @ qm[bh, i // 32]) * 2.0 ** (eq[bh, i // 32] + ek[bh // g])
    return out


@pytest.mark.parametrize("name", list(QK4))
def test_qk4_against_the_oracle(name):
    kw, layout = QK4[name]
    kw = dict(kw)
    w = synth.WORKLOADS[kw.pop("base")].with_(name=name, **kw)
    Q, K, V = synth.make_inputs(w)
    nqt = -(-w.N // 128)
    tiles = sorted({0, nqt - 1, (w.B * w.H - 1) * nqt})
    g = run_gpu_qk4(w, Q, K, V, layout, dump_tiles=tiles)
    r = orc.quantize_qk4(synth.bits(Q), synth.bits(K), w.dtype_code, smooth_q=w.smooth_q)
    vc, vs = orc.quantize_v(synth.bits(V), w.dtype_code)
    check_qk4_quant(w, g, r)
    assert np.array_equal(g["v_codes"][:, :, :w.Nkv], vc) and np.array_equal(g["v_scale"], vs)
    O_ref, P_ref = orc.attn_rows_qk4(r, vc, vs, w.causal, w.sm_scale, want_p=True)
    # scores: the matrix core's fp32 accumulation of the block products against the exact sum rounded once
    worst = 0.0
    for k, tid in enumerate(tiles):
        bh, qt = divmod(tid, nqt)
        nr = min(128, w.N - qt * 128)
        rows = bh * w.N + qt * 128 + np.arange(nr)
        s_ref = orc.qk4_scores(r, rows)
        s_got = g["s_dump"][k][:nr]
        written = s_got != S_SENTINEL
        i = qt * 128 + np.arange(nr)[:, None]
        j = np.arange(w.Nkv)[None, :]
        visible = (j <= i + (w.Nkv - w.N)) if w.causal else np.ones_like(written)
        assert written[visible].all()
        sg = s_got.view(np.float32)
        scale = np.abs(s_ref).max(axis=1, keepdims=True)
        err = np.abs(sg.astype(np.float64) - s_ref)
        dev = err / np.maximum(scale, 1e-30)
        worst = max(worst, float(dev[written].max()))
        if w.smooth_q:
            # the mean's term is exact in fp32 (integer sum on the INT8 matrix core, one exact fma);
            # the FP4 products are added to it in fp32, so each of the two 64-channel instructions
            # rounds at the magnitude of the term plus its partial sum
            T = np.abs(qm_terms(r, w, rows))
            bound = 2.0 ** -18 * scale + 2.0 ** -22 * T
            ratio = float((err / (2.0 ** -18 * scale + 2.0 ** -22 * T))[written].max())
            print(f"{name}: worst score error {ratio:.3g} of its bound")
            assert (err[written] <= bound[written]).all(), f"score error {ratio:.3g} of its bound"
        else:
            assert (dev[written] <= 2.0 ** -18).all(), f"score deviation {dev[written].max():.3g} of the row max"
        check_p_codes(g["p_dump"][k][:nr], P_ref[rows], visible, flip_frac=P_FLIP_FRAC)
    print(f"{name}: worst score deviation {worst:.3g} of the row max")
    O = g["O"].reshape(-1, w.d)
    err = np.abs(O - O_ref)
    print(f"{name}: max |O - oracle| {err.max():.3g}")
    assert err.max() <= O_TOL, f"max |O - oracle| = {err.max():.3g}"
    ex = orc.exact_attention(Q.float().numpy(), K.float().numpy(), V.float().numpy(), w.causal, w.sm_scale)
    assert cosine(O, ex) >= QK4_COS
    if w.smooth_q and w.q_bias_var:   # smoothing must beat the plain 4-bit path on biased queries
        plain = run_gpu_qk4(w, Q, K, V, layout, smooth_q=False)["O"].reshape(-1, w.d)
        print(f"{name}: cosine vs fp64 {cosine(O, ex):.5f} smoothed, {cosine(plain, ex):.5f} plain")
        assert cosine(O, ex) > cosine(plain, ex)


@pytest.mark.gpu
def test_qk4_smoothing_degenerate_cases():
    """One query per head: its block mean is the row itself, the smoothed
    codes are all zero and the scores are the mean's term alone (against the
    oracle).  Q = 0: mean, codes and scores all zero, so O is the plain mean
    of the dequantized V rows (a closed form)."""
    base = synth.WORKLOADS["vit-2k-f16"].with_(B=1, H=4, Hkv_=2, N=1, Nkv_=200, smooth_q=True, q_bias_var=4.0)
    Q, K, V = synth.make_inputs(base)
    g = run_gpu_qk4(base, Q, K, V)
    r = orc.quantize_qk4(synth.bits(Q), synth.bits(K), base.dtype_code, smooth_q=True)
    check_qk4_quant(base, g, r)
    assert not unpack4(g["q4_codes"])[:, :, 0].any()   # q - mean(q) = +0 for a one-row block
    vc, vs = orc.quantize_v(synth.bits(V), base.dtype_code)
    O_ref = orc.attn_rows_qk4(r, vc, vs, False, base.sm_scale)
    assert np.abs(g["O"].reshape(-1, base.d) - O_ref).max() <= O_TOL

    zq = base.with_(N=64, q_bias_var=0.0)
    Q, K, V = synth.make_inputs(zq)
    Q = torch.zeros_like(Q)
    g = run_gpu_qk4(zq, Q, K, V)
    assert not g["q_mean"].any() and not g["qm_codes"].any() and not unpack4(g["q4_codes"]).any()
    vc, vs = orc.quantize_v(synth.bits(V), zq.dtype_code)
    deq = orc.e4m3_decode(vc) * vs[:, :, None, :].astype(np.float64)        # [B, Hkv, Nkv, d]
    want = np.repeat(deq.mean(axis=2), zq.H // zq.Hkv, axis=1)              # per query head
    O = g["O"].reshape(zq.B, zq.H, zq.N, zq.d)
    assert np.abs(O - want[:, :, None, :]).max() <= 1e-5 * max(1.0, np.abs(want).max())


# ------------------------------------------------------------------ FP4 attention (FP4 QK^T and FP4 P~V)
FP4 = {
    "fp4-noncausal-bf16-d128": (dict(base="video-dit-32k", H=2, N=768), "bhnd"),
    "fp4-causal-gqa-d128": (dict(base="llm-prefill-4k-causal", B=1, H=8, Hkv_=2, N=512), "bnhd"),
    "fp4-ragged-chunk-causal-d64": (dict(base="vit-2k-f16", B=1, H=4, Hkv_=2, N=200, Nkv_=333, causal=True), "bhnd"),
    "fp4-ragged-noncausal-d64": (dict(base="vit-2k-f16", B=2, H=2, N=300), "bnhd"),
    "fp4-causal-d64": (dict(base="vit-2k-f16", B=1, H=4, N=512, causal=True), "bhnd"),
    "fp4-outliers-causal": (dict(base="long-prefill-128k-causal", H=2, N=1024), "bhnd"),
}


def run_gpu_fp4(w, Q, K, V, layout="bhnd", dump_tiles=(), out_dtype=torch.float32):
    sage = _sage()
    dev = torch.device("cuda:0")
    tok = layout == "bnhd"
    Qd, Kd, Vd = ((t.transpose(1, 2) if tok else t).contiguous().to(dev) for t in (Q, K, V))
    qk4 = sage.quantize_qk4(Qd, Kd, layout=layout)
    v4 = sage.quantize_v4(Vd, layout=layout)
    dump = None
    if dump_tiles:
        sel = torch.tensor(list(dump_tiles), dtype=torch.int32, device=dev)
        s_d = torch.full((len(dump_tiles), 128, w.Nkv), S_SENTINEL, dtype=torch.int32, device=dev)
        p_d = torch.full((len(dump_tiles), 128, w.Nkv), P_SENTINEL, dtype=torch.uint8, device=dev)
        dump = (sel, s_d, p_d)
    O = sage.attn_fwd_fp4(qk4, v4, causal=w.causal, sm_scale=w.sm_scale, out_dtype=out_dtype, layout=layout, dump=dump)
    torch.cuda.synchronize()
    res = {k: v.cpu().numpy() for k, v in qk4.items() if torch.is_tensor(v)}
    vn, vsn = sage.v4_to_natural(v4)
    res["v4_codes"], res["v4_scale"] = vn.cpu().numpy(), vsn.cpu().numpy()
    res["O"] = (O.transpose(1, 2) if tok else O).float().cpu().numpy()
    if dump:
        res["s_dump"], res["p_dump"] = dump[1].cpu().numpy(), dump[2].cpu().numpy()
    return res


def check_fp4_quant(w, g, Q, K, V):
    """Q/K codes as the 4-bit path; V codes and scales bit-exact, padding zero."""
    r = orc.quantize_qk4(synth.bits(Q), synth.bits(K), w.dtype_code)
    check_qk4_quant(w, g, r)
    vc, vs = orc.quantize_v4(synth.bits(V), w.dtype_code)
    nb = vs.shape[2]
    assert np.array_equal(g["v4_codes"][:, :, :w.Nkv], vc), "v4 codes"
    assert not g["v4_codes"][:, :, w.Nkv:].any(), "v4 padding"
    assert np.array_equal(g["v4_scale"][:, :, :nb], vs), "v4 scales"
    assert not g["v4_scale"][:, :, nb:].any(), "v4 padding scales"
    return r, (vc, vs)


@pytest.mark.parametrize("name", list(FP4))
def test_fp4_against_the_oracle(name):
    kw, layout = FP4[name]
    kw = dict(kw)
    w = synth.WORKLOADS[kw.pop("base")].with_(name=name, qk4=True, pv4=True, **kw)
    Q, K, V = synth.make_inputs(w)
    nqt = -(-w.N // 128)
    tiles = sorted({0, nqt - 1, (w.B * w.H - 1) * nqt})
    g = run_gpu_fp4(w, Q, K, V, layout, dump_tiles=tiles)
    r, v4 = check_fp4_quant(w, g, Q, K, V)
    O_ref, P_ref = orc.attn_rows_fp4(r, *v4, w.causal, w.sm_scale, want_p=True)
    flips = 0
    for k, tid in enumerate(tiles):
        bh, qt = divmod(tid, nqt)
        nr = min(128, w.N - qt * 128)
        rows = bh * w.N + qt * 128 + np.arange(nr)
        s_ref = orc.qk4_scores(r, rows)
        s_got = g["s_dump"][k][:nr]
        written = s_got != S_SENTINEL
        i = qt * 128 + np.arange(nr)[:, None]
        j = np.arange(w.Nkv)[None, :]
        visible = (j <= i + (w.Nkv - w.N)) if w.causal else np.ones_like(written)
        assert written[visible].all()
        dev = np.abs(s_got.view(np.float32).astype(np.float64) - s_ref) / np.maximum(
            np.abs(s_ref).max(axis=1, keepdims=True), 1e-30)
        assert (dev[written] <= 2.0 ** -18).all(), f"score deviation {dev[written].max():.3g} of the row max"
        # E2M1 codes of P~ (0..15; P~ >= 0, so 0..7): equal except one-step flips at rounding ties
        flips += check_p_codes(g["p_dump"][k][:nr], P_ref[rows], visible)
    O = g["O"].reshape(-1, w.d)
    err = np.abs(O - O_ref)
    ex = orc.exact_attention(Q.float().numpy(), K.float().numpy(), V.float().numpy(), w.causal, w.sm_scale)
    print(f"{name}: max |O - oracle| {err.max():.3g}, P^ flips {flips}, cosine vs fp64 {cosine(O, ex):.5f}")
    assert err.max() <= O_TOL, f"max |O - oracle| = {err.max():.3g}"
    assert cosine(O, ex) >= FP4_COS


# Seeded sweeps of the other entry points: split-KV decode (few queries against a cache, any
# kv_chunk), 4-bit QK^T (half of them with Q smoothing) and FP4 attention.  V outlier channels are
# drawn only with sm_scale = 1/sqrt(d), sharper softmaxes (sm_scale up to 0.3) only without them.
# Decode and the 4-bit scores keep P~V on the FP8 instruction, so their bar is that of the INT8
# sweep, max(2e-3, 7 * 2^-13 * A), with A from the single-pass FP8 P~ codes (for decode the split
# reweights the same V rows, equal up to the FP8 rounding of the weights).  A 4-bit case
# concentrating 69% of a row on one key exceeded 2e-3 that way on a x8 outlier channel (2.93e-3,
# A = 13.2).  FP4 P~V runs on the FP4 instruction, whose inner window is not measured here: its
# cases draw no outlier channels and keep the plain 2e-3.
def _random_variant_cases(n=12, seed=4711):
    rng = np.random.default_rng(seed)
    cases = []
    for kind in ("decode", "qk4", "fp4"):
        for i in range(n):
            d = int(rng.choice([64, 128]))
            Hkv = int(rng.integers(1, 4))
            g = int(rng.choice([1, 2, 4, 8]))
            causal = bool(rng.integers(0, 2))
            outliers = bool(rng.random() < 0.35) and kind != "fp4"
            sm = float(np.float32(1.0 / np.sqrt(d))) if outliers else float(np.float32(rng.uniform(0.05, 0.3)))
            if kind == "decode":
                Nq = int(rng.integers(1, 9))
                Nkv = int(rng.integers(Nq, 3000))
            else:
                Nkv = int(rng.integers(1, 700))
                Nq = int(rng.integers(1, Nkv + 1)) if causal or rng.random() < 0.5 else int(rng.integers(1, 700))
            kw = dict(name=f"{kind}{i}", B=int(rng.integers(1, 4 if kind == "decode" else 3)), H=Hkv * g, Hkv_=Hkv,
                      N=Nq, Nkv_=Nkv, d=d, dtype=str(rng.choice(["float16", "bfloat16"])), causal=causal,
                      blk_q=int(rng.choice([32, 64, 128])), blk_k=int(rng.choice([16, 32, 64])),
                      bias_var=float(rng.choice([0.0, 2.0, 4.0])), sm_scale=sm,
                      v_outlier_channels=d // 10 if outliers else 0, v_outlier_scale=8.0,
                      seed=int(rng.integers(0, 1 << 30)))
            if kind == "qk4":
                kw.update(qk4=True, smooth_q=bool(i % 2), q_bias_var=float(rng.choice([0.0, 4.0])))
            if kind == "fp4":
                kw.update(qk4=True, pv4=True)
            extra = dict(layout=str(rng.choice(["bhnd", "bnhd"])),
                         kv_chunk=int(rng.choice([0, 64, 128, 256, 512, 1024])) if kind == "decode" else 0)
            cases.append((kind, kw, extra))
    return cases


RANDOM_VARIANT_CASES = {kw["name"]: (kind, kw, extra) for kind, kw, extra in _random_variant_cases()}


@pytest.mark.parametrize("name", list(RANDOM_VARIANT_CASES))
def test_seeded_random_variant_shapes_against_the_oracle(name):
    kind, kw, extra = RANDOM_VARIANT_CASES[name]
    w = synth.Workload(**kw)
    print(f"{name}: {kw} {extra}", flush=True)
    Q, K, V = synth.make_inputs(w)
    if kind == "decode":
        g = run_gpu_decode(w, Q, K, V, extra["kv_chunk"], extra["layout"])
        qk, vc, vs = run_oracle_quant(w, Q, K, V)
        check_quant_bit_exact(g, qk, vc, vs)
        O_ref = orc.attn_rows_split(qk, vc, vs, w.blk_q, w.blk_k, w.causal, w.sm_scale, kv_chunk=g["kv_chunk"])
        P_ref = orc.attn_rows(qk, vc, vs, w.blk_q, w.blk_k, w.causal, w.sm_scale, want_p=True)[1]
        cos_min = 0.995
    elif kind == "qk4":
        g = run_gpu_qk4(w, Q, K, V, extra["layout"])
        r = orc.quantize_qk4(synth.bits(Q), synth.bits(K), w.dtype_code, smooth_q=w.smooth_q)
        vc, vs = orc.quantize_v(synth.bits(V), w.dtype_code)
        check_qk4_quant(w, g, r)
        assert np.array_equal(g["v_codes"][:, :, :w.Nkv], vc) and np.array_equal(g["v_scale"], vs)
        O_ref, P_ref = orc.attn_rows_qk4(r, vc, vs, w.causal, w.sm_scale, want_p=True)
    else:
        g = run_gpu_fp4(w, Q, K, V, extra["layout"])
        r, v4 = check_fp4_quant(w, g, Q, K, V)
        O_ref = orc.attn_rows_fp4(r, *v4, w.causal, w.sm_scale)
    O = g["O"].reshape(-1, w.d)
    err = np.abs(O.astype(np.float64) - O_ref)
    if kind == "fp4":
        bar = np.full_like(err, O_TOL)
    else:
        bar = np.maximum(O_TOL, INNER_MAX * weighted_abs_v(P_ref, np.arange(w.B * w.H * w.N), vc, vs, w))
    worst = np.unravel_index(int(np.argmax(err / bar)), err.shape)
    ex = orc.exact_attention(Q.float().numpy(), K.float().numpy(), V.float().numpy(), w.causal, w.sm_scale)
    cs, cs_ref = cosine(O, ex), cosine(O_ref, ex)
    print(f"{name}: max |O - oracle| {err.max():.3g} ({(err > O_TOL).sum()} elements above 2e-3; worst "
          f"{err[worst]:.3g} against the bar {bar[worst]:.3g}), cosine vs fp64 {cs:.5f} (oracle {cs_ref:.5f})",
          flush=True)
    assert (err <= bar).all(), f"|O - oracle| {err[worst]:.3g} above the bar {bar[worst]:.3g} at {worst}"
    # The INT8 path's accuracy bound holds on any of these inputs; the 4-bit scores' accuracy is
    # the method's and varies with the draw (a short causal head gave 0.962), so there the GPU
    # must match the oracle's cosine instead
    if kind == "decode":
        assert cs >= cos_min
    else:
        assert cs >= cs_ref - 1e-3


def test_fp4_q_zero_and_constant_v_closed_forms():
    """Q = 0: every P~ is 2^8 and lands on the E2M1 value 4, so O is the plain
    mean of the dequantized FP4 V rows (causal: of the visible ones).  V a
    power of two per channel: O equals it up to the matrix core's windowed
    inner sums (the P~V and the row-sum instructions truncate their block
    sums independently; the oracle, summing exactly, gives it exactly)."""
    sage = _sage()
    for causal in (False, True):
        w = synth.WORKLOADS["vit-2k-f16"].with_(B=1, H=4, Hkv_=2, N=70, Nkv_=200, causal=causal, qk4=True, pv4=True)
        Q, K, V = synth.make_inputs(w)
        Q = torch.zeros_like(Q)
        g = run_gpu_fp4(w, Q, K, V)
        vn = g["v4_codes"][:, :, :w.Nkv]
        sc = np.repeat(g["v4_scale"], 32, axis=2)[:, :, :w.Nkv].astype(np.float64)
        deq = orc.e2m1_decode(vn) * 2.0 ** (sc - 127)                          # [B, Hkv, Nkv, d]
        O = g["O"].reshape(w.B, w.H, w.N, w.d)
        for h in range(w.H):
            for i in range(w.N):
                last = i + w.Nkv - w.N if causal else w.Nkv - 1
                want = deq[0, h // 2, :last + 1].mean(axis=0)
                assert np.abs(O[0, h, i] - want).max() <= 2e-6 * max(1.0, np.abs(want).max()), (causal, h, i)
        c = (2.0 ** np.random.default_rng(3).integers(-4, 4, w.d)).astype(np.float32)
        Vc = torch.from_numpy(np.broadcast_to(c, V.shape).copy()).to(V.dtype)
        Q2, K2, _ = synth.make_inputs(w)
        g2 = run_gpu_fp4(w, Q2, K2, Vc)
        rel = np.abs(g2["O"] / np.broadcast_to(c, g2["O"].shape) - 1.0).max()
        assert rel <= 2.0 ** -20, (causal, rel)
    del sage


@pytest.mark.parametrize("dt", [torch.float16, torch.bfloat16])
def test_fp4_output_dtypes_round_the_fp32_result(dt):
    w = synth.WORKLOADS["llm-prefill-4k-causal"].with_(B=1, H=4, Hkv_=2, N=384, qk4=True, pv4=True)
    Q, K, V = synth.make_inputs(w)
    ref = torch.from_numpy(run_gpu_fp4(w, Q, K, V, "bnhd")["O"])
    got = torch.from_numpy(run_gpu_fp4(w, Q, K, V, "bnhd", out_dtype=dt)["O"])
    assert torch.equal(got, ref.to(dt).float())


@pytest.mark.gpu
def test_graph_capture_replays_match_eager():
    """The calls allocate nothing, set no memory and never synchronize, so a
    prefill step (quantize Q/K, quantize V, attention; also with the fused
    quantize call, in FP4, and with Q smoothing) and a decode step (quantize
    the new queries, split-KV attention against a quantized cache) can be
    captured in a HIP graph.  Every replay, with eager work and
    synchronizations in between, equals the eager result bit for bit."""
    sage = _sage()
    dev = torch.device("cuda:0")
    w = synth.WORKLOADS["llm-prefill-4k-causal"].with_(B=1, H=4, Hkv_=2, N=512)
    Q, K, V = (t.to(dev) for t in synth.make_inputs(w))

    def prefill():
        qk = sage.quantize_qk(Q, K, w.blk_q, w.blk_k)
        vq = sage.quantize_v(V)
        return sage.attn_fwd(qk, vq, causal=True, sm_scale=w.sm_scale, out_dtype=torch.float32)

    def prefill_fused():   # the two quantize calls in one (three launches)
        qk, vq = sage.quantize_qkv(Q, K, V, w.blk_q, w.blk_k)
        return sage.attn_fwd(qk, vq, causal=True, sm_scale=w.sm_scale, out_dtype=torch.float32)

    def prefill_fp4():     # FP4 QK^T and FP4 P~V
        return sage.attn_fwd_fp4(sage.quantize_qk4(Q, K), sage.quantize_v4(V), causal=True, sm_scale=w.sm_scale)

    def prefill_qk4s():    # 4-bit QK^T with Q smoothing
        return sage.attn_fwd_qk4(sage.quantize_qk4(Q, K, smooth_q=True), sage.quantize_v(V), causal=True,
                                 sm_scale=w.sm_scale)

    kc = sage.quantize_k(K)
    vq = sage.quantize_v(V)
    Qn = Q[:, :, -3:].contiguous()

    def decode():
        q = sage.quantize_q(Qn)
        return sage.attn_decode(q, kc, vq, causal=True, sm_scale=w.sm_scale, kv_chunk=128)

    for step in (prefill, prefill_fused, prefill_fp4, prefill_qk4s, decode):
        ref = step().clone()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            step()   # warm up on the side stream before capture
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            out = step()
        for _ in range(3):
            out.fill_(float("nan"))
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, ref), step.__name__
            eager = step()      # the program's own eager work between replays
            torch.cuda.synchronize()
            assert torch.equal(eager, ref)


@pytest.mark.gpu
def test_fp8_conversion_at_every_midpoint():
    """The V path's FP8 conversion (the hardware convert) on exact e4m3 values,
    every midpoint between neighbours (ties to even), subnormals and both signs:
    with 448 in every channel the channel scale is exactly 1, so each code is
    the conversion of the input itself.  Checked against the oracle's encoder
    and against torch's CPU float8_e4m3fn conversion."""
    sage = _sage()
    mags = np.unique(np.abs(orc.e4m3_decode(np.arange(256, dtype=np.uint8))))
    mags = mags[np.isfinite(mags) & (mags <= 448)]
    mids = (mags[1:] + mags[:-1]) / 2
    vals = np.concatenate([mags, mids, -mags, -mids])
    assert np.array_equal(vals.astype(np.float16).astype(np.float64), vals)   # all exact in f16
    d, N = 64, 64 * -(-(len(vals) + 1) // 64)
    V = np.zeros((1, 1, N, d), np.float32)
    V[0, 0, 0, :] = 448.0
    for c in range(d):
        V[0, 0, 1:1 + len(vals), c] = np.roll(vals, 7 * c)
    Vt = torch.from_numpy(V).to(torch.float16)
    vq = sage.quantize_v(Vt.to("cuda:0"))
    torch.cuda.synchronize()
    codes = sage.v_codes_to_natural(vq[0]).cpu().numpy()[0, 0]
    assert np.array_equal(vq[1].cpu().numpy(), np.ones((1, 1, d), np.float32))
    want_oracle = orc.e4m3_encode(V[0, 0].ravel()).reshape(N, d)
    want_torch = Vt[0, 0].float().to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, want_oracle)
    assert np.array_equal(codes, want_torch)


@pytest.mark.gpu
@pytest.mark.parametrize("smooth", [False, True])
def test_qk4_output_dtypes_round_the_fp32_result(smooth):
    """The 4-bit variants (plain and Q-smoothed) share the epilogue: f16 and
    bf16 outputs are the round-to-nearest-even of the fp32 output."""
    w = synth.WORKLOADS["llm-prefill-4k-causal"].with_(B=1, H=4, Hkv_=2, N=384, smooth_q=smooth,
                                                       q_bias_var=4.0 if smooth else 0.0)
    Q, K, V = synth.make_inputs(w)
    ref = torch.from_numpy(run_gpu_qk4(w, Q, K, V, "bnhd")["O"])
    for dt in (torch.bfloat16, torch.float16):
        got = torch.from_numpy(run_gpu_qk4(w, Q, K, V, "bnhd", out_dtype=dt)["O"])
        exp = ref.to(dt).float()
        assert torch.equal(got, exp), f"{dt}: {(got != exp).sum().item()} mismatches"


@pytest.mark.gpu
def test_binding_rejects_mismatched_tensors_before_launching():
    """The C ABI cannot see buffer sizes, so the tensor helpers check every
    tensor they pass: V codes of another length, an output of the wrong shape
    or layout, a workspace on the host, Q/K of different dtypes, queries and a
    cache of different batches.  Each raises before any kernel is launched;
    the matching call still runs."""
    sage = _sage()
    dev = torch.device("cuda:0")
    w = synth.WORKLOADS["llm-prefill-4k-causal"].with_(B=2, H=2, N=256)
    Q, K, V = (t.to(dev) for t in synth.make_inputs(w))
    qk = sage.quantize_qk(Q, K)
    vq = sage.quantize_v(V)
    with pytest.raises(ValueError):
        sage.attn_fwd(qk, sage.quantize_v(V[:, :, :64].contiguous()))           # fewer keys than K
    with pytest.raises(ValueError):
        sage.attn_fwd(qk, vq, out=torch.empty(16, dtype=torch.float32, device=dev))
    with pytest.raises(ValueError):                                              # [B,N,H,d] view, not contiguous
        sage.attn_fwd(qk, vq, out=torch.empty(2, 256, 2, 128, device=dev).transpose(1, 2))
    with pytest.raises(ValueError):
        sage.quantize_qk(Q, K, workspace=torch.empty(1 << 20, dtype=torch.uint8))
    with pytest.raises(ValueError):
        sage.quantize_qk4(Q, K.to(torch.float16))
    with pytest.raises(ValueError):
        sage.attn_fwd_qk4(sage.quantize_qk4(Q, K), sage.quantize_v(V[:1].contiguous()))
    kc = sage.quantize_k(K)
    with pytest.raises(ValueError):
        sage.attn_decode(sage.quantize_q(Q[:1, :, -2:].contiguous()), kc, vq)
    out = torch.empty((2, 2, 256, 128), dtype=torch.bfloat16, device=dev)
    assert sage.attn_fwd(qk, vq, causal=True, out=out) is out
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
