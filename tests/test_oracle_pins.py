"""Pins for the CPU oracle: each check ties the oracle to something other than
itself (brute force, an independent library routine, exact rationals, a closed
form, or an invariance the mathematics fixes), so that a dropped term, a wrong
sign or index, or a transposed operand fails at least one of them."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import oracle as orc
from quantized_scaled_dot_amd import synth


def _f16_bits(a):
    return synth.bits(torch.from_numpy(np.asarray(a, np.float32)).to(torch.float16))


def _bf16_bits(a):
    return synth.bits(torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16))


def _f16_vals(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.float16).float().numpy()


# ------------------------------------------------------------------ e4m3 codec
def test_e4m3_decode_matches_torch_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = orc.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2  # S.1111.111 only
    assert np.array_equal(ours[~nan], ref[~nan])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6


def _nearest_even_bruteforce(x):
    """Nearest finite e4m3 value by exhaustive search; ties to the even code."""
    codes = np.arange(0, 127, dtype=np.uint8)  # positive finite codes
    vals = orc.e4m3_decode(codes)
    a = abs(float(x))
    if a >= 448.0:
        c = 0x7E
    else:
        dist = np.abs(vals - a)
        best = np.flatnonzero(dist == dist.min())
        c = int(best[0]) if len(best) == 1 else int(best[best % 2 == 0][0])
    return c | (0x80 if math.copysign(1.0, x) < 0 else 0)


def test_e4m3_encode_midpoints_ties_to_even_and_saturation():
    vals = orc.e4m3_decode(np.arange(0, 127, dtype=np.uint8))
    xs = []
    for k in range(126):
        mid = np.float32((vals[k] + vals[k + 1]) / 2)
        v = np.float32(vals[k])
        xs += [v, np.nextafter(v, np.float32(1e30)), np.nextafter(v, np.float32(-1e30)),
               mid, np.nextafter(mid, np.float32(1e30)), np.nextafter(mid, np.float32(-1e30))]
    xs += [np.float32(v) for v in (448, 449, 463.99, 464, 1e6, 3e38, 0, 2 ** -10, 3 * 2 ** -11, 2 ** -11, 1e-30)]
    # the whole saturating range: past the largest finite value every input
    # maps to 448, including the band where the next binade's codes would be NaN
    big = np.concatenate([np.arange(448.0, 512.0, 0.125), 2.0 ** np.arange(9, 128)]).astype(np.float32)
    xs += list(big) + list(np.nextafter(big, np.float32(1e30))) + list(np.nextafter(big, np.float32(0)))
    xs = np.array(xs, np.float32)
    xs = np.concatenate([xs, -xs])
    got = orc.e4m3_encode(xs)
    ref = np.array([_nearest_even_bruteforce(float(x)) for x in xs], np.uint8)
    assert np.array_equal(got, ref)
    assert orc.e4m3_encode(np.array([np.nan], np.float32))[0] == 0x7F


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(200000).astype(np.float32) * 40,
                        rng.uniform(-448, 448, 200000).astype(np.float32),
                        (rng.standard_normal(100000) * 1e-2).astype(np.float32)])
    ours = orc.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


# ------------------------------------------------------------------ softmax exp2
def test_exp2_exact_points():
    # powers of two are exact, down to the smallest subnormal; below it, zero
    ints = np.arange(-149, 128, dtype=np.float32)
    assert [float(v) for v in orc.exp2f(ints)] == [2.0 ** int(k) for k in ints]
    assert orc.exp2f(np.array([-150.5, -1e4, -1e30, -np.inf], np.float32)).tolist() == [0, 0, 0, 0]
    assert orc.exp2f(np.array([0.0, -0.0], np.float32)).tolist() == [1.0, 1.0]


def test_exp2_against_square_roots_and_logs():
    # 2^(1/2) and 2^(-1/2) are sqrt(2) and 1/sqrt(2), correctly rounded
    got = orc.exp2f(np.array([0.5, -0.5, 8.5], np.float32))
    assert got[0] == np.float32(np.sqrt(2.0)) and got[1] == np.float32(np.sqrt(0.5))
    assert got[2] == np.float32(256.0 * np.sqrt(2.0))
    # 2^(log2 x) returns x up to the rounding of log2 x to fp32 (|dt| <= 2^-24 |t|)
    x = np.array([3.0, 5.0, 10.0, 0.1, 1e-3, 200.0])
    t = np.log2(x).astype(np.float32)
    rel = np.abs(orc.exp2f(t) / x - 1)
    assert (rel <= np.abs(t) * 2.0 ** -24 * np.log(2) + 2.0 ** -24).all()


def test_exp2_shift_by_one_is_doubling_and_monotone():
    rng = np.random.default_rng(5)
    t = rng.uniform(-120, 120, 200_000).astype(np.float32)
    t1 = t + np.float32(1)
    keep = t1.astype(np.float64) - t.astype(np.float64) == 1.0   # t + 1 exact in fp32
    t, t1 = t[keep], t1[keep]
    assert t.size > 100_000
    a, b = orc.exp2f(t), orc.exp2f(t1)
    assert np.array_equal(b, a * np.float32(2))
    s = np.sort(rng.uniform(-30, 9, 500_000).astype(np.float32))
    y = orc.exp2f(s)
    assert (np.diff(y.astype(np.float64)) >= 0).all()
    # within half an fp32 ulp of the exact value (a spot check in long double)
    u = np.array([-0.3, 0.7, -17.123, 7.999], np.float32)
    exact = np.array([np.exp2(np.longdouble(v)) for v in u])
    err = np.abs(orc.exp2f(u).astype(np.longdouble) - exact)
    assert (err <= np.spacing(orc.exp2f(u)).astype(np.longdouble) / 2 * (1 + 1e-9)).all()


# ------------------------------------------------------------------ int32 QK^T
def test_qk_int32_against_bigint_bruteforce():
    rng = np.random.default_rng(2)
    B, H, N, d = 1, 2, 8, 64
    qc = rng.integers(-127, 128, (B, H, N, d), dtype=np.int8)
    kc = rng.integers(-127, 128, (B, H, N, d), dtype=np.int8)
    qc[0, 1, 3] = 127
    kc[0, 1, 5] = -127  # extreme products
    rows = np.array([0, 3, 7, N + 3, 2 * N - 1], np.int64)
    got = orc.qk_int32(qc, kc, rows)
    for r, row in enumerate(rows):
        bh, i = divmod(int(row), N)
        b, h = divmod(bh, H)
        for j in range(N):
            s = sum(int(qc[b, h, i, c]) * int(kc[b, h, j, c]) for c in range(d))
            assert got[r, j] == s


# ------------------------------------------------------------------ K mean
def test_kmean_equals_exact_rational_mean_f16():
    rng = np.random.default_rng(3)
    B, H, N, d = 1, 2, 96, 16
    k = rng.standard_normal((B, H, N, d)).astype(np.float32) * 3 + 1.5
    kb = _f16_bits(k)
    kv = _f16_vals(k)
    mu, sums = orc.kmean(kb, 0)
    for b in range(B):
        for h in range(H):
            for c in range(d):
                exact = sum(Fraction(float(x)) for x in kv[b, h, :, c])
                # every float16 is a multiple of 2^-24: the fixed-point sum is the exact sum
                assert Fraction(int(sums[b, h, c]), 2 ** 24) == exact
                m = exact / N
                rn = np.float32(float(m))  # round the exact mean once (via double)
                assert abs(Fraction(float(mu[b, h, c])) - m) <= Fraction(float(np.spacing(rn)))
                assert mu[b, h, c] == np.float32(np.float64(float(exact)) / N)


def test_kmean_constant_channels_and_bf16_tiny_values():
    B, H, N, d = 1, 1, 64, 8
    k = np.tile(np.array([0.5, -3.25, 1024.0, 0, 7.0, -0.125, 2.0 ** -20, 96.0], np.float32), (B, H, N, 1))
    for conv, dt in ((_f16_bits, 0), (_bf16_bits, 1)):
        mu, _ = orc.kmean(conv(k), dt)
        kv = torch.from_numpy(k).to(torch.float16 if dt == 0 else torch.bfloat16).float().numpy()
        expect = kv[0, 0, 0].copy()
        if dt == 1:  # bfloat16 values below 2^-24 granularity are truncated in the fixed-point sum
            expect[6] = np.float32(0.0) if kv[0, 0, 0, 6] < 2.0 ** -24 else expect[6]
        assert np.array_equal(mu[0, 0], expect)


def test_kmean_at_the_length_limit_with_saturated_channels():
    """N = 2^19 tokens (the C ABI's limit) with channels far beyond the fixed-point clamp of
    2^19 on every token: each term is 2^43, so the int64 sum is exactly +-2^62 (no overflow)
    and the mean is the clamp value itself; ordinary channels keep their exact mean."""
    N, d = 1 << 19, 4
    k = np.zeros((1, 1, N, d), np.float32)
    k[..., 0] = 2.0 ** 100          # bfloat16 keeps it; far past the clamp
    k[..., 1] = -3.0e38             # near the bfloat16 maximum
    k[..., 2] = 2.0 ** 19           # exactly at the clamp
    k[..., 3] = np.where(np.arange(N) % 2 == 0, 1.5, -0.5)
    mu, sums = orc.kmean(_bf16_bits(k), 1)
    assert sums[0, 0].tolist() == [2 ** 62, -(2 ** 62), 2 ** 62, (N // 2) * 2 ** 24]
    assert mu[0, 0].tolist() == [2.0 ** 19, -(2.0 ** 19), 2.0 ** 19, 0.5]


# ------------------------------------------------------------------ Q/K block quantizer
def _quantize(B=2, H=2, N=256, d=64, blk_q=64, blk_k=64, seed=4, dtype=0, scale=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, N, d)).astype(np.float32) * scale
    k = (rng.standard_normal((B, H, N, d)) + rng.standard_normal((B, H, 1, d)) * 2).astype(np.float32) * scale
    conv = _f16_bits if dtype == 0 else _bf16_bits
    return q, k, orc.quantize_qk(conv(q), conv(k), dtype, blk_q, blk_k)


def test_quantizer_roundtrip_bound_and_full_range():
    for dtype in (0, 1):
        q, k, r = _quantize(dtype=dtype)
        tdt = torch.float16 if dtype == 0 else torch.bfloat16
        qv = torch.from_numpy(q).to(tdt).float().numpy()
        kv = torch.from_numpy(k).to(tdt).float().numpy()
        ks = kv - r["k_mean"][:, :, None, :]  # smoothed K in fp32 (exact per element rounding)
        for x, codes, scale, blk in ((qv, r["q_codes"], r["q_scale"], 64), (ks, r["k_codes"], r["k_scale"], 64)):
            B, H, N, d = x.shape
            xb = x.reshape(B, H, N // blk, blk * d).astype(np.float64)
            cb = codes.reshape(B, H, N // blk, blk * d).astype(np.float64)
            dl = scale.astype(np.float64)[..., None]
            assert np.abs(codes).max() <= 127
            assert (np.abs(cb).max(axis=-1) == 127).all()  # every nonzero block uses the full range
            err = np.abs(xb - cb * dl)
            assert (err <= dl / 2 + 127 * dl * 2.0 ** -21).all()
            a = np.abs(xb).max(axis=-1, keepdims=True)
            assert np.array_equal(dl.astype(np.float32), (a.astype(np.float32) / np.float32(127)))


def test_quantizer_power_of_two_metamorphic():
    _, _, r0 = _quantize(seed=5)
    _, _, r1 = _quantize(seed=5, scale=8.0)
    _, _, r2 = _quantize(seed=5, scale=1 / 16)
    for r in (r1, r2):
        assert np.array_equal(r["q_codes"], r0["q_codes"]) and np.array_equal(r["k_codes"], r0["k_codes"])
    assert np.array_equal(r1["q_scale"], r0["q_scale"] * 8) and np.array_equal(r1["k_scale"], r0["k_scale"] * 8)
    assert np.array_equal(r2["q_scale"], r0["q_scale"] / 16)


def test_zero_block_gives_zero_scale_and_codes():
    B, H, N, d = 1, 1, 128, 64
    q = np.zeros((B, H, N, d), np.float32)
    q[0, 0, 64:] = 1.0
    k = np.ones((B, H, N, d), np.float32) * 3  # constant K: smoothed K is exactly 0
    r = orc.quantize_qk(_f16_bits(q), _f16_bits(k), 0, 64, 64)
    assert r["q_scale"][0, 0, 0] == 0 and (r["q_codes"][0, 0, :64] == 0).all()
    assert (r["q_codes"][0, 0, 64:] == 127).all()
    assert (r["k_scale"] == 0).all() and (r["k_codes"] == 0).all() and (r["k_mean"] == 3).all()


# ------------------------------------------------------------------ V quantizer
def test_v_quantizer_roundtrip_and_scales():
    rng = np.random.default_rng(6)
    B, H, N, d = 1, 2, 128, 32
    v = rng.standard_normal((B, H, N, d)).astype(np.float32)
    v[0, 1, :, 5] *= 8
    vv = _f16_vals(v).astype(np.float64)
    vc, vs = orc.quantize_v(_f16_bits(v), 0)
    a = np.abs(vv).max(axis=2)
    assert np.array_equal(vs, (a.astype(np.float32) / np.float32(448)))
    deq = orc.e4m3_decode(vc) * vs[:, :, None, :].astype(np.float64)
    err = np.abs(deq - vv)
    normal = np.abs(orc.e4m3_decode(vc)) >= 2.0 ** -6
    tol_norm = 2.0 ** -4 * np.abs(vv) * (1 + 2.0 ** -20)
    tol_sub = 2.0 ** -10 * np.broadcast_to(vs[:, :, None, :], vv.shape) * (1 + 2.0 ** -20)
    assert (err[normal] <= tol_norm[normal] + 1e-30).all()
    assert (err[~normal] <= tol_sub[~normal]).all()
    # each channel's largest magnitude maps to the top code
    assert (np.abs(orc.e4m3_decode(vc)).max(axis=2) == 448).all()


# ------------------------------------------------------------------ attention
def _small(w_kw, seed=0):
    w = synth.WORKLOADS["tiny-f16-256"].with_(**w_kw)
    Q, K, V = synth.make_inputs(w, seed=seed)
    return w, Q, K, V


def _run(w, Q, K, V, **kw):
    return orc.run(synth.bits(Q), synth.bits(K), synth.bits(V), w.dtype_code, w.blk_q, w.blk_k, w.causal,
                   w.sm_scale, **kw)


@pytest.mark.parametrize("kw", [dict(), dict(causal=True), dict(d=128, blk_q=128, dtype="bfloat16", causal=True),
                                dict(N=512, v_outlier_channels=6, v_outlier_scale=8.0, causal=True)])
def test_oracle_close_to_exact_fp64_attention(kw):
    w, Q, K, V = _small(kw)
    _, _, O = _run(w, Q, K, V)
    ref = orc.exact_attention(Q.float().numpy(), K.float().numpy(), V.float().numpy(), w.causal, w.sm_scale)
    O = O.astype(np.float64)
    cos = (O * ref).sum() / np.sqrt((O * O).sum() * (ref * ref).sum())
    assert cos >= 0.995
    # a dropped term or a wrong index moves the result far beyond FP8 noise
    assert np.abs(O - ref).max() < 0.25 * np.abs(ref).max()


def test_softmax_invariant_to_subtracting_the_k_mean_fp64():
    w, Q, K, V = _small({})
    mu, _ = orc.kmean(synth.bits(K), 0)
    Qf, Kf, Vf = (t.double().numpy() for t in (Q, K, V))
    a = orc.exact_attention(Qf, Kf, Vf, False, w.sm_scale)
    b = orc.exact_attention(Qf, Kf - mu[:, :, None, :].astype(np.float64), Vf, False, w.sm_scale)
    assert np.abs(a - b).max() < 1e-12


def test_k_bias_invariance_bit_exact_on_dyadic_grid():
    """On a dyadic grid the smoothing step removes a per-channel K bias exactly,
    so every code, scale and output is bit-identical with and without it."""
    rng = np.random.default_rng(7)
    B, H, N, d = 1, 2, 256, 64
    q = rng.integers(-512, 513, (B, H, N, d)) / 256.0
    k = rng.integers(-512, 513, (B, H, N, d)) / 256.0
    v = rng.integers(-512, 513, (B, H, N, d)) / 256.0
    bias = rng.integers(-900, 901, (B, H, 1, d)) / 256.0
    args = dict(dtype=0, blk_q=64, blk_k=64, causal=True, sm_scale=0.125)
    r0 = orc.run(_f16_bits(q), _f16_bits(k), _f16_bits(v), want_p=True, **args)
    r1 = orc.run(_f16_bits(q), _f16_bits(k + bias), _f16_bits(v), want_p=True, **args)
    assert np.array_equal(r1[0]["k_mean"], r0[0]["k_mean"] + bias[:, :, 0, :].astype(np.float32))
    for key in ("k_codes", "k_scale", "q_codes", "q_scale"):
        assert np.array_equal(r0[0][key], r1[0][key])
    assert np.array_equal(r0[2][1], r1[2][1])  # FP8 codes of P~
    assert np.array_equal(r0[2][0], r1[2][0])  # O bit for bit


def test_zero_q_gives_mean_of_dequantized_v():
    for causal in (False, True):
        w, Q, K, V = _small(dict(causal=causal))
        Q = torch.zeros_like(Q)
        qk, (vc, vs), (O, P) = _run(w, Q, K, V, want_p=True)
        assert (qk["q_codes"] == 0).all() and (qk["q_scale"] == 0).all()
        deq = orc.e4m3_decode(vc) * vs[:, :, None, :].astype(np.float64)  # [B,H,N,d]
        B, H, N, d = deq.shape
        if causal:
            ref = np.cumsum(deq, axis=2) / np.arange(1, N + 1)[None, None, :, None]
            vis = np.tril(np.ones((N, N), bool))
        else:
            ref = np.broadcast_to(deq.mean(axis=2, keepdims=True), deq.shape)
            vis = np.ones((N, N), bool)
        assert np.allclose(O.reshape(B, H, N, d), ref, rtol=2e-6, atol=1e-6)
        P = P.reshape(B, H, N, N)
        assert (P[:, :, vis] == 0x78).all() and (P[:, :, ~vis] == 0).all()  # every P~ = 2^8 exactly


def test_causal_first_row_is_first_value_row():
    w, Q, K, V = _small(dict(causal=True))
    qk, (vc, vs), O = _run(w, Q, K, V)
    B, H, N, d = vc.shape
    O = O.reshape(B, H, N, d)
    expect = (orc.e4m3_decode(vc[:, :, 0, :]) * vs.astype(np.float64)).astype(np.float32)
    assert np.array_equal(O[:, :, 0, :], expect)


def test_v_power_of_two_scales_output_exactly():
    w, Q, K, V = _small(dict(causal=True))
    _, (vc0, vs0), O0 = _run(w, Q, K, V)
    _, (vc1, vs1), O1 = _run(w, Q, K, V * 4)
    assert np.array_equal(vc0, vc1) and np.array_equal(vs1, vs0 * 4)
    assert np.array_equal(O1, O0 * 4)


@pytest.mark.parametrize("causal", [False, True])
def test_constant_v_channels_give_that_constant(causal):
    """V constant over the tokens of each channel: every V code is +-448 and O is a weighted
    average whose weights are the FP8 codes P^ divided by their own sum l (INT8 path: l sums
    the codes, not the fp32 P~), so O equals the channel's dequantized value to fp32 rounding
    for any Q and K, through several tiles, rescales and the causal mask.  With l summed over
    the fp32 P~ the weights would miss one by the FP8 rounding of P~ (about 1e-2)."""
    w, Q, K, _ = _small(dict(causal=causal, N=512, d=128, blk_q=128, dtype="bfloat16"))
    rng = np.random.default_rng(5)
    a = (rng.standard_normal((w.B, w.H, 1, w.d)) * 3).astype(np.float32)
    V = torch.from_numpy(np.broadcast_to(a, (w.B, w.H, w.N, w.d)).copy()).to(torch.bfloat16)
    qk, (vc, vs), O = _run(w, Q * 3, K, V)
    assert (np.abs(orc.e4m3_decode(vc)) == 448).all()
    expect = orc.e4m3_decode(vc[:, :, :1, :]) * vs[:, :, None, :].astype(np.float64)   # the dequantized constant
    O = O.reshape(w.B, w.H, w.N, w.d).astype(np.float64)
    assert np.abs(O - expect).max() <= 4e-6 * np.abs(expect).max()


def test_split_chunks_with_constant_v_give_that_constant():
    """The split-KV form merges chunk states with the same weights for O and l, so constant V
    channels come out exactly (to fp32 rounding) whatever the chunking."""
    w, Q, K, _ = _small(dict(causal=True, N=512, d=128, blk_q=128, dtype="bfloat16"))
    a = np.linspace(-5, 5, w.d, dtype=np.float32)[None, None, None, :]
    V = torch.from_numpy(np.broadcast_to(a, (w.B, w.H, w.N, w.d)).copy()).to(torch.bfloat16)
    qk = orc.quantize_qk(synth.bits(Q), synth.bits(K), w.dtype_code, w.blk_q, w.blk_k)
    vc, vs = orc.quantize_v(synth.bits(V), w.dtype_code)
    expect = orc.e4m3_decode(vc[:, :, :1, :]) * vs[:, :, None, :].astype(np.float64)
    rows = np.arange(w.B * w.H * w.N)
    for chunk in (64, 128, 256):
        O = orc.attn_rows_split(qk, vc, vs, w.blk_q, w.blk_k, w.causal, w.sm_scale, kv_chunk=chunk, rows=rows)
        O = O.reshape(w.B, w.H, w.N, w.d)
        assert np.abs(O - expect).max() <= 4e-6 * np.abs(expect).max(), chunk


def test_identity_v_exposes_p_tilde_on_the_fp8_grid():
    """With V the identity (one key per channel, one 64-key tile) row i of O is
    P~_i . diag(1) scaled by one common factor, so O shows the values that enter
    the P~V product: the row's largest is 2^8 (the running-max offset) and every
    other value must be an e4m3 value, the FP8 rounding of
    2^(8 + s_ij - max_j s_ij) for the exact dequantized scores s."""
    rng = np.random.default_rng(11)
    N = d = 64
    q = rng.standard_normal((1, 1, N, d)) * 0.8
    k = rng.standard_normal((1, 1, N, d)) * 0.8
    v = np.eye(N, d)[None, None]
    args = dict(dtype=0, blk_q=64, blk_k=64, causal=False, sm_scale=0.125)
    qk, (vc, vs), (O, P) = orc.run(_f16_bits(q), _f16_bits(k), _f16_bits(v), want_p=True, **args)
    O = O.reshape(N, d).astype(np.float64)
    ratio = 256.0 * O / O.max(axis=1, keepdims=True)
    grid = orc.e4m3_decode(np.arange(0, 127, dtype=np.uint8))
    nearest = grid[np.abs(ratio[..., None] - grid).argmin(axis=-1)]
    assert np.all(np.abs(ratio - nearest) <= 1e-6 * nearest)
    # the dump's FP8 codes are exactly what entered the product
    assert np.array_equal(orc.e4m3_decode(P.reshape(N, N)), nearest)
    # and they round the exact exponentials of the dequantized INT8 scores
    qc = qk["q_codes"].reshape(N, d).astype(np.int64)
    kc = qk["k_codes"].reshape(N, d).astype(np.int64)
    s = (qc @ kc.T) * float(qk["q_scale"].ravel()[0]) * float(qk["k_scale"].ravel()[0]) * 0.125 * math.log2(math.e)
    p = 2.0 ** (8.0 + s - s.max(axis=1, keepdims=True))
    assert np.all(np.abs(nearest - p) <= p / 8 + 2.0 ** -9)
    # random scores put most values off the grid: the check above has teeth
    assert np.mean(np.abs(p - nearest) > 1e-3 * p) > 0.5


def test_head_permutation_equivariance():
    w, Q, K, V = _small(dict(B=2, H=3, N=128))
    perm = torch.tensor([4, 0, 5, 2, 1, 3])
    def flat(t):
        return t.reshape(6, *t.shape[2:])
    def unflat(t):
        return t.reshape(2, 3, *t.shape[1:])
    Qp, Kp, Vp = (unflat(flat(t)[perm]) for t in (Q, K, V))
    _, _, O = _run(w, Q, K, V)
    _, _, Op = _run(w, Qp, Kp, Vp)
    N, d = 128, w.d
    assert np.array_equal(Op.reshape(6, N, d), O.reshape(6, N, d)[perm.numpy()])


def test_row_subset_matches_full_run():
    w, Q, K, V = _small(dict(causal=True))
    qk, (vc, vs), (O, P) = _run(w, Q, K, V, want_p=True)
    rows = np.array([0, 5, 63, 64, 255, 256, 300, 511], np.int64)
    Os, Ps = orc.attn_rows(qk, vc, vs, w.blk_q, w.blk_k, True, w.sm_scale, rows=rows, want_p=True)
    assert np.array_equal(Os, O[rows]) and np.array_equal(Ps, P[rows])


def test_exact_attention_reference_against_python_loops():
    rng = np.random.default_rng(8)
    B, H, N, d = 1, 1, 5, 3
    Q, K, V = (rng.standard_normal((B, H, N, d)) for _ in range(3))
    got = orc.exact_attention(Q, K, V, True, 0.7)
    for i in range(N):
        logits = [sum(Q[0, 0, i, c] * K[0, 0, j, c] for c in range(d)) * 0.7 for j in range(i + 1)]
        mx = max(logits)
        w = [math.exp(x - mx) for x in logits]
        s = sum(w)
        for c in range(d):
            assert abs(got[i, c] - sum(w[j] * V[0, 0, j, c] for j in range(i + 1)) / s) < 1e-12


def test_online_softmax_matches_single_tile_reference_in_the_exact_limit():
    """With the KV tile as wide as the sequence, one tile holds every key: the
    result is softmax with the exact row max.  Narrow tiles must agree within
    FP8 noise, and both must track the fp64 reference."""
    w, Q, K, V = _small({})
    qk, (vc, vs), O64 = _run(w, Q, K, V, kv_tile=64)
    O256 = orc.attn_rows(qk, vc, vs, w.blk_q, w.blk_k, False, w.sm_scale, kv_tile=256)
    assert np.abs(O64 - O256).max() < 0.05


# ------------------------------------------------------------------ head sharing and unequal lengths
def _gqa_inputs(B=1, Hq=4, Hkv=2, Nq=256, Nkv=256, d=64, seed=11):
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((B, Hq, Nq, d)).astype(np.float32)
    K = (rng.standard_normal((B, Hkv, Nkv, d)) + 2 * rng.standard_normal((B, Hkv, 1, d))).astype(np.float32)
    V = rng.standard_normal((B, Hkv, Nkv, d)).astype(np.float32)
    return Q, K, V


@pytest.mark.parametrize("causal", [False, True])
def test_grouped_heads_equal_repeated_kv_heads(causal):
    """Query head h reading K/V head h // (Hq/Hkv) is the same computation as
    every query head owning a copy of that K/V head: bit for bit."""
    Q, K, V = _gqa_inputs()
    g = Q.shape[1] // K.shape[1]
    Kr, Vr = np.repeat(K, g, axis=1), np.repeat(V, g, axis=1)
    qb, kb, vb, krb, vrb = (_f16_bits(a) for a in (Q, K, V, Kr, Vr))
    qk, (vc, vs), (O, P) = orc.run(qb, kb, vb, 0, 64, 64, causal, 0.125, want_p=True)
    qk_r, (vc_r, vs_r), (O_r, P_r) = orc.run(qb, krb, vrb, 0, 64, 64, causal, 0.125, want_p=True)
    assert qk["k_codes"].shape[1] == 2 and qk_r["k_codes"].shape[1] == 4
    assert np.array_equal(np.repeat(qk["k_codes"], g, axis=1), qk_r["k_codes"])
    assert np.array_equal(O, O_r) and np.array_equal(P, P_r)
    # and the head mapping is h // g, not h % Hkv: swapping the two K/V heads changes the result
    qk_s, (vc_s, vs_s), O_s = orc.run(qb, kb[:, ::-1].copy(), vb[:, ::-1].copy(), 0, 64, 64, causal, 0.125)
    assert not np.array_equal(O, O_s)


@pytest.mark.parametrize("causal", [False, True])
def test_fewer_queries_equal_the_last_rows_of_the_square_problem(causal):
    """Nq < Nkv with causal visibility aligned at the end (key j visible to query
    i iff j <= i + Nkv - Nq): the Nq queries are the last Nq rows of the square
    problem whose queries extend over all Nkv positions (the Q blocks line up
    because Nkv - Nq is a multiple of the block)."""
    Q, K, V = _gqa_inputs(Hq=2, Hkv=2, Nq=384, Nkv=384, seed=12)
    Qs = Q[:, :, 128:]
    qb, qsb, kb, vb = (_f16_bits(a) for a in (Q, Qs, K, V))
    _, _, (O, P) = orc.run(qb, kb, vb, 0, 128, 64, causal, 0.125, want_p=True)
    _, _, (Os, Ps) = orc.run(qsb, kb, vb, 0, 128, 64, causal, 0.125, want_p=True)
    rows = (np.arange(2)[:, None] * 384 + 128 + np.arange(256)[None, :]).ravel()
    assert np.array_equal(Os, O[rows]) and np.array_equal(Ps, P[rows])


def test_unequal_lengths_and_groups_against_fp64_and_loops():
    Q, K, V = _gqa_inputs(B=2, Hq=4, Hkv=1, Nq=128, Nkv=320, seed=13)
    qb, kb, vb = (_f16_bits(a) for a in (Q, K, V))
    Qv, Kv, Vv = (_f16_vals(a) for a in (Q, K, V))
    for causal in (False, True):
        _, _, O = orc.run(qb, kb, vb, 0, 64, 64, causal, 0.125)
        ref = orc.exact_attention(Qv, Kv, Vv, causal, 0.125)
        a, b = O.astype(np.float64).ravel(), ref.ravel()
        assert a @ b / np.sqrt((a @ a) * (b @ b)) >= 0.995
    # the fp64 reference itself, one row by loops: query 5 of head 3 of batch 1
    # reads K/V head 0 and, causally, keys 0 .. 5 + 320 - 128
    got = orc.exact_attention(Qv, Kv, Vv, True, 0.125, rows=np.array([(1 * 4 + 3) * 128 + 5]))
    last = 5 + 320 - 128
    q64, k64 = Qv[1, 3, 5].astype(np.float64), Kv[1, 0].astype(np.float64)
    logits = [float(q64 @ k64[j]) * 0.125 for j in range(last + 1)]
    mx = max(logits)
    wts = [math.exp(x - mx) for x in logits]
    want = sum(wts[j] * Vv[1, 0, j].astype(np.float64) for j in range(last + 1)) / sum(wts)
    assert np.abs(got[0] - want).max() < 1e-12


def test_unequal_shapes_rejected():
    Q, K, V = _gqa_inputs(Hq=3, Hkv=2)
    qk = orc.quantize_qk(_f16_bits(Q), _f16_bits(K), 0, 64, 64)
    vc, vs = orc.quantize_v(_f16_bits(V), 0)
    with pytest.raises(ValueError):   # 3 query heads cannot share 2 K/V heads evenly
        orc.attn_rows(qk, vc, vs, 64, 64, False, 0.125)
    Q, K, V = _gqa_inputs(Nq=256, Nkv=128)
    qk = orc.quantize_qk(_f16_bits(Q), _f16_bits(K), 0, 64, 64)
    vc, vs = orc.quantize_v(_f16_bits(V), 0)
    with pytest.raises(ValueError):   # causal with more queries than keys: the first queries see nothing
        orc.attn_rows(qk, vc, vs, 64, 64, True, 0.125)
    orc.attn_rows(qk, vc, vs, 64, 64, False, 0.125, rows=np.array([0, 255]))   # non-causal is fine


# ------------------------------------------------------------------ lengths that are not block multiples
def test_ragged_q_blocks_equal_the_zero_padded_tensor():
    """A last Q block of N mod blk tokens: appending zero tokens up to a block
    multiple changes no code of the real tokens and no scale (|0| never raises
    a block's max), and the block count is ceil(N / blk)."""
    rng = np.random.default_rng(21)
    for N, blk in ((200, 64), (130, 128), (1, 64), (127, 128)):
        Q = rng.standard_normal((1, 2, N, 64)).astype(np.float32) * 3
        Np = -(-N // blk) * blk
        Qp = np.zeros((1, 2, Np, 64), np.float32)
        Qp[:, :, :N] = Q
        K = rng.standard_normal((1, 2, 64, 64)).astype(np.float32)
        a = orc.quantize_qk(_f16_bits(Q), _f16_bits(K), 0, blk, 64)
        b = orc.quantize_qk(_f16_bits(Qp), _f16_bits(K), 0, blk, 64)
        assert a["q_scale"].shape == (1, 2, Np // blk)
        assert np.array_equal(a["q_scale"], b["q_scale"])
        assert np.array_equal(a["q_codes"], b["q_codes"][:, :, :N])
        assert not b["q_codes"][:, :, N:].any()


def test_ragged_k_last_block_holds_exactly_the_tail_tokens():
    """K of N = 64 m + r tokens: the last scale times 127 is the largest
    |k - mean| over the r tail tokens alone (not over 64 tokens), and that
    element's code is +-127; the mean runs over all N tokens."""
    rng = np.random.default_rng(22)
    N, r = 64 * 3 + 5, 5
    K = rng.standard_normal((1, 1, N, 64)).astype(np.float32)
    K[0, 0, N - r:] *= 0.25        # a quiet tail: any token of the previous block would raise its max
    Kv = _f16_vals(K)
    qk = orc.quantize_qk(_f16_bits(K[:, :, :64]), _f16_bits(K), 0, 64, 64)
    mu = qk["k_mean"][0, 0]
    assert np.abs(mu.astype(np.float64) - Kv[0, 0].astype(np.float64).mean(0)).max() < 1e-6
    assert qk["k_scale"].shape == (1, 1, 4)
    tail = Kv[0, 0, N - r:] - mu                       # fp32, as the method smooths
    a = np.abs(tail).max()
    assert qk["k_scale"][0, 0, 3] == np.float32(a / np.float32(127))
    i = np.unravel_index(np.abs(tail).argmax(), tail.shape)
    assert abs(int(qk["k_codes"][0, 0, N - r + i[0], i[1]])) == 127


@pytest.mark.parametrize("causal", [False, True])
def test_ragged_fewer_queries_equal_the_last_rows(causal):
    """Ragged Nq and Nkv: dropping the first 64 queries (one Q block) leaves the
    remaining rows bit-identical, the causal offset Nkv - Nq growing by 64."""
    Q, K, V = _gqa_inputs(Hq=2, Hkv=1, Nq=200, Nkv=261, seed=23)
    qb, qsb, kb, vb = (_f16_bits(a) for a in (Q, Q[:, :, 64:], K, V))
    _, _, (O, P) = orc.run(qb, kb, vb, 0, 64, 64, causal, 0.125, want_p=True)
    _, _, (Os, Ps) = orc.run(qsb, kb, vb, 0, 64, 64, causal, 0.125, want_p=True)
    rows = (np.arange(2)[:, None] * 200 + 64 + np.arange(136)[None, :]).ravel()
    assert np.array_equal(Os, O[rows]) and np.array_equal(Ps, P[rows])


def test_ragged_tail_key_is_attended():
    """Nkv = 65: the one key of the short last tile dominates every score it
    enters (weight above 0.999), so O is its V row; a dropped or misplaced tail
    tile would give O near the mean of the other V rows (about 0) instead.
    Causal, Nq = Nkv = 65: only query 64 sees that key.  Against fp64 exact
    attention."""
    rng = np.random.default_rng(24)
    d = 64
    K = rng.standard_normal((1, 1, 65, d)).astype(np.float32) * 0.5
    K[0, 0, 64] = 0.0
    K[0, 0, 64, 0] = 12.0            # score 8 * 12 * 0.125 = 12 above the others' ~0
    V = rng.standard_normal((1, 1, 65, d)).astype(np.float32)
    V[0, 0, 64] = 5.0
    kb, vb = _f16_bits(K), _f16_bits(V)
    for causal, nq in ((False, 128), (True, 65)):
        Q = rng.standard_normal((1, 1, nq, d)).astype(np.float32)
        Q[..., 0] = 8.0
        _, _, O = orc.run(_f16_bits(Q), kb, vb, 0, 64, 64, causal, 0.125)
        ex = orc.exact_attention(_f16_vals(Q), _f16_vals(K), _f16_vals(V), causal, 0.125).reshape(O.shape)
        assert np.abs(O - ex).max() < 2.0 ** -4 * 5.0   # FP8 V: relative error below 2^-4 of max|v| = 5
        seen = O if not causal else O[64:]
        assert np.abs(seen - 5.0).max() < 0.02
        if causal:
            assert np.abs(O[:64]).max() < 4.0 and np.abs(O[:64] - 5.0).min() > 0.5


def test_ragged_shapes_against_fp64():
    for (B, Hq, Hkv, Nq, Nkv, causal, seed) in ((1, 2, 2, 77, 77, True, 25), (2, 4, 2, 130, 300, False, 26),
                                                (1, 3, 1, 50, 190, True, 27), (1, 2, 1, 300, 70, False, 28)):
        Q, K, V = _gqa_inputs(B=B, Hq=Hq, Hkv=Hkv, Nq=Nq, Nkv=Nkv, seed=seed)
        qb, kb, vb = (_f16_bits(a) for a in (Q, K, V))
        _, _, O = orc.run(qb, kb, vb, 0, 64, 64, causal, 0.125)
        ex = orc.exact_attention(_f16_vals(Q), _f16_vals(K), _f16_vals(V), causal, 0.125)
        a, b = O.astype(np.float64).ravel(), ex.ravel()
        assert a @ b / np.sqrt((a @ a) * (b @ b)) >= 0.995, (Nq, Nkv, causal)


# ------------------------------------------------------------------ split-KV form (decode)
def _split_case(Hq=4, Hkv=2, Nq=3, Nkv=700, seed=31, causal=True):
    Q, K, V = _gqa_inputs(Hq=Hq, Hkv=Hkv, Nq=Nq, Nkv=Nkv, seed=seed)
    qb, kb, vb = (_f16_bits(a) for a in (Q, K, V))
    qk = orc.quantize_qk(qb, kb, 0, 64, 64)
    vc, vs = orc.quantize_v(vb, 0)
    return Q, K, V, qk, vc, vs


@pytest.mark.parametrize("causal", [False, True])
def test_split_with_one_chunk_is_the_single_pass(causal):
    """kv_chunk covering every key: the merge weight is exp2(0) = 1 and the
    fma merge of one chunk is exact, so the split form is bit-identical."""
    Q, K, V, qk, vc, vs = _split_case(causal=causal)
    one = orc.attn_rows(qk, vc, vs, 64, 64, causal, 0.125)
    for chunk in (704, 768, 4096):
        split = orc.attn_rows_split(qk, vc, vs, 64, 64, causal, 0.125, kv_chunk=chunk)
        assert np.array_equal(split.view(np.uint32), one.view(np.uint32)), chunk


def test_split_zero_q_gives_mean_of_dequantized_v():
    """Q = 0: every chunk has m = 0 and P~ = 2^8 per key, so the merged O is the
    mean of the dequantized V rows the query sees, whatever the chunk size."""
    Q, K, V, qk, vc, vs = _split_case(Hq=2, Hkv=1, Nq=2, Nkv=300, causal=True)
    qk = dict(qk, q_codes=np.zeros_like(qk["q_codes"]), q_scale=np.zeros_like(qk["q_scale"]))
    deq = orc.e4m3_decode(vc) * vs[:, :, None, :].astype(np.float64)   # [1,1,300,d]
    for chunk in (64, 128, 192):
        O = orc.attn_rows_split(qk, vc, vs, 64, 64, True, 0.125, kv_chunk=chunk)
        for r in range(4):   # rows: head h = r // 2, query i = r % 2 sees keys 0 .. i + 298
            last = r % 2 + 298
            assert np.allclose(O[r], deq[0, 0, :last + 1].mean(0), rtol=2e-6, atol=1e-6), (chunk, r)


def test_split_merge_weights_follow_the_dominant_chunk():
    """One key in the last chunk dominates every score: the merge must carry
    its chunk's O (weight ~1) and scale the others by exp2(m_c - m*) ~ 0."""
    rng = np.random.default_rng(32)
    d = 64
    K = rng.standard_normal((1, 1, 640, d)).astype(np.float32) * 0.5
    K[0, 0, 600] = 0.0
    K[0, 0, 600, 0] = 12.0
    V = rng.standard_normal((1, 1, 640, d)).astype(np.float32)
    V[0, 0, 600] = 5.0
    Q = rng.standard_normal((1, 1, 4, d)).astype(np.float32)
    Q[..., 0] = 8.0
    qk = orc.quantize_qk(_f16_bits(Q), _f16_bits(K), 0, 64, 64)
    vc, vs = orc.quantize_v(_f16_bits(V), 0)
    ex = orc.exact_attention(_f16_vals(Q), _f16_vals(K), _f16_vals(V), False, 0.125).reshape(4, d)
    for chunk in (64, 192, 320):
        O = orc.attn_rows_split(qk, vc, vs, 64, 64, False, 0.125, kv_chunk=chunk)
        # exact: about 4.972 (the other 639 keys keep ~0.5% of the weight); a
        # merge that dropped or misweighted the dominant chunk lands near 0
        assert np.abs(O - 5.0).max() < 0.05 and np.abs(O - ex).max() < 0.03, chunk


def test_split_chunks_without_visible_keys_are_left_out():
    """Causal, Nq = 40 queries at the end of Nkv = 130 keys, chunks of 64: the
    last chunk (keys 128, 129) is invisible to queries 0 .. 37 and must not
    enter their merge; the result stays on fp64 exact attention."""
    Q, K, V, qk, vc, vs = _split_case(Hq=1, Hkv=1, Nq=40, Nkv=130, seed=33)
    O = orc.attn_rows_split(qk, vc, vs, 64, 64, True, 0.125, kv_chunk=64)
    assert np.isfinite(O).all()
    ex = orc.exact_attention(_f16_vals(Q), _f16_vals(K), _f16_vals(V), True, 0.125).reshape(O.shape)
    assert np.abs(O - ex).max() < 0.05
    a, b = O.astype(np.float64).ravel(), ex.ravel()
    assert a @ b / np.sqrt((a @ a) * (b @ b)) >= 0.999


def test_split_row_with_one_visible_key_and_a_very_negative_score():
    """Causal and square: query 0 sees key 0 alone, so its output is key 0's dequantized V row
    whatever the score.  The score is made thousands below zero (in log2 units), so the row's
    running max is too: the chunks without a visible key must still stay out of the merge, whose
    weight exp2(m_c - m*) would overflow for them."""
    rng = np.random.default_rng(41)
    N, d, sm = 256, 64, 50.0
    q, k, v = (rng.standard_normal((1, 1, N, d)) for _ in range(3))
    ks0 = k[0, 0, 0] - k[0, 0].mean(axis=0)               # key 0 after smoothing
    q[0, 0, 0] = -4.0 * ks0 / np.abs(ks0).max()           # query 0 points against it
    qk = orc.quantize_qk(_f16_bits(q), _f16_bits(k), 0, 64, 64)
    vc, vs = orc.quantize_v(_f16_bits(v), 0)
    s0 = int(qk["q_codes"][0, 0, 0].astype(np.int64) @ qk["k_codes"][0, 0, 0].astype(np.int64))
    u0 = s0 * float(qk["q_scale"][0, 0, 0]) * float(qk["k_scale"][0, 0, 0]) * sm * math.log2(math.e)
    assert u0 < -1000
    O = orc.attn_rows_split(qk, vc, vs, 64, 64, True, sm, kv_chunk=64, rows=np.array([0], np.int64))
    expect = orc.e4m3_decode(vc[0, 0, 0]) * vs[0, 0].astype(np.float64)
    assert np.isfinite(O).all()
    # P~ = exp2(fma(S, c2, -(m' - 8))) with m' the fp32-rounded score: 2^(8 + e) with |e| at most
    # half an fp32 ulp of |u0|; P^ still rounds to 256 but l = P~, so O = expect * 2^-e
    e = 2.0 ** (math.floor(math.log2(-u0)) - 24)
    assert np.all(np.abs(O[0] - expect) <= (e * math.log(2) * 1.01 + 2e-7) * np.abs(expect) + 1e-12)


@pytest.mark.parametrize("chunk", [64, 128, 320])
def test_split_against_fp64(chunk):
    Q, K, V, qk, vc, vs = _split_case(Hq=8, Hkv=2, Nq=4, Nkv=1000, seed=34)
    for causal in (False, True):
        O = orc.attn_rows_split(qk, vc, vs, 64, 64, causal, 0.125, kv_chunk=chunk)
        ex = orc.exact_attention(_f16_vals(Q), _f16_vals(K), _f16_vals(V), causal, 0.125).reshape(O.shape)
        a, b = O.astype(np.float64).ravel(), ex.ravel()
        assert a @ b / np.sqrt((a @ a) * (b @ b)) >= 0.999
        one = orc.attn_rows(qk, vc, vs, 64, 64, causal, 0.125)
        # the split changes where P~ is rounded to FP8, not the size of the error
        assert np.abs(O - ex).max() < 1.5 * np.abs(one - ex).max() + 1e-3


def test_split_rejects_chunks_that_are_not_tile_multiples():
    Q, K, V, qk, vc, vs = _split_case()
    for chunk in (0, 32, 100):
        with pytest.raises(ValueError):
            orc.attn_rows_split(qk, vc, vs, 64, 64, True, 0.125, kv_chunk=chunk)


# ------------------------------------------------------------------ 4-bit QK^T (E2M1 with 32-value power-of-two blocks)
def _e2m1_from_bits(c):
    """E2M1 from its bit fields: sign s, exponent e (2 bits, bias 1), mantissa m (1 bit)."""
    s, e, m = (c >> 3) & 1, (c >> 1) & 3, c & 1
    mag = 0.5 * m if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)
    return -mag if s else mag


def test_e2m1_decode_is_the_bit_field_definition():
    got = orc.e2m1_decode(np.arange(16))
    assert [float(g) for g in got] == [_e2m1_from_bits(c) for c in range(16)]


def test_e2m1_encode_is_nearest_with_ties_to_even():
    rng = np.random.default_rng(41)
    mags = np.array([_e2m1_from_bits(c) for c in range(8)])
    mids = (mags[1:] + mags[:-1]) / 2
    x = np.concatenate([rng.uniform(-7, 7, 200000), mids, -mids, [0.0, -0.0, 6.0, 6.5, 100.0, -100.0]]).astype(np.float32)
    got = orc.e2m1_encode(x)
    for xi, ci in zip(x[-2000:].tolist() + mids.tolist(), list(got[-2000:]) + list(orc.e2m1_encode(mids))):
        a = abs(xi)
        d = np.abs(mags - a)
        best = np.flatnonzero(d == d.min())
        want = best[0] if len(best) == 1 else best[best % 2 == 0][0]   # ties: even code
        assert (ci & 7) == want, (xi, ci)
    # all values: decoded code is a nearest magnitude, sign kept
    dec = orc.e2m1_decode(got)
    err = np.abs(np.abs(dec) - np.minimum(np.abs(x), 6.0))
    nearest = np.min(np.abs(mags[None, :] - np.minimum(np.abs(x), 6.0)[:, None]), axis=1)
    assert np.array_equal(err, nearest)
    assert ((got >> 3) == np.signbit(x)).all()


def _q4_case(seed=42, N=64, d=128, scale=1.0):
    rng = np.random.default_rng(seed)
    Q = (rng.standard_normal((1, 2, N, d)) * scale).astype(np.float32)
    K = (rng.standard_normal((1, 2, N, d)) * scale + rng.standard_normal((1, 2, 1, d))).astype(np.float32)
    return Q, K


def test_mx4_blocks_properties():
    Q, K = _q4_case()
    r = orc.quantize_qk4(_f16_bits(Q), _f16_bits(K), 0)
    x = _f16_vals(Q).reshape(1, 2, 64, 4, 32).astype(np.float64)
    c = r["q4_codes"].reshape(1, 2, 64, 4, 32)
    sc = 2.0 ** (r["q4_scale"].astype(np.float64)[..., None] - 127)
    amax = np.abs(x).max(-1, keepdims=True)
    # the shared exponent puts the block max in [4, 8): its code is 4 or 6
    assert ((amax / sc >= 4) & (amax / sc < 8)).all()
    top = np.take_along_axis(c, np.abs(x).argmax(-1)[..., None], -1) & 7
    assert np.isin(top, [6, 7]).all()
    # round trip: within half the E2M1 spacing at each value's magnitude (1 above 4, 0.5 in [2,4), 0.25 below)
    y = orc.e2m1_decode(c) * sc
    t = np.minimum(np.abs(x) / sc, 6.0)
    half = np.where(t >= 4, 1.0, np.where(t >= 2, 0.5, 0.25))
    assert (np.abs(np.abs(y) / sc - t) <= half + 1e-12).all()
    # scaling the input by 2^5 moves every scale byte by 5 and keeps the codes
    r2 = orc.quantize_qk4(_f16_bits(Q * 32), _f16_bits(K), 0)
    assert np.array_equal(r2["q4_codes"], r["q4_codes"]) and np.array_equal(r2["q4_scale"], r["q4_scale"] + 5)
    # an all-zero block: scale byte 0, zero codes
    Qz = Q.copy(); Qz[0, 0, 3, 32:64] = 0
    r3 = orc.quantize_qk4(_f16_bits(Qz), _f16_bits(K), 0)
    assert r3["q4_scale"][0, 0, 3, 1] == 0 and (r3["q4_codes"][0, 0, 3, 32:64] == 0).all()


def test_k4_uses_the_same_smoothing_as_int8():
    Q, K = _q4_case(seed=43)
    r4 = orc.quantize_qk4(_f16_bits(Q), _f16_bits(K), 0)
    r8 = orc.quantize_qk(_f16_bits(Q), _f16_bits(K), 0, 64, 64)
    assert np.array_equal(r4["k_mean"].view(np.uint32), r8["k_mean"].view(np.uint32))


def test_qk4_scores_against_exact_python_arithmetic():
    from fractions import Fraction
    Q, K = _q4_case(seed=44, N=8, d=64)
    r = orc.quantize_qk4(_f16_bits(Q), _f16_bits(K), 0)
    rows = np.array([0, 5, 8 + 7], dtype=np.int64)   # (head 0, rows 0 and 5), (head 1, row 7)
    got = orc.qk4_scores(r, rows)
    dec = [Fraction(float(v)) for v in orc.e2m1_decode(np.arange(16))]
    for k, row in enumerate(rows):
        h, i = divmod(int(row), 8)
        for j in range(8):
            s = Fraction(0)
            for b in range(2):
                blk = sum(dec[r["q4_codes"][0, h, i, c]] * dec[r["k4_codes"][0, h, j, c]] for c in range(32 * b, 32 * b + 32))
                s += blk * Fraction(2) ** (int(r["q4_scale"][0, h, i, b]) + int(r["k4_scale"][0, h, j, b]) - 254)
            assert got[k, j] == np.float32(float(s)), (row, j)


@pytest.mark.parametrize("causal", [False, True])
def test_qk4_zero_q_gives_mean_of_dequantized_v(causal):
    Q, K, V = _gqa_inputs(Hq=2, Hkv=1, Nq=128, Nkv=192, seed=45)
    r = orc.quantize_qk4(_f16_bits(np.zeros_like(Q)), _f16_bits(K), 0)
    vc, vs = orc.quantize_v(_f16_bits(V), 0)
    O = orc.attn_rows_qk4(r, vc, vs, causal, 0.125)
    deq = orc.e4m3_decode(vc) * vs[:, :, None, :].astype(np.float64)
    for row in (0, 77, 128 + 5):
        i = row % 128
        last = i + 64 if causal else 191
        assert np.allclose(O[row], deq[0, 0, :last + 1].mean(0), rtol=2e-6, atol=1e-6)


def test_qk4_attention_against_fp64():
    """4-bit scores lose about three bits against INT8: the bar is the accuracy
    of E2M1 blocks (cosine >= 0.98 on these inputs), not that of the 8-bit path."""
    for causal in (False, True):
        Q, K, V = _gqa_inputs(B=1, Hq=4, Hkv=2, Nq=128, Nkv=320, seed=46)
        r = orc.quantize_qk4(_f16_bits(Q), _f16_bits(K), 0)
        vc, vs = orc.quantize_v(_f16_bits(V), 0)
        O = orc.attn_rows_qk4(r, vc, vs, causal, 0.125)
        ex = orc.exact_attention(_f16_vals(Q), _f16_vals(K), _f16_vals(V), causal, 0.125).reshape(O.shape)
        a, b = O.astype(np.float64).ravel(), ex.ravel()
        assert a @ b / np.sqrt((a @ a) * (b @ b)) >= 0.98


# ------------------------------------------------------------ Q smoothing (4-bit)
def test_q_block_mean_is_the_exact_mean_of_32_query_rows():
    """q_mean of each block of 32 consecutive queries (the last block ragged) is
    the exact rational mean of the block's f16 rows, rounded once to fp32."""
    from fractions import Fraction
    rng = np.random.default_rng(50)
    Q = (rng.standard_normal((1, 2, 75, 64)) * 3 + rng.standard_normal((1, 2, 1, 64)) * 8).astype(np.float32)
    K = rng.standard_normal((1, 1, 40, 64)).astype(np.float32)
    r = orc.quantize_qk4(_f16_bits(Q), _f16_bits(K), 0, smooth_q=True)
    q = _f16_vals(Q)
    assert r["q_mean"].shape == (1, 2, 3, 64)
    for h in range(2):
        for blk, (a, b) in enumerate(((0, 32), (32, 64), (64, 75))):
            for c in (0, 17, 63):
                exact = sum(Fraction(float(v)) for v in q[0, h, a:b, c]) / (b - a)
                assert r["q_mean"][0, h, blk, c] == np.float32(float(exact)), (h, blk, c)


def test_q_smoothing_removes_a_per_channel_bias_exactly():
    """Dyadic inputs: adding a per-channel bias to every query leaves the
    smoothed 4-bit codes and scales unchanged and moves the mean by the bias."""
    rng = np.random.default_rng(51)
    Q0 = (np.clip(np.round(rng.standard_normal((1, 2, 64, 64)) * 64), -255, 255) / 64).astype(np.float32)
    beta = (np.clip(np.round(rng.standard_normal((1, 2, 1, 64)) * 4 * 64), -960, 960) / 64).astype(np.float32)
    K = rng.standard_normal((1, 1, 64, 64)).astype(np.float32)
    r0 = orc.quantize_qk4(_f16_bits(Q0), _f16_bits(K), 0, smooth_q=True)
    r1 = orc.quantize_qk4(_f16_bits(Q0 + beta), _f16_bits(K), 0, smooth_q=True)
    assert np.array_equal(_f16_vals(Q0 + beta), Q0 + beta)   # the biased inputs are exact in f16
    # equal values (a -0 input minus a +0 mean gives -0, whose code keeps the sign bit)
    assert np.array_equal(orc.e2m1_decode(r0["q4_codes"]), orc.e2m1_decode(r1["q4_codes"]))
    assert np.array_equal(r0["q4_scale"], r1["q4_scale"])
    assert np.array_equal(r1["q_mean"], r0["q_mean"] + beta)
    # without smoothing the bias changes the codes
    p1 = orc.quantize_qk4(_f16_bits(Q0 + beta), _f16_bits(K), 0)
    assert not np.array_equal(p1["q4_codes"], r1["q4_codes"])


def _check_int8_pow2_block(x, codes, byte):
    """INT8 codes of one block with one power-of-two scale 2^e, e = byte - 127:
    e is the smallest exponent in [-63, 52] with max|x| 2^-e <= 127, and each
    code is the nearest integer to x 2^-e (ties to the even one)."""
    x = np.asarray(x, np.float64).ravel()
    codes = np.asarray(codes).astype(np.int64).ravel()
    e = int(byte) - 127
    a = float(np.abs(x).max())
    assert -63 <= e <= 52
    assert a * 2.0 ** -e <= 127
    if e > -63:
        assert a * 2.0 ** -(e - 1) > 127, "not the smallest exponent"
    y = x * 2.0 ** -e                      # exact: a power-of-two scaling
    lo = np.floor(y)
    frac = y - lo
    want = np.where(frac > 0.5, lo + 1, np.where(frac < 0.5, lo, np.where(lo % 2 == 0, lo, lo + 1)))
    assert np.array_equal(codes, want.astype(np.int64))
    assert np.abs(codes).max(initial=0) <= 127


def test_q_mean_int8_blocks_properties():
    """The block means of Q in INT8, one power-of-two scale per 32-query block
    over all d channels; an all-zero mean gets the lowest exponent and zero
    codes; a block max just below 128 steps after the scale goes to the next
    exponent instead of saturating."""
    rng = np.random.default_rng(52)
    Q = (rng.standard_normal((1, 1, 256, 128)) + rng.standard_normal((1, 1, 1, 128)) * 5).astype(np.float32)
    Q[0, 0, 64:96] = 0.0                                   # block 2: zero mean
    Q[0, 0, 96:128] = np.clip(Q[0, 0, 96], -7, 7)          # block 3: 32 equal rows, mean = the row
    Q[0, 0, 96:128, 7] = 511 / 64                          # 127.75 * 2^-4: exact in f16, just above 127 at e = -4
    K = rng.standard_normal((1, 1, 64, 128)).astype(np.float32)
    r = orc.quantize_qk4(_f16_bits(Q), _f16_bits(K), 0, smooth_q=True)
    assert r["qm_codes"].shape == (1, 1, 8, 128) and r["qm_scale"].shape == (1, 1, 8)
    assert r["qm_codes"].dtype == np.int8
    for blk in range(8):
        _check_int8_pow2_block(r["q_mean"][0, 0, blk], r["qm_codes"][0, 0, blk], r["qm_scale"][0, 0, blk])
    assert r["qm_scale"][0, 0, 2] == 127 - 63 and not r["qm_codes"][0, 0, 2].any()
    assert r["q_mean"][0, 0, 3, 7] == np.float32(511 / 64)
    assert np.abs(r["q_mean"][0, 0, 3]).max() == np.float32(511 / 64)
    assert r["qm_scale"][0, 0, 3] == 127 - 3 and r["qm_codes"][0, 0, 3, 7] == 64   # 63.875 -> 64 at e = -3


def test_smoothed_qk4_scores_against_exact_python_arithmetic():
    """Score = the E2M1 blocks of the smoothed row against K's E2M1 blocks,
    each scaled by its power-of-two scales, plus the integer dot product of
    the row block's INT8 mean codes with the key's INT8 codes times the two
    blocks' scales (the key's block of 64 keys; 100 keys = a ragged second
    block), summed exactly and rounded once."""
    from fractions import Fraction
    rng = np.random.default_rng(53)
    Q = (rng.standard_normal((1, 2, 40, 64)) + rng.standard_normal((1, 2, 1, 64)) * 6).astype(np.float32)
    K = (rng.standard_normal((1, 2, 100, 64)) + rng.standard_normal((1, 2, 1, 64))).astype(np.float32)
    K[0, 1, 64:] *= 5                                  # head 1: the second K block gets its own scale
    r = orc.quantize_qk4(_f16_bits(Q), _f16_bits(K), 0, smooth_q=True)
    assert r["k8_scale"].shape == (1, 2, 2) and r["k8_scale"][0, 1, 0] != r["k8_scale"][0, 1, 1]
    rows = np.array([0, 33, 40 + 39], dtype=np.int64)   # head 0 rows 0 and 33 (second block), head 1 row 39
    got = orc.qk4_scores(r, rows)
    d4 = [Fraction(float(v)) for v in orc.e2m1_decode(np.arange(16))]
    for k, row in enumerate(rows):
        h, i = divmod(int(row), 40)
        for j in (0, 1, 63, 64, 65, 99):
            s = Fraction(0)
            for b in range(2):
                ek = int(r["k4_scale"][0, h, j, b])
                blk = sum(d4[r["q4_codes"][0, h, i, c]] * d4[r["k4_codes"][0, h, j, c]] for c in range(32 * b, 32 * b + 32))
                s += blk * Fraction(2) ** (int(r["q4_scale"][0, h, i, b]) + ek - 254)
            dot = sum(int(r["qm_codes"][0, h, i // 32, c]) * int(r["k8_codes"][0, h, j, c]) for c in range(64))
            s += dot * Fraction(2) ** (int(r["qm_scale"][0, h, i // 32]) + int(r["k8_scale"][0, h, j // 64]) - 254)
            assert got[k, j] == np.float32(float(s)), (row, j)


def test_q_mean_term_is_close_to_the_exact_mean_times_smoothed_k():
    """The mean's term (INT8 codes times their scales) is the fp64 product of
    the block mean and the smoothed key within the quantization bound: each
    code is within half a step of its value, so |t - qm.k| <= sum_c
    (|qm_c| dk / 2 + |k_c| dq / 2 + dq dk / 4)."""
    rng = np.random.default_rng(57)
    Q = (rng.standard_normal((1, 2, 96, 128)) + rng.standard_normal((1, 2, 1, 128)) * 4).astype(np.float32)
    K = (rng.standard_normal((1, 2, 150, 128)) + rng.standard_normal((1, 2, 1, 128)) * 2).astype(np.float32)
    r = orc.quantize_qk4(_f16_bits(Q), _f16_bits(K), 0, smooth_q=True)
    ks = (_f16_vals(K) - r["k_mean"][:, :, None, :]).astype(np.float32).astype(np.float64)
    for h in range(2):
        for blk in range(3):
            qm = r["q_mean"][0, h, blk].astype(np.float64)
            dq = 2.0 ** (int(r["qm_scale"][0, h, blk]) - 127)
            for j in range(150):
                dk = 2.0 ** (int(r["k8_scale"][0, h, j // 64]) - 127)
                t = float(r["qm_codes"][0, h, blk].astype(np.int64) @ r["k8_codes"][0, h, j].astype(np.int64)) * dq * dk
                exact = float(qm @ ks[0, h, j])
                bound = float((np.abs(qm) * dk / 2 + np.abs(ks[0, h, j]) * dq / 2 + dq * dk / 4).sum())
                assert abs(t - exact) <= bound, (h, blk, j, t, exact, bound)


def test_q_smoothing_helps_4bit_scores_when_q_has_a_channel_bias():
    """With a per-channel bias in Q, the smoothed 4-bit path is closer to fp64
    attention than the plain one; dropping the mean term would wreck it."""
    rng = np.random.default_rng(54)
    Q, K, V = _gqa_inputs(B=1, Hq=2, Hkv=1, Nq=128, Nkv=256, seed=55)
    Q = (Q + 3 * rng.standard_normal((1, 2, 1, Q.shape[-1]))).astype(np.float32)
    vc, vs = orc.quantize_v(_f16_bits(V), 0)
    ex = orc.exact_attention(_f16_vals(Q), _f16_vals(K), _f16_vals(V), False, 0.125).reshape(-1, Q.shape[-1])
    cos = lambda a, b: float(a.ravel() @ b.ravel() / np.sqrt((a.ravel() @ a.ravel()) * (b.ravel() @ b.ravel())))
    rp = orc.quantize_qk4(_f16_bits(Q), _f16_bits(K), 0)
    rs = orc.quantize_qk4(_f16_bits(Q), _f16_bits(K), 0, smooth_q=True)
    cp = cos(orc.attn_rows_qk4(rp, vc, vs, False, 0.125).astype(np.float64), ex)
    cs = cos(orc.attn_rows_qk4(rs, vc, vs, False, 0.125).astype(np.float64), ex)
    dropped = {k: v for k, v in rs.items() if k not in ("qm_codes", "qm_scale", "k8_codes", "k8_scale")}
    cd = cos(orc.attn_rows_qk4(dropped, vc, vs, False, 0.125).astype(np.float64), ex)
    # on these inputs: about 0.915 plain, 0.99 smoothed (the smoothed path stays near the unbiased 0.985)
    assert cs > cp + 0.05 and cs >= 0.98 and cd < cs - 0.05, (cp, cs, cd)


def test_k8_blocks_are_the_smoothed_k_in_int8():
    """INT8 K blocks of the mean term: the same K mean as the 4-bit and INT8
    paths, one power-of-two scale per 64 keys over all channels (the last
    block ragged), codes the nearest integers."""
    rng = np.random.default_rng(56)
    K = (rng.standard_normal((1, 2, 150, 128)) + rng.standard_normal((1, 2, 1, 128))).astype(np.float32)
    K[0, 0, 128:] *= 16
    Q = rng.standard_normal((1, 2, 32, 128)).astype(np.float32)
    r = orc.quantize_qk4(_f16_bits(Q), _f16_bits(K), 0, smooth_q=True)
    assert r["k8_codes"].shape == (1, 2, 150, 128) and r["k8_scale"].shape == (1, 2, 3)
    assert r["k8_codes"].dtype == np.int8
    ks = (_f16_vals(K) - r["k_mean"][:, :, None, :]).astype(np.float32)
    for h in range(2):
        for blk in range(3):
            sl = slice(64 * blk, min(64 * blk + 64, 150))
            _check_int8_pow2_block(ks[0, h, sl], r["k8_codes"][0, h, sl], r["k8_scale"][0, h, blk])
    assert r["k8_scale"][0, 0, 2] >= r["k8_scale"][0, 0, 1] + 3   # the scaled tail block has its own exponent


# ------------------------------------------------------------ FP4 P~V (MXFP4 P~ and V)
def _v4_case(seed=60, B=1, H=2, N=100, d=64):
    rng = np.random.default_rng(seed)
    V = rng.standard_normal((B, H, N, d)).astype(np.float32)
    V[:, :, :, 5] *= 40                                     # an outlier channel gets its own scales
    return V


def test_v4_blocks_properties():
    """V in E2M1 blocks of 32 consecutive tokens per channel (the last block
    ragged): the shared exponent puts each block max in [4, 8), codes round to
    within half the E2M1 spacing, a zero block gets scale byte 0."""
    V = _v4_case()
    V[0, 1, 64:96, 9] = 0.0
    vc, vs = orc.quantize_v4(_f16_bits(V), 0)
    assert vc.shape == V.shape and vs.shape == (1, 2, 4, 64)
    x = _f16_vals(V).astype(np.float64)
    for blk, (a, b) in enumerate(((0, 32), (32, 64), (64, 96), (96, 100))):
        xb = x[:, :, a:b, :]
        cb = vc[:, :, a:b, :]
        sc = 2.0 ** (vs[:, :, blk, :].astype(np.float64) - 127)[:, :, None, :]
        amax = np.abs(xb).max(2, keepdims=True)
        live = amax > 0
        r = amax / sc
        assert ((r >= 4) & (r < 8))[live].all()
        y = orc.e2m1_decode(cb) * sc
        t = np.minimum(np.abs(xb) / sc, 6.0)
        half = np.where(t >= 4, 1.0, np.where(t >= 2, 0.5, 0.25))
        assert (np.abs(np.abs(y) / sc - t) <= half + 1e-12)[np.broadcast_to(live, t.shape)].all()
    assert vs[0, 1, 2, 9] == 0 and not vc[0, 1, 64:96, 9].any()
    assert vs[0, 0, 0, 5] >= vs[0, 0, 0, 4] + 4             # the outlier channel's own exponent


def _fp4_attention(Q, K, V, causal, rows=None, want_p=False):
    r = orc.quantize_qk4(_f16_bits(Q), _f16_bits(K), 0)
    vc, vs = orc.quantize_v4(_f16_bits(V), 0)
    return r, (vc, vs), orc.attn_rows_fp4(r, vc, vs, causal, 1.0 / math.sqrt(Q.shape[-1]), rows=rows, want_p=want_p)


@pytest.mark.parametrize("causal", [False, True])
def test_fp4_attention_of_a_power_of_two_constant_v_is_that_constant(causal):
    """V constant per channel and a power of two (exact in every MX block):
    the same P^ weights both O_acc and l, so O is that constant exactly."""
    rng = np.random.default_rng(61)
    Q = rng.standard_normal((1, 2, 70, 64)).astype(np.float32)
    K = (rng.standard_normal((1, 1, 150, 64)) + 1).astype(np.float32)
    c = 2.0 ** rng.integers(-6, 6, 64) * np.where(rng.random(64) < 0.5, -1, 1)
    V = np.broadcast_to(c.astype(np.float32), (1, 1, 150, 64)).copy()
    _, _, O = _fp4_attention(Q, K, V, causal)
    assert np.array_equal(O, np.broadcast_to(c.astype(np.float32), O.shape))


@pytest.mark.parametrize("causal", [False, True])
def test_fp4_attention_with_q_zero_is_the_mean_of_the_fp4_v(causal):
    """Q = 0: every score is 0, every P~ is 2^8 and lands on the E2M1 value 4
    of its block's scale 2^6, so O is the plain mean of the dequantized FP4 V
    over the visible keys (a closed form)."""
    rng = np.random.default_rng(62)
    Nq, Nkv = 40, 131
    Q = np.zeros((1, 2, Nq, 64), np.float32)
    K = rng.standard_normal((1, 1, Nkv, 64)).astype(np.float32)
    V = _v4_case(seed=63, H=1, N=Nkv)
    r, (vc, vs), (O, P) = _fp4_attention(Q, K, V, causal, want_p=True)
    deq = orc.e2m1_decode(vc[0, 0]) * 2.0 ** (np.repeat(vs[0, 0], 32, axis=0)[:Nkv].astype(np.float64) - 127)
    for h in range(2):
        for i in range(Nq):
            last = i + Nkv - Nq if causal else Nkv - 1
            want = deq[:last + 1].mean(axis=0)
            got = O[h * Nq + i]
            assert np.abs(got - want).max() <= 2e-6 * max(1.0, np.abs(want).max()), (h, i)
            assert (P[h * Nq + i, :last + 1] == 6).all()      # E2M1 4.0


def test_fp4_p_blocks_take_the_mx_exponent_of_their_largest_value():
    """Every visited 32-key block of P^ has its largest code at 4 or 6 (E2M1
    codes 6, 7): the block max, divided by 2^(floor(log2 max) - 2), lies in
    [4, 8).  Codes are non-negative (P~ >= 0) and masked keys get none."""
    rng = np.random.default_rng(64)
    Q = rng.standard_normal((1, 2, 96, 64)).astype(np.float32) * 2
    K = rng.standard_normal((1, 2, 200, 64)).astype(np.float32)
    V = _v4_case(seed=65, H=2, N=200)
    for causal in (False, True):
        _, _, (O, P) = _fp4_attention(Q, K, V, causal, want_p=True)
        assert (P < 8).all()                                 # no sign bit
        for row in range(P.shape[0]):
            i = row % 96
            last = i + 200 - 96 if causal else 199
            for b0 in range(0, last + 1, 32):
                blk = P[row, b0:min(b0 + 32, last + 1)]
                assert blk.max() in (6, 7), (causal, row, b0, blk)
            if causal:
                assert not P[row, last + 1:].any()


def test_fp4_attention_single_tile_against_exact_python_arithmetic():
    """One KV tile (no rescale): O = RN(sum_k P^_k V^_kc) / RN(sum_k P^_k) with
    P^ rebuilt here from the scores: fp32 argument (fma), exp2, the block
    exponent floor(max arg) - 2, E2M1 nearest-even codes; V^ decoded from the
    oracle's FP4 V.  Exact rationals for the sums."""
    from fractions import Fraction
    rng = np.random.default_rng(66)
    Q = rng.standard_normal((1, 1, 5, 32)).astype(np.float32)
    K = rng.standard_normal((1, 1, 50, 32)).astype(np.float32)
    V = _v4_case(seed=67, H=1, N=50, d=32)
    r, (vc, vs), O = _fp4_attention(Q, K, V, False)
    S = orc.qk4_scores(r, np.arange(5)).astype(np.float64)
    c2 = np.float32(np.float32(1.0 / math.sqrt(32)) * np.float32(1.4426950408889634))
    mags = [0, 0.5, 1, 1.5, 2, 3, 4, 6]

    def e2m1_nearest_even(t):
        best = min(range(8), key=lambda k: (abs(mags[k] - t), k & 1))
        return mags[best]
    vdec = orc.e2m1_decode(vc[0, 0]) * 2.0 ** (np.repeat(vs[0, 0], 32, axis=0)[:50].astype(np.float64) - 127)
    for i in range(5):
        u = (S[i] * np.float64(c2)).astype(np.float32)
        mm = np.float32(u.max()) - np.float32(8)
        arg = (S[i] * np.float64(c2) - np.float64(mm)).astype(np.float32)     # fma: exact product, one rounding
        p = np.exp2(arg.astype(np.float64)).astype(np.float32)
        ph = []
        for b0 in (0, 32):
            e = int(np.floor(arg[b0:b0 + 32].max())) - 2
            ph += [Fraction(e2m1_nearest_even(float(x) * 2.0 ** -e)) * Fraction(2) ** e for x in p[b0:b0 + 32]]
        l = np.float32(float(sum(ph)))
        for c in range(32):
            acc = np.float32(float(sum(ph[k] * Fraction(float(vdec[k, c])) for k in range(50))))
            assert O[i, c] == np.float32(np.float64(acc) / np.float64(l)), (i, c)
