"""Python face of the CPU oracle (test infrastructure only).

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import this module.  It loads ``liboracle.so`` (plain C, see
``sage_oracle.c``) through ctypes and adds the fp64 exact-attention reference
used for the accuracy check.  It imports nothing from the GPU package.

Arrays are numpy.  Inputs Q, K, V are passed as the raw 16-bit patterns of
float16 / bfloat16 tensors (``uint16``), with ``dtype`` 0 for float16 and 1
for bfloat16: Q of shape [B, Hq, Nq, d], K and V of shape [B, Hkv, Nkv, d].
Query head h reads key/value head h // (Hq // Hkv) (grouped-query attention
when Hkv < Hq); with causal masking, key j is visible to query i iff
j <= i + (Nkv - Nq).
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None

F16, BF16 = 0, 1
#: width of the KV tile over which the online softmax updates its running max
#: and the inner FP8 P~V block is accumulated (the kernel's tile width).
KV_TILE = 64


def lib():
    global _lib
    if _lib is None:
        # SAGE_ORACLE_LIB names a library built elsewhere from a modified copy
        # of the source (the mutation test plants one mistake per copy).
        path = os.environ.get("SAGE_ORACLE_LIB")
        if not path:
            path = _build.LIB
            if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
                _build.build()
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32, i64, f32 = ctypes.c_int, ctypes.c_int64, ctypes.c_float
        L.oracle_e4m3_decode.restype = ctypes.c_double
        L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_e4m3_encode.argtypes = [f32]
        L.oracle_e4m3_encode_n.argtypes = [P, P, i64]
        L.oracle_e4m3_decode_n.argtypes = [P, P, i64]
        L.oracle_exp2f.restype = f32
        L.oracle_exp2f.argtypes = [f32]
        L.oracle_exp2f_n.argtypes = [P, P, i64]
        L.oracle_kmean.restype = i32
        L.oracle_kmean.argtypes = [P, i32, i32, i32, i32, P, P]
        L.oracle_quantize_qk.restype = i32
        L.oracle_quantize_qk.argtypes = [P, P, i32, i32, i32, i32, i32, i32, P, P, P, P, P]
        L.oracle_quantize_q.restype = i32
        L.oracle_quantize_q.argtypes = [P, i32, i32, i32, i32, i32, P, P]
        L.oracle_quantize_k.restype = i32
        L.oracle_quantize_k.argtypes = [P, i32, i32, i32, i32, i32, P, P, P]
        L.oracle_quantize_v.restype = i32
        L.oracle_quantize_v.argtypes = [P, i32, i32, i32, i32, P, P]
        L.oracle_qk_int32.restype = None
        L.oracle_qk_int32.argtypes = [P, P, i32, i32, i32, i32, i32, i32, P, i32, P]
        L.oracle_e2m1_decode.restype = ctypes.c_double
        L.oracle_e2m1_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e2m1_encode_n.argtypes = [P, P, i64]
        L.oracle_quantize_q4.restype = i32
        L.oracle_quantize_q4.argtypes = [P, i32, i32, i32, i32, P, P]
        L.oracle_quantize_k4.restype = i32
        L.oracle_quantize_k4.argtypes = [P, i32, i32, i32, i32, P, P, P]
        L.oracle_attn_rows_qk4.restype = i32
        L.oracle_attn_rows_qk4.argtypes = [P] * 10 + [i32] * 8 + [f32, P, i32, P, P]
        L.oracle_quantize_v4.restype = i32
        L.oracle_quantize_v4.argtypes = [P, i32, i32, i32, i32, P, P]
        L.oracle_attn_rows_fp4.restype = i32
        L.oracle_attn_rows_fp4.argtypes = [P] * 6 + [i32] * 8 + [f32, P, i32, P, P]
        L.oracle_qk4_scores.restype = i32
        L.oracle_qk4_scores.argtypes = [P] * 8 + [i32] * 6 + [P, i32, P]
        L.oracle_quantize_k8.restype = i32
        L.oracle_quantize_k8.argtypes = [P, i32, i32, i32, i32, P, P]
        L.oracle_quantize_q4_smooth.restype = i32
        L.oracle_quantize_q4_smooth.argtypes = [P, i32, i32, i32, i32, P, P, P, P, P]
        L.oracle_attn_rows_split.restype = i32
        L.oracle_attn_rows_split.argtypes = [P, P, P, P, P, P] + [i32] * 11 + [f32, P, i32, P]
        L.oracle_attn_rows.restype = i32
        L.oracle_attn_rows.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32, i32, i32, i32, i32, i32, f32,
                                       P, i32, P, P]
        L.oracle_num_threads.restype = i32
        _lib = L
    return _lib


def _p(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


# ---------------------------------------------------------------- primitives
def e4m3_encode(x):
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint8)
    lib().oracle_e4m3_encode_n(_p(x), _p(out), x.size)
    return out


def e4m3_decode(c):
    c = _c(c, np.uint8)
    out = np.empty(c.shape, np.float64)
    lib().oracle_e4m3_decode_n(_p(c), _p(out), c.size)
    return out


def exp2f(t):
    """The softmax exponential: 2^t of fp32 t, evaluated in double, rounded once to fp32."""
    t = _c(t, np.float32)
    out = np.empty(t.shape, np.float32)
    lib().oracle_exp2f_n(_p(t), _p(out), t.size)
    return out


def num_threads():
    return int(lib().oracle_num_threads())


# ---------------------------------------------------------------- the method
def kmean(K_bits, dtype):
    K_bits = _c(K_bits, np.uint16)
    B, H, N, d = K_bits.shape
    mu = np.empty((B, H, d), np.float32)
    sums = np.empty((B, H, d), np.int64)
    rc = lib().oracle_kmean(_p(K_bits), dtype, B * H, N, d, _p(mu), _p(sums))
    assert rc == 0
    return mu, sums


def quantize_qk(Q_bits, K_bits, dtype, blk_q, blk_k):
    """INT8 blocks of Q [B,Hq,Nq,d]; K mean and INT8 blocks of the smoothed K [B,Hkv,Nkv,d].
    Scales: [B,Hq,ceil(Nq/blk_q)] and [B,Hkv,ceil(Nkv/blk_k)] (a shorter last block)."""
    Q_bits = _c(Q_bits, np.uint16)
    K_bits = _c(K_bits, np.uint16)
    B, Hq, Nq, d = Q_bits.shape
    Bk, Hkv, Nkv, dk = K_bits.shape
    if Bk != B or dk != d:
        raise ValueError("Q and K must share B and d")
    qc = np.empty((B, Hq, Nq, d), np.int8)
    kc = np.empty((B, Hkv, Nkv, d), np.int8)
    qs = np.empty((B, Hq, -(-Nq // blk_q)), np.float32)
    ks = np.empty((B, Hkv, -(-Nkv // blk_k)), np.float32)
    mu = np.empty((B, Hkv, d), np.float32)
    rc = lib().oracle_quantize_q(_p(Q_bits), dtype, B * Hq, Nq, d, blk_q, _p(qc), _p(qs))
    rc |= lib().oracle_quantize_k(_p(K_bits), dtype, B * Hkv, Nkv, d, blk_k, _p(kc), _p(ks), _p(mu))
    if rc != 0:
        raise ValueError("oracle quantize: unsupported shape")
    return dict(q_codes=qc, q_scale=qs, k_codes=kc, k_scale=ks, k_mean=mu)


def quantize_q(Q_bits, dtype, blk_q):
    """INT8 blocks of Q [B,Hq,Nq,d] alone: (q_codes, q_scale [B,Hq,ceil(Nq/blk_q)])."""
    Q_bits = _c(Q_bits, np.uint16)
    B, Hq, Nq, d = Q_bits.shape
    qc = np.empty((B, Hq, Nq, d), np.int8)
    qs = np.empty((B, Hq, -(-Nq // blk_q)), np.float32)
    if lib().oracle_quantize_q(_p(Q_bits), dtype, B * Hq, Nq, d, blk_q, _p(qc), _p(qs)) != 0:
        raise ValueError("oracle quantize_q: unsupported shape")
    return qc, qs


def quantize_v(V_bits, dtype):
    """Returns (v_codes [B,H,N,d] e4m3 in natural token-major layout, v_scale [B,H,d])."""
    V_bits = _c(V_bits, np.uint16)
    B, H, N, d = V_bits.shape
    vc = np.empty((B, H, N, d), np.uint8)
    vs = np.empty((B, H, d), np.float32)
    rc = lib().oracle_quantize_v(_p(V_bits), dtype, B * H, N, d, _p(vc), _p(vs))
    assert rc == 0
    return vc, vs


def qk_int32(q_codes, k_codes, rows):
    """Exact int32 scores of flat query rows ``bh*Nq + i`` against every key of their K head: [nrows, Nkv]."""
    q_codes = _c(q_codes, np.int8)
    k_codes = _c(k_codes, np.int8)
    B, Hq, Nq, d = q_codes.shape
    _, Hkv, Nkv, _ = k_codes.shape
    rows = _c(rows, np.int64)
    out = np.empty((rows.size, Nkv), np.int32)
    lib().oracle_qk_int32(_p(q_codes), _p(k_codes), B, Hq, Hkv, Nq, Nkv, d, _p(rows), rows.size, _p(out))
    return out


def attn_rows(qk, v_codes, v_scale, blk_q, blk_k, causal, sm_scale, rows=None, kv_tile=KV_TILE,
              want_p=False):
    """Oracle attention for flat query rows ``bh*Nq + i`` (all rows when None).

    ``qk`` is the dict returned by :func:`quantize_qk`; ``v_codes`` is in the
    natural [B,Hkv,Nkv,d] layout.  Returns O [nrows, d] fp32 (and the FP8 codes
    of P~ [nrows, Nkv] when ``want_p``).
    """
    qc = _c(qk["q_codes"], np.int8)
    kc = _c(qk["k_codes"], np.int8)
    qs = _c(qk["q_scale"], np.float32)
    ks = _c(qk["k_scale"], np.float32)
    vc = _c(v_codes, np.uint8)
    vs = _c(v_scale, np.float32)
    B, Hq, Nq, d = qc.shape
    _, Hkv, Nkv, _ = kc.shape
    if rows is None:
        rows = np.arange(B * Hq * Nq, dtype=np.int64)
    rows = _c(rows, np.int64)
    out = np.empty((rows.size, d), np.float32)
    p = np.empty((rows.size, Nkv), np.uint8) if want_p else None
    rc = lib().oracle_attn_rows(_p(qc), _p(qs), _p(kc), _p(ks), _p(vc), _p(vs), B, Hq, Hkv, Nq, Nkv, d, blk_q,
                                blk_k, kv_tile, int(bool(causal)), float(sm_scale), _p(rows), rows.size, _p(out),
                                _p(p))
    if rc != 0:
        raise ValueError("oracle_attn_rows: unsupported arguments")
    return (out, p) if want_p else out


def attn_rows_split(qk, v_codes, v_scale, blk_q, blk_k, causal, sm_scale, kv_chunk, rows=None, kv_tile=KV_TILE):
    """Split-KV oracle attention: chunks of ``kv_chunk`` keys, each with its own
    online softmax, merged by the log-sum-exp rule.  Same arguments and result
    as :func:`attn_rows` (no P~ codes)."""
    qc = _c(qk["q_codes"], np.int8)
    kc = _c(qk["k_codes"], np.int8)
    qs = _c(qk["q_scale"], np.float32)
    ks = _c(qk["k_scale"], np.float32)
    vc = _c(v_codes, np.uint8)
    vs = _c(v_scale, np.float32)
    B, Hq, Nq, d = qc.shape
    _, Hkv, Nkv, _ = kc.shape
    if rows is None:
        rows = np.arange(B * Hq * Nq, dtype=np.int64)
    rows = _c(rows, np.int64)
    out = np.empty((rows.size, d), np.float32)
    rc = lib().oracle_attn_rows_split(_p(qc), _p(qs), _p(kc), _p(ks), _p(vc), _p(vs), B, Hq, Hkv, Nq, Nkv, d, blk_q,
                                      blk_k, kv_tile, kv_chunk, int(bool(causal)), float(sm_scale), _p(rows),
                                      rows.size, _p(out))
    if rc != 0:
        raise ValueError("oracle_attn_rows_split: unsupported arguments")
    return out


# ---------------------------------------------------------------- 4-bit QK^T variant
def e2m1_decode(codes):
    codes = np.asarray(codes, np.uint8)
    tab = np.array([lib().oracle_e2m1_decode(c) for c in range(16)])
    return tab[codes]


def e2m1_encode(x):
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint8)
    lib().oracle_e2m1_encode_n(_p(x), _p(out), x.size)
    return out


def quantize_qk4(Q_bits, K_bits, dtype, smooth_q=False):
    """E2M1 blocks of 32 channels of Q [B,Hq,Nq,d] and of the smoothed K
    [B,Hkv,Nkv,d]: codes (one per value, 0..15) and E8M0 scale bytes per block.
    smooth_q: Q minus the mean of its 32-query block, which is returned as
    q_mean [B,Hq,ceil(Nq/32),d] with its INT8 codes qm_codes and one exponent
    byte per block qm_scale [B,Hq,ceil(Nq/32)] (scale 2^(byte - 127)), and the
    smoothed K also in INT8 blocks of 64 keys, k8_codes [B,Hkv,Nkv,d] and
    k8_scale [B,Hkv,ceil(Nkv/64)], for the mean's term."""
    Q_bits = _c(Q_bits, np.uint16)
    K_bits = _c(K_bits, np.uint16)
    B, Hq, Nq, d = Q_bits.shape
    _, Hkv, Nkv, _ = K_bits.shape
    qc = np.empty((B, Hq, Nq, d), np.uint8)
    qs = np.empty((B, Hq, Nq, d // 32), np.uint8)
    kc = np.empty((B, Hkv, Nkv, d), np.uint8)
    ks = np.empty((B, Hkv, Nkv, d // 32), np.uint8)
    mu = np.empty((B, Hkv, d), np.float32)
    extra = {}
    if smooth_q:
        nb = -(-Nq // 32)
        qmean = np.empty((B, Hq, nb, d), np.float32)
        qmc = np.empty((B, Hq, nb, d), np.int8)
        qms = np.empty((B, Hq, nb), np.uint8)
        rc = lib().oracle_quantize_q4_smooth(_p(Q_bits), dtype, B * Hq, Nq, d, _p(qc), _p(qs), _p(qmean), _p(qmc),
                                             _p(qms))
        k8c = np.empty((B, Hkv, Nkv, d), np.int8)
        k8s = np.empty((B, Hkv, -(-Nkv // 64)), np.uint8)
        rc |= lib().oracle_quantize_k8(_p(K_bits), dtype, B * Hkv, Nkv, d, _p(k8c), _p(k8s))
        extra = dict(q_mean=qmean, qm_codes=qmc, qm_scale=qms, k8_codes=k8c, k8_scale=k8s)
    else:
        rc = lib().oracle_quantize_q4(_p(Q_bits), dtype, B * Hq, Nq, d, _p(qc), _p(qs))
    rc |= lib().oracle_quantize_k4(_p(K_bits), dtype, B * Hkv, Nkv, d, _p(kc), _p(ks), _p(mu))
    if rc != 0:
        raise ValueError("oracle quantize_qk4: unsupported shape")
    return dict(q4_codes=qc, q4_scale=qs, k4_codes=kc, k4_scale=ks, k_mean=mu, **extra)


def _qm(qk4):
    """The Q-mean and INT8 K codes and exponent bytes of a smoothed quantization, else NULLs."""
    if "qm_codes" not in qk4:
        return None, None, None, None
    return (_c(qk4["qm_codes"], np.int8), _c(qk4["qm_scale"], np.uint8), _c(qk4["k8_codes"], np.int8),
            _c(qk4["k8_scale"], np.uint8))


def qk4_scores(qk4, rows):
    qc, qs, kc, ks = (_c(qk4[k], np.uint8) for k in ("q4_codes", "q4_scale", "k4_codes", "k4_scale"))
    B, Hq, Nq, d = qc.shape
    _, Hkv, Nkv, _ = kc.shape
    rows = _c(rows, np.int64)
    out = np.empty((rows.size, Nkv), np.float32)
    mc, ms, k8c, k8s = _qm(qk4)
    if lib().oracle_qk4_scores(_p(qc), _p(qs), _p(kc), _p(ks), _p(mc), _p(ms), _p(k8c), _p(k8s), B, Hq, Hkv, Nq, Nkv,
                               d, _p(rows),
                               rows.size, _p(out)) != 0:
        raise ValueError("oracle qk4_scores: unsupported arguments")
    return out


def attn_rows_qk4(qk4, v_codes, v_scale, causal, sm_scale, rows=None, kv_tile=KV_TILE, want_p=False):
    """Oracle attention with 4-bit QK^T for flat query rows bh*Nq + i."""
    qc, qs, kc, ks = (_c(qk4[k], np.uint8) for k in ("q4_codes", "q4_scale", "k4_codes", "k4_scale"))
    vc = _c(v_codes, np.uint8)
    vs = _c(v_scale, np.float32)
    B, Hq, Nq, d = qc.shape
    _, Hkv, Nkv, _ = kc.shape
    if rows is None:
        rows = np.arange(B * Hq * Nq, dtype=np.int64)
    rows = _c(rows, np.int64)
    out = np.empty((rows.size, d), np.float32)
    p = np.empty((rows.size, Nkv), np.uint8) if want_p else None
    mc, ms, k8c, k8s = _qm(qk4)
    rc = lib().oracle_attn_rows_qk4(_p(qc), _p(qs), _p(kc), _p(ks), _p(mc), _p(ms), _p(k8c), _p(k8s), _p(vc), _p(vs),
                                    B, Hq, Hkv, Nq,
                                    Nkv, d, kv_tile,
                                    int(bool(causal)), float(sm_scale), _p(rows), rows.size, _p(out), _p(p))
    if rc != 0:
        raise ValueError("oracle_attn_rows_qk4: unsupported arguments")
    return (out, p) if want_p else out


def quantize_v4(V_bits, dtype):
    """V [B,H,N,d] in E2M1 blocks of 32 consecutive tokens per channel (MXFP4):
    codes [B,H,N,d] (one per value, 0..15) and E8M0 scale bytes [B,H,ceil(N/32),d]."""
    V_bits = _c(V_bits, np.uint16)
    B, H, N, d = V_bits.shape
    vc = np.empty((B, H, N, d), np.uint8)
    vs = np.empty((B, H, -(-N // 32), d), np.uint8)
    if lib().oracle_quantize_v4(_p(V_bits), dtype, B * H, N, d, _p(vc), _p(vs)) != 0:
        raise ValueError("oracle quantize_v4: unsupported shape")
    return vc, vs


def attn_rows_fp4(qk4, v4_codes, v4_scale, causal, sm_scale, rows=None, kv_tile=KV_TILE, want_p=False):
    """Oracle FP4 attention (4-bit QK^T, FP4 P~V) for flat query rows bh*Nq + i;
    with want_p also the E2M1 code of P~ of every visited key."""
    qc, qs, kc, ks = (_c(qk4[k], np.uint8) for k in ("q4_codes", "q4_scale", "k4_codes", "k4_scale"))
    vc, vs = _c(v4_codes, np.uint8), _c(v4_scale, np.uint8)
    B, Hq, Nq, d = qc.shape
    _, Hkv, Nkv, _ = kc.shape
    if rows is None:
        rows = np.arange(B * Hq * Nq, dtype=np.int64)
    rows = _c(rows, np.int64)
    out = np.empty((rows.size, d), np.float32)
    p = np.empty((rows.size, Nkv), np.uint8) if want_p else None
    rc = lib().oracle_attn_rows_fp4(_p(qc), _p(qs), _p(kc), _p(ks), _p(vc), _p(vs), B, Hq, Hkv, Nq, Nkv, d, kv_tile,
                                    int(bool(causal)), float(sm_scale), _p(rows), rows.size, _p(out), _p(p))
    if rc != 0:
        raise ValueError("oracle_attn_rows_fp4: unsupported arguments")
    return (out, p) if want_p else out


def run(Q_bits, K_bits, V_bits, dtype, blk_q, blk_k, causal, sm_scale, rows=None, kv_tile=KV_TILE,
        want_p=False):
    """The whole path on the CPU: quantize Q, K, V, then attention for ``rows``."""
    qk = quantize_qk(Q_bits, K_bits, dtype, blk_q, blk_k)
    vc, vs = quantize_v(V_bits, dtype)
    res = attn_rows(qk, vc, vs, blk_q, blk_k, causal, sm_scale, rows=rows, kv_tile=kv_tile, want_p=want_p)
    return qk, (vc, vs), res


# ---------------------------------------------------------------- exact reference
def exact_attention(Q, K, V, causal, sm_scale, rows=None, chunk=256):
    """softmax(Q K^T * sm_scale [+ causal mask]) V in fp64 from float inputs.

    Plain definition, evaluated in row chunks so that long sequences fit in
    memory.  Q [B,Hq,Nq,d]; K, V [B,Hkv,Nkv,d]; query head h reads K/V head
    h // (Hq // Hkv); causal: key j visible to query i iff j <= i + Nkv - Nq.
    Returns [nrows, d] for flat rows ``bh*Nq + i`` (all rows when None).
    """
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    B, Hq, Nq, d = Q.shape
    _, Hkv, Nkv, _ = K.shape
    group = Hq // Hkv
    Qf, Kf, Vf = Q.reshape(B * Hq, Nq, d), K.reshape(B * Hkv, Nkv, d), V.reshape(B * Hkv, Nkv, d)
    if rows is None:
        rows = np.arange(B * Hq * Nq, dtype=np.int64)
    rows = np.asarray(rows, np.int64)
    out = np.empty((rows.size, d), np.float64)
    for s in range(0, rows.size, chunk):
        r = rows[s:s + chunk]
        bh, i = r // Nq, r % Nq
        for h in np.unique(bh):
            sel = np.nonzero(bh == h)[0]
            qi = i[sel]
            hk = (h // Hq) * Hkv + (h % Hq) // group
            logits = (Qf[h][qi] @ Kf[hk].T) * sm_scale
            if causal:
                logits = np.where(np.arange(Nkv)[None, :] <= qi[:, None] + (Nkv - Nq), logits, -np.inf)
            logits -= logits.max(axis=1, keepdims=True)
            w = np.exp(logits)
            w /= w.sum(axis=1, keepdims=True)
            out[s + sel] = w @ Vf[hk]
    return out
