"""Thin Python binding of libsage.so (argument marshalling only).

Every step of the computation runs in the library's HIP kernels; PyTorch only
provides device memory and the current HIP stream.  Importing this module
fails loudly if the library has not been built: there is no fallback path.

The ``sage_*`` functions mirror the C ABI in ``include/sage.h`` one to one and
take raw integers (device pointers, sizes, stream handle).  The tensor-level
helpers below them allocate outputs with torch and call the C entry points.
"""
import ctypes
import math
import os

import torch  # loads torch's HIP runtime first, so the library binds to the same one

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsage.so")

SAGE_OK, SAGE_ERR_INVALID_ARG, SAGE_ERR_UNSUPPORTED, SAGE_ERR_MISALIGNED, SAGE_ERR_HIP, SAGE_ERR_WORKSPACE = range(6)
SAGE_F16, SAGE_BF16, SAGE_F32 = 0, 1, 2
SAGE_LAYOUT_BHND, SAGE_LAYOUT_BNHD = 0, 1
#: exported symbols, in header order
SYMBOLS = ("sage_status_string", "sage_kv_tile", "sage_quantize_qk_workspace_bytes", "sage_quantize_qk",
           "sage_quantize_qk_ex", "sage_quantize_v_workspace_bytes", "sage_quantize_v", "sage_quantize_v_ex",
           "sage_quantize_qkv_workspace_bytes", "sage_quantize_qkv",
           "sage_attn_fwd", "sage_attn_fwd_ex", "sage_attn_fwd_dump", "sage_attn_fwd_ex_dump", "sage_quantize_q",
           "sage_quantize_k", "sage_decode_kv_chunk", "sage_attn_decode_workspace_bytes", "sage_attn_decode",
           "sage_attn_decode_noalloc", "sage_quantize_qk4", "sage_attn_fwd_qk4", "sage_attn_fwd_qk4_dump", "sage_quantize_qk4_smooth_q",
           "sage_attn_fwd_qk4_smooth_q", "sage_attn_fwd_qk4_smooth_q_dump", "sage_quantize_v4", "sage_attn_fwd_fp4",
           "sage_attn_fwd_fp4_dump", "sage_probe_mfma_peak", "sage_probe_hbm_read")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
                      "(hipcc, gfx950); there is no CPU fallback")

_lib = ctypes.CDLL(LIB_PATH)
_P, _I, _SZ, _F = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
_lib.sage_status_string.restype = ctypes.c_char_p
_lib.sage_status_string.argtypes = [_I]
_lib.sage_kv_tile.restype = _I
_lib.sage_kv_tile.argtypes = []
_lib.sage_quantize_qk_workspace_bytes.restype = _SZ
_lib.sage_quantize_qk_workspace_bytes.argtypes = [_I, _I, _I, _I]
_lib.sage_quantize_v_workspace_bytes.restype = _SZ
_lib.sage_quantize_v_workspace_bytes.argtypes = [_I, _I, _I, _I]
_lib.sage_quantize_qk.restype = _I
_lib.sage_quantize_qk.argtypes = [_P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _SZ, _P]
_lib.sage_quantize_qk_ex.restype = _I
_lib.sage_quantize_qk_ex.argtypes = [_P, _P, _I, _I] + [_I] * 8 + [_P, _P, _P, _P, _P, _P, _SZ, _P]
_lib.sage_quantize_v.restype = _I
_lib.sage_quantize_v.argtypes = [_P, _I, _I, _I, _I, _I, _P, _P, _P, _SZ, _P]
_lib.sage_quantize_v_ex.restype = _I
_lib.sage_quantize_v_ex.argtypes = [_P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _SZ, _P]
_lib.sage_attn_fwd.restype = _I
_lib.sage_attn_fwd.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F, _P]
_lib.sage_attn_fwd_ex.restype = _I
_lib.sage_attn_fwd_ex.argtypes = [_P] * 7 + [_I] * 11 + [_F, _P]
_lib.sage_attn_fwd_dump.restype = _I
_lib.sage_attn_fwd_dump.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F, _P, _I, _P, _P, _P]
_lib.sage_quantize_q.restype = _I
_lib.sage_quantize_q.argtypes = [_P, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P]
_lib.sage_quantize_k.restype = _I
_lib.sage_quantize_k.argtypes = [_P, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _SZ, _P]
_lib.sage_decode_kv_chunk.restype = _I
_lib.sage_decode_kv_chunk.argtypes = [_I] * 6
_lib.sage_attn_decode_workspace_bytes.restype = _SZ
_lib.sage_attn_decode_workspace_bytes.argtypes = [_I] * 7
_lib.sage_attn_decode.restype = _I
_lib.sage_attn_decode.argtypes = [_P] * 7 + [_I] * 11 + [_F, _I, _P, _SZ, _P]
_lib.sage_attn_decode_noalloc.restype = _I
_lib.sage_attn_decode_noalloc.argtypes = [_P] * 7 + [_I] * 11 + [_F, _I, _P]
#: bytes of the library's per-device scratch array for sage_attn_decode_noalloc
SAGE_NOALLOC_SCRATCH_BYTES = 32 << 20
_lib.sage_quantize_qk4.restype = _I
_lib.sage_quantize_qk4.argtypes = [_P, _P] + [_I] * 8 + [_P] * 6 + [_SZ, _P]
_lib.sage_attn_fwd_qk4.restype = _I
_lib.sage_attn_fwd_qk4.argtypes = [_P] * 7 + [_I] * 9 + [_F, _P]
_lib.sage_attn_fwd_qk4_dump.restype = _I
_lib.sage_attn_fwd_qk4_dump.argtypes = [_P] * 7 + [_I] * 9 + [_F, _P, _I, _P, _P, _P]
_lib.sage_quantize_qk4_smooth_q.restype = _I
_lib.sage_quantize_qk4_smooth_q.argtypes = [_P, _P] + [_I] * 8 + [_P] * 11 + [_SZ, _P]
_lib.sage_attn_fwd_qk4_smooth_q.restype = _I
_lib.sage_attn_fwd_qk4_smooth_q.argtypes = [_P] * 11 + [_I] * 9 + [_F, _P]
_lib.sage_attn_fwd_qk4_smooth_q_dump.restype = _I
_lib.sage_attn_fwd_qk4_smooth_q_dump.argtypes = [_P] * 11 + [_I] * 9 + [_F, _P, _I, _P, _P, _P]
_lib.sage_quantize_v4.restype = _I
_lib.sage_quantize_v4.argtypes = [_P] + [_I] * 6 + [_P, _P, _P]
_lib.sage_attn_fwd_fp4.restype = _I
_lib.sage_attn_fwd_fp4.argtypes = [_P] * 7 + [_I] * 9 + [_F, _P]
_lib.sage_attn_fwd_fp4_dump.restype = _I
_lib.sage_attn_fwd_fp4_dump.argtypes = [_P] * 7 + [_I] * 9 + [_F, _P, _I, _P, _P, _P]
_lib.sage_attn_fwd_ex_dump.restype = _I
_lib.sage_attn_fwd_ex_dump.argtypes = [_P] * 7 + [_I] * 11 + [_F, _P, _I, _P, _P, _P]
_lib.sage_probe_mfma_peak.restype = _I
_lib.sage_probe_mfma_peak.argtypes = [_I, _I, _P, _P]
_lib.sage_quantize_qkv_workspace_bytes.restype = _SZ
_lib.sage_quantize_qkv_workspace_bytes.argtypes = [_I] * 4
_lib.sage_quantize_qkv.restype = _I
_lib.sage_quantize_qkv.argtypes = [_P] * 3 + [_I] * 10 + [_P] * 8 + [_SZ, _P]
_lib.sage_probe_hbm_read.restype = _I
_lib.sage_probe_hbm_read.argtypes = [_P, _SZ, _P, _P]


class SageError(RuntimeError):
    def __init__(self, status):
        self.status = status
        super().__init__(sage_status_string(status))


def _check(status):
    if status != SAGE_OK:
        raise SageError(status)


# ---------------------------------------------------------------- C ABI, 1:1
def sage_status_string(status):
    return _lib.sage_status_string(status).decode()


def sage_kv_tile():
    return _lib.sage_kv_tile()


def sage_probe_mfma_peak(workgroups, iters, sink=None, stream=None):
    return _lib.sage_probe_mfma_peak(workgroups, iters, sink, stream)


def sage_quantize_qkv_workspace_bytes(B, Hkv, Nkv, d):
    return _lib.sage_quantize_qkv_workspace_bytes(B, Hkv, Nkv, d)


def sage_quantize_qkv(Q, K, V, in_dtype, layout, B, Hq, Hkv, Nq, Nkv, d, blk_q, blk_k, q_codes, q_scale, k_codes,
                      k_scale, k_mean, v_codes, v_scale, workspace, workspace_bytes, stream):
    return _lib.sage_quantize_qkv(Q, K, V, in_dtype, layout, B, Hq, Hkv, Nq, Nkv, d, blk_q, blk_k, q_codes, q_scale,
                                  k_codes, k_scale, k_mean, v_codes, v_scale, workspace, workspace_bytes, stream)


def sage_probe_hbm_read(buf, nbytes, sink, stream=None):
    return _lib.sage_probe_hbm_read(buf, nbytes, sink, stream)


def sage_quantize_qk_workspace_bytes(B, H, N, d):
    return _lib.sage_quantize_qk_workspace_bytes(B, H, N, d)


def sage_quantize_v_workspace_bytes(B, H, N, d):
    return _lib.sage_quantize_v_workspace_bytes(B, H, N, d)


def sage_quantize_qk(Q, K, in_dtype, B, H, N, d, blk_q, blk_k, q_codes, q_scale, k_codes, k_scale, k_mean,
                     workspace, workspace_bytes, stream):
    return _lib.sage_quantize_qk(Q, K, in_dtype, B, H, N, d, blk_q, blk_k, q_codes, q_scale, k_codes, k_scale, k_mean,
                                 workspace, workspace_bytes, stream)


def sage_quantize_qk_ex(Q, K, in_dtype, layout, B, Hq, Hkv, Nq, Nkv, d, blk_q, blk_k, q_codes, q_scale, k_codes,
                        k_scale, k_mean, workspace, workspace_bytes, stream):
    return _lib.sage_quantize_qk_ex(Q, K, in_dtype, layout, B, Hq, Hkv, Nq, Nkv, d, blk_q, blk_k, q_codes, q_scale,
                                    k_codes, k_scale, k_mean, workspace, workspace_bytes, stream)


def sage_quantize_v(V, in_dtype, B, H, N, d, v_codes, v_scale, workspace, workspace_bytes, stream):
    return _lib.sage_quantize_v(V, in_dtype, B, H, N, d, v_codes, v_scale, workspace, workspace_bytes, stream)


def sage_quantize_v_ex(V, in_dtype, layout, B, H, N, d, v_codes, v_scale, workspace, workspace_bytes, stream):
    return _lib.sage_quantize_v_ex(V, in_dtype, layout, B, H, N, d, v_codes, v_scale, workspace, workspace_bytes,
                                   stream)


def sage_attn_fwd(q_codes, q_scale, k_codes, k_scale, v_codes, v_scale, O, out_dtype, B, H, N, d, blk_q, blk_k,
                  causal, sm_scale, stream):
    return _lib.sage_attn_fwd(q_codes, q_scale, k_codes, k_scale, v_codes, v_scale, O, out_dtype, B, H, N, d, blk_q,
                              blk_k, causal, sm_scale, stream)


def sage_attn_fwd_ex(q_codes, q_scale, k_codes, k_scale, v_codes, v_scale, O, out_dtype, layout, B, Hq, Hkv, Nq, Nkv,
                     d, blk_q, blk_k, causal, sm_scale, stream):
    return _lib.sage_attn_fwd_ex(q_codes, q_scale, k_codes, k_scale, v_codes, v_scale, O, out_dtype, layout, B, Hq,
                                 Hkv, Nq, Nkv, d, blk_q, blk_k, causal, sm_scale, stream)


def sage_attn_fwd_dump(q_codes, q_scale, k_codes, k_scale, v_codes, v_scale, O, out_dtype, B, H, N, d, blk_q, blk_k,
                       causal, sm_scale, sel, n_sel, s_dump, p_dump, stream):
    return _lib.sage_attn_fwd_dump(q_codes, q_scale, k_codes, k_scale, v_codes, v_scale, O, out_dtype, B, H, N, d,
                                   blk_q, blk_k, causal, sm_scale, sel, n_sel, s_dump, p_dump, stream)


def sage_attn_fwd_ex_dump(q_codes, q_scale, k_codes, k_scale, v_codes, v_scale, O, out_dtype, layout, B, Hq, Hkv, Nq,
                          Nkv, d, blk_q, blk_k, causal, sm_scale, sel, n_sel, s_dump, p_dump, stream):
    return _lib.sage_attn_fwd_ex_dump(q_codes, q_scale, k_codes, k_scale, v_codes, v_scale, O, out_dtype, layout, B,
                                      Hq, Hkv, Nq, Nkv, d, blk_q, blk_k, causal, sm_scale, sel, n_sel, s_dump, p_dump,
                                      stream)


def sage_quantize_q(Q, in_dtype, layout, B, Hq, Nq, d, blk_q, q_codes, q_scale, stream):
    return _lib.sage_quantize_q(Q, in_dtype, layout, B, Hq, Nq, d, blk_q, q_codes, q_scale, stream)


def sage_quantize_k(K, in_dtype, layout, B, Hkv, Nkv, d, blk_k, k_codes, k_scale, k_mean, workspace, workspace_bytes,
                    stream):
    return _lib.sage_quantize_k(K, in_dtype, layout, B, Hkv, Nkv, d, blk_k, k_codes, k_scale, k_mean, workspace,
                                workspace_bytes, stream)


def sage_decode_kv_chunk(B, Hq, Hkv, Nq, Nkv, d):
    return _lib.sage_decode_kv_chunk(B, Hq, Hkv, Nq, Nkv, d)


def sage_attn_decode_workspace_bytes(B, Hq, Hkv, Nq, Nkv, d, kv_chunk):
    return _lib.sage_attn_decode_workspace_bytes(B, Hq, Hkv, Nq, Nkv, d, kv_chunk)


def sage_attn_decode(q_codes, q_scale, k_codes, k_scale, v_codes, v_scale, O, out_dtype, layout, B, Hq, Hkv, Nq, Nkv,
                     d, blk_q, blk_k, causal, sm_scale, kv_chunk, workspace, workspace_bytes, stream):
    return _lib.sage_attn_decode(q_codes, q_scale, k_codes, k_scale, v_codes, v_scale, O, out_dtype, layout, B, Hq,
                                 Hkv, Nq, Nkv, d, blk_q, blk_k, causal, sm_scale, kv_chunk, workspace,
                                 workspace_bytes, stream)


def sage_attn_decode_noalloc(q_codes, q_scale, k_codes, k_scale, v_codes, v_scale, O, out_dtype, layout, B, Hq, Hkv,
                             Nq, Nkv, d, blk_q, blk_k, causal, sm_scale, kv_chunk, stream):
    return _lib.sage_attn_decode_noalloc(q_codes, q_scale, k_codes, k_scale, v_codes, v_scale, O, out_dtype, layout,
                                         B, Hq, Hkv, Nq, Nkv, d, blk_q, blk_k, causal, sm_scale, kv_chunk, stream)


def sage_quantize_qk4(Q, K, in_dtype, layout, B, Hq, Hkv, Nq, Nkv, d, q4_codes, q4_scale, k4_codes, k4_scale, k_mean,
                      workspace, workspace_bytes, stream):
    return _lib.sage_quantize_qk4(Q, K, in_dtype, layout, B, Hq, Hkv, Nq, Nkv, d, q4_codes, q4_scale, k4_codes,
                                  k4_scale, k_mean, workspace, workspace_bytes, stream)


def sage_attn_fwd_qk4(q4_codes, q4_scale, k4_codes, k4_scale, v_codes, v_scale, O, out_dtype, layout, B, Hq, Hkv, Nq,
                      Nkv, d, causal, sm_scale, stream):
    return _lib.sage_attn_fwd_qk4(q4_codes, q4_scale, k4_codes, k4_scale, v_codes, v_scale, O, out_dtype, layout, B,
                                  Hq, Hkv, Nq, Nkv, d, causal, sm_scale, stream)


def sage_attn_fwd_qk4_dump(q4_codes, q4_scale, k4_codes, k4_scale, v_codes, v_scale, O, out_dtype, layout, B, Hq,
                           Hkv, Nq, Nkv, d, causal, sm_scale, sel, n_sel, s_dump, p_dump, stream):
    return _lib.sage_attn_fwd_qk4_dump(q4_codes, q4_scale, k4_codes, k4_scale, v_codes, v_scale, O, out_dtype, layout,
                                       B, Hq, Hkv, Nq, Nkv, d, causal, sm_scale, sel, n_sel, s_dump, p_dump, stream)


def sage_quantize_qk4_smooth_q(Q, K, in_dtype, layout, B, Hq, Hkv, Nq, Nkv, d, q4_codes, q4_scale, k4_codes, k4_scale,
                               k_mean, q_mean, qm_codes, qm_scale, k8_codes, k8_scale, workspace, workspace_bytes,
                               stream):
    return _lib.sage_quantize_qk4_smooth_q(Q, K, in_dtype, layout, B, Hq, Hkv, Nq, Nkv, d, q4_codes, q4_scale,
                                           k4_codes, k4_scale, k_mean, q_mean, qm_codes, qm_scale, k8_codes, k8_scale,
                                           workspace, workspace_bytes, stream)


def sage_attn_fwd_qk4_smooth_q(q4_codes, q4_scale, k4_codes, k4_scale, qm_codes, qm_scale, k8_codes, k8_scale, v_codes,
                               v_scale, O, out_dtype, layout, B, Hq, Hkv, Nq, Nkv, d, causal, sm_scale, stream):
    return _lib.sage_attn_fwd_qk4_smooth_q(q4_codes, q4_scale, k4_codes, k4_scale, qm_codes, qm_scale, k8_codes,
                                           k8_scale, v_codes, v_scale, O, out_dtype, layout, B, Hq, Hkv, Nq, Nkv, d,
                                           causal, sm_scale, stream)


def sage_attn_fwd_qk4_smooth_q_dump(q4_codes, q4_scale, k4_codes, k4_scale, qm_codes, qm_scale, k8_codes, k8_scale,
                                    v_codes, v_scale, O, out_dtype, layout, B, Hq, Hkv, Nq, Nkv, d, causal, sm_scale,
                                    sel, n_sel, s_dump, p_dump, stream):
    return _lib.sage_attn_fwd_qk4_smooth_q_dump(q4_codes, q4_scale, k4_codes, k4_scale, qm_codes, qm_scale, k8_codes,
                                                k8_scale, v_codes, v_scale, O, out_dtype, layout, B, Hq, Hkv, Nq, Nkv,
                                                d, causal, sm_scale, sel, n_sel, s_dump, p_dump, stream)


def sage_quantize_v4(V, in_dtype, layout, B, H, N, d, v4_codes, v4_scale, stream):
    return _lib.sage_quantize_v4(V, in_dtype, layout, B, H, N, d, v4_codes, v4_scale, stream)


def sage_attn_fwd_fp4(q4_codes, q4_scale, k4_codes, k4_scale, v4_codes, v4_scale, O, out_dtype, layout, B, Hq, Hkv,
                      Nq, Nkv, d, causal, sm_scale, stream):
    return _lib.sage_attn_fwd_fp4(q4_codes, q4_scale, k4_codes, k4_scale, v4_codes, v4_scale, O, out_dtype, layout, B,
                                  Hq, Hkv, Nq, Nkv, d, causal, sm_scale, stream)


def sage_attn_fwd_fp4_dump(q4_codes, q4_scale, k4_codes, k4_scale, v4_codes, v4_scale, O, out_dtype, layout, B, Hq,
                           Hkv, Nq, Nkv, d, causal, sm_scale, sel, n_sel, s_dump, p_dump, stream):
    return _lib.sage_attn_fwd_fp4_dump(q4_codes, q4_scale, k4_codes, k4_scale, v4_codes, v4_scale, O, out_dtype, layout,
                                       B, Hq, Hkv, Nq, Nkv, d, causal, sm_scale, sel, n_sel, s_dump, p_dump, stream)


# ---------------------------------------------------------------- tensor helpers
_DT = {torch.float16: SAGE_F16, torch.bfloat16: SAGE_BF16, torch.float32: SAGE_F32}


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _ptr(t):
    return t.data_ptr() if t is not None else None


_LAYOUTS = {"bhnd": SAGE_LAYOUT_BHND, "bnhd": SAGE_LAYOUT_BNHD}


def _layout(layout):
    if layout not in _LAYOUTS:
        raise ValueError(f"layout must be one of {sorted(_LAYOUTS)}")
    return _LAYOUTS[layout]


def _bhnd(x, layout):
    """(B, H, N, d) of a contiguous CUDA tensor in ``layout``."""
    if x.dim() != 4 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("expected a contiguous CUDA tensor [B, H, N, d] or [B, N, H, d]")
    B, a, b, d = x.shape
    return (B, a, b, d) if _layout(layout) == SAGE_LAYOUT_BHND else (B, b, a, d)


def _round_up(n, m):
    return -(-n // m) * m


def _expect(t, shape, dtypes, dev, name):
    """A tensor handed to the library: contiguous, on ``dev``, of ``shape`` and
    one of ``dtypes`` (the C ABI cannot see buffer sizes, so they are checked
    here before any pointer is passed)."""
    if not torch.is_tensor(t) or t.device != dev or not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor on {dev}")
    if tuple(t.shape) != tuple(shape) or t.dtype not in dtypes:
        raise ValueError(f"{name}: expected shape {tuple(shape)} and dtype in {dtypes}, "
                         f"got {tuple(t.shape)} {t.dtype}")


def _workspace(workspace, nbytes, dev):
    """The caller's workspace (any contiguous tensor on ``dev``), or a new one."""
    if workspace is None:
        return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    if not torch.is_tensor(workspace) or workspace.device != dev or not workspace.is_contiguous():
        raise ValueError(f"workspace: expected a contiguous tensor on {dev}")
    return workspace


_OUT_DTYPES = (torch.float32, torch.float16, torch.bfloat16)


def _out(out, B, H, N, d, out_dtype, layout, dev):
    """O as given (checked) or new: [B,H,N,d] or [B,N,H,d]."""
    shape = (B, H, N, d) if _layout(layout) == SAGE_LAYOUT_BHND else (B, N, H, d)
    if out is None:
        return torch.empty(shape, dtype=out_dtype, device=dev)
    _expect(out, shape, _OUT_DTYPES, dev, "out")
    return out


def _check_dump(dump, Nkv, dev):
    """(sel int32 [n], s_dump int32 [n,128,Nkv], p_dump uint8 [n,128,Nkv]) of the dump calls."""
    sel, s_dump, p_dump = dump
    n = sel.numel()
    _expect(sel, (n,), (torch.int32,), dev, "sel")
    _expect(s_dump, (n, 128, Nkv), (torch.int32,), dev, "s_dump")
    _expect(p_dump, (n, 128, Nkv), (torch.uint8,), dev, "p_dump")
    return sel, s_dump, p_dump


def _check_v(v, B, Hkv, Nkt, d, dev):
    """(v_codes, v_scale) from quantize_v for B x Hkv heads of Nkt (tile-padded) keys."""
    v_codes, v_scale = v
    kt = sage_kv_tile()
    _expect(v_codes, (B, Hkv, Nkt // kt, d, kt), (torch.uint8,), dev, "v_codes")
    _expect(v_scale, (B, Hkv, d), (torch.float32,), dev, "v_scale")
    return v_codes, v_scale


def _plain(B, Hq, Hkv, Nq, Nkv, layout):
    return _layout(layout) == SAGE_LAYOUT_BHND and Hq == Hkv and Nq == Nkv


def quantize_qk(Q, K, blk_q=128, blk_k=64, layout="bhnd", workspace=None, stream=None):
    """INT8 per-block Q and smoothed K.  Q: [B,Hq,Nq,d], K: [B,Hkv,Nkv,d] (or
    [B,N,H,d] with layout="bnhd").  Returns a dict of device tensors; the codes
    and scales are head-major whatever the layout, with Q codes padded to a
    multiple of 128 rows and K codes to a multiple of 64 (zero codes), plus
    the true lengths "Nq" and "Nkv"."""
    B, Hq, Nq, d = _bhnd(Q, layout)
    Bk, Hkv, Nkv, dk = _bhnd(K, layout)
    if (Bk, dk) != (B, d) or K.dtype != Q.dtype or K.device != Q.device:
        raise ValueError("Q and K must have the same batch, head dim, dtype and device")
    dev = Q.device
    Nqp, Nkt = _round_up(Nq, 128), _round_up(Nkv, sage_kv_tile())
    out = dict(q_codes=torch.empty((B, Hq, Nqp, d), dtype=torch.int8, device=dev),
               q_scale=torch.empty((B, Hq, Nqp // blk_q), dtype=torch.float32, device=dev),
               k_codes=torch.empty((B, Hkv, Nkt, d), dtype=torch.int8, device=dev),
               k_scale=torch.empty((B, Hkv, Nkt // blk_k), dtype=torch.float32, device=dev),
               k_mean=torch.empty((B, Hkv, d), dtype=torch.float32, device=dev))
    workspace = _workspace(workspace, sage_quantize_qk_workspace_bytes(B, Hkv, Nkv, d), dev)
    ptrs = (_ptr(out["q_codes"]), _ptr(out["q_scale"]), _ptr(out["k_codes"]), _ptr(out["k_scale"]),
            _ptr(out["k_mean"]), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    dt = _DT.get(Q.dtype, -1)
    if _plain(B, Hq, Hkv, Nq, Nkv, layout):
        _check(sage_quantize_qk(_ptr(Q), _ptr(K), dt, B, Hq, Nq, d, blk_q, blk_k, *ptrs))
    else:
        _check(sage_quantize_qk_ex(_ptr(Q), _ptr(K), dt, _layout(layout), B, Hq, Hkv, Nq, Nkv, d, blk_q, blk_k,
                                   *ptrs))
    out.update(blk_q=blk_q, blk_k=blk_k, Nq=Nq, Nkv=Nkv)
    return out


def quantize_v(V, layout="bhnd", workspace=None, stream=None):
    """FP8 e4m3 V with per-channel scales.  Returns (v_codes, v_scale); v_codes
    is in KV-tile channel-major order (see ``v_codes_to_natural``), padded with
    zero codes to whole tiles of 64 tokens."""
    B, H, N, d = _bhnd(V, layout)
    dev = V.device
    kt = sage_kv_tile()
    v_codes = torch.empty((B, H, -(-N // kt), d, kt), dtype=torch.uint8, device=dev)
    v_scale = torch.empty((B, H, d), dtype=torch.float32, device=dev)
    workspace = _workspace(workspace, sage_quantize_v_workspace_bytes(B, H, N, d), dev)
    rest = (_ptr(v_codes), _ptr(v_scale), _ptr(workspace), workspace.numel() * workspace.element_size(),
            _stream(stream))
    dt = _DT.get(V.dtype, -1)
    if _layout(layout) == SAGE_LAYOUT_BHND:
        _check(sage_quantize_v(_ptr(V), dt, B, H, N, d, *rest))
    else:
        _check(sage_quantize_v_ex(_ptr(V), dt, _layout(layout), B, H, N, d, *rest))
    return v_codes, v_scale


def quantize_qkv(Q, K, V, blk_q=128, blk_k=64, layout="bhnd", workspace=None, stream=None):
    """quantize_qk(Q, K) and quantize_v(V) in one library call (the same outputs bit for bit,
    fewer launches).  Returns (qk dict, (v_codes, v_scale)) as those two helpers do."""
    B, Hq, Nq, d = _bhnd(Q, layout)
    Bk, Hkv, Nkv, dk = _bhnd(K, layout)
    if (Bk, dk) != (B, d) or K.dtype != Q.dtype or K.device != Q.device:
        raise ValueError("Q and K must have the same batch, head dim, dtype and device")
    if tuple(V.shape) != tuple(K.shape) or V.dtype != K.dtype or V.device != K.device:
        raise ValueError("V must have the shape, dtype and device of K")
    dev = Q.device
    Nqp, Nkt = _round_up(Nq, 128), _round_up(Nkv, sage_kv_tile())
    out = dict(q_codes=torch.empty((B, Hq, Nqp, d), dtype=torch.int8, device=dev),
               q_scale=torch.empty((B, Hq, Nqp // blk_q), dtype=torch.float32, device=dev),
               k_codes=torch.empty((B, Hkv, Nkt, d), dtype=torch.int8, device=dev),
               k_scale=torch.empty((B, Hkv, Nkt // blk_k), dtype=torch.float32, device=dev),
               k_mean=torch.empty((B, Hkv, d), dtype=torch.float32, device=dev))
    v_codes = torch.empty((B, Hkv, Nkt // sage_kv_tile(), d, sage_kv_tile()), dtype=torch.uint8, device=dev)
    v_scale = torch.empty((B, Hkv, d), dtype=torch.float32, device=dev)
    workspace = _workspace(workspace, sage_quantize_qkv_workspace_bytes(B, Hkv, Nkv, d), dev)
    _check(sage_quantize_qkv(_ptr(Q), _ptr(K), _ptr(V), _DT.get(Q.dtype, -1), _layout(layout), B, Hq, Hkv, Nq, Nkv, d,
                             blk_q, blk_k, _ptr(out["q_codes"]), _ptr(out["q_scale"]), _ptr(out["k_codes"]),
                             _ptr(out["k_scale"]), _ptr(out["k_mean"]), _ptr(v_codes), _ptr(v_scale), _ptr(workspace),
                             workspace.numel() * workspace.element_size(), _stream(stream)))
    out.update(blk_q=blk_q, blk_k=blk_k, Nq=Nq, Nkv=Nkv)
    return out, (v_codes, v_scale)


def v_codes_to_natural(v_codes):
    """[B, H, Nt/64, d, 64] tile layout -> [B, H, Nt, d] token-major (Nt: tokens rounded up to 64)."""
    B, H, T, d, kt = v_codes.shape
    return v_codes.permute(0, 1, 2, 4, 3).reshape(B, H, T * kt, d)


def default_sm_scale(d):
    return float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32))


def attn_fwd(qk, v, causal=False, sm_scale=None, out_dtype=torch.float32, out=None, layout="bhnd", stream=None,
             dump=None):
    """Attention on quantized operands.  ``qk`` from quantize_qk, ``v`` = (v_codes, v_scale).
    O is [B,Hq,Nq,d] (or [B,Nq,Hq,d] with layout="bnhd").  ``dump`` = (sel int32
    tensor, s_dump, p_dump) routes through the dump entry points."""
    B, Hq, _, d = qk["q_codes"].shape
    Hkv, Nkt = qk["k_codes"].shape[1], qk["k_codes"].shape[2]
    Nq, Nkv = qk["Nq"], qk["Nkv"]
    dev = qk["q_codes"].device
    v_codes, v_scale = _check_v(v, B, Hkv, Nkt, d, dev)
    if sm_scale is None:
        sm_scale = default_sm_scale(d)
    out = _out(out, B, Hq, Nq, d, out_dtype, layout, dev)
    ops = (_ptr(qk["q_codes"]), _ptr(qk["q_scale"]), _ptr(qk["k_codes"]), _ptr(qk["k_scale"]), _ptr(v_codes),
           _ptr(v_scale), _ptr(out), _DT.get(out.dtype, -1))
    tail = (d, qk["blk_q"], qk["blk_k"], int(bool(causal)), float(sm_scale))
    plain = _plain(B, Hq, Hkv, Nq, Nkv, layout)
    shape = (B, Hq, Nq) if plain else (_layout(layout), B, Hq, Hkv, Nq, Nkv)
    if dump is None:
        fn = sage_attn_fwd if plain else sage_attn_fwd_ex
        _check(fn(*ops, *shape, *tail, _stream(stream)))
    else:
        sel, s_dump, p_dump = _check_dump(dump, Nkv, dev)
        fn = sage_attn_fwd_dump if plain else sage_attn_fwd_ex_dump
        _check(fn(*ops, *shape, *tail, _ptr(sel), sel.numel(), _ptr(s_dump), _ptr(p_dump), _stream(stream)))
    return out


def quantize_q(Q, blk_q=128, layout="bhnd", stream=None):
    """INT8 blocks of Q alone (the queries of a decode step).  Returns a dict
    with q_codes (padded to a multiple of 128 rows), q_scale, blk_q and Nq."""
    B, Hq, Nq, d = _bhnd(Q, layout)
    dev = Q.device
    Nqp = _round_up(Nq, 128)
    out = dict(q_codes=torch.empty((B, Hq, Nqp, d), dtype=torch.int8, device=dev),
               q_scale=torch.empty((B, Hq, Nqp // blk_q), dtype=torch.float32, device=dev))
    _check(sage_quantize_q(_ptr(Q), _DT.get(Q.dtype, -1), _layout(layout), B, Hq, Nq, d, blk_q, _ptr(out["q_codes"]),
                           _ptr(out["q_scale"]), _stream(stream)))
    out.update(blk_q=blk_q, Nq=Nq)
    return out


def quantize_k(K, blk_k=64, layout="bhnd", workspace=None, stream=None):
    """K mean and smoothed INT8 blocks of K alone (a K cache).  Returns a dict
    with k_codes (padded to a multiple of 64 rows), k_scale, k_mean, blk_k and Nkv."""
    B, Hkv, Nkv, d = _bhnd(K, layout)
    dev = K.device
    Nkt = _round_up(Nkv, sage_kv_tile())
    out = dict(k_codes=torch.empty((B, Hkv, Nkt, d), dtype=torch.int8, device=dev),
               k_scale=torch.empty((B, Hkv, Nkt // blk_k), dtype=torch.float32, device=dev),
               k_mean=torch.empty((B, Hkv, d), dtype=torch.float32, device=dev))
    workspace = _workspace(workspace, sage_quantize_qk_workspace_bytes(B, Hkv, Nkv, d), dev)
    _check(sage_quantize_k(_ptr(K), _DT.get(K.dtype, -1), _layout(layout), B, Hkv, Nkv, d, blk_k,
                           _ptr(out["k_codes"]), _ptr(out["k_scale"]), _ptr(out["k_mean"]), _ptr(workspace),
                           workspace.numel() * workspace.element_size(), _stream(stream)))
    out.update(blk_k=blk_k, Nkv=Nkv)
    return out


def attn_decode(q, kc, v, causal=True, sm_scale=None, out_dtype=torch.float32, out=None, layout="bhnd",
                kv_chunk=0, workspace=None, stream=None):
    """Split-KV attention of quantized queries ``q`` (from quantize_q) against a
    quantized cache: ``kc`` from quantize_k (or quantize_qk), ``v`` = (v_codes,
    v_scale) from quantize_v.  kv_chunk 0 = the library's default split."""
    B, Hq, _, d = q["q_codes"].shape
    Bk, Hkv, Nkt, dk = kc["k_codes"].shape
    if (Bk, dk) != (B, d) or kc["k_codes"].device != q["q_codes"].device:
        raise ValueError("queries and cache must have the same batch, head dim and device")
    Nq, Nkv = q["Nq"], kc["Nkv"]
    dev = q["q_codes"].device
    v_codes, v_scale = _check_v(v, B, Hkv, Nkt, d, dev)
    if sm_scale is None:
        sm_scale = default_sm_scale(d)
    if kv_chunk == 0:
        kv_chunk = sage_decode_kv_chunk(B, Hq, Hkv, Nq, Nkv, d)
    out = _out(out, B, Hq, Nq, d, out_dtype, layout, dev)
    wsb = sage_attn_decode_workspace_bytes(B, Hq, Hkv, Nq, Nkv, d, kv_chunk)
    workspace = _workspace(workspace, wsb, dev)
    _check(sage_attn_decode(_ptr(q["q_codes"]), _ptr(q["q_scale"]), _ptr(kc["k_codes"]), _ptr(kc["k_scale"]),
                            _ptr(v_codes), _ptr(v_scale), _ptr(out), _DT.get(out.dtype, -1), _layout(layout), B, Hq,
                            Hkv, Nq, Nkv, d, q["blk_q"], kc["blk_k"], int(bool(causal)), float(sm_scale), kv_chunk,
                            _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def quantize_qk4(Q, K, layout="bhnd", workspace=None, stream=None, smooth_q=False):
    """4-bit Q and smoothed K (E2M1, a power-of-two scale per 32 channels).
    Returns a dict with q4_codes [B,Hq,Nqp,d/2], q4_scale [B,Hq,Nqp,d/32],
    k4_codes, k4_scale, k_mean, Nq and Nkv; with ``smooth_q`` also q_mean
    [B,Hq,Nqp/32,d] with its INT8 codes qm_codes and exponent bytes qm_scale
    [B,Hq,Nqp/32], and the smoothed K in INT8, k8_codes [B,Hkv,Nkt,d] with
    one exponent byte per 64-key tile, k8_scale [B,Hkv,Nkt/64]."""
    B, Hq, Nq, d = _bhnd(Q, layout)
    Bk, Hkv, Nkv, dk = _bhnd(K, layout)
    if (Bk, dk) != (B, d) or K.dtype != Q.dtype or K.device != Q.device:
        raise ValueError("Q and K must have the same batch, head dim, dtype and device")
    dev = Q.device
    Nqp, Nkt = _round_up(Nq, 128), _round_up(Nkv, sage_kv_tile())
    out = dict(q4_codes=torch.empty((B, Hq, Nqp, d // 2), dtype=torch.uint8, device=dev),
               q4_scale=torch.empty((B, Hq, Nqp, d // 32), dtype=torch.uint8, device=dev),
               k4_codes=torch.empty((B, Hkv, Nkt, d // 2), dtype=torch.uint8, device=dev),
               k4_scale=torch.empty((B, Hkv, Nkt, d // 32), dtype=torch.uint8, device=dev),
               k_mean=torch.empty((B, Hkv, d), dtype=torch.float32, device=dev))
    workspace = _workspace(workspace, sage_quantize_qk_workspace_bytes(B, Hkv, Nkv, d), dev)
    head = (_ptr(Q), _ptr(K), _DT.get(Q.dtype, -1), _layout(layout), B, Hq, Hkv, Nq, Nkv, d, _ptr(out["q4_codes"]),
            _ptr(out["q4_scale"]), _ptr(out["k4_codes"]), _ptr(out["k4_scale"]), _ptr(out["k_mean"]))
    tail = (_ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    if smooth_q:
        nb = Nqp // 32
        out.update(q_mean=torch.empty((B, Hq, nb, d), dtype=torch.float32, device=dev),
                   qm_codes=torch.empty((B, Hq, nb, d), dtype=torch.int8, device=dev),
                   qm_scale=torch.empty((B, Hq, nb), dtype=torch.uint8, device=dev),
                   k8_codes=torch.empty((B, Hkv, Nkt, d), dtype=torch.int8, device=dev),
                   k8_scale=torch.empty((B, Hkv, Nkt // sage_kv_tile()), dtype=torch.uint8, device=dev))
        _check(sage_quantize_qk4_smooth_q(*head, _ptr(out["q_mean"]), _ptr(out["qm_codes"]), _ptr(out["qm_scale"]),
                                          _ptr(out["k8_codes"]), _ptr(out["k8_scale"]), *tail))
    else:
        _check(sage_quantize_qk4(*head, *tail))
    out.update(Nq=Nq, Nkv=Nkv)
    return out


def attn_fwd_qk4(qk4, v, causal=False, sm_scale=None, out_dtype=torch.float32, out=None, layout="bhnd", stream=None,
                 dump=None):
    """Attention with 4-bit QK^T: ``qk4`` from quantize_qk4 (with or without
    Q smoothing), ``v`` from quantize_v."""
    B, Hq, _, h2 = qk4["q4_codes"].shape
    d = 2 * h2
    Hkv, Nkt = qk4["k4_codes"].shape[1], qk4["k4_codes"].shape[2]
    Nq, Nkv = qk4["Nq"], qk4["Nkv"]
    dev = qk4["q4_codes"].device
    v_codes, v_scale = _check_v(v, B, Hkv, Nkt, d, dev)
    if sm_scale is None:
        sm_scale = default_sm_scale(d)
    out = _out(out, B, Hq, Nq, d, out_dtype, layout, dev)
    smooth = "qm_codes" in qk4
    ops = (_ptr(qk4["q4_codes"]), _ptr(qk4["q4_scale"]), _ptr(qk4["k4_codes"]), _ptr(qk4["k4_scale"]))
    if smooth:
        ops += (_ptr(qk4["qm_codes"]), _ptr(qk4["qm_scale"]), _ptr(qk4["k8_codes"]), _ptr(qk4["k8_scale"]))
    args = ops + (_ptr(v_codes), _ptr(v_scale), _ptr(out), _DT.get(out.dtype, -1), _layout(layout), B, Hq, Hkv, Nq,
                  Nkv, d, int(bool(causal)), float(sm_scale))
    if dump is None:
        _check((sage_attn_fwd_qk4_smooth_q if smooth else sage_attn_fwd_qk4)(*args, _stream(stream)))
    else:
        sel, s_dump, p_dump = _check_dump(dump, Nkv, dev)
        fn = sage_attn_fwd_qk4_smooth_q_dump if smooth else sage_attn_fwd_qk4_dump
        _check(fn(*args, _ptr(sel), sel.numel(), _ptr(s_dump), _ptr(p_dump), _stream(stream)))
    return out


def quantize_v4(V, layout="bhnd", stream=None):
    """V in E2M1 with one E8M0 scale per channel and 32 tokens (MXFP4), for
    attn_fwd_fp4.  Returns (v4_codes [B,H,Nt/64,d,32] bytes: per KV tile, d
    channel rows of 64 codes, two per byte, low nibble first; v4_scale
    [B,H,Nt/64,2,32,d/32] bytes: per tile, byte (g, m, c) for channel 32c + m
    and tokens 32g ..); see ``v4_to_natural``."""
    B, H, N, d = _bhnd(V, layout)
    dev = V.device
    kt = sage_kv_tile()
    T = -(-N // kt)
    v4_codes = torch.empty((B, H, T, d, kt // 2), dtype=torch.uint8, device=dev)
    v4_scale = torch.empty((B, H, T, 2, 32, d // 32), dtype=torch.uint8, device=dev)
    _check(sage_quantize_v4(_ptr(V), _DT.get(V.dtype, -1), _layout(layout), B, H, N, d, _ptr(v4_codes),
                            _ptr(v4_scale), _stream(stream)))
    return v4_codes, v4_scale


def v4_to_natural(v4):
    """(v4_codes, v4_scale) of quantize_v4 -> (codes [B,H,Nt,d] one per value,
    scales [B,H,Nt/32,d]) token-major (Nt: tokens rounded up to 64)."""
    codes, scale = v4
    B, H, T, d, kb = codes.shape
    lo, hi = codes & 0xF, codes >> 4
    nib = torch.stack((lo, hi), dim=-1).reshape(B, H, T, d, 2 * kb)              # [.., d, 64 tokens]
    nat = nib.permute(0, 1, 2, 4, 3).reshape(B, H, T * 2 * kb, d)
    sc = scale.permute(0, 1, 2, 3, 5, 4).reshape(B, H, T, 2, d).reshape(B, H, 2 * T, d)   # channel 32c + m
    return nat, sc


def attn_fwd_fp4(qk4, v4, causal=False, sm_scale=None, out_dtype=torch.float32, out=None, layout="bhnd", stream=None,
                 dump=None):
    """FP4 attention: ``qk4`` from quantize_qk4 (without Q smoothing), ``v4``
    from quantize_v4; the scores and P~V both on the FP4 matrix instructions."""
    if "qm_codes" in qk4:
        raise ValueError("attn_fwd_fp4 takes the plain 4-bit Q/K codes (no Q smoothing)")
    B, Hq, _, h2 = qk4["q4_codes"].shape
    d = 2 * h2
    Hkv, Nkt = qk4["k4_codes"].shape[1], qk4["k4_codes"].shape[2]
    Nq, Nkv = qk4["Nq"], qk4["Nkv"]
    dev = qk4["q4_codes"].device
    kt = sage_kv_tile()
    v4_codes, v4_scale = v4
    _expect(v4_codes, (B, Hkv, Nkt // kt, d, kt // 2), (torch.uint8,), dev, "v4_codes")
    _expect(v4_scale, (B, Hkv, Nkt // kt, 2, 32, d // 32), (torch.uint8,), dev, "v4_scale")
    if sm_scale is None:
        sm_scale = default_sm_scale(d)
    out = _out(out, B, Hq, Nq, d, out_dtype, layout, dev)
    args = (_ptr(qk4["q4_codes"]), _ptr(qk4["q4_scale"]), _ptr(qk4["k4_codes"]), _ptr(qk4["k4_scale"]),
            _ptr(v4_codes), _ptr(v4_scale), _ptr(out), _DT.get(out.dtype, -1), _layout(layout), B, Hq, Hkv, Nq, Nkv,
            d, int(bool(causal)), float(sm_scale))
    if dump is None:
        _check(sage_attn_fwd_fp4(*args, _stream(stream)))
    else:
        sel, s_dump, p_dump = _check_dump(dump, Nkv, dev)
        _check(sage_attn_fwd_fp4_dump(*args, _ptr(sel), sel.numel(), _ptr(s_dump), _ptr(p_dump), _stream(stream)))
    return out


def attention(q, k, v, causal=False, sm_scale=None, blk_q=128, blk_k=64, out_dtype=None, layout="bhnd",
              stream=None):
    """Drop-in quantized attention forward for float16/bfloat16 inputs: q
    [B,Hq,Nq,d], k and v [B,Hkv,Nkv,d] (layout="bhnd", the layout of PyTorch's
    scaled_dot_product_attention) or [B,N,H,d] (layout="bnhd").  Hq must be a
    multiple of Hkv; causal needs Nkv >= Nq (queries are the last Nq positions)."""
    qk = quantize_qk(q, k, blk_q, blk_k, layout=layout, stream=stream)
    vq = quantize_v(v, layout=layout, stream=stream)
    return attn_fwd(qk, vq, causal=causal, sm_scale=sm_scale, out_dtype=out_dtype or q.dtype, layout=layout,
                    stream=stream)


def loaded_hip_runtimes():
    """Paths of libamdhip64 mapped into this process (must be exactly one)."""
    paths = set()
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64" in line:
                paths.add(line.split()[-1])
    return sorted(paths)
