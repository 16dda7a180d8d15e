"""Host-side checks of the C ABI: the library loads, exports every function
include/sage.h declares, and rejects bad arguments before touching the GPU."""
import ctypes
import os
import re

import pytest

from quantized_scaled_dot_amd import sage

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    src = open(os.path.join(ROOT, "include", "sage.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(sage_\w+)\s*\(", src, flags=re.M)


def test_every_declared_symbol_is_exported():
    names = _header_functions()
    assert len(names) == 31 and tuple(names) == sage.SYMBOLS
    lib = ctypes.CDLL(sage.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_constants():
    assert sage.sage_status_string(0) == "SAGE_OK"
    for s in range(1, 6):
        assert sage.sage_status_string(s).startswith("SAGE_ERR_")
    assert sage.sage_kv_tile() == 64


def test_hbm_probe_rejects_bad_arguments():
    assert sage.sage_probe_hbm_read(None, 1 << 20, A, None) == sage.SAGE_ERR_INVALID_ARG
    assert sage.sage_probe_hbm_read(A, 0, A, None) == sage.SAGE_ERR_INVALID_ARG
    assert sage.sage_probe_hbm_read(A, 100, A, None) == sage.SAGE_ERR_INVALID_ARG
    assert sage.sage_probe_hbm_read(A, 1 << 20, None, None) == sage.SAGE_ERR_INVALID_ARG
    assert sage.sage_probe_hbm_read(A + 8, 1 << 20, A, None) == sage.SAGE_ERR_MISALIGNED


def test_mfma_probe_rejects_bad_arguments():
    assert sage.sage_probe_mfma_peak(0, 10) == sage.SAGE_ERR_INVALID_ARG
    assert sage.sage_probe_mfma_peak(65537, 10) == sage.SAGE_ERR_INVALID_ARG
    assert sage.sage_probe_mfma_peak(512, 0) == sage.SAGE_ERR_INVALID_ARG
    assert sage.sage_probe_mfma_peak(512, (1 << 24) + 1) == sage.SAGE_ERR_INVALID_ARG
    assert sage.sage_probe_mfma_peak(512, 10, 4097) == sage.SAGE_ERR_MISALIGNED


def test_workspace_sizes():
    assert sage.sage_quantize_qk_workspace_bytes(1, 24, 32768, 128) == 24 * 128 * 128 * 8   # 256-token chunks
    assert sage.sage_quantize_v_workspace_bytes(1, 2, 256, 64) == (2 * 1 * 64 + 2 * 64) * 4
    assert sage.sage_quantize_qk_workspace_bytes(1, 1, 0, 64) == 0     # invalid N
    assert sage.sage_quantize_qk_workspace_bytes(1, 1, 100, 64) == 64 * 8   # one partial 256-token chunk
    assert sage.sage_quantize_v_workspace_bytes(1, 1, 257, 64) == (2 * 64 + 64) * 4


A = 4096  # a fake 16-byte aligned address; never dereferenced because validation fails first


def _qk(**kw):
    args = dict(Q=A, K=A, in_dtype=1, B=1, H=1, N=256, d=128, blk_q=128, blk_k=64, q_codes=A, q_scale=A,
                k_codes=A, k_scale=A, k_mean=A, workspace=A, workspace_bytes=1 << 20, stream=None)
    args.update(kw)
    return sage.sage_quantize_qk(**args)


def _v(**kw):
    args = dict(V=A, in_dtype=0, B=1, H=1, N=256, d=64, v_codes=A, v_scale=A, workspace=A, workspace_bytes=1 << 20,
                stream=None)
    args.update(kw)
    return sage.sage_quantize_v(**args)


def _attn(**kw):
    args = dict(q_codes=A, q_scale=A, k_codes=A, k_scale=A, v_codes=A, v_scale=A, O=A, out_dtype=2, B=1, H=1, N=256,
                d=128, blk_q=128, blk_k=64, causal=0, sm_scale=0.125, stream=None)
    args.update(kw)
    return sage.sage_attn_fwd(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(d=96), sage.SAGE_ERR_UNSUPPORTED), (dict(N=(1 << 19) + 1), sage.SAGE_ERR_UNSUPPORTED),
    (dict(N=1 << 20), sage.SAGE_ERR_UNSUPPORTED), (dict(B=0), sage.SAGE_ERR_INVALID_ARG),
    (dict(H=-1), sage.SAGE_ERR_INVALID_ARG), (dict(in_dtype=2), sage.SAGE_ERR_INVALID_ARG),
    (dict(in_dtype=7), sage.SAGE_ERR_INVALID_ARG), (dict(blk_q=16), sage.SAGE_ERR_UNSUPPORTED),
    (dict(blk_k=128), sage.SAGE_ERR_UNSUPPORTED), (dict(Q=None), sage.SAGE_ERR_INVALID_ARG),
    (dict(k_mean=None), sage.SAGE_ERR_INVALID_ARG), (dict(K=A + 8), sage.SAGE_ERR_MISALIGNED),
    (dict(workspace=None), sage.SAGE_ERR_INVALID_ARG), (dict(workspace_bytes=16), sage.SAGE_ERR_WORKSPACE),
])
def test_quantize_qk_rejects(kw, status):
    assert _qk(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(d=32), sage.SAGE_ERR_UNSUPPORTED), (dict(N=0), sage.SAGE_ERR_INVALID_ARG),
    (dict(V=None), sage.SAGE_ERR_INVALID_ARG), (dict(v_codes=A + 4), sage.SAGE_ERR_MISALIGNED),
    (dict(in_dtype=-1), sage.SAGE_ERR_INVALID_ARG), (dict(workspace_bytes=0), sage.SAGE_ERR_WORKSPACE),
])
def test_quantize_v_rejects(kw, status):
    assert _v(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(d=256), sage.SAGE_ERR_UNSUPPORTED), (dict(N=-128), sage.SAGE_ERR_INVALID_ARG),
    (dict(blk_q=256), sage.SAGE_ERR_UNSUPPORTED), (dict(blk_k=8), sage.SAGE_ERR_UNSUPPORTED),
    (dict(out_dtype=3), sage.SAGE_ERR_INVALID_ARG), (dict(causal=2), sage.SAGE_ERR_INVALID_ARG),
    (dict(sm_scale=0.0), sage.SAGE_ERR_INVALID_ARG), (dict(sm_scale=-1.0), sage.SAGE_ERR_INVALID_ARG),
    (dict(sm_scale=float("inf")), sage.SAGE_ERR_INVALID_ARG), (dict(sm_scale=float("nan")), sage.SAGE_ERR_INVALID_ARG),
    (dict(O=None), sage.SAGE_ERR_INVALID_ARG), (dict(v_scale=A + 2), sage.SAGE_ERR_MISALIGNED),
    (dict(q_codes=None), sage.SAGE_ERR_INVALID_ARG),
])
def test_attn_fwd_rejects(kw, status):
    assert _attn(**kw) == status


def test_attn_fwd_dump_rejects_bad_selection():
    r = sage.sage_attn_fwd_dump(A, A, A, A, A, A, A, 2, 1, 1, 256, 128, 128, 64, 0, 0.125, None, 1, A, A, None)
    assert r == sage.SAGE_ERR_INVALID_ARG
    r = sage.sage_attn_fwd_dump(A, A, A, A, A, A, A, 2, 1, 1, 256, 128, 128, 64, 0, 0.125, A, -1, A, A, None)
    assert r == sage.SAGE_ERR_INVALID_ARG


def _qk_ex(**kw):
    args = dict(Q=A, K=A, in_dtype=1, layout=1, B=1, Hq=4, Hkv=2, Nq=128, Nkv=384, d=128, blk_q=128, blk_k=64,
                q_codes=A, q_scale=A, k_codes=A, k_scale=A, k_mean=A, workspace=A, workspace_bytes=1 << 20, stream=None)
    args.update(kw)
    return sage.sage_quantize_qk_ex(**args)


def _v_ex(**kw):
    args = dict(V=A, in_dtype=0, layout=1, B=1, H=2, N=384, d=64, v_codes=A, v_scale=A, workspace=A,
                workspace_bytes=1 << 20, stream=None)
    args.update(kw)
    return sage.sage_quantize_v_ex(**args)


def _attn_ex(**kw):
    args = dict(q_codes=A, q_scale=A, k_codes=A, k_scale=A, v_codes=A, v_scale=A, O=A, out_dtype=2, layout=0, B=1,
                Hq=4, Hkv=2, Nq=128, Nkv=384, d=128, blk_q=128, blk_k=64, causal=1, sm_scale=0.125, stream=None)
    args.update(kw)
    return sage.sage_attn_fwd_ex(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(layout=2), sage.SAGE_ERR_INVALID_ARG), (dict(layout=-1), sage.SAGE_ERR_INVALID_ARG),
    (dict(Hq=3), sage.SAGE_ERR_INVALID_ARG), (dict(Hkv=0), sage.SAGE_ERR_INVALID_ARG),
    (dict(Hkv=8), sage.SAGE_ERR_INVALID_ARG), (dict(Nq=(1 << 19) + 64), sage.SAGE_ERR_UNSUPPORTED),
    (dict(Nkv=-100), sage.SAGE_ERR_INVALID_ARG), (dict(Nkv=1 << 20), sage.SAGE_ERR_UNSUPPORTED),
    (dict(Nq=0), sage.SAGE_ERR_INVALID_ARG), (dict(d=32), sage.SAGE_ERR_UNSUPPORTED),
    (dict(in_dtype=2), sage.SAGE_ERR_INVALID_ARG), (dict(K=None), sage.SAGE_ERR_INVALID_ARG),
    (dict(workspace_bytes=16), sage.SAGE_ERR_WORKSPACE),
])
def test_quantize_qk_ex_rejects(kw, status):
    assert _qk_ex(**kw) == status


def test_quantize_qk_ex_workspace_follows_k():
    need = sage.sage_quantize_qk_workspace_bytes(1, 2, 384, 128)
    assert need == 2 * 2 * 128 * 8
    # the workspace covers K only (B*Hkv heads of Nkv tokens), however long Q is
    assert _qk_ex(workspace_bytes=need - 1, Q=None) == sage.SAGE_ERR_INVALID_ARG
    assert _qk_ex(workspace_bytes=need - 1, Nq=4096) == sage.SAGE_ERR_WORKSPACE


@pytest.mark.parametrize("kw,status", [
    (dict(layout=5), sage.SAGE_ERR_INVALID_ARG), (dict(N=(1 << 19) + 2), sage.SAGE_ERR_UNSUPPORTED),
    (dict(V=A + 8), sage.SAGE_ERR_MISALIGNED), (dict(workspace_bytes=0), sage.SAGE_ERR_WORKSPACE),
])
def test_quantize_v_ex_rejects(kw, status):
    assert _v_ex(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(layout=3), sage.SAGE_ERR_INVALID_ARG), (dict(Hq=6, Hkv=4), sage.SAGE_ERR_INVALID_ARG),
    (dict(Nq=512), sage.SAGE_ERR_INVALID_ARG),              # causal with Nq > Nkv: first rows see no key
    (dict(Nq=385, Nkv=384), sage.SAGE_ERR_INVALID_ARG), (dict(Hkv=-2), sage.SAGE_ERR_INVALID_ARG),
    (dict(blk_q=96), sage.SAGE_ERR_UNSUPPORTED), (dict(sm_scale=float("nan")), sage.SAGE_ERR_INVALID_ARG),
    (dict(O=A + 4), sage.SAGE_ERR_MISALIGNED), (dict(k_scale=None), sage.SAGE_ERR_INVALID_ARG),
])
def test_attn_fwd_ex_rejects(kw, status):
    assert _attn_ex(**kw) == status


def test_attn_fwd_ex_dump_rejects_bad_selection():
    shape = (0, 1, 4, 2, 128, 384, 128, 128, 64, 0, 0.125)
    assert sage.sage_attn_fwd_ex_dump(A, A, A, A, A, A, A, 2, *shape, None, 1, A, A, None) == sage.SAGE_ERR_INVALID_ARG
    assert sage.sage_attn_fwd_ex_dump(A, A, A, A, A, A, A, 2, *shape, A, -1, A, A, None) == sage.SAGE_ERR_INVALID_ARG


def test_python_helpers_validate_shapes():
    import torch
    with pytest.raises(ValueError):
        sage.quantize_qk(torch.zeros(2, 2), torch.zeros(2, 2))
    with pytest.raises(ValueError):
        sage.quantize_v(torch.zeros(1, 2, 128, 64), layout="nhd")


def _dec(**kw):
    args = dict(q_codes=A, q_scale=A, k_codes=A, k_scale=A, v_codes=A, v_scale=A, O=A, out_dtype=2, layout=0, B=2,
                Hq=8, Hkv=2, Nq=1, Nkv=1000, d=128, blk_q=128, blk_k=64, causal=1, sm_scale=0.125, kv_chunk=128,
                workspace=A, workspace_bytes=1 << 30, stream=None)
    args.update(kw)
    return sage.sage_attn_decode(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(kv_chunk=96), sage.SAGE_ERR_INVALID_ARG), (dict(kv_chunk=-64), sage.SAGE_ERR_INVALID_ARG),
    (dict(kv_chunk=32), sage.SAGE_ERR_INVALID_ARG), (dict(Hq=7), sage.SAGE_ERR_INVALID_ARG),
    (dict(Nq=1001), sage.SAGE_ERR_INVALID_ARG), (dict(blk_k=128), sage.SAGE_ERR_UNSUPPORTED),
    (dict(workspace=None), sage.SAGE_ERR_INVALID_ARG), (dict(workspace_bytes=1024), sage.SAGE_ERR_WORKSPACE),
    (dict(O=A + 4), sage.SAGE_ERR_MISALIGNED), (dict(out_dtype=5), sage.SAGE_ERR_INVALID_ARG),
    (dict(sm_scale=0.0), sage.SAGE_ERR_INVALID_ARG), (dict(d=96), sage.SAGE_ERR_UNSUPPORTED),
])
def test_attn_decode_rejects(kw, status):
    assert _dec(**kw) == status


def test_decode_split_and_workspace_sizes():
    # 2 batches x 2 K/V heads x 1 row group (4 query heads x 1 query) = 4 row groups:
    # 256 splits would fit, the 16 tiles of 1000 keys allow 16, one tile each
    assert sage.sage_decode_kv_chunk(2, 8, 2, 1, 1000, 128) == 64
    # 16 x 8 x 1 = 128 row groups, 8 splits of the 512 tiles of 32768 keys (1024 waves)
    assert sage.sage_decode_kv_chunk(16, 32, 8, 1, 32768, 128) == 64 * 64
    units = 2 * 2 * 1 * 8   # 8 splits of 128 keys over ceil(1000/64) = 16 tiles
    assert sage.sage_attn_decode_workspace_bytes(2, 8, 2, 1, 1000, 128, 128) == units * (32 * 128 + 64) * 4
    assert sage.sage_attn_decode_workspace_bytes(2, 8, 2, 1, 1000, 128, 100) == 0
    assert sage.sage_decode_kv_chunk(2, 6, 4, 1, 100, 128) == 0   # Hq not a multiple of Hkv


def test_quantize_q_and_k_reject():
    assert sage.sage_quantize_q(A, 1, 0, 1, 2, 5, 128, 48, A, A, None) == sage.SAGE_ERR_UNSUPPORTED
    assert sage.sage_quantize_q(None, 1, 0, 1, 2, 5, 128, 64, A, A, None) == sage.SAGE_ERR_INVALID_ARG
    assert sage.sage_quantize_q(A, 1, 2, 1, 2, 5, 128, 64, A, A, None) == sage.SAGE_ERR_INVALID_ARG
    assert sage.sage_quantize_k(A, 0, 0, 1, 2, 300, 64, 16, A, A, A, A, 8, None) == sage.SAGE_ERR_WORKSPACE
    assert sage.sage_quantize_k(A, 0, 0, 1, 2, 300, 64, 24, A, A, A, A, 1 << 20, None) == sage.SAGE_ERR_UNSUPPORTED
    assert sage.sage_quantize_k(A, 0, 0, 1, 2, 300, 64, 16, A, A, None, A, 1 << 20, None) == sage.SAGE_ERR_INVALID_ARG


def _qk4(**kw):
    args = dict(Q=A, K=A, in_dtype=1, layout=0, B=1, Hq=4, Hkv=2, Nq=256, Nkv=300, d=128, q4_codes=A, q4_scale=A,
                k4_codes=A, k4_scale=A, k_mean=A, workspace=A, workspace_bytes=1 << 20, stream=None)
    args.update(kw)
    return sage.sage_quantize_qk4(**args)


def _attn4(**kw):
    args = dict(q4_codes=A, q4_scale=A, k4_codes=A, k4_scale=A, v_codes=A, v_scale=A, O=A, out_dtype=2, layout=1, B=1,
                Hq=4, Hkv=2, Nq=256, Nkv=300, d=64, causal=1, sm_scale=0.125, stream=None)
    args.update(kw)
    return sage.sage_attn_fwd_qk4(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(d=96), sage.SAGE_ERR_UNSUPPORTED), (dict(Hq=3), sage.SAGE_ERR_INVALID_ARG),
    (dict(in_dtype=2), sage.SAGE_ERR_INVALID_ARG), (dict(layout=4), sage.SAGE_ERR_INVALID_ARG),
    (dict(k4_scale=None), sage.SAGE_ERR_INVALID_ARG), (dict(q4_codes=A + 1), sage.SAGE_ERR_MISALIGNED),
    (dict(workspace_bytes=8), sage.SAGE_ERR_WORKSPACE), (dict(Nkv=0), sage.SAGE_ERR_INVALID_ARG),
])
def test_quantize_qk4_rejects(kw, status):
    assert _qk4(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(Nq=400), sage.SAGE_ERR_INVALID_ARG), (dict(q4_scale=None), sage.SAGE_ERR_INVALID_ARG),
    (dict(k4_codes=A + 8), sage.SAGE_ERR_MISALIGNED), (dict(out_dtype=9), sage.SAGE_ERR_INVALID_ARG),
    (dict(sm_scale=-1.0), sage.SAGE_ERR_INVALID_ARG), (dict(d=32), sage.SAGE_ERR_UNSUPPORTED),
])
def test_attn_fwd_qk4_rejects(kw, status):
    assert _attn4(**kw) == status


def _qk4s(**kw):
    args = dict(Q=A, K=A, in_dtype=1, layout=0, B=1, Hq=4, Hkv=2, Nq=256, Nkv=300, d=128, q4_codes=A, q4_scale=A,
                k4_codes=A, k4_scale=A, k_mean=A, q_mean=A, qm_codes=A, qm_scale=A, k8_codes=A, k8_scale=A,
                workspace=A, workspace_bytes=1 << 20, stream=None)
    args.update(kw)
    return sage.sage_quantize_qk4_smooth_q(**args)


def _attn4s(**kw):
    args = dict(q4_codes=A, q4_scale=A, k4_codes=A, k4_scale=A, qm_codes=A, qm_scale=A, k8_codes=A, k8_scale=A,
                v_codes=A, v_scale=A, O=A, out_dtype=2, layout=1, B=1, Hq=4, Hkv=2, Nq=256, Nkv=300, d=64, causal=1,
                sm_scale=0.125, stream=None)
    args.update(kw)
    return sage.sage_attn_fwd_qk4_smooth_q(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(q_mean=None), sage.SAGE_ERR_INVALID_ARG), (dict(k8_scale=None), sage.SAGE_ERR_INVALID_ARG),
    (dict(qm_codes=A + 4), sage.SAGE_ERR_MISALIGNED), (dict(d=96), sage.SAGE_ERR_UNSUPPORTED),
    (dict(Hq=3), sage.SAGE_ERR_INVALID_ARG), (dict(workspace_bytes=8), sage.SAGE_ERR_WORKSPACE),
])
def test_quantize_qk4_smooth_q_rejects(kw, status):
    """The five smoothing outputs go together: a null among them is an error
    (all five null is the plain call, which the GPU tests run)."""
    assert _qk4s(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(qm_codes=None), sage.SAGE_ERR_INVALID_ARG), (dict(k8_codes=None), sage.SAGE_ERR_INVALID_ARG),
    (dict(qm_scale=A + 8), sage.SAGE_ERR_MISALIGNED), (dict(Nq=400), sage.SAGE_ERR_INVALID_ARG),
    (dict(out_dtype=7), sage.SAGE_ERR_INVALID_ARG),
])
def test_attn_fwd_qk4_smooth_q_rejects(kw, status):
    assert _attn4s(**kw) == status


def test_decode_noalloc_rejects_shapes_beyond_its_scratch_before_any_hip_call():
    """The allocation-free decode checks its size limit (the header constant, mirrored by the
    binding) before it looks up its device array or enqueues anything."""
    src = open(os.path.join(ROOT, "include", "sage.h")).read()
    m = re.search(r"#define SAGE_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == sage.SAGE_NOALLOC_SCRATCH_BYTES
    # 16 batches x 8 K/V heads x 512 one-tile splits of 32768 keys: 65536 waves of chunk states
    need = sage.sage_attn_decode_workspace_bytes(16, 32, 8, 1, 32768, 128, 64)
    assert need > sage.SAGE_NOALLOC_SCRATCH_BYTES
    st = sage.sage_attn_decode_noalloc(A, A, A, A, A, A, A, sage.SAGE_F32, 0, 16, 32, 8, 1, 32768, 128, 128, 64, 1,
                                       0.088, 64, None)
    assert st == sage.SAGE_ERR_WORKSPACE
    # the argument checks of sage_attn_decode come first
    assert sage.sage_attn_decode_noalloc(A, A, A, A, A, A, None, sage.SAGE_F32, 0, 16, 32, 8, 1, 32768, 128, 128, 64,
                                         1, 0.088, 64, None) == sage.SAGE_ERR_INVALID_ARG
    assert sage.sage_attn_decode_noalloc(A, A, A, A, A, A, A, sage.SAGE_F32, 0, 16, 32, 8, 1, 32768, 128, 128, 64, 1,
                                         0.088, 96, None) == sage.SAGE_ERR_INVALID_ARG
