"""The allocation-free decode entry point (sage_attn_decode_noalloc) against the
one that takes a caller's workspace (sage_attn_decode), through the C ABI:
bit-identical O on two calls in a row, the second on a smaller, ragged shape
(the library's scratch array then still holds the first call's states), and
both within 2e-3 of the split-KV oracle."""
import numpy as np
import pytest
import torch

from oracle import oracle as orc
from quantized_scaled_dot_amd import synth

pytestmark = pytest.mark.gpu

SHAPES = [
    # (base workload, overrides): a decode step of 4 sequences against an 8k-token cache, then a
    # smaller one with 3 queries per sequence on a 1000-token cache (not a tile multiple)
    ("decode-32k-gqa", dict(B=4, Nkv_=8192)),
    ("decode-32k-gqa", dict(B=2, H=8, Hkv_=2, N=3, Nkv_=1000)),
]


def _decode_both(sage, w, Q, K, V):
    dev = torch.device("cuda:0")
    q = sage.quantize_q(Q.to(dev), w.blk_q)
    kc = sage.quantize_k(K.to(dev), w.blk_k)
    vq = sage.quantize_v(V.to(dev))
    B, Hq, Hkv, Nq, Nkv, d = w.B, w.H, w.Hkv, w.N, w.Nkv, w.d
    chunk = sage.sage_decode_kv_chunk(B, Hq, Hkv, Nq, Nkv, d)
    need = sage.sage_attn_decode_workspace_bytes(B, Hq, Hkv, Nq, Nkv, d, chunk)
    assert 0 < need <= sage.SAGE_NOALLOC_SCRATCH_BYTES
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    o_ws = torch.empty((B, Hq, Nq, d), dtype=torch.float32, device=dev)
    o_na = torch.full_like(o_ws, float("nan"))
    st = torch.cuda.current_stream().cuda_stream
    common = (q["q_codes"].data_ptr(), q["q_scale"].data_ptr(), kc["k_codes"].data_ptr(), kc["k_scale"].data_ptr(),
              vq[0].data_ptr(), vq[1].data_ptr())
    shape = (sage.SAGE_F32, sage.SAGE_LAYOUT_BHND, B, Hq, Hkv, Nq, Nkv, d, w.blk_q, w.blk_k, int(w.causal),
             float(w.sm_scale), chunk)
    print(f"decode {w.name}: B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nkv={Nkv} split {chunk} keys, {need} scratch bytes",
          flush=True)
    assert sage.sage_attn_decode(*common, o_ws.data_ptr(), *shape, ws.data_ptr(), need, st) == sage.SAGE_OK
    assert sage.sage_attn_decode_noalloc(*common, o_na.data_ptr(), *shape, st) == sage.SAGE_OK
    torch.cuda.synchronize()
    return o_ws.cpu().numpy(), o_na.cpu().numpy(), chunk


def test_noalloc_decode_matches_the_workspace_entry_point_on_two_calls_in_a_row():
    from quantized_scaled_dot_amd import sage

    for base, kw in SHAPES:
        w = synth.WORKLOADS[base].with_(name=f"noalloc-{base}", **kw)
        Q, K, V = synth.make_inputs(w)
        o_ws, o_na, chunk = _decode_both(sage, w, Q, K, V)
        assert np.array_equal(o_na.view(np.uint32), o_ws.view(np.uint32)), "O differs from sage_attn_decode"
        qk = orc.quantize_qk(synth.bits(Q), synth.bits(K), w.dtype_code, w.blk_q, w.blk_k)
        vc, vs = orc.quantize_v(synth.bits(V), w.dtype_code)
        rows = np.arange(w.B * w.H * w.N)
        ref = orc.attn_rows_split(qk, vc, vs, w.blk_q, w.blk_k, w.causal, w.sm_scale, kv_chunk=chunk, rows=rows)
        err = float(np.abs(o_na.reshape(-1, w.d) - ref).max())
        print(f"  bit-identical to sage_attn_decode; max |O - oracle| {err:.3g}", flush=True)
        assert err <= 2e-3
