"""The matrix-core throughput probe (a measurement aid that bench.py times)
runs through the C ABI, fills its checksum sink and is deterministic."""
import pytest
import torch

pytestmark = pytest.mark.gpu


def test_mfma_probe_runs_and_is_deterministic():
    from quantized_scaled_dot_amd import sage
    dev = torch.device("cuda:0")
    wg, iters = 4, 3
    outs = []
    for _ in range(2):
        sink = torch.full((wg * 256,), -7, dtype=torch.int32, device=dev)
        st = sage.sage_probe_mfma_peak(wg, iters, sink.data_ptr(), torch.cuda.current_stream().cuda_stream)
        assert st == sage.SAGE_OK, sage.sage_status_string(st)
        torch.cuda.synchronize()
        outs.append(sink.cpu())
    assert torch.equal(outs[0], outs[1])
    assert (outs[0] != -7).all()
