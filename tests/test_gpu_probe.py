"""The throughput probes (measurement aids that bench.py times) run through
the C ABI: the matrix-core probe fills its checksum sink deterministically,
the HBM read probe reads every word of its buffer exactly once."""
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


def test_hbm_probe_reads_every_word_exactly_once():
    """The XOR of the probe's per-thread checksums is the XOR of every 32-bit word of the buffer
    (each 16-byte vector is read by exactly one thread, once), also for a length that leaves the
    last loop partly empty."""
    import numpy as np
    from quantized_scaled_dot_amd import sage
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(3)
    for nbytes in (16 * 1024 * 256 * 8 * 2, 16 * 1024 * 256 * 8 * 2 + 16 * 777, 16 * 12345):
        host = rng.integers(-2 ** 31, 2 ** 31, nbytes // 4, dtype=np.int64).astype(np.int32)
        buf = torch.from_numpy(host).to(dev)
        sink = torch.zeros(1024 * 256, dtype=torch.int32, device=dev)
        st = sage.sage_probe_hbm_read(buf.data_ptr(), nbytes, sink.data_ptr(), torch.cuda.current_stream().cuda_stream)
        assert st == sage.SAGE_OK, sage.sage_status_string(st)
        torch.cuda.synchronize()
        assert np.bitwise_xor.reduce(sink.cpu().numpy()) == np.bitwise_xor.reduce(host), nbytes
