"""The matrix-unit rate probe (a diagnostic beside the layer) through the C
ABI: it runs, its per-wave clock marks are plausible, and its rate is
below the datasheet peak of the arithmetic it issues."""
import numpy as np
import pytest

import rank_gemm_svdq_amd as B

pytestmark = pytest.mark.gpu

PEAK_TOPS = {0: 10100.0, 1: 5000.0}   # dense FP4 and int8 datasheet figures


@pytest.mark.parametrize("kind", [0, 1])
@pytest.mark.parametrize("zero", [0, 1])
def test_rate_probe_runs_within_the_datasheet_peak(kind, zero):
    import torch
    blocks = torch.cuda.get_device_properties(0).multi_processor_count
    iters = 200
    sink = torch.empty(blocks * 512, dtype=torch.float32, device="cuda")
    marks = torch.zeros(blocks * 16, dtype=torch.int64, device="cuda")
    B.mfma_rate_probe(kind, zero, blocks, iters, sink, marks)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    B.mfma_rate_probe(kind, zero, blocks, iters, sink, marks)
    e1.record()
    torch.cuda.synchronize()
    ops = blocks * 8 * (32 if kind == 0 else 16) * iters * 65536
    tops = ops / (e0.elapsed_time(e1) * 1e-3) / 1e12
    assert 0.05 * PEAK_TOPS[kind] < tops < PEAK_TOPS[kind]
    m = marks.view(-1, 2).cpu().numpy().astype(np.float64)
    assert np.all(m[:, 0] > 0) and np.all(m[:, 1] > 0)
    clock_ghz = m[:, 0] / (m[:, 1] / 100e6) / 1e9
    assert 0.5 < float(np.median(clock_ghz)) < 3.0
    s = sink.cpu().numpy()
    if zero:
        assert np.all(s == 0.0)
    else:
        assert np.all(np.isfinite(s)) and np.any(s != 0.0)


def test_rate_probe_rejects_bad_buffers():
    import torch
    sink = torch.empty(16, dtype=torch.float32, device="cuda")
    with pytest.raises(B.SvdqError):
        B.mfma_rate_probe(0, 0, 4, 10, sink)            # sink shorter than blocks * 512
    with pytest.raises(B.SvdqError):
        B.mfma_rate_probe(0, 0, 1, 10, torch.empty(512, dtype=torch.float64, device="cuda"))
