"""GPU runs of the measurement probes (hq_probe_stream, hq_probe_mfma) through
the C ABI: every probed type launches, completes and leaves finite sums; the
stream probe reads a buffer whose size is not a multiple of the grid."""
import numpy as np
import pytest
import torch

from bit_quantized_gemm_w4a16_amd import hq
from gpu_util import note

pytestmark = pytest.mark.gpu


def test_stream_probe_reads_ragged_buffer():
    nbytes = (1 << 20) + 48
    note(f"probe stream {nbytes} bytes")
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(16, dtype=torch.uint8, device="cuda")
    hq.hq_probe_stream(src, nbytes, sink, 3)
    torch.cuda.synchronize()
    assert int(sink.sum()) == 0


@pytest.mark.parametrize("dt", [hq.HQ_DT_FP16, hq.HQ_DT_BF16, hq.HQ_DT_FP8_E4M3, hq.HQ_DT_FP4_E2M1, hq.HQ_DT_INT8])
def test_mfma_probe_runs(dt):
    note(f"probe mfma dtype={dt}")
    wgs = 8
    sink = torch.full((wgs * 256,), float("nan"), dtype=torch.float32, device="cuda")
    flops = hq.hq_probe_mfma(dt, wgs, 10, sink)
    torch.cuda.synchronize()
    assert flops == wgs * 4 * 10 * 8 * hq.PROBE_MFMA_FLOPS[dt]
    assert np.all(np.isfinite(sink.cpu().numpy()))
