"""GPU parity of the eight-wave small-M weight stream with direct A loads
(HQ_TUNE_STREAM8; the library's own choice up to 8 rows on wide layers for the
16-bit-activation formats with the longer decodes), against the CPU oracle
through the C ABI.

Each wave takes an eighth of K: K = 1024 (one chunk per wave in a two-chunk
batch, one dead), 2048, 4096, 7168 (seven chunks) and 8192 (eight) reach every
batch size; M = 1..16 covers the rows that read a clamped A row; N = 3100 ends
in a partial 16-column strip."""
import numpy as np
import pytest

from bit_quantized_gemm_w4a16_amd import autotune, hq
from gpu_layers import A16_FORMATS, Layer
from gpu_util import note

pytestmark = pytest.mark.gpu

N = 3100
WNA16 = [(fmt, M, K) for fmt in ("wna16_f16_zp", "wna16_bf16_sym") for M in (1, 13, 16)
         for K in (1024, 4096, 7168, 8192)]
OTHERS = [(fmt, M, K) for fmt in A16_FORMATS[2:] for M in (5, 16) for K in (2048, 7168)]


@pytest.mark.parametrize("fmt,M,K", WNA16 + OTHERS)
def test_direct_stream_matches_the_oracle(fmt, M, K):
    L = Layer(fmt, M, N, K, seed=M * 7 + K // 1024)
    d = autotune.with_tune(L.desc, hq.HQ_TUNE(hq.HQ_TUNE_STREAM8, 0))
    plan = hq.hq_gemm_plan(d, M)
    note(f"direct stream {fmt} M={M} N={N} K={K} {plan}")
    assert len(plan) == 1 and ",direct>" in plan[0] and "splits=1" in plan[0]
    L.check(L.run(d, M), np.arange(M))


HEAVY = {"nvfp4_a16", "mxint4_a16", "w8a16_bf16", "w8a16_f16", "fp8w_bf16", "fp8w_f16", "mxfp8_a16", "mxfp6e2_a16",
         "mxfp6e3_a16", "mxfp6e2_a16_f16"}


@pytest.mark.parametrize("fmt", A16_FORMATS)
def test_library_choice_up_to_eight_rows(fmt):
    """On a wide layer (256 strips) at M = 1 and 8 the library takes the direct
    stream for the formats with the longer decodes (NVFP4, MXINT4, 8-bit and
    MX float weights) and the four-wave stream for the others; both match the oracle."""
    K = 7168
    for M in (1, 8):
        L = Layer(fmt, M, 4096, K, seed=M)
        plan = hq.hq_gemm_plan(L.desc, M)
        note(f"library choice {fmt} M={M} N=4096 K={K} {plan}")
        assert len(plan) == 1 and (",direct>" in plan[0]) == (fmt in HEAVY)
        L.check(L.run(L.desc, M), np.arange(M))
