"""GPU parity of MXINT4 weights (two's-complement INT4 codes with one E8M0 scale
per 32 K) with bf16 activations against the CPU oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import cases
import oracle
import synthetic as syn
from bit_quantized_gemm_w4a16_amd import hq
from gpu_util import GATE, dev, empty, gate_error, note, sample_rows, sweep_rows, to_f64, workspace

pytestmark = pytest.mark.gpu


def run_mxint4(M, N, K, seed=0, rows=None, data=None):
    d = syn.w4a16_mxint4(seed, M, N, K) if data is None else data
    note(f"mxint4 a16 M={M} N={N} K={K} seed={seed}")
    desc = hq.desc_mxint4_a16(N, K)
    wp, sp, _ = hq.hq_repack(desc, d["q"], d["e"])
    D = empty(M * N * 2)
    ws, nb = workspace(desc, M)
    hq.hq_gemm(desc, M, dev(d["A"]), None, dev(wp), dev(sp), None, D, ws, nb)
    torch.cuda.synchronize()
    Dh = to_f64(D[: M * N * 2].cpu().numpy().view(np.uint16).reshape(M, N), torch.bfloat16)
    r = sample_rows(M) if rows is None else rows
    return Dh[r], oracle.gemm_mxint4_a16(d["A"], d["q"], d["e"], N=N, K=K, rows=r)


def check(Dr, O):
    assert np.all(np.isfinite(Dr))
    err = gate_error(Dr, O)
    # exact bf16 operands (INT4 x 2^(E-127)), fp32 accumulation, one bf16 rounding
    assert err <= min(GATE, 8e-3), err


@pytest.mark.parametrize("M,N,K", cases.MXINT4_SMALL + cases.MXINT4_TILES)
def test_mxint4_a16_shapes(M, N, K):
    """Small-M stream (split and unsplit), 128 x 128 split tiles, 128 x 256 and
    256 x 256 tiles, ragged last row and column tiles."""
    Dr, O = run_mxint4(M, N, K, seed=M + K, rows=sweep_rows(M) if M > 300 else None)
    check(Dr, O)


@pytest.mark.parametrize("M,N,K", cases.MXINT4_SWEEP)
def test_mxint4_a16_full_size(M, N, K):
    """The dense W4A16 shape (N=4096, K=7168) with MXINT4 weights at the M sweep."""
    Dr, O = run_mxint4(M, N, K, seed=0, rows=sweep_rows(M))
    check(Dr, O)


def test_mxint4_a16_extreme_codes_and_exponents():
    """Every code -8 (the most negative) under the largest and smallest exponents of the
    draw, and alternating exponents: exact operands, so the bf16 bound still holds."""
    M, N, K = 20, 272, 1024
    d = syn.w4a16_mxint4(7, M, N, K)
    d["q"][:] = 0x88888888
    d["e"][::2] = 127
    d["e"][1::2] = 118
    Dr, O = run_mxint4(M, N, K, data=d)
    check(Dr, O)
