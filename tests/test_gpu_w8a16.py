"""GPU parity of 8-bit weight-only GEMMs (bf16 / fp16 activations x INT8 or FP8-E4M3
weights with fp32 per-channel scales) against the CPU oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import cases
import oracle
import synthetic as syn
from bit_quantized_gemm_w4a16_amd import hq
from gpu_util import GATE, dev, empty, gate_error, note, sample_rows, sweep_rows, to_f64, workspace

pytestmark = pytest.mark.gpu

DTYPES = ["bf16", "fp16"]


WFMTS = ["int8", "fp8"]


def run_w8a16(M, N, K, dt, seed=0, rows=None, data=None, wfmt="int8"):
    bf = dt == "bf16"
    tdt = torch.bfloat16 if bf else torch.float16
    fp8 = wfmt == "fp8"
    if data is None:
        d = syn.w8a16_fp8(seed, M, N, K, tdt) if fp8 else syn.w8a16_int8(seed, M, N, K, tdt)
    else:
        d = data
    note(f"w8a16 {wfmt} {dt} M={M} N={N} K={K} seed={seed}")
    desc = hq.desc_fp8w_a16(N, K, bf16=bf) if fp8 else hq.desc_w8a16(N, K, bf16=bf)
    wp, sp, _ = hq.hq_repack(desc, d["w"], d["s_w"])
    D = empty(M * N * 2)
    ws, nb = workspace(desc, M)
    hq.hq_gemm(desc, M, dev(d["A"]), None, dev(wp), dev(sp), None, D, ws, nb)
    torch.cuda.synchronize()
    Dh = to_f64(D[: M * N * 2].cpu().numpy().view(np.uint16).reshape(M, N), tdt)
    r = sample_rows(M) if rows is None else rows
    ref = oracle.gemm_fp8w_a16 if fp8 else oracle.gemm_w8a16
    return Dh[r], ref(d["A"], d["w"], d["s_w"], a_bf16=bf, rows=r)


def check(Dr, O, dt):
    assert np.all(np.isfinite(Dr))
    err = gate_error(Dr, O)
    # exact 16-bit operands, fp32 accumulation, the per-channel scale in fp32, one rounding
    assert err <= min(GATE, 8e-3 if dt == "bf16" else 3e-3), err


@pytest.mark.parametrize("wfmt", WFMTS)
@pytest.mark.parametrize("dt", DTYPES)
@pytest.mark.parametrize("M,N,K", cases.W8A16_SMALL + cases.W8A16_TILES)
def test_w8a16_shapes(wfmt, dt, M, N, K):
    """Small-M stream (split and unsplit), 128 x 128 split tiles and 128 x 256 tiles,
    ragged last row and column tiles."""
    Dr, O = run_w8a16(M, N, K, dt, seed=M + K, rows=sweep_rows(M) if M > 300 else None, wfmt=wfmt)
    check(Dr, O, dt)


@pytest.mark.parametrize("wfmt", WFMTS)
@pytest.mark.parametrize("dt", DTYPES)
@pytest.mark.parametrize("M,N,K", cases.W8A16_SWEEP)
def test_w8a16_full_size(wfmt, dt, M, N, K):
    """N=4096, K=7168 at the M sweep."""
    Dr, O = run_w8a16(M, N, K, dt, seed=0, rows=sweep_rows(M), wfmt=wfmt)
    check(Dr, O, dt)


@pytest.mark.parametrize("dt", DTYPES)
def test_fp8w_extreme_codes(dt):
    """FP8 weights at +-448 (the largest finite E4M3), the smallest subnormal and -0."""
    M, N, K = 24, 272, 512
    d = syn.w8a16_fp8(4, M, N, K, torch.bfloat16 if dt == "bf16" else torch.float16)
    d["w"][:, 0::4] = 0x7E
    d["w"][:, 1::4] = 0xFE
    d["w"][:, 2::4] = 0x01
    d["w"][:, 3::4] = 0x80
    Dr, O = run_w8a16(M, N, K, dt, data=d, wfmt="fp8")
    check(Dr, O, dt)


@pytest.mark.parametrize("dt", DTYPES)
def test_w8a16_extreme_codes(dt):
    """Every weight -128 (the code the +128 offset decode must wrap to 0) or 127."""
    M, N, K = 33, 272, 1024
    d = syn.w8a16_int8(9, M, N, K, torch.bfloat16 if dt == "bf16" else torch.float16)
    d["w"][:, ::2] = -128
    d["w"][:, 1::2] = 127
    Dr, O = run_w8a16(M, N, K, dt, data=d)
    check(Dr, O, dt)
