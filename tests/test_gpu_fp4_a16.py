"""GPU parity of FP4 weights with bf16 activations (WnA16 with FP4 weights):
MXFP4 (E8M0 per 32 K) and NVFP4 (E4M3 per 16 K with a per-tensor fp32
second-level scale), against the CPU oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import cases
import oracle
import synthetic as syn
from bit_quantized_gemm_w4a16_amd import hq
from gpu_util import GATE, dev, empty, gate_error, note, sample_rows, sweep_rows, to_f64, workspace

pytestmark = pytest.mark.gpu

KINDS = ["mxfp4", "nvfp4"]


def run_fp4(M, N, K, kind, seed=0, rows=None):
    nv = kind == "nvfp4"
    d = syn.w4a16_fp4(seed, M, N, K, nvfp4=nv)
    note(f"fp4 a16 {kind} M={M} N={N} K={K} seed={seed}")
    desc = hq.desc_fp4_a16(N, K, nv)
    if nv:
        wp, sp, _, s2p = hq.hq_repack(desc, d["q"], d["s"], None, d["s2"])
    else:
        wp, sp, _ = hq.hq_repack(desc, d["q"], d["s"])
    D = empty(M * N * 2)
    ws, nb = workspace(desc, M)
    hq.hq_gemm(desc, M, dev(d["A"]), None, dev(wp), dev(sp), None, D, ws, nb, s2=dev(s2p) if nv else None)
    torch.cuda.synchronize()
    Dh = to_f64(D[: M * N * 2].cpu().numpy().view(np.uint16).reshape(M, N), torch.bfloat16)
    r = sample_rows(M) if rows is None else rows
    O = oracle.gemm_fp4_a16(d["A"], d["q"], d["s"], N=N, K=K, a_bf16=True, nvfp4=nv,
                            s2=d["s2"] if nv else None, rows=r)
    return Dh[r], O


def check(Dr, O):
    assert np.all(np.isfinite(Dr))
    err = gate_error(Dr, O)
    # exact bf16 operands (e2m1 x E8M0 / E4M3), fp32 accumulation, one bf16 rounding
    # (NVFP4: times the fp32 second-level scale first)
    assert err <= min(GATE, 8e-3), err


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("M,N,K", cases.FP4A16_SMALL + cases.FP4A16_TILES)
def test_fp4_a16_shapes(kind, M, N, K):
    """Small-M stream (split and unsplit), 128 x 128 split tiles, 128 x 256 and
    256 x 256 tiles, ragged last row and column tiles."""
    Dr, O = run_fp4(M, N, K, kind, seed=M + K, rows=sweep_rows(M) if M > 300 else None)
    check(Dr, O)


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("M,N,K", cases.FP4A16_SWEEP)
def test_fp4_a16_full_size(kind, M, N, K):
    """The dense W4A16 shape (N=4096, K=7168) with FP4 weights at the M sweep."""
    Dr, O = run_fp4(M, N, K, kind, seed=0, rows=sweep_rows(M))
    check(Dr, O)
