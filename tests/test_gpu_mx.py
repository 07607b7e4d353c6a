"""GPU parity of the MX-activation paths against the CPU oracle, through the C ABI:
the OCP MX activation quantiser (E8M0 per 32 along K, E4M3 or E2M1 elements,
bit-exact) and the GEMMs of MX activations with MXFP4 weights -- W4A4
(MXFP4 x MXFP4) and MXFP8 x MXFP4 -- on the scaled fp8/fp4 MFMA."""
import numpy as np
import pytest
import torch

import cases
import oracle
import synthetic as syn
from bit_quantized_gemm_w4a16_amd import hq
from gpu_util import GATE, dev, empty, gate_error, note, sample_rows, sweep_rows, to_f64, workspace

pytestmark = pytest.mark.gpu

ELEMS = ["e2m1", "e4m3"]
DT = {"e2m1": hq.HQ_DT_FP4_E2M1, "e4m3": hq.HQ_DT_FP8_E4M3}


def gpu_quant_mx(x, elem):
    M, K = x.shape
    qb = M * K // 2 if elem == "e2m1" else M * K
    q, e = empty(qb), empty(M * K // 32)
    hq.hq_quantize_act_mx(DT[elem], M, K, dev(x.astype(np.float32)), q, e)
    torch.cuda.synchronize()
    return q[:qb].cpu().numpy().reshape(M, -1), e[: M * K // 32].cpu().numpy().reshape(M, K // 32)


@pytest.mark.parametrize("elem", ELEMS)
@pytest.mark.parametrize("M,K", [(1, 32), (5, 4096), (300, 4096), (7, 96), (64, 7168)])
def test_quantize_act_mx_bit_exact(elem, M, K):
    note(f"quant_mx {elem} M={M} K={K}")
    x = syn.normal_rows(5, 9, syn.T_A, M, K) * np.float32(2.0)
    if M >= 5:
        x[1, :32] = 0.0                                         # all-zero block -> E 0
        x[2, 32:64] *= np.float32(1e-38)                        # subnormal block
        x[3, :8] = [448.0 * 64, -3.0, 0.25, 0.75, 1.25, -1.75, 2.5, 5.0]   # ties and saturation
        x[4, 64:96] = np.float32(2.0 ** 100)                    # large exponents
    q_o, e_o = oracle.quant_act_mx(x, elem)
    q_g, e_g = gpu_quant_mx(x, elem)
    np.testing.assert_array_equal(e_g, e_o)
    np.testing.assert_array_equal(q_g, q_o)


@pytest.mark.parametrize("elem", ELEMS)
def test_quantize_act_mx_non_finite_blocks(elem):
    M, K = 3, 128
    x = syn.normal_rows(6, 9, syn.T_A, M, K)
    x[0, 5] = np.nan
    x[1, 33] = np.inf
    x[2, 127] = -np.inf
    q_o, e_o = oracle.quant_act_mx(x, elem)
    assert e_o[0, 0] == 0xFF and e_o[1, 1] == 0xFF and e_o[2, 3] == 0xFF
    q_g, e_g = gpu_quant_mx(x, elem)
    np.testing.assert_array_equal(e_g, e_o)
    np.testing.assert_array_equal(q_g, q_o)


def run_mx(M, N, K, elem, seed=0, rows=None):
    d = syn.w4a8_mxfp4(seed, M, N, K)
    note(f"mx gemm {elem} M={M} N={N} K={K} seed={seed}")
    qa, ea = oracle.quant_act_mx(d["A0"], elem)
    desc = hq.desc_mx_act_mxfp4(N, K, fp4_act=elem == "e2m1")
    wp, sp, _ = hq.hq_repack(desc, d["q"], d["e"])
    D = empty(M * N * 2)
    ws, nb = workspace(desc, M)
    hq.hq_gemm(desc, M, dev(qa), dev(ea), dev(wp), dev(sp), None, D, ws, nb)
    torch.cuda.synchronize()
    Dh = to_f64(D[: M * N * 2].cpu().numpy().view(np.uint16).reshape(M, N), torch.bfloat16)
    r = sample_rows(M) if rows is None else rows
    O = oracle.gemm_mx_mxfp4(qa, ea, d["q"], d["e"], N=N, K=K, a_elem=elem, rows=r)
    return Dh[r], O


def check(Dr, O):
    assert np.all(np.isfinite(Dr))
    err = gate_error(Dr, O)
    # fp8 x fp4 and fp4 x fp4 products are exact in the MFMA; fp32 accumulation,
    # one bf16 rounding of the output: the bf16 bound used for the W4A8 path
    assert err <= min(GATE, 8e-3), err


@pytest.mark.parametrize("elem", ELEMS)
@pytest.mark.parametrize("M,N,K", cases.MXA_SMALL + cases.MXA_MID + cases.MXA_BIG)
def test_mx_gemm_shapes(elem, M, N, K):
    """Small-M weight stream (whole slice, split K), the 128 x 128 four-stage and
    two-stage tiles and the 256 x 256 ring, with ragged last tiles."""
    Dr, O = run_mx(M, N, K, elem, seed=M + K, rows=sweep_rows(M) if M > 300 else None)
    check(Dr, O)


@pytest.mark.parametrize("elem", ELEMS)
@pytest.mark.parametrize("M,N,K", cases.MXA_SWEEP)
def test_mx_gemm_full_size(elem, M, N, K):
    """The W4A8 workload's shape (N=7168, K=4096) with MX activations at every M
    of the benchmark sweep; sampled rows from M = 16 on."""
    Dr, O = run_mx(M, N, K, elem, seed=0, rows=sweep_rows(M))
    check(Dr, O)


@pytest.mark.parametrize("elem", ELEMS)
def test_mx_gemm_on_gpu_quantised_activations(elem):
    """The GPU quantiser feeding the GPU GEMM equals the oracle's quantiser
    feeding the oracle's GEMM (the codes are bit-identical, so the GEMM inputs are)."""
    M, N, K = 40, 512, 1024
    d = syn.w4a8_mxfp4(11, M, N, K)
    qa, ea = gpu_quant_mx(d["A0"], elem)
    qo, eo = oracle.quant_act_mx(d["A0"], elem)
    np.testing.assert_array_equal(qa, qo)
    np.testing.assert_array_equal(ea, eo)
    desc = hq.desc_mx_act_mxfp4(N, K, fp4_act=elem == "e2m1")
    wp, sp, _ = hq.hq_repack(desc, d["q"], d["e"])
    D = empty(M * N * 2)
    ws, nb = workspace(desc, M)
    hq.hq_gemm(desc, M, dev(qa), dev(ea), dev(wp), dev(sp), None, D, ws, nb)
    torch.cuda.synchronize()
    Dh = to_f64(D[: M * N * 2].cpu().numpy().view(np.uint16).reshape(M, N), torch.bfloat16)
    check(Dh, oracle.gemm_mx_mxfp4(qo, eo, d["q"], d["e"], N=N, K=K, a_elem=elem))
