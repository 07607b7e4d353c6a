"""GPU parity of FP8 W8A8 with blockwise scales against the CPU oracle, through
the C ABI: E4M3 activations with one fp32 scale per row and 128-K block
(quantised on the GPU bit-exactly), E4M3 weights with one fp32 scale per
128 x 128 block, each 128-K block's fp8 MFMA partial scaled on the fp32
accumulator."""
import numpy as np
import pytest
import torch

import cases
import oracle
import synthetic as syn
from bit_quantized_gemm_w4a16_amd import hq
from gpu_util import GATE, dev, empty, gate_error, note, sample_rows, sweep_rows, to_f64, workspace

pytestmark = pytest.mark.gpu

SMALL, TILES, SWEEP = cases.FP8B_SMALL, cases.FP8B_TILES, cases.FP8B_SWEEP


def gpu_quant_blocks(x, block):
    M, K = x.shape
    q, s = empty(M * K), empty(M * (K // block) * 4)
    hq.hq_quantize_act_blocks(hq.HQ_DT_FP8_E4M3, M, K, block, dev(x.astype(np.float32)), q, s)
    torch.cuda.synchronize()
    return q[: M * K].cpu().numpy().reshape(M, K), s[: M * (K // block) * 4].cpu().numpy().view(np.float32).reshape(M, -1)


@pytest.mark.parametrize("M,K,block", [(1, 128, 128), (7, 640, 128), (300, 7168, 128), (5, 4096, 4096), (3, 256, 32)])
def test_quantize_act_blocks_bit_exact(M, K, block):
    note(f"quant blocks M={M} K={K} block={block}")
    x = syn.normal_rows(7, 10, syn.T_A, M, K)
    if M > 2:
        x[1, :block] = 0.0                                    # all-zero block -> scale 1, codes 0
        x[2, 3] = np.nan
    q_o, s_o = oracle.quant_act_e4m3_blocks(x, block)
    q_g, s_g = gpu_quant_blocks(x, block)
    np.testing.assert_array_equal(s_g.view(np.uint32), s_o.view(np.uint32))
    np.testing.assert_array_equal(q_g, q_o)


def run_fp8b(M, N, K, seed=0, rows=None):
    d = syn.w8a8_fp8_blockwise(seed, M, N, K)
    note(f"fp8 blockwise M={M} N={N} K={K} seed={seed}")
    qa, sa = oracle.quant_act_e4m3_blocks(d["A0"], 128)
    desc = hq.desc_fp8_blockwise(N, K)
    wp, sp, _ = hq.hq_repack(desc, d["w"], d["s_w"])
    D = empty(M * N * 2)
    ws, nb = workspace(desc, M)
    hq.hq_gemm(desc, M, dev(qa), dev(sa), dev(wp), dev(sp), None, D, ws, nb)
    torch.cuda.synchronize()
    Dh = to_f64(D[: M * N * 2].cpu().numpy().view(np.uint16).reshape(M, N), torch.bfloat16)
    r = sample_rows(M) if rows is None else rows
    return Dh[r], oracle.gemm_fp8_blockwise(qa, sa, d["w"], d["s_w"], rows=r)


def check(Dr, O):
    assert np.all(np.isfinite(Dr))
    err = gate_error(Dr, O)
    # exact fp8 products, fp32 block partials scaled in fp32 (two roundings per
    # block), fp32 accumulation, one bf16 rounding: the bf16 bound
    assert err <= min(GATE, 8e-3), err


@pytest.mark.parametrize("M,N,K", SMALL + TILES)
def test_fp8_blockwise_shapes(M, N, K):
    """Small-M weight stream (split and unsplit), 128 x 128 and 256 x 128 rings,
    ragged last row, column tile and column scale block."""
    Dr, O = run_fp8b(M, N, K, seed=M + K, rows=sweep_rows(M) if M > 300 else None)
    check(Dr, O)


@pytest.mark.parametrize("M,N,K", SWEEP)
def test_fp8_blockwise_full_size(M, N, K):
    """A DeepSeek-style FP8 layer (N = K = 7168, 128 x 128 weight blocks) at the M sweep."""
    Dr, O = run_fp8b(M, N, K, seed=0, rows=sweep_rows(M))
    check(Dr, O)


def test_fp8_blockwise_on_gpu_quantised_activations():
    M, N, K = 40, 512, 1024
    d = syn.w8a8_fp8_blockwise(3, M, N, K)
    qa, sa = gpu_quant_blocks(d["A0"], 128)
    qo, so = oracle.quant_act_e4m3_blocks(d["A0"], 128)
    np.testing.assert_array_equal(qa, qo)
    np.testing.assert_array_equal(sa.view(np.uint32), so.view(np.uint32))
    desc = hq.desc_fp8_blockwise(N, K)
    wp, sp, _ = hq.hq_repack(desc, d["w"], d["s_w"])
    D = empty(M * N * 2)
    ws, nb = workspace(desc, M)
    hq.hq_gemm(desc, M, dev(qa), dev(sa), dev(wp), dev(sp), None, D, ws, nb)
    torch.cuda.synchronize()
    Dh = to_f64(D[: M * N * 2].cpu().numpy().view(np.uint16).reshape(M, N), torch.bfloat16)
    check(Dh, oracle.gemm_fp8_blockwise(qo, so, d["w"], d["s_w"]))
