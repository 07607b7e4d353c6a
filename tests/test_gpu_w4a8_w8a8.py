"""GPU parity of the dense W4A8-MXFP4 and W8A8-INT8 paths and of the tokenwise
E4M3 activation quantisation, against the CPU oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from bit_quantized_gemm_w4a16_amd import hq
from gpu_util import GATE, dev, empty, gate_error, note, sample_rows, to_f64, workspace

pytestmark = pytest.mark.gpu


def gpu_quant(A0):
    M, K = A0.shape
    x = dev(A0.astype(np.float32))
    q = empty(M * K)
    s = torch.empty(max(M, 4), dtype=torch.float32, device="cuda")
    hq.hq_quantize_act(hq.HQ_DT_FP8_E4M3, M, K, x, q, s)
    torch.cuda.synchronize()
    return q[: M * K].cpu().numpy().reshape(M, K), s[:M].cpu().numpy()


# K a multiple of 4 up to 8192: the register-held row kernel (1, 2, 4 and 8
# float4 per thread, with ragged tails); other K: the generic kernel.
@pytest.mark.parametrize("M,K", [(1, 4), (1, 128), (5, 4096), (64, 1000), (300, 4096), (9, 2052), (2, 8192),
                                 (7, 1001), (3, 10000), (4, 8196)])
def test_quantize_act_bit_exact(M, K):
    note(f"quant_e4m3 M={M} K={K}")
    A0 = syn.normal_rows(3, 3, syn.T_A, M, K)
    if M > 2:
        A0[1] = 0.0                   # all-zero row -> scale 1, codes 0
        A0[2, :7] = [448.0, -1e-30, 3e-3, -2.5, 0.0, 1e-7, -448.0]
    q_o, s_o = oracle.quant_act_e4m3(A0)
    q_g, s_g = gpu_quant(A0)
    np.testing.assert_array_equal(s_g.view(np.uint32), s_o.view(np.uint32))
    np.testing.assert_array_equal(q_g, q_o)


def run_w4a8(M, N, K, seed=0, data=None, rows=None):
    d = syn.w4a8_mxfp4(seed, M, N, K) if data is None else data
    note(f"w4a8 M={M} N={N} K={K} seed={seed}")
    qa, s_a = oracle.quant_act_e4m3(d["A0"])
    desc = hq.desc_w4a8_mxfp4(N, K)
    wp, sp, _ = hq.hq_repack(desc, d["q"], d["e"])
    D = empty(M * N * 2)
    ws, nb = workspace(desc, M)
    hq.hq_gemm(desc, M, dev(qa), dev(s_a), dev(wp), dev(sp), None, D, ws, nb)
    torch.cuda.synchronize()
    Dh = to_f64(D[: M * N * 2].cpu().numpy().view(np.uint16).reshape(M, N), torch.bfloat16)
    r = sample_rows(M) if rows is None else rows
    O = oracle.gemm_w4a8_mxfp4(qa, s_a, d["q"], d["e"], N=N, K=K, rows=r)
    return Dh[r], O


@pytest.mark.parametrize("M", [1, 3, 16, 24, 32, 64, 100, 257])
def test_w4a8_small_shapes(M):
    Dr, O = run_w4a8(M, 272, 512, seed=M)
    err = gate_error(Dr, O)
    assert err <= min(GATE, 8e-3), err


def test_w4a8_ragged_n_and_extremes():
    M, N, K = 20, 1000, 1024
    d = syn.w4a8_mxfp4(5, M, N, K)
    d["q"][:] = 0x77777777                          # every code +6
    d["e"][:] = 127
    Dr, O = run_w4a8(M, N, K, data=d)
    assert gate_error(Dr, O) <= 8e-3
    d = syn.w4a8_mxfp4(6, M, N, K)
    d["e"][::3] = 118                               # mixed exponents, smallest value 2^-10
    Dr, O = run_w4a8(M, N, K, data=d)
    assert gate_error(Dr, O) <= 8e-3


@pytest.mark.parametrize("M,N,K", [(1100, 7200, 128), (1100, 7168, 640)])
def test_w4a8_big_tiles_ragged(M, N, K):
    """256 x 256 W4A8 tiles on the three-stage ring with ragged last row and
    column tiles: one K step (the ring's prologue fetches steps past the slice,
    never computed) and five steps (not a multiple of the ring)."""
    Dr, O = run_w4a8(M, N, K, seed=M + K, rows=np.arange(M))
    err = gate_error(Dr, O)
    assert err <= min(GATE, 8e-3), err


@pytest.mark.parametrize("M", [1, 16, 32, 256, 2048, 8192])
def test_w4a8_full_size(M):
    """The dense W4A8-MXFP4 workload: N=7168, K=4096 (sampled rows at large M)."""
    Dr, O = run_w4a8(M, 7168, 4096, seed=0)
    err = gate_error(Dr, O)
    assert err <= min(GATE, 8e-3), err


def run_w8a8(M, N, K, seed=0, raw=False, rows=None, data=None):
    d = syn.w8a8_int8(seed, M, N, K) if data is None else data
    note(f"w8a8 M={M} N={N} K={K} raw={raw} seed={seed}")
    desc = hq.desc_w8a8(N, K, raw_int32=raw)
    wp, sp, _ = hq.hq_repack(desc, d["w"], d["s_w"])
    D = empty(M * N * (4 if raw else 2))
    ws, nb = workspace(desc, M)
    hq.hq_gemm(desc, M, dev(d["a"]), dev(d["s_a"]), dev(wp), dev(sp), None, D, ws, nb)
    torch.cuda.synchronize()
    r = sample_rows(M) if rows is None else rows
    acc, O = oracle.gemm_w8a8(d["a"], d["s_a"], d["w"], d["s_w"], rows=r)
    if raw:
        got = D[: M * N * 4].cpu().numpy().view(np.int32).reshape(M, N)[r]
        return got, acc
    got = to_f64(D[: M * N * 2].cpu().numpy().view(np.uint16).reshape(M, N), torch.bfloat16)[r]
    return got, O


@pytest.mark.parametrize("M", [1, 7, 64, 130])
def test_w8a8_raw_int32_bit_exact_small(M):
    got, acc = run_w8a8(M, 304, 640, seed=M, raw=True)
    np.testing.assert_array_equal(got.astype(np.int64), acc)


def test_w8a8_split_k_needs_workspace():
    """Shapes whose grid is split along K (partials summed by a finalize pass)
    report a workspace; without it the call is rejected, not run."""
    desc = hq.desc_w8a8(304, 640, raw_int32=True)
    assert hq.hq_workspace_bytes(desc, 130) > 0
    D = empty(130 * 304 * 4)
    a, sa, w, s = empty(130 * 640), empty(130 * 4), empty(304 * 640), empty(304 * 4)
    with pytest.raises(hq.HQError):
        hq.hq_gemm(desc, 130, a, sa, w, s, None, D)


@pytest.mark.parametrize("M", [1, 33, 200])
def test_w8a8_bf16_small(M):
    got, O = run_w8a8(M, 304, 640, seed=M)
    assert gate_error(got, O) <= 8e-3


def test_w8a8_extreme_accumulators_exact():
    """All codes +-127 at K=7168: |acc| = 127^2 * 7168 = 115,613,696, still exact in int32."""
    M, N, K = 8, 64, 7168
    d = syn.w8a8_int8(1, M, N, K)
    d["a"][:] = 127
    d["a"][1::2] = -127
    d["w"][:] = 127
    got, acc = run_w8a8(M, N, K, raw=True, data=d)
    np.testing.assert_array_equal(got.astype(np.int64), acc)
    assert abs(int(acc[0, 0])) == 127 * 127 * K


@pytest.mark.parametrize("M", [1, 64, 512, 8192])
def test_w8a8_full_size(M):
    """The dense W8A8 workload: N=18432, K=7168; raw int32 bit-exact and bf16 epilogue."""
    got, acc = run_w8a8(M, 18432, 7168, seed=0, raw=True)
    np.testing.assert_array_equal(got.astype(np.int64), acc)
    got, O = run_w8a8(M, 18432, 7168, seed=0)
    assert gate_error(got, O) <= 8e-3


@pytest.mark.parametrize("M,N,K", [(2100, 16400, 256), (600, 11000, 384), (600, 11000, 128)])
def test_w8a8_raw_int32_big_tiles_ragged(M, N, K):
    """Grids of 256 x 256 (first shape) and 256 x 128 (the others, a three-stage
    ring: three steps, and one step whose ring fetches run past the slice) INT8
    tiles with ragged last row and column tiles: raw int32 accumulators bit-exact."""
    got, acc = run_w8a8(M, N, K, seed=M, raw=True)
    np.testing.assert_array_equal(got.astype(np.int64), acc)
