"""GPU parity of the dense W4A8-MXFP4 and W8A8-INT8 paths and of the tokenwise
E4M3 activation quantisation, against the CPU oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from bit_quantized_gemm_w4a16_amd import hq
import cases
from gpu_util import GATE, dev, empty, gate_error, note, sample_rows, sweep_rows, to_f64, workspace

pytestmark = pytest.mark.gpu


def gpu_quant(A0):
    M, K = A0.shape
    x = dev(A0.astype(np.float32))
    q = empty(M * K)
    s = torch.empty(max(M, 4), dtype=torch.float32, device="cuda")
    hq.hq_quantize_act(hq.HQ_DT_FP8_E4M3, M, K, x, q, s)
    torch.cuda.synchronize()
    return q[: M * K].cpu().numpy().reshape(M, K), s[:M].cpu().numpy()


@pytest.mark.parametrize("K", [4096, 1001])
def test_quantize_act_non_finite_rows(K):
    """NaN elements are left out of the row maximum and encode as 0x7F (the E4M3
    NaN); a row holding an infinity gets an infinite scale, its finite elements
    encode as +-0 and its infinities (Inf / Inf) as NaN -- bit for bit as the oracle."""
    note(f"quant_e4m3 non-finite K={K}")
    A0 = syn.normal_rows(4, 3, syn.T_A, 6, K)
    A0[0, 5] = np.nan
    A0[1, :3] = [np.nan, -np.nan, 7.0]
    A0[2, 17] = np.inf
    A0[3, 0] = -np.inf
    A0[3, 9] = np.nan
    A0[4, :] = np.nan
    q_o, s_o = oracle.quant_act_e4m3(A0)
    assert q_o[0, 5] == 0x7F and q_o[2, 17] == 0x7F and np.isinf(s_o[2]) and s_o[4] == 1.0
    q_g, s_g = gpu_quant(A0)
    np.testing.assert_array_equal(s_g.view(np.uint32), s_o.view(np.uint32))
    np.testing.assert_array_equal(q_g, q_o)


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


@pytest.mark.parametrize("M,N,K", cases.W4A8_SMALL)
def test_w4a8_small_shapes(M, N, K):
    Dr, O = run_w4a8(M, N, K, seed=M)
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


@pytest.mark.parametrize("M,N,K", cases.W4A8_MID)
def test_w4a8_two_stage_128_tiles(M, N, K):
    """The two-stage 128 x 128 W4A8 tile (more than one round of 128 x 128 tiles,
    too few for 256 x 256), with a ragged last column tile in the second shape."""
    Dr, O = run_w4a8(M, N, K, seed=M + K, rows=sweep_rows(M))
    err = gate_error(Dr, O)
    assert err <= min(GATE, 8e-3), err


@pytest.mark.parametrize("M,N,K", cases.W4A8_BIG)
def test_w4a8_big_tiles_ragged(M, N, K):
    """256 x 256 W4A8 tiles on the three-stage ring with ragged last row and
    column tiles: one K step (the ring's prologue fetches steps past the slice,
    never computed) and five steps (not a multiple of the ring)."""
    Dr, O = run_w4a8(M, N, K, seed=M + K, rows=np.arange(M))
    err = gate_error(Dr, O)
    assert err <= min(GATE, 8e-3), err


@pytest.mark.parametrize("M,N,K", cases.W4A8_C3_SWEEP)
def test_w4a8_full_size(M, N, K):
    """The dense W4A8-MXFP4 workload (N=7168, K=4096) at every M of the benchmark
    sweep, in the launch configuration the benchmark times; sampled rows from M = 16 on."""
    Dr, O = run_w4a8(M, N, K, seed=0, rows=sweep_rows(M))
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


@pytest.mark.parametrize("M,N,K", cases.W8A8_SMALL_RAW + cases.W8A8_SKINNY_K7168)
def test_w8a8_raw_int32_bit_exact_small(M, N, K):
    got, acc = run_w8a8(M, N, K, seed=M, raw=True)
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


@pytest.mark.parametrize("M,N,K", cases.W8A8_SMALL_BF16)
def test_w8a8_bf16_small(M, N, K):
    got, O = run_w8a8(M, N, K, seed=M)
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


@pytest.mark.parametrize("M,N,K", cases.W8A8_C4_SWEEP)
def test_w8a8_full_size(M, N, K):
    """The dense W8A8 workload (N=18432, K=7168) at every M of the benchmark sweep:
    raw int32 bit-exact and the bf16 epilogue, sampled rows from M = 16 on."""
    d = syn.w8a8_int8(0, M, N, K)
    r = sweep_rows(M)
    got, acc = run_w8a8(M, N, K, raw=True, rows=r, data=d)
    np.testing.assert_array_equal(got.astype(np.int64), acc)
    got, O = run_w8a8(M, N, K, rows=r, data=d)
    assert gate_error(got, O) <= 8e-3


@pytest.mark.parametrize("M,N,K", cases.W8A8_BIG_RAW)
def test_w8a8_raw_int32_big_tiles_ragged(M, N, K):
    """Grids of 256 x 256 INT8 tiles (two stages) with ragged last row and column
    tiles, at one, two and three K steps: raw int32 accumulators bit-exact."""
    got, acc = run_w8a8(M, N, K, seed=M, raw=True)
    np.testing.assert_array_equal(got.astype(np.int64), acc)


@pytest.mark.parametrize("M,N,K", cases.W8A8_RING)
def test_w8a8_raw_int32_ring_tiles(M, N, K):
    """The 256 x 128 INT8 tile on its three-stage ring, reached from the 128-row
    branch (M = 200) and the 256-row branch (M = 1024, 256), with three, two and
    five K steps and ragged last tiles: raw int32 accumulators bit-exact."""
    got, acc = run_w8a8(M, N, K, seed=M, raw=True, rows=sweep_rows(M))
    np.testing.assert_array_equal(got.astype(np.int64), acc)
