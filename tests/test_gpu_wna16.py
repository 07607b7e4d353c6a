"""GPU parity of the W4A16 path (symmetric INT4 / UINT4 + zero-points) against
the CPU oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from bit_quantized_gemm_w4a16_amd import hq
import cases
from gpu_util import GATE, dev, empty, gate_error, note, sample_rows, sweep_rows, to_f64, workspace

pytestmark = pytest.mark.gpu


def run_wna16(M, N, K, G, bf16, zp, seed=0, data=None, rows=None):
    dt = torch.bfloat16 if bf16 else torch.float16
    if data is None:
        data = (syn.w4a16_zp(seed, M, N, K, G, dt) if zp else syn.w4a16_sym(seed, M, N, K, G, dt))
    note(f"wna16 M={M} N={N} K={K} G={G} bf16={bf16} zp={zp} seed={seed}")
    desc = hq.desc_w4a16(N, K, G, bf16=bf16, zp=zp)
    wp, sp, zpk = hq.hq_repack(desc, data["q"], data["s"], data.get("z") if zp else None)
    A = dev(data["A"])
    w, s = dev(wp), dev(sp)
    z = dev(zpk) if zp else None
    D = empty(M * N * 2)
    ws, nb = workspace(desc, M)
    hq.hq_gemm(desc, M, A, None, w, s, z, D, ws, nb)
    torch.cuda.synchronize()
    Dh = to_f64(D[: M * N * 2].cpu().numpy().view(np.uint16).reshape(M, N), dt)
    r = sample_rows(M) if rows is None else rows
    O = oracle.gemm_wna16(data["A"], data["q"], data["s"], data.get("z") if zp else None, N=N, K=K, G=G,
                          a_bf16=bf16, w_signed=not zp, rows=r)
    return Dh[r], O


def check(Dr, O, bf16):
    err = gate_error(Dr, O)
    assert np.all(np.isfinite(Dr))
    assert err <= GATE, err
    # tighter bound derived from the output rounding (bf16 2^-8, fp16 2^-11) plus accumulation
    assert err <= (8e-3 if bf16 else 3e-3), err
    return err


def test_c1_dense_w4a16_sym_bf16_m16():
    """The small dense case: M=16, N=K=1024, symmetric INT4, G=128, bf16."""
    Dr, O = run_wna16(16, 1024, 1024, 128, bf16=True, zp=False, seed=0)
    check(Dr, O, True)


@pytest.mark.parametrize("M,N,K,G,bf16,zp", cases.WNA16_SMALL + cases.WNA16_SKINNY_K7168)
def test_small_m_tiles_and_ragged_tail(M, N, K, G, bf16, zp):
    Dr, O = run_wna16(M, N, K, G, bf16=bf16, zp=zp, seed=M)
    check(Dr, O, bf16)


@pytest.mark.parametrize("M,N,K,G,bf16,zp", cases.WNA16_LARGER)
def test_larger_m(M, N, K, G, bf16, zp):
    Dr, O = run_wna16(M, N, K, G, bf16=bf16, zp=zp, seed=M)
    check(Dr, O, bf16)


@pytest.mark.parametrize("M,N,K,G,bf16,zp", cases.WNA16_SHAPES)
def test_shapes_groups_and_split_k(M, N, K, G, bf16, zp):
    Dr, O = run_wna16(M, N, K, G, bf16=bf16, zp=zp, seed=N + M)
    check(Dr, O, bf16)


@pytest.mark.parametrize("M,N,K,G,bf16,zp", cases.WNA16_BF16_LARGE)
def test_bf16_above_small_m(M, N, K, G, bf16, zp):
    """bf16 activations on the tiled path (operand 128 + u, the -(128 + z) offset
    from a row-sum MFMA, the group scale on the fp32 partial), split and unsplit,
    symmetric and zero-point, ragged N."""
    Dr, O = run_wna16(M, N, K, G, bf16=bf16, zp=zp, seed=M + N, rows=sweep_rows(M))
    check(Dr, O, bf16)


def test_zero_point_equals_code_gives_exact_zero():
    M, N, K, G = 5, 64, 512, 128
    d = syn.w4a16_zp(1, M, N, K, G, torch.float16)
    zc = ((d["z"][:, :, None] >> (4 * np.arange(8, dtype=np.uint32))[None, None, :]) & 15).reshape(K // G, -1)
    q = np.zeros((K // 8, N), dtype=np.uint32)
    for k in range(K):
        q[k // 8] |= zc[k // G, :N].astype(np.uint32) << np.uint32(4 * (k % 8))
    d["q"] = q
    Dr, O = run_wna16(M, N, K, G, bf16=False, zp=True, data=d)
    assert np.all(O == 0) and np.all(Dr == 0)


def test_extreme_codes():
    M, N, K, G = 16, 128, 1024, 128
    for code in (0x88888888, 0x77777777):          # all -8 / all +7
        d = syn.w4a16_sym(2, M, N, K, G, torch.bfloat16)
        d["q"] = np.full_like(d["q"], code)
        Dr, O = run_wna16(M, N, K, G, bf16=True, zp=False, data=d)
        check(Dr, O, True)


def test_workspace_reused_across_calls_and_sizes():
    """One workspace serves back-to-back calls of different M (split and unsplit):
    each call writes the partial tiles it reads, so leftovers never leak in."""
    N, K, G = 1024, 7168, 128
    desc = hq.desc_w4a16(N, K, G, bf16=False, zp=True)
    nb = max(hq.hq_workspace_bytes(desc, m) for m in (1, 64))
    ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    for M in (40, 3, 64, 1):
        d = syn.w4a16_zp(M, M, N, K, G, torch.float16)
        note(f"wna16 reuse M={M}")
        wp, sp, zpk = hq.hq_repack(desc, d["q"], d["s"], d["z"])
        D = empty(M * N * 2)
        hq.hq_gemm(desc, M, dev(d["A"]), None, dev(wp), dev(sp), dev(zpk), D, ws, nb)
        torch.cuda.synchronize()
        Dh = to_f64(D[: M * N * 2].cpu().numpy().view(np.uint16).reshape(M, N), torch.float16)
        O = oracle.gemm_wna16(d["A"], d["q"], d["s"], d["z"], N=N, K=K, G=G, a_bf16=False, w_signed=False)
        check(Dh, O, False)


@pytest.mark.parametrize("M,N,K,G,bf16,zp", cases.WNA16_C2_SWEEP)
def test_dense_w4a16_zp_full_size(M, N, K, G, bf16, zp):
    """The dense W4A16 workload (UINT4 + zero-points, fp16, N=4096, K=7168, G=128)
    at every M of the benchmark sweep, in the launch configuration the benchmark
    times; sampled rows from M = 16 on."""
    Dr, O = run_wna16(M, N, K, G, bf16=bf16, zp=zp, seed=0, rows=sweep_rows(M))
    check(Dr, O, bf16)


@pytest.mark.parametrize("M,N,K,G,bf16,zp", cases.WNA16_WIDE)
def test_wide_tiles_ragged(M, N, K, G, bf16, zp):
    """Grids large enough for 256-column tiles (256 x 256 from about 256 tiles of
    that size, else 128 x 256), with ragged last row and column tiles."""
    Dr, O = run_wna16(M, N, K, G, bf16=bf16, zp=zp, seed=M + N)
    check(Dr, O, bf16)
