"""GPU parity of the MX float weight formats with bf16 activations (MXFP8:
E4M3 codes; MXFP6: E2M3 / E3M2 codes; one E8M0 scale per 32 K) against the CPU
oracle, through the C ABI.  The small-M stream converts the codes with the
lane's scale (FP6 32 at a time); the tiles take E4M3 codes (FP6 widened to
E4M3 in the workspace first, exact)."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from bit_quantized_gemm_w4a16_amd import hq
import cases
from gpu_util import GATE, dev, empty, gate_error, note, sample_rows, sweep_rows, to_f64

pytestmark = pytest.mark.gpu


def run(M, N, K, elem, seed, rows=None, codes=None, e=None):
    note(f"mxf elem={elem} M={M} N={N} K={K} seed={seed}")
    d = syn.mxf_a16(seed, M, N, K, elem)
    if codes is not None:
        d["codes"] = codes
    if e is not None:
        d["e"] = e
    desc = hq.desc_mxf_a16(N, K, elem)
    wp, sp, _ = hq.hq_repack(desc, d["codes"], d["e"])
    D = empty(M * N * 2)
    nb = hq.hq_workspace_bytes(desc, M)
    ws = torch.zeros(max(nb, 16), dtype=torch.uint8, device="cuda") if nb else None
    hq.hq_gemm(desc, M, dev(d["A"]), None, dev(wp), dev(sp), None, D, ws, nb)
    torch.cuda.synchronize()
    Dh = to_f64(D[: M * N * 2].cpu().numpy().view(np.uint16).reshape(M, N), torch.bfloat16)
    r = sample_rows(M) if rows is None else rows
    O = oracle.gemm_mxf_a16(d["A"], d["codes"], d["e"], elem=elem, rows=r)
    Dr = Dh[r]
    assert np.all(np.isfinite(Dr))
    err = gate_error(Dr, O)
    assert err <= GATE and err <= 8e-3, err
    return err


@pytest.mark.parametrize("M,N,K,elem", cases.MXF_SMALL)
def test_small_m_stream(M, N, K, elem):
    run(M, N, K, elem, seed=M)


@pytest.mark.parametrize("M,N,K,elem", cases.MXF_TILES)
def test_tiles_ragged(M, N, K, elem):
    run(M, N, K, elem, seed=M + N)


@pytest.mark.parametrize("M,N,K,elem", cases.MXF_SWEEP)
def test_full_size_sweep(M, N, K, elem):
    """N = 4096, K = 7168 at every M of the benchmark sweep, in the launch
    configuration the benchmark times; sampled rows from M = 16 on."""
    run(M, N, K, elem, seed=0, rows=sweep_rows(M))


@pytest.mark.parametrize("elem", cases.MXF_ELEMS)
def test_every_code_under_extreme_block_scales(elem):
    """Every code of the format cycles through K (FP6: all 64; E4M3: the finite
    ones) under block exponents far from 127 on both sides (scales 2^-27..2^-24
    and 2^93..2^96, products and sums still normal in bf16 and fp32), on the
    stream (M = 8) and the tiles (M = 160)."""
    N, K = 144, 1024
    if elem == "e4m3":
        allc = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    else:
        allc = np.arange(64, dtype=np.uint8)
    codes = allc[(np.arange(K)[:, None] + 7 * np.arange(N)[None, :]) % allc.size]
    for M in (8, 160):
        for lo, hi in ((100, 104), (220, 224)):
            e = np.random.default_rng([M, lo]).integers(lo, hi, size=(K // 32, N)).astype(np.uint8)
            run(M, N, K, elem, seed=3, rows=np.arange(M), codes=codes, e=e)
