"""GPU parity of the zero-exponent float weights e0mN (sign bit and integer
magnitude: e0m1..e0m6 with 16-bit group scales on the WnA16 kernels of width
n + 1, e0m7 with fp32 per-channel scales on the INT8 weight-only kernels)
against the CPU oracle (its e0mN decode, then the integer GEMM of the
container), through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from bit_quantized_gemm_w4a16_amd import hq
from gpu_util import GATE, dev, empty, gate_error, note, sample_rows, to_f64

pytestmark = pytest.mark.gpu

CASES = [(M, N, K, n, bf) for n in (1, 2, 3, 4, 5, 6, 7) for bf in (True, False)
         for M, N, K in ((1, 272, 1024), (24, 272, 1024), (300, 1000, 512))]


def words_of(ints, K, N):
    nib = (ints.astype(np.int64) & 15).astype(np.uint32)
    q = np.zeros((K // 8, N), dtype=np.uint32)
    for i in range(8):
        q |= nib[i::8] << np.uint32(4 * i)
    return q


@pytest.mark.parametrize("M,N,K,n,bf", CASES)
def test_e0m_matches_the_oracle(M, N, K, n, bf):
    note(f"e0m{n} M={M} N={N} K={K} bf16={bf}")
    dt = torch.bfloat16 if bf else torch.float16
    rng = np.random.default_rng([M, N, K, n])
    codes = rng.integers(0, 1 << (n + 1), size=(K, N)).astype(np.uint8)
    ints = oracle.e0m_to_int(codes, n)
    A = syn.activations(M + n, syn.C11, M, K, dt)
    desc = hq.desc_e0m(N, K, n, bf16=bf)
    if n == 7:
        s = (np.abs(rng.standard_normal(N)) * 0.01 + 1e-4).astype(np.float32)
        packed = hq.hq_repack(desc, codes, s)
        ref = lambda r: oracle.gemm_w8a16(A, ints, s, a_bf16=bf, rows=r)
    else:
        s = torch.from_numpy((np.abs(rng.standard_normal((K // 128, N))) * 0.02 + 1e-3).astype(np.float32)).to(dt)
        s = s.view(torch.int16).numpy().view(np.uint16)
        packed = hq.hq_repack(desc, words_of(codes.astype(np.int64), K, N) if n == 3 else codes, s)
        if n >= 4:
            ref = lambda r: oracle.gemm_wnwide(A, ints, s, None, N=N, K=K, G=128, bits=n + 1, a_bf16=bf,
                                               w_signed=True, rows=r)
        elif n == 3:
            ref = lambda r: oracle.gemm_wna16(A, words_of(ints, K, N), s, None, N=N, K=K, G=128, a_bf16=bf,
                                              w_signed=True, rows=r)
        else:
            ref = lambda r: oracle.gemm_wnlow(A, ints, s, None, N=N, K=K, G=128, bits=n + 1, a_bf16=bf,
                                              w_signed=True, rows=r)
    D = empty(M * N * 2)
    nb = hq.hq_workspace_bytes(desc, M)
    ws = torch.zeros(max(nb, 16), dtype=torch.uint8, device="cuda") if nb else None
    hq.hq_gemm(desc, M, dev(A), None, dev(packed[0]), dev(packed[1]), None, D, ws, nb)
    torch.cuda.synchronize()
    Dh = to_f64(D[: M * N * 2].cpu().numpy().view(np.uint16).reshape(M, N), dt)
    rows = sample_rows(M)
    O = ref(rows)
    err = gate_error(Dh[rows], O)
    assert np.all(np.isfinite(Dh[rows])) and err <= GATE and err <= (8e-3 if bf else 3e-3), err
