"""GPU test of hq_gemm_noalloc, the entry point for callers that cannot
allocate: its split-K partial tiles live in a scratch array compiled into the
library.  Two calls in a row (the second smaller, so it runs on what the first
left in the array) must return exactly what hq_gemm returns with a workspace,
and both must meet the oracle's bar on sampled rows."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from bit_quantized_gemm_w4a16_amd import hq
from gpu_util import dev, empty, gate_error, note, sweep_rows, to_f64, workspace

pytestmark = pytest.mark.gpu


def _w8a8_pair(M, N, K, d):
    desc = hq.desc_w8a8(N, K, raw_int32=True)
    wp, sp, _ = hq.hq_repack(desc, d["w"], d["s_w"])
    a, sa, w, s = dev(d["a"][:M]), dev(d["s_a"][:M]), dev(wp), dev(sp)
    ref = empty(M * N * 4)
    ws, nb = workspace(desc, M)
    assert 0 < nb <= hq.HQ_NOALLOC_SCRATCH_BYTES, nb
    hq.hq_gemm(desc, M, a, sa, w, s, None, ref, ws, nb)
    got = empty(M * N * 4)
    hq.hq_gemm_noalloc(desc, M, a, sa, w, s, None, got)
    torch.cuda.synchronize()
    return ref[: M * N * 4].cpu().numpy().view(np.int32), got[: M * N * 4].cpu().numpy().view(np.int32)


def test_noalloc_w8a8_two_calls_bit_exact():
    """W8A8 (N=8192, K=7168) at M=128 (4-way K split, 16 MiB of partials) and
    then M=16 (2-way): raw int32 identical to hq_gemm and to the oracle."""
    N, K = 8192, 7168
    d = syn.w8a8_int8(0, 128, N, K)
    for M in (128, 16):
        note(f"noalloc w8a8 M={M} N={N} K={K}")
        ref, got = _w8a8_pair(M, N, K, d)
        np.testing.assert_array_equal(got, ref)
        r = sweep_rows(M)
        acc, _ = oracle.gemm_w8a8(d["a"][:M], d["s_a"][:M], d["w"], d["s_w"], rows=r)
        np.testing.assert_array_equal(got.reshape(M, N)[r].astype(np.int64), acc)


def test_noalloc_w4a16_two_calls_match_workspace_path():
    """fp16 W4A16 with zero-points (N=4096, K=7168) at M=64 then M=32, both split
    along K: outputs bit-identical to hq_gemm, within the gate of the oracle."""
    N, K, G = 4096, 7168, 128
    d = syn.w4a16_zp(0, 64, N, K, G, torch.float16)
    desc = hq.desc_w4a16(N, K, G, bf16=False, zp=True)
    wp, sp, zp = hq.hq_repack(desc, d["q"], d["s"], d["z"])
    w, s, z = dev(wp), dev(sp), dev(zp)
    A = dev(d["A"])
    for M in (64, 32):
        note(f"noalloc wna16 M={M} N={N} K={K}")
        ws, nb = workspace(desc, M)
        assert nb > 0
        ref, got = empty(M * N * 2), empty(M * N * 2)
        hq.hq_gemm(desc, M, A, None, w, s, z, ref, ws, nb)
        hq.hq_gemm_noalloc(desc, M, A, None, w, s, z, got)
        torch.cuda.synchronize()
        rb = ref[: M * N * 2].cpu().numpy().view(np.uint16)
        gb = got[: M * N * 2].cpu().numpy().view(np.uint16)
        np.testing.assert_array_equal(gb, rb)
        r = sweep_rows(M)
        O = oracle.gemm_wna16(d["A"][:M], d["q"], d["s"], d["z"], N=N, K=K, G=G, a_bf16=False, w_signed=False, rows=r)
        assert gate_error(to_f64(gb.reshape(M, N), torch.float16)[r], O) <= 3e-3


def test_noalloc_rejects_plans_beyond_the_scratch():
    """A plan needing more partial-tile bytes than the array holds is refused
    before any launch, with the need in the message."""
    N, K, M = 36864, 7168, 64
    desc = hq.desc_w4a16(N, K, 128, bf16=False, zp=True)
    assert hq.hq_workspace_bytes(desc, M) > hq.HQ_NOALLOC_SCRATCH_BYTES
    a, w, s, z, D = empty(M * K * 2), empty(16), empty(16), empty(16), empty(M * N * 2)
    with pytest.raises(hq.HQError) as e:
        hq.hq_gemm_noalloc(desc, M, a, None, w, s, z, D)
    assert e.value.status == hq.HQ_ERR_WORKSPACE and "scratch" in str(e.value)
