"""Host-side tests of the zero-exponent float weights e0mN (no GPU): descriptor
validation, and that the repack of e0mN codes equals the repack of the same
values as two's-complement codes of width n + 1 (the values decoded by the
oracle), so the kernels of that width run them unchanged."""
import numpy as np
import pytest

import oracle
from bit_quantized_gemm_w4a16_amd import hq


def words_of(ints, K, N):
    """int values [K][N] -> the 4-bit logical input uint32 [K/8][N]."""
    nib = (ints.astype(np.int64) & 15).astype(np.uint32)
    q = np.zeros((K // 8, N), dtype=np.uint32)
    for i in range(8):
        q |= nib[i::8] << np.uint32(4 * i)
    return q


def e0m_codes(rng, n, K, N):
    return rng.integers(0, 1 << (n + 1), size=(K, N)).astype(np.uint8)


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6, 7])
def test_descriptor_validation(n):
    d = hq.desc_e0m(1024, 1024, n)
    hq.hq_desc_validate(d)
    bad = hq.hq_layer_desc.from_buffer_copy(d)
    bad.zp_dtype = hq.HQ_DT_UINT4
    with pytest.raises(hq.HQError):
        hq.hq_desc_validate(bad)
    bad = hq.hq_layer_desc.from_buffer_copy(d)
    if n == 7:   # INT8 weight-only: fp32 per-channel scales only
        bad.w_scale_dtype, bad.w_scale_gran, bad.group_size = hq.HQ_DT_BF16, hq.HQ_GRAN_PER_GROUP_K, 128
    else:
        bad.w_scale_dtype, bad.w_scale_gran, bad.group_size = hq.HQ_DT_FP32, hq.HQ_GRAN_PER_CHANNEL, 1024
    with pytest.raises(hq.HQError):
        hq.hq_desc_validate(bad)


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6, 7])
@pytest.mark.parametrize("N,K", [(16, 128), (40, 384), (1000, 256)])
def test_repack_equals_the_twos_complement_container(n, N, K):
    rng = np.random.default_rng([n, N, K])
    codes = e0m_codes(rng, n, K, N)
    ints = oracle.e0m_to_int(codes, n)
    if n == 7:
        s = rng.random(N).astype(np.float32)
        got = hq.hq_repack(hq.desc_e0m(N, K, 7), codes, s)
        want = hq.hq_repack(hq.desc_w8a16(N, K, bf16=True), ints, s)
    else:
        s = np.full((K // 128, N), 0x3F80, np.uint16)
        w_in = words_of(codes.astype(np.int64), K, N) if n == 3 else codes
        got = hq.hq_repack(hq.desc_e0m(N, K, n), w_in, s)
        want = (hq.hq_repack(hq.desc_w4a16(N, K, 128, bf16=True, zp=False), words_of(ints, K, N), s) if n == 3
                else hq.hq_repack(hq.desc_wnwide(N, K, n + 1, True), ints, s) if n >= 4
                else hq.hq_repack(hq.desc_wnlow(N, K, n + 1, True), ints, s))
    for g, w in zip(got, want):
        if w is None:
            assert g is None
        else:
            np.testing.assert_array_equal(g, w)


@pytest.mark.parametrize("n", [1, 2, 4, 5, 6])
def test_repack_rejects_bits_above_the_sign(n):
    N, K = 32, 128
    codes = np.zeros((K, N), np.uint8)
    codes[5, 7] = 1 << (n + 1)
    with pytest.raises(hq.HQError) as e:
        hq.hq_repack(hq.desc_e0m(N, K, n), codes, np.full((1, N), 0x3F80, np.uint16))
    assert e.value.status == hq.HQ_ERR_INVALID_ARG


def test_plans_are_those_of_the_container():
    N, K = 4096, 4096
    for n, ref in ((3, hq.desc_w4a16(N, K, 128, bf16=True, zp=False)), (2, hq.desc_wnlow(N, K, 3, True)),
                   (1, hq.desc_wnlow(N, K, 2, True)), (7, hq.desc_w8a16(N, K, bf16=True)),
                   (4, hq.desc_wnwide(N, K, 5, True)), (5, hq.desc_wnwide(N, K, 6, True)),
                   (6, hq.desc_wnwide(N, K, 7, True))):
        for M in (1, 64, 1024):
            assert hq.hq_gemm_plan(hq.desc_e0m(N, K, n), M) == hq.hq_gemm_plan(ref, M)
