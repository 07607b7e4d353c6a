"""Host-side tests of libhq (no GPU): exported symbols, descriptor validation,
error paths that must return before any HIP call, and the repack layout."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import synthetic as syn
from bit_quantized_gemm_w4a16_amd import hq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    txt = open(os.path.join(ROOT, "include", "hq.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(hq_[a-z0-9_]+)\s*\(", txt)))


def test_library_exports_every_declared_function():
    names = header_functions()
    assert "hq_gemm" in names and "hq_repack" in names and "hq_moe_gemm" in names
    L = C.CDLL(hq.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    assert hq.lib().hq_abi_version() == hq.HQ_ABI_VERSION


def status_of(fn, *args):
    try:
        fn(*args)
    except hq.HQError as e:
        return e.status
    return hq.HQ_OK


def test_descriptor_validation():
    ok = hq.desc_w4a16(1024, 1024)
    assert status_of(hq.hq_desc_validate, ok) == hq.HQ_OK
    bad = hq.desc_w4a16(1024, 1024)
    bad.abi_version = 99
    assert status_of(hq.hq_desc_validate, bad) == hq.HQ_ERR_ABI
    assert status_of(hq.hq_desc_validate, hq.desc_w4a16(1024, 1000)) == hq.HQ_ERR_UNSUPPORTED       # K % G
    assert status_of(hq.hq_desc_validate, hq.desc_w4a16(1024, 1024, group_size=64)) == hq.HQ_ERR_UNSUPPORTED
    assert status_of(hq.hq_desc_validate, hq.desc_w4a16(0, 1024)) == hq.HQ_ERR_INVALID_ARG
    # N up to 2^21 (a 256-row output tile is addressed through one 32-bit buffer range)
    assert status_of(hq.hq_desc_validate, hq.desc_w4a16(1 << 21, 1024)) == hq.HQ_OK
    assert status_of(hq.hq_desc_validate, hq.desc_w4a16((1 << 21) + 1, 1024)) == hq.HQ_ERR_INVALID_ARG
    r = hq.desc_w4a16(64, 128)
    r.reserved = 3
    assert status_of(hq.hq_desc_validate, r) == hq.HQ_ERR_INVALID_ARG
    r = hq.desc_w4a16(64, 128)
    r.flags = 4
    assert status_of(hq.hq_desc_validate, r) == hq.HQ_ERR_INVALID_ARG
    r = hq.desc_w4a16(64, 128)
    r.tune = hq.HQ_TUNE(9, 1)
    assert status_of(hq.hq_desc_validate, r) == hq.HQ_ERR_INVALID_ARG
    r = hq.desc_moe_mxfp4(8, 128, 128)
    r.flags = hq.HQ_FLAG_BATCH_INVARIANT
    assert status_of(hq.hq_desc_validate, r) == hq.HQ_ERR_UNSUPPORTED
    mix = hq.desc_w4a16(64, 128)
    mix.w_scale_dtype = hq.HQ_DT_FP16                                                             # bf16 A, fp16 scales
    assert status_of(hq.hq_desc_validate, mix) == hq.HQ_ERR_UNSUPPORTED
    zp_missing = hq.desc_w4a16(64, 128, zp=True)
    zp_missing.zp_dtype = hq.HQ_DT_NONE
    assert status_of(hq.hq_desc_validate, zp_missing) == hq.HQ_ERR_UNSUPPORTED
    assert status_of(hq.hq_desc_validate, hq.desc_w4a8_mxfp4(7168, 4096)) == hq.HQ_OK
    assert status_of(hq.hq_desc_validate, hq.desc_w4a8_mxfp4(7168, 4000)) == hq.HQ_ERR_UNSUPPORTED
    assert status_of(hq.hq_desc_validate, hq.desc_w8a8(18432, 7168)) == hq.HQ_OK
    assert status_of(hq.hq_desc_validate, hq.desc_w8a8(18432, 7168 + 32)) == hq.HQ_ERR_UNSUPPORTED
    assert status_of(hq.hq_desc_validate, hq.desc_moe_mxfp4(256, 4096, 7168)) == hq.HQ_OK
    pair = hq.desc_w4a16(64, 128)
    pair.a_dtype = hq.HQ_DT_INT8
    assert status_of(hq.hq_desc_validate, pair) == hq.HQ_ERR_UNSUPPORTED
    assert "dtype" in hq.lib().hq_last_error().decode()


def test_descriptor_validation_low_precision_variants():
    """W4A4 / MXFP8 activations (E8M0 per 32 K) and FP8 W8A8 with blockwise scales."""
    assert status_of(hq.hq_desc_validate, hq.desc_mx_act_mxfp4(7168, 4096, fp4_act=True)) == hq.HQ_OK
    assert status_of(hq.hq_desc_validate, hq.desc_mx_act_mxfp4(7168, 4096, fp4_act=False)) == hq.HQ_OK
    assert status_of(hq.hq_desc_validate, hq.desc_mx_act_mxfp4(7168, 4000, fp4_act=True)) == hq.HQ_ERR_UNSUPPORTED
    d = hq.desc_mx_act_mxfp4(256, 256, fp4_act=True)
    d.a_scale = hq.HQ_ASCALE_PER_TOKEN_F32                  # fp4 activations need MX scales
    assert status_of(hq.hq_desc_validate, d) == hq.HQ_ERR_UNSUPPORTED
    d = hq.desc_mx_act_mxfp4(256, 256, fp4_act=True)
    d.num_experts = 4
    assert status_of(hq.hq_desc_validate, d) == hq.HQ_ERR_UNSUPPORTED
    assert status_of(hq.hq_desc_validate, hq.desc_fp8_blockwise(7168, 7168)) == hq.HQ_OK
    assert status_of(hq.hq_desc_validate, hq.desc_fp8_blockwise(7168, 7000)) == hq.HQ_ERR_UNSUPPORTED
    d = hq.desc_fp8_blockwise(256, 256)
    d.w_scale_gran = hq.HQ_GRAN_PER_CHANNEL
    assert status_of(hq.hq_desc_validate, d) == hq.HQ_ERR_UNSUPPORTED
    d = hq.desc_fp8_blockwise(256, 256)
    d.a_scale = hq.HQ_ASCALE_PER_TOKEN_F32
    assert status_of(hq.hq_desc_validate, d) == hq.HQ_ERR_UNSUPPORTED


def test_descriptor_validation_mxint4():
    """MXINT4 (INT4 codes, E8M0 per 32 K, bf16 activations): dense only, 32-K blocks,
    no zero-points; INT4 with bf16 scales stays the symmetric W4A16 format."""
    assert status_of(hq.hq_desc_validate, hq.desc_mxint4_a16(4096, 7168)) == hq.HQ_OK
    assert status_of(hq.hq_desc_validate, hq.desc_mxint4_a16(4096, 7000)) == hq.HQ_ERR_UNSUPPORTED
    for field, value in (("group_size", 16), ("num_experts", 4), ("zp_dtype", hq.HQ_DT_UINT4),
                         ("a_scale", hq.HQ_ASCALE_PER_TOKEN_F32), ("out_dtype", hq.HQ_DT_FP16),
                         ("scale2", hq.HQ_S2_PER_TENSOR_F32)):
        d = hq.desc_mxint4_a16(256, 256)
        setattr(d, field, value)
        assert status_of(hq.hq_desc_validate, d) == hq.HQ_ERR_UNSUPPORTED, field
    assert status_of(hq.hq_desc_validate, hq.desc_w4a16(256, 256, bf16=True, zp=False)) == hq.HQ_OK
    # the packed layout is the MXFP4 one (natural nibble order, E8M0 per lane)
    N, K = 40, 256
    d = syn.w4a16_mxint4(0, 1, N, K)
    wi, si, _ = hq.hq_repack(hq.desc_mxint4_a16(N, K), d["q"], d["e"])
    wf, sf, _ = hq.hq_repack(hq.desc_fp4_a16(N, K, False), d["q"], d["e"])
    np.testing.assert_array_equal(wi, wf)
    np.testing.assert_array_equal(si, sf)


def test_descriptor_validation_and_layout_w8a16():
    """INT8 weight-only: 16-bit activations, fp32 per-channel scales, dense only; the packed
    layout gives each lane 32 consecutive K of its column per 128-K chunk (two 16-byte halves)."""
    for bf in (True, False):
        assert status_of(hq.hq_desc_validate, hq.desc_w8a16(4096, 7168, bf16=bf)) == hq.HQ_OK
    assert status_of(hq.hq_desc_validate, hq.desc_w8a16(4096, 7000)) == hq.HQ_ERR_UNSUPPORTED
    for field, value in (("w_scale_gran", hq.HQ_GRAN_PER_GROUP_K), ("num_experts", 2), ("zp_dtype", hq.HQ_DT_UINT4),
                         ("a_scale", hq.HQ_ASCALE_PER_TOKEN_F32), ("out_dtype", hq.HQ_DT_INT32),
                         ("w_scale_dtype", hq.HQ_DT_BF16)):
        d = hq.desc_w8a16(256, 256)
        setattr(d, field, value)
        assert status_of(hq.hq_desc_validate, d) == hq.HQ_ERR_UNSUPPORTED, field
    N, K = 40, 256
    d = syn.w8a16_int8(0, 1, N, K)
    wp, sp, _ = hq.hq_repack(hq.desc_w8a16(N, K), d["w"], d["s_w"])
    Np = 48
    got = wp.view(np.int8).reshape(Np // 16, K // 128, 2, 64, 16)
    for st in range(Np // 16):
        for c in range(K // 128):
            for h in range(2):
                for lane in range(64):
                    n = 16 * st + (lane & 15)
                    k = 128 * c + 32 * (lane >> 4) + 16 * h + np.arange(16)
                    want = d["w"][k, n] if n < N else np.zeros(16, np.int8)
                    np.testing.assert_array_equal(got[st, c, h, lane], want)
    np.testing.assert_array_equal(sp.view(np.float32)[:N], d["s_w"])
    np.testing.assert_array_equal(sp.view(np.float32)[N:], np.ones(Np - N, np.float32))


def test_fp8_weight_only_descriptor_and_layout():
    """FP8 weight-only takes the INT8 weight-only layout byte for byte."""
    for bf in (True, False):
        assert status_of(hq.hq_desc_validate, hq.desc_fp8w_a16(4096, 7168, bf16=bf)) == hq.HQ_OK
    d = hq.desc_fp8w_a16(256, 256)
    d.w_scale_gran = hq.HQ_GRAN_BLOCK_128x128
    assert status_of(hq.hq_desc_validate, d) == hq.HQ_ERR_UNSUPPORTED
    N, K = 40, 256
    d = syn.w8a16_fp8(0, 1, N, K)
    wf, sf, _ = hq.hq_repack(hq.desc_fp8w_a16(N, K), d["w"], d["s_w"])
    wi, si, _ = hq.hq_repack(hq.desc_w8a16(N, K), d["w"].view(np.int8), d["s_w"])
    np.testing.assert_array_equal(wf, wi)
    np.testing.assert_array_equal(sf, si)


def test_fp8_blockwise_repack_keeps_int8_layout_and_block_scales():
    N, K = 300, 256
    d = syn.w8a8_fp8_blockwise(0, 1, N, K)
    wp, sp, _ = hq.hq_repack(hq.desc_fp8_blockwise(N, K), d["w"], d["s_w"])
    wi, _, _ = hq.hq_repack(hq.desc_w8a8(N, K), d["w"].view(np.int8), np.ones(N, np.float32))
    np.testing.assert_array_equal(wp, wi)
    np.testing.assert_array_equal(sp.view(np.float32).reshape(K // 128, 3), d["s_w"])


def test_gemm_error_paths_return_before_any_hip_call():
    d = hq.desc_w4a16(1024, 7168, zp=True, bf16=False)
    A = w = s = z = D = 0x10000
    # M == 0: nothing to do
    assert status_of(hq.hq_gemm, d, 0, A, None, w, s, z, D, None, 0, 0) == hq.HQ_OK
    assert status_of(hq.hq_gemm, d, -1, A, None, w, s, z, D, None, 0, 0) == hq.HQ_ERR_INVALID_ARG
    assert status_of(hq.hq_gemm, d, 4, None, None, w, s, z, D, None, 0, 0) == hq.HQ_ERR_INVALID_ARG
    assert status_of(hq.hq_gemm, d, 4, A, None, w, s, None, D, None, 0, 0) == hq.HQ_ERR_INVALID_ARG   # zp missing
    assert status_of(hq.hq_gemm, d, 4, A + 2, None, w, s, z, D, None, 0, 0) == hq.HQ_ERR_ALIGNMENT
    need = hq.hq_workspace_bytes(d, 4)
    assert need > 0                                   # K split across workgroups for this shape
    assert status_of(hq.hq_gemm, d, 4, A, None, w, s, z, D, None, 0, 0) == hq.HQ_ERR_WORKSPACE
    assert status_of(hq.hq_gemm, d, 4, A, None, w, s, z, D, 0x20000, need - 16, 0) == hq.HQ_ERR_WORKSPACE
    moe = hq.desc_moe_mxfp4(8, 256, 256)
    assert status_of(hq.hq_gemm, moe, 4, A, None, w, s, None, D, None, 0, 0) == hq.HQ_ERR_INVALID_ARG


# ---------------------------------------------------------------------------
# repack layout
# ---------------------------------------------------------------------------

PAIR = [0, 2, 4, 6, 1, 3, 5, 7]


def unpack_packed_4bit(buf, E, N, K, pair_order):
    """Inverse of the packed 4-bit layout described in include/hq.h -> codes [E, K, N]."""
    Np = (N + 15) // 16 * 16
    words = buf.view(np.uint32).reshape(E, Np // 16, K // 128, 64, 4)
    codes = np.zeros((E, K, Np), dtype=np.uint8)
    for lane in range(64):
        n = np.arange(Np // 16) * 16 + (lane & 15)
        for t in range(4):
            for p in range(8):
                j = PAIR[p] if pair_order else p
                kk = np.arange(K // 128) * 128 + 32 * (lane >> 4) + 8 * t + j
                codes[:, kk[:, None], n[None, :]] = ((words[:, :, :, lane, t] >> (4 * p)) & 15).transpose(0, 2, 1)
    return codes[:, :, :N]


def logical_codes(q, K):
    sh = (4 * np.arange(8, dtype=np.uint32))[None, :, None]
    return ((q[:, None, :] >> sh) & 15).reshape(K, q.shape[1]).astype(np.uint8)


def test_repack_hand_walkthrough_16x128():
    """16 columns x 128 K, code(k, n) = (k + n) % 16; expected words worked out by hand."""
    N, K = 16, 128
    codes = (np.arange(K)[:, None] + np.arange(N)[None, :]) % 16
    q = np.zeros((K // 8, N), dtype=np.uint32)
    for k in range(K):
        q[k // 8] |= (codes[k].astype(np.uint32) << np.uint32(4 * (k % 8)))
    s = np.full((1, N), 0x3F80, dtype=np.uint16)
    wp, sp, _ = hq.hq_repack(hq.desc_w4a16(N, K), q, s)
    words = wp.view(np.uint32).reshape(64, 4)
    # lane 0: column 0, k 0..7 -> codes 0..7 in pair order {0,2,4,6,1,3,5,7}
    assert words[0, 0] == 0x75316420
    # lane 17: column 1, quad 1 -> k 32..39 -> codes 1..8
    assert words[17, 0] == 0x86427531
    # lane 63: column 15, quad 3, word 3 -> k 120..127 -> codes (135..142) % 16 = 7..14
    assert words[63, 3] == 0xECA8DB97
    # MXFP4 keeps natural order: lane 0 word 0 = codes 0..7 in nibbles 0..7
    e = np.full((K // 32, N), 127, dtype=np.uint8)
    wf, ef, _ = hq.hq_repack(hq.desc_w4a8_mxfp4(N, K), q, e)
    assert wf.view(np.uint32)[0] == 0x76543210
    assert ef.size == 64 and np.all(ef == 127)


@pytest.mark.parametrize("N,K,G", [(16, 128, 128), (40, 256, 128), (1000, 512, 256)])
def test_repack_4bit_roundtrip_and_padding(N, K, G):
    d = syn.w4a16_zp(3, 1, N, K, G)
    wp, sp, zp = hq.hq_repack(hq.desc_w4a16(N, K, G, bf16=False, zp=True), d["q"], d["s"], d["z"])
    got = unpack_packed_4bit(wp, 1, N, K, True)[0]
    np.testing.assert_array_equal(got, logical_codes(d["q"], K))
    Np = (N + 15) // 16 * 16
    if Np > N:   # padded columns decode to code 0
        full = unpack_packed_4bit(wp, 1, Np, K, True)
        assert np.all(full[0][:, N:] == 0)
    # scales: [Np/16][K/G][16], padding = fp16 1.0
    s16 = sp.view(np.uint16).reshape(Np // 16, K // G, 16)
    ref = np.full((K // G, Np), 0x3C00, dtype=np.uint16)
    ref[:, :N] = d["s"]
    np.testing.assert_array_equal(s16.transpose(1, 0, 2).reshape(K // G, Np), ref)
    # zeros: [Np/16][K/G] uint64, column 16*strip+i in nibble i
    z64 = zp.view(np.uint64).reshape(Np // 16, K // G)
    zc = ((d["z"][:, :, None] >> (4 * np.arange(8, dtype=np.uint32))[None, None, :]) & 15).reshape(K // G, -1)[:, :N]
    for strip in range(Np // 16):
        for i in range(16):
            n = strip * 16 + i
            exp = zc[:, n] if n < N else np.zeros(K // G, dtype=np.uint32)
            np.testing.assert_array_equal((z64[strip] >> np.uint64(4 * i)) & np.uint64(15), exp.astype(np.uint64))


def test_repack_fp4_int8_e8m0_layouts():
    N, K = 40, 640                                   # 5 chunks; N padded to 48
    d = syn.w4a8_mxfp4(2, 1, N, K)
    wp, ep, _ = hq.hq_repack(hq.desc_w4a8_mxfp4(N, K), d["q"], d["e"])
    np.testing.assert_array_equal(unpack_packed_4bit(wp, 1, N, K, False)[0], logical_codes(d["q"], K))
    e = ep.reshape(3, 5, 64)
    for strip in range(3):
        for lane in range(64):
            for c in range(5):
                n = strip * 16 + (lane & 15)
                exp = d["e"][4 * c + (lane >> 4), n] if n < N else 127
                assert e[strip, c, lane] == exp
    w8 = syn.w8a8_int8(1, 1, 40, 128)
    wp8, sp8, _ = hq.hq_repack(hq.desc_w8a8(40, 128), w8["w"], w8["s_w"])
    b = wp8.view(np.int8).reshape(3, 2, 64, 16)
    for strip in range(3):
        for c in range(2):
            for lane in range(64):
                n = strip * 16 + (lane & 15)
                k = c * 64 + 16 * (lane >> 4) + np.arange(16)
                exp = w8["w"][k, n] if n < 40 else np.zeros(16, np.int8)
                np.testing.assert_array_equal(b[strip, c, lane], exp)
    sw = sp8.view(np.float32)
    np.testing.assert_array_equal(sw[:40], w8["s_w"])
    assert np.all(sw[40:] == 1.0)


def test_repack_moe_expert_stacking():
    E, N, K = 3, 32, 256
    d = syn.moe_mxfp4(0, 2, E, 2, N, K)
    wp, ep, _ = hq.hq_repack(hq.desc_moe_mxfp4(E, N, K), d["q"], d["e"])
    got = unpack_packed_4bit(wp, E, N, K, False)
    for e in range(E):
        np.testing.assert_array_equal(got[e], logical_codes(d["q"][e], K))


def test_repack_rejects_bad_buffers():
    d = hq.desc_w4a16(16, 128, zp=True, bf16=False)
    q = np.zeros((16, 16), np.uint32)
    s = np.zeros((1, 16), np.uint16)
    assert status_of(hq.hq_repack, d, q, s, None) == hq.HQ_ERR_INVALID_ARG


def test_probe_argument_checks_need_no_gpu():
    """The measurement probes reject bad arguments before any device call."""
    with pytest.raises(hq.HQError) as e:
        hq.hq_probe_stream(None, 100, None, 1, stream=0)        # not a multiple of 16
    assert e.value.status == hq.HQ_ERR_INVALID_ARG
    with pytest.raises(hq.HQError) as e:
        hq.hq_probe_stream(None, 1024, None, 1, stream=0)       # no buffers
    assert e.value.status == hq.HQ_ERR_INVALID_ARG
    with pytest.raises(hq.HQError) as e:
        hq.hq_probe_mfma(hq.HQ_DT_FP32, 1, 1, None, stream=0)   # no fp32 probe
    assert e.value.status == hq.HQ_ERR_UNSUPPORTED
    with pytest.raises(hq.HQError) as e:
        hq.hq_probe_mfma(hq.HQ_DT_FP16, 0, 1, None, stream=0)
    assert e.value.status == hq.HQ_ERR_INVALID_ARG


def test_direct_stream_override_rejects_what_it_cannot_take():
    """HQ_TUNE_STREAM8 (eight waves, direct A loads): more than 16 rows, a K split,
    K beyond 64 chunks or 8-bit activations give HQ_ERR_UNSUPPORTED; 16-bit A at
    M <= 16 plans one unsplit launch."""
    from bit_quantized_gemm_w4a16_amd import autotune
    t8 = hq.HQ_TUNE(hq.HQ_TUNE_STREAM8, 0)
    desc = hq.desc_w4a16(4096, 7168, 128, bf16=False, zp=True)
    plan = hq.hq_gemm_plan(autotune.with_tune(desc, t8), 8)
    assert len(plan) == 1 and ",direct>" in plan[0] and "splits=1" in plan[0]
    for d, M in ((autotune.with_tune(desc, t8), 17), (autotune.with_tune(desc, hq.HQ_TUNE(hq.HQ_TUNE_STREAM8, 2)), 8),
                 (autotune.with_tune(hq.desc_w4a16(4096, 8320, 128, bf16=False, zp=True), t8), 8),
                 (autotune.with_tune(hq.desc_w4a8_mxfp4(7168, 4096), t8), 8)):
        with pytest.raises(hq.HQError):
            hq.hq_gemm_plan(d, M)
    bad = hq.hq_layer_desc.from_buffer_copy(desc)
    bad.tune = 7
    with pytest.raises(hq.HQError):
        hq.hq_gemm_plan(bad, 8)
