"""Host-side tests of the MX float weight formats (MXFP8 E4M3, MXFP6 E2M3 / E3M2
with E8M0 per 32 K, bf16 activations; no GPU): descriptor validation, the
packed layouts, the code-range check of the repack and the launch plans.

The FP6 planes are decoded here from the layout hq.h states (a 192-bit group
per lane and chunk, code j at bits 6j..6j+5) and compared with the logical
codes; the E4M3 weights must take the INT8 weight-only layout byte for byte
and the E8M0 scales the MXFP4 scale layout."""
import numpy as np
import pytest

import synthetic as syn
from bit_quantized_gemm_w4a16_amd import autotune, hq

ELEMS = ["e4m3", "e2m3", "e3m2"]


def fp6_planes_to_codes(wp, N, K):
    """Packed FP6 planes -> logical codes [K][N] (padding columns dropped)."""
    Np = (N + 15) // 16 * 16
    nst, nc = Np // 16, K // 128
    slots = nst * nc * 64
    assert wp.size == slots * 24
    a = wp[:slots * 16].view(np.uint32).reshape(slots, 4).astype(np.uint64)
    b = wp[slots * 16:].view(np.uint32).reshape(slots, 2).astype(np.uint64)
    words = np.concatenate([a, b], axis=1)                     # [slots][6]
    codes = np.zeros((K, Np), dtype=np.uint8)
    for st in range(nst):
        for c in range(nc):
            for lane in range(64):
                slot = (st * nc + c) * 64 + lane
                big = 0
                for d in range(6):
                    big |= int(words[slot, d]) << (32 * d)
                n = st * 16 + (lane & 15)
                for j in range(32):
                    codes[c * 128 + 32 * (lane >> 4) + j, n] = (big >> (6 * j)) & 63
    return codes[:, :N], codes[:, N:]


@pytest.mark.parametrize("elem", ELEMS)
def test_descriptor_validation(elem):
    d = hq.desc_mxf_a16(4096, 1024, elem)
    hq.hq_desc_validate(d)
    for field, value in (("group_size", 64), ("w_scale_gran", hq.HQ_GRAN_PER_CHANNEL), ("out_dtype", hq.HQ_DT_FP16),
                         ("zp_dtype", hq.HQ_DT_UINT4), ("num_experts", 4), ("a_scale", hq.HQ_ASCALE_PER_TOKEN_F32),
                         ("K", 1000)):
        bad = hq.hq_layer_desc.from_buffer_copy(d)
        setattr(bad, field, value)
        with pytest.raises(hq.HQError):
            hq.hq_desc_validate(bad)
    if elem != "e4m3":   # FP6 only with E8M0 scales (E4M3 with fp32 per-channel scales is FP8 weight-only)
        bad = hq.hq_layer_desc.from_buffer_copy(d)
        bad.w_scale_dtype, bad.w_scale_gran, bad.group_size = hq.HQ_DT_FP32, hq.HQ_GRAN_PER_CHANNEL, 1024
        with pytest.raises(hq.HQError):
            hq.hq_desc_validate(bad)


@pytest.mark.parametrize("elem", ["e2m3", "e3m2"])
@pytest.mark.parametrize("N,K", [(16, 128), (40, 384), (1000, 256)])
def test_fp6_planes_hold_the_codes(elem, N, K):
    d = syn.mxf_a16(4, 1, N, K, elem)
    wp, sp, zp = hq.hq_repack(hq.desc_mxf_a16(N, K, elem), d["codes"], d["e"])
    got, pad = fp6_planes_to_codes(wp, N, K)
    np.testing.assert_array_equal(got, d["codes"])
    assert np.all(pad == 0) and zp is None
    # E8M0 scales: the MXFP4 scale layout, byte for byte
    _, s4, _ = hq.hq_repack(hq.desc_fp4_a16(N, K, False), np.zeros((K // 8, N), np.uint32), d["e"])
    np.testing.assert_array_equal(sp, s4)


def test_fp6_hand_walkthrough():
    """One strip, one chunk: lane 0 holds codes 0..31 of column 0, code j = j,
    so its 192-bit group is the sum of j << 6j: the first dword holds codes 0-4
    whole and the low two bits of code 5, the 8-byte plane the last 64 bits."""
    N, K = 16, 128
    codes = np.zeros((K, N), np.uint8)
    codes[:32, 0] = np.arange(32)
    e = np.full((K // 32, N), 127, np.uint8)
    wp, _, _ = hq.hq_repack(hq.desc_mxf_a16(N, K, "e2m3"), codes, e)
    big = sum(j << (6 * j) for j in range(32))
    words = [(big >> (32 * d)) & 0xFFFFFFFF for d in range(6)]
    assert words[0] == (0 | 1 << 6 | 2 << 12 | 3 << 18 | 4 << 24 | (5 & 3) << 30)
    np.testing.assert_array_equal(wp[:16].view(np.uint32), words[:4])
    np.testing.assert_array_equal(wp[64 * 16:64 * 16 + 8].view(np.uint32), words[4:])


@pytest.mark.parametrize("N,K", [(40, 384), (1000, 256)])
def test_e4m3_takes_the_8bit_weight_only_layout(N, K):
    d = syn.mxf_a16(5, 1, N, K, "e4m3")
    wp, sp, _ = hq.hq_repack(hq.desc_mxf_a16(N, K, "e4m3"), d["codes"], d["e"])
    w8, _, _ = hq.hq_repack(hq.desc_fp8w_a16(N, K, bf16=True), d["codes"], np.ones(N, np.float32))
    np.testing.assert_array_equal(wp, w8)
    _, s4, _ = hq.hq_repack(hq.desc_fp4_a16(N, K, False), np.zeros((K // 8, N), np.uint32), d["e"])
    np.testing.assert_array_equal(sp, s4)


@pytest.mark.parametrize("elem", ["e2m3", "e3m2"])
def test_repack_rejects_codes_above_six_bits(elem):
    N, K = 32, 256
    d = syn.mxf_a16(1, 1, N, K, elem)
    for v in (64, 128, 255):
        c = d["codes"].copy()
        c[K - 1, N - 1] = v
        with pytest.raises(hq.HQError) as e:
            hq.hq_repack(hq.desc_mxf_a16(N, K, elem), c, d["e"])
        assert e.value.status == hq.HQ_ERR_INVALID_ARG


@pytest.mark.parametrize("elem", ELEMS)
def test_plans(elem):
    N, K = 4096, 4096
    desc = hq.desc_mxf_a16(N, K, elem)
    small = hq.hq_gemm_plan(desc, 1)
    assert len(small) == 1 and small[0].startswith("skinny_kernel<MXF")
    big = hq.hq_gemm_plan(desc, 2048)
    if elem == "e4m3":
        assert big[0].startswith("tile_gemm_kernel<MXF8_BF16,")
    else:
        # FP6 on the tiles: widened to E4M3 in the workspace, then the MXFP8 tiles
        assert big[0].startswith(f"widen_fp6_kernel<{elem}>") and big[1].startswith("tile_gemm_kernel<MXF8_BF16,")
        assert hq.hq_workspace_bytes(desc, 2048) >= (N // 16) * (K // 128) * 2048
    # the direct stream takes these formats; every tuning override plans
    assert len(hq.hq_gemm_plan(autotune.with_tune(desc, hq.HQ_TUNE(hq.HQ_TUNE_STREAM8, 0)), 8)) == 1
