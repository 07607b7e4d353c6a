"""Host-side tests of the low-bit WnA16 weights (INT1/2/3, UINT1/2/3; no GPU):
descriptor validation, the two-plane packed layout, the code-range check of the
repack and the launch plans.

The planes are decoded here from the layout hq.h states (bit positions of the
2-bit and 1-bit planes over the 4-bit word order) and compared with the 4-bit
repack of the same codes (the INT4/UINT4 container), whose layout the hand
walkthrough in test_abi pins."""
import numpy as np
import pytest

import synthetic as syn
from bit_quantized_gemm_w4a16_amd import autotune, hq

WIDTHS = [(b, sg) for b in (1, 2, 3) for sg in (True, False)]


def nibble_words(codes, K, N):
    """Codes [K][N] (int8) -> the 4-bit logical input uint32 [K/8][N] (two's-
    complement nibble for negative codes)."""
    nib = (codes.astype(np.int64) & 15).astype(np.uint32)
    q = np.zeros((K // 8, N), dtype=np.uint32)
    for i in range(8):
        q |= nib[i::8] << np.uint32(4 * i)
    return q


def planes_to_codes(wp, bits, signed, Np, K):
    """Decode the packed planes into the codes [slots][4 sub-steps][8] (int),
    from the bit positions hq.h states."""
    slots = (Np // 16) * (K // 128) * 64
    two, one = bits >= 2, bits != 2
    off = slots * 8 if two else 0
    assert wp.size == (slots * 8 if two else 0) + (slots * 4 if one else 0)
    x = wp[:off].view(np.uint32).reshape(slots, 2).astype(np.int64) if two else None
    y = wp[off:].view(np.uint32).reshape(slots).astype(np.int64) if one else None
    out = np.zeros((slots, 4, 8), dtype=np.int64)
    for t in range(4):
        for j in range(8):
            v = 0
            if two:
                v = (x[:, t >> 1] >> (16 * (j & 1) + 8 * (t & 1) + 2 * (j >> 1))) & 3
            if one:
                bit = (y >> (16 * (j & 1) + 4 * t + (j >> 1))) & 1
                v = v | (bit << (0 if bits == 1 else 2))
            if signed:
                v = np.where(v >> (bits - 1) & 1, v - (1 << bits), v)
            out[:, t, j] = v
    return out


def codes_of_4bit_words(w4, signed, Np, K):
    """The packed 4-bit pair-order words [slots][4] -> codes [slots][4][8]."""
    slots = (Np // 16) * (K // 128) * 64
    words = w4.view(np.uint32).reshape(slots, 4).astype(np.int64)
    out = np.zeros((slots, 4, 8), dtype=np.int64)
    for p, j in enumerate((0, 2, 4, 6, 1, 3, 5, 7)):
        v = (words >> (4 * p)) & 15
        out[:, :, j] = np.where(v >= 8, v - 16, v) if signed else v
    return out


@pytest.mark.parametrize("bits,signed", WIDTHS)
def test_descriptor_validation(bits, signed):
    d = hq.desc_wnlow(4096, 1024, bits, signed)
    hq.hq_desc_validate(d)
    hq.hq_desc_validate(hq.desc_wnlow(40, 512, bits, signed, group_size=256, bf16=False))
    bad = hq.hq_layer_desc.from_buffer_copy(d)
    bad.zp_dtype = hq.HQ_DT_UINT4 if signed else hq.HQ_DT_NONE   # signed take none, unsigned need UINT4
    with pytest.raises(hq.HQError):
        hq.hq_desc_validate(bad)
    bad = hq.hq_layer_desc.from_buffer_copy(d)
    bad.group_size = 64
    with pytest.raises(hq.HQError):
        hq.hq_desc_validate(bad)
    bad = hq.hq_layer_desc.from_buffer_copy(d)
    bad.num_experts = 4
    with pytest.raises(hq.HQError):
        hq.hq_desc_validate(bad)


@pytest.mark.parametrize("bits,signed", WIDTHS)
@pytest.mark.parametrize("N,K,G", [(16, 128, 128), (40, 384, 128), (1000, 512, 256)])
def test_planes_decode_to_the_4bit_layout_of_the_same_codes(bits, signed, N, K, G):
    d = syn.wnlow(5 + bits, 1, N, K, bits, signed, G=G)
    desc = hq.desc_wnlow(N, K, bits, signed, group_size=G, bf16=False)
    wb, sb, zb, _ = hq.hq_repacked_bytes(desc)
    Np = (N + 15) // 16 * 16
    slots = (Np // 16) * (K // 128) * 64
    assert wb == (slots * 8 if bits >= 2 else 0) + (slots * 4 if bits != 2 else 0)
    wp, sp, zp = hq.hq_repack(desc, d["codes"], d["s"], d.get("z"))
    d4 = hq.desc_w4a16(N, K, G, bf16=False, zp=not signed)
    w4, s4, z4 = hq.hq_repack(d4, nibble_words(d["codes"], K, N), d["s"], d.get("z"))
    np.testing.assert_array_equal(planes_to_codes(wp, bits, signed, Np, K), codes_of_4bit_words(w4, signed, Np, K))
    np.testing.assert_array_equal(sp, s4)
    if signed:
        assert zp is None and zb == 0
    else:
        np.testing.assert_array_equal(zp, z4)


def test_plane_hand_walkthrough_3bit():
    """16 columns x 128 K of UINT3, code(k, n) = (k + n) % 8.  Lane 0 (column 0,
    k = 0..31): sub-step 0 holds codes 0..7, sub-step 1 codes 0..7 again.  2-bit
    word 0: evens j = 0,2,4,6 of t = 0 (low bits 0,2,0,2) in bits 0-7, the same
    for t = 1 in bits 8-15, odds j = 1,3,5,7 (low bits 1,3,1,3) in bits 16-23 and
    24-31: bytes 0x88, 0x88, 0xDD, 0xDD.  1-bit word: bit 2 of the evens (codes
    0,2,4,6 -> 0,0,1,1) at bits 4t + 0..3 = 0b1100 per t, of the odds (1,3,5,7
    -> 0,0,1,1) at 16 + 4t + 0..3: 0xCCCC in each half."""
    N, K = 16, 128
    codes = ((np.arange(K)[:, None] + np.arange(N)[None, :]) % 8).astype(np.int8)
    s = np.full((1, N), 0x3C00, dtype=np.uint16)
    z = np.zeros((1, 2), dtype=np.uint32)
    wp, _, _ = hq.hq_repack(hq.desc_wnlow(N, K, 3, False, bf16=False), codes, s, z)
    x = wp[:64 * 8].view(np.uint32).reshape(64, 2)
    y = wp[64 * 8:].view(np.uint32)
    assert x[0, 0] == 0xDDDD8888 and x[0, 1] == 0xDDDD8888 and y[0] == 0xCCCCCCCC
    # lane 17: column 1, k = 32..63 -> sub-step t holds codes (1 + j) % 8:
    # evens j=0,2,4,6 -> 1,3,5,7 (low bits 1,3,1,3; bit 2: 0,0,1,1),
    # odds j=1,3,5,7 -> 2,4,6,0 (low bits 2,0,2,0; bit 2: 0,1,1,0)
    ev = sum(v << (2 * s) for s, v in enumerate([1, 3, 1, 3]))
    od = sum(v << (2 * s) for s, v in enumerate([2, 0, 2, 0]))
    assert x[17, 0] == ev | ev << 8 | od << 16 | od << 24
    hb_e = sum(v << s for s, v in enumerate([0, 0, 1, 1]))
    hb_o = sum(v << s for s, v in enumerate([0, 1, 1, 0]))
    assert y[17] == sum(hb_e << 4 * t | hb_o << (16 + 4 * t) for t in range(4))


@pytest.mark.parametrize("bits,signed", WIDTHS)
def test_repack_rejects_codes_outside_the_width(bits, signed):
    N, K = 32, 256
    d = syn.wnlow(1, 1, N, K, bits, signed)
    desc = hq.desc_wnlow(N, K, bits, signed)
    hi = (1 << (bits - 1)) if signed else (1 << bits)        # one past the top
    lo = -(1 << (bits - 1)) - 1 if signed else -1            # one below the bottom (-1 = 255 unsigned)
    for bad_code in (hi, lo):
        c = d["codes"].copy()
        c[K - 1, N - 1] = bad_code
        with pytest.raises(hq.HQError) as e:
            hq.hq_repack(desc, c, d["s"], d.get("z"))
        assert e.value.status == hq.HQ_ERR_INVALID_ARG


@pytest.mark.parametrize("bits", [1, 2, 3])
def test_plans_stream_natively_and_widen_for_the_tiles(bits):
    N, K = 4096, 4096
    desc = hq.desc_wnlow(N, K, bits, bits != 2, bf16=True)
    small = hq.hq_gemm_plan(desc, 4)
    assert f",w{bits}>" in small[0] and not any("widen" in p for p in small)
    big = hq.hq_gemm_plan(desc, 1024)
    assert big[0].startswith(f"widen_lowbit_kernel<{bits}>") and "tile_gemm_kernel" in big[1]
    wide = (N // 16) * (K // 128) * 1024
    assert hq.hq_workspace_bytes(desc, 1024) >= wide
    assert hq.hq_workspace_bytes(desc, 4) < wide
    # split tiles: the partial tiles follow the widened weights
    mid = hq.hq_gemm_plan(desc, 128)
    if "splits=1" not in mid[1]:
        sp = int(mid[1].split("splits=")[1].split()[0])
        assert hq.hq_workspace_bytes(desc, 128) >= ((wide + 255) // 256 * 256) + sp * 128 * N * 4
    with pytest.raises(hq.HQError):
        hq.hq_gemm_plan(autotune.with_tune(desc, hq.HQ_TUNE(hq.HQ_TUNE_STREAM8, 0)), 4)
