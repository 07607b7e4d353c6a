"""Pins for the CPU oracle (no GPU).

Each test ties an oracle function to something other than itself: the OCP
format tables (tests/golden), PyTorch's own fp8/bf16/fp16 conversions, exact
rational arithmetic, numpy's int64/fp64 matmul, closed forms and invariants
of the GEMM.  A dropped term, a wrong sign, a swapped index or a transposed
operand in the oracle fails at least one of them.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from conftest import golden


# ---------------------------------------------------------------------------
# helpers that decode the documented logical layouts (test-side, table based)
# ---------------------------------------------------------------------------

E2M1_TABLE = dict(golden("e2m1_ocp_mx_v1.txt"))


def unpack_k(q, K):
    """uint32 [K/8, N] -> nibble codes [K, N] (code k=8j+i in bits 4i of word j)."""
    sh = (4 * np.arange(8, dtype=np.uint32))[None, :, None]
    return ((q[:, None, :] >> sh) & 15).reshape(K, q.shape[1]).astype(np.int64)


def unpack_n(z, N):
    sh = (4 * np.arange(8, dtype=np.uint32))[None, None, :]
    return ((z[:, :, None] >> sh) & 15).reshape(z.shape[0], -1)[:, :N].astype(np.int64)


def torch16(bits, dt):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(dt).to(torch.float64).numpy()


def e2m1_tab(codes):
    lut = np.array([E2M1_TABLE[c] for c in range(16)])
    return lut[codes]


def rel_err(x, ref):
    scale = max(np.abs(ref).max(), 1e-300)
    return np.abs(x - ref).max() / scale


# ---------------------------------------------------------------------------
# scalar formats
# ---------------------------------------------------------------------------

def test_e2m1_matches_ocp_table():
    for code, v in golden("e2m1_ocp_mx_v1.txt"):
        got = oracle.e2m1(code)
        assert got == v and math.copysign(1, got) == math.copysign(1, v), code


def test_e8m0_matches_ocp_values_and_doubles():
    for code, v in golden("e8m0_ocp_mx_v1.txt"):
        got = oracle.e8m0(code)
        assert (math.isnan(v) and math.isnan(got)) or got == v, code
    for e in range(0, 254):
        assert oracle.e8m0(e + 1) == 2 * oracle.e8m0(e)


def test_e4m3_decode_matches_ocp_and_torch_exhaustive():
    for code, v in golden("e4m3_ocp_ofp8.txt"):
        got = oracle.e4m3(code)
        assert (math.isnan(v) and math.isnan(got)) or (got == v and math.copysign(1, got) == math.copysign(1, v)), hex(code)
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        got = oracle.e4m3(c)
        assert (math.isnan(ref[c]) and math.isnan(got)) or got == ref[c], hex(c)


def test_e4m3_encode_roundtrip_saturation_ties():
    for c in range(256):
        v = oracle.e4m3(c)
        if math.isnan(v):
            continue
        assert oracle.e4m3_encode(v) == c, hex(c)
    assert oracle.e4m3_encode(449.0) == 0x7E
    assert oracle.e4m3_encode(1e30) == 0x7E
    assert oracle.e4m3_encode(-1e30) == 0xFE
    assert oracle.e4m3_encode(1.0625) == 0x38          # tie between 1.0 and 1.125 -> even (1.0)
    assert oracle.e4m3_encode(1.1875) == 0x3A          # tie between 1.125 and 1.25 -> even (1.25)
    assert oracle.e4m3_encode(2.0 ** -10) == 0x00      # tie between 0 and 2^-9 -> even (0)
    assert oracle.e4m3_encode(3 * 2.0 ** -10) == 0x02  # tie between 2^-9 and 2^-8 -> even


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 100,
                        rng.standard_normal(5000).astype(np.float32) * 0.01,
                        np.float32(448.0) * (rng.random(2000).astype(np.float32) * 2 - 1)])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ok = np.abs(x) <= 448
    got = np.array([oracle.e4m3_encode(float(v)) for v in x[ok]], dtype=np.uint8)
    np.testing.assert_array_equal(got, ref[ok])


def test_bf16_fp16_decode_match_torch_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    for fn, dt in ((oracle.bf16, torch.bfloat16), (oracle.fp16, torch.float16)):
        ref = torch16(bits, dt)
        for b in range(0, 65536, 7):
            got = fn(b)
            assert (math.isnan(ref[b]) and math.isnan(got)) or got == ref[b], (dt, b)


# ---------------------------------------------------------------------------
# W4A16
# ---------------------------------------------------------------------------

def exact_wna16(A, q, s, z, N, K, G, a_dt, w_signed):
    """Exact rational result with table/torch decoding (tiny shapes only)."""
    a = torch16(A, a_dt)
    sc = torch16(s, a_dt)
    codes = unpack_k(q, K)
    if w_signed:
        codes = np.where(codes >= 8, codes - 16, codes)
        zz = np.zeros((K // G, N), dtype=np.int64)
    else:
        zz = unpack_n(z, N) if z is not None else np.zeros((K // G, N), dtype=np.int64)
    M = a.shape[0]
    out = np.empty((M, N))
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                g = k // G
                acc += Fraction(float(a[m, k])) * (int(codes[k, n]) - int(zz[g, n])) * Fraction(float(sc[g, n]))
            out[m, n] = float(acc)
    return out


@pytest.mark.parametrize("M,N,K,G", [(1, 16, 128, 128), (2, 16, 256, 128), (3, 32, 256, 128), (2, 24, 256, 64)])
@pytest.mark.parametrize("variant", ["sym_bf16", "zp_fp16"])
def test_wna16_matches_exact_rational(M, N, K, G, variant):
    if variant == "sym_bf16":
        d = syn.w4a16_sym(7, M, N, K, G, torch.bfloat16)
        z, a_dt, signed = None, torch.bfloat16, True
    else:
        d = syn.w4a16_zp(7, M, N, K, G, torch.float16)
        z, a_dt, signed = d["z"], torch.float16, False
    got = oracle.gemm_wna16(d["A"], d["q"], d["s"], z, N=N, K=K, G=G, a_bf16=a_dt is torch.bfloat16, w_signed=signed)
    ref = exact_wna16(d["A"], d["q"], d["s"], z, N, K, G, a_dt, signed)
    assert rel_err(got, ref) < 1e-13


def test_wna16_single_weight_placement():
    """Hand-placed code: only column 17 sees code 5 at k=133 (word 16, nibble 5)."""
    M, N, K, G = 3, 24, 256, 128
    A = syn.activations(3, 9, M, K, torch.bfloat16)
    q = np.zeros((K // 8, N), dtype=np.uint32)
    q[133 // 8, 17] = np.uint32(5) << np.uint32(4 * (133 % 8))
    s = syn.abs_normal_scales(3, 9, 3, (K // G, N), 0.02, 1e-3, torch.bfloat16)
    got = oracle.gemm_wna16(A, q, s, None, N=N, K=K, G=G, a_bf16=True, w_signed=True)
    a = torch16(A, torch.bfloat16)
    sc = torch16(s, torch.bfloat16)
    ref = np.zeros((M, N))
    ref[:, 17] = a[:, 133] * 5 * sc[1, 17]
    np.testing.assert_array_equal(got, ref)
    # the same code placed as a zero-point-shifted UINT4 value: (5 - z) with z at column 17 of group 1
    z = np.zeros((K // G, 3), dtype=np.uint32)
    z[1, 2] = np.uint32(3) << np.uint32(4 * 1)        # column 17 = word 2, nibble 1
    got = oracle.gemm_wna16(A, q, s, z, N=N, K=K, G=G, a_bf16=True, w_signed=False)
    ref2 = np.zeros((M, N))
    ref2[:, 17] = a[:, 133] * 5 * sc[1, 17] - 3 * sc[1, 17] * a[:, 128:256].sum(axis=1)
    assert rel_err(got, ref2) < 1e-13


@pytest.mark.parametrize("code", [0, 3, 7, 8, 15])
def test_wna16_constant_code_closed_form(code):
    M, N, K, G = 4, 32, 512, 128
    A = syn.activations(5, 2, M, K, torch.float16)
    q = np.full((K // 8, N), sum(code << (4 * i) for i in range(8)), dtype=np.uint32)
    s = np.full((K // G, N), np.float16(0.03125).view(np.uint16), dtype=np.uint16)
    got = oracle.gemm_wna16(A, q, s, None, N=N, K=K, G=G, a_bf16=False, w_signed=True)
    val = code - 16 if code >= 8 else code
    rowsum = torch16(A, torch.float16).sum(axis=1)
    np.testing.assert_allclose(got, np.repeat((val * 0.03125 * rowsum)[:, None], N, axis=1), rtol=1e-14, atol=0)


def test_wna16_zero_point_invariants():
    M, N, K, G = 3, 40, 256, 128
    d = syn.w4a16_zp(11, M, N, K, G, torch.float16)
    # q == z everywhere -> exactly zero
    zcodes = unpack_n(d["z"], N)
    qz = np.zeros((K // 8, N), dtype=np.uint32)
    for k in range(K):
        qz[k // 8] |= (zcodes[k // G].astype(np.uint32) << np.uint32(4 * (k % 8)))
    got = oracle.gemm_wna16(d["A"], qz, d["s"], d["z"], N=N, K=K, G=G, a_bf16=False, w_signed=False)
    assert np.all(got == 0.0)
    # UINT4 with z == 8 is bit-identical to signed INT4 with code (q - 8) = q ^ 8
    z8 = np.full((K // G, (N + 7) // 8), 0x88888888, dtype=np.uint32)
    o1 = oracle.gemm_wna16(d["A"], d["q"], d["s"], z8, N=N, K=K, G=G, a_bf16=False, w_signed=False)
    o2 = oracle.gemm_wna16(d["A"], d["q"] ^ np.uint32(0x88888888), d["s"], None, N=N, K=K, G=G, a_bf16=False, w_signed=True)
    np.testing.assert_array_equal(o1, o2)


def test_wna16_unit_scales_equal_numpy_matmul():
    M, N, K, G = 5, 48, 384, 128
    d = syn.w4a16_sym(2, M, N, K, G, torch.bfloat16)
    ones = np.full((K // G, N), 0x3F80, dtype=np.uint16)      # bf16 1.0
    got = oracle.gemm_wna16(d["A"], d["q"], ones, None, N=N, K=K, G=G, a_bf16=True, w_signed=True)
    codes = unpack_k(d["q"], K)
    w = np.where(codes >= 8, codes - 16, codes).astype(np.float64)
    ref = torch16(d["A"], torch.bfloat16) @ w
    assert rel_err(got, ref) < 1e-13


def test_wna16_group_scale_linearity():
    M, N, K, G = 2, 32, 512, 128
    d = syn.w4a16_sym(4, M, N, K, G, torch.bfloat16)
    base = oracle.gemm_wna16(d["A"], d["q"], d["s"], None, N=N, K=K, G=G, a_bf16=True, w_signed=True)
    s2 = d["s"].copy()
    s2[2] = np.full(N, 0x4000, dtype=np.uint16)                # bf16 2.0 for group 2 only
    moved = oracle.gemm_wna16(d["A"], d["q"], s2, None, N=N, K=K, G=G, a_bf16=True, w_signed=True)
    codes = unpack_k(d["q"], K)
    w = np.where(codes >= 8, codes - 16, codes).astype(np.float64)[2 * G:3 * G]
    ds = 2.0 - torch16(d["s"], torch.bfloat16)[2]
    delta = torch16(d["A"], torch.bfloat16)[:, 2 * G:3 * G] @ (w * ds[None, :])
    assert rel_err(moved - base, delta) < 1e-12


def test_wna16_row_subset_equals_full():
    M, N, K, G = 9, 32, 256, 128
    d = syn.w4a16_zp(6, M, N, K, G, torch.float16)
    full = oracle.gemm_wna16(d["A"], d["q"], d["s"], d["z"], N=N, K=K, G=G, a_bf16=False, w_signed=False)
    rows = np.array([8, 0, 5])
    sub = oracle.gemm_wna16(d["A"], d["q"], d["s"], d["z"], N=N, K=K, G=G, a_bf16=False, w_signed=False, rows=rows)
    np.testing.assert_array_equal(sub, full[rows])


# ---------------------------------------------------------------------------
# W4A8-MXFP4
# ---------------------------------------------------------------------------

def test_quant_act_e4m3_matches_torch_cast():
    x = syn.normal_rows(0, 3, syn.T_A, 70, 512)
    x[3] = 0.0
    q, s = oracle.quant_act_e4m3(x)
    amax = np.abs(x).max(axis=1)
    exp_s = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    np.testing.assert_array_equal(s, exp_s)
    ref = torch.from_numpy(x / exp_s[:, None]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(q, ref)
    am = np.abs(x).argmax(axis=1)
    for m in range(70):
        if m != 3:
            assert q[m, am[m]] & 0x7F == 0x7E


def mx_dense_ref(qa, s_a, q, e, K):
    a = np.array([oracle.e4m3(c) for c in range(256)])[qa.astype(np.int64)]
    w = e2m1_tab(unpack_k(q, K)) * (2.0 ** (np.repeat(e.astype(np.int64), 32, axis=0) - 127))
    return (a @ w) * s_a.astype(np.float64)[:, None]


def test_w4a8_matches_table_decoded_matmul():
    M, N, K = 6, 48, 512
    d = syn.w4a8_mxfp4(1, M, N, K)
    qa, s_a = oracle.quant_act_e4m3(d["A0"])
    got = oracle.gemm_w4a8_mxfp4(qa, s_a, d["q"], d["e"], N=N, K=K)
    assert rel_err(got, mx_dense_ref(qa, s_a, d["q"], d["e"], K)) < 1e-13


def test_w4a8_exact_rational_tiny():
    M, N, K = 2, 16, 64
    d = syn.w4a8_mxfp4(2, M, N, K)
    qa, s_a = oracle.quant_act_e4m3(d["A0"])
    got = oracle.gemm_w4a8_mxfp4(qa, s_a, d["q"], d["e"], N=N, K=K)
    codes = unpack_k(d["q"], K)
    e4 = torch.from_numpy(qa).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += Fraction(float(e4[m, k])) * Fraction(E2M1_TABLE[int(codes[k, n])]) * Fraction(2) ** (int(d["e"][k // 32, n]) - 127)
            assert abs(got[m, n] - float(acc * Fraction(float(s_a[m])))) <= 1e-13 * max(abs(float(acc)), 1e-30)


def test_w4a8_constant_code_sign_flip_and_exponent_step():
    M, N, K = 3, 32, 256
    d = syn.w4a8_mxfp4(3, M, N, K)
    qa, s_a = oracle.quant_act_e4m3(d["A0"])
    ones = np.full((K // 8, N), 0x22222222, dtype=np.uint32)       # e2m1 code 0x2 == 1.0
    e127 = np.full((K // 32, N), 127, dtype=np.uint8)
    got = oracle.gemm_w4a8_mxfp4(qa, s_a, ones, e127, N=N, K=K)
    a = torch.from_numpy(qa).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_allclose(got, np.repeat((a.sum(axis=1) * s_a)[:, None], N, axis=1), rtol=1e-14)
    base = oracle.gemm_w4a8_mxfp4(qa, s_a, d["q"], d["e"], N=N, K=K)
    neg = oracle.gemm_w4a8_mxfp4(qa, s_a, d["q"] ^ np.uint32(0x88888888), d["e"], N=N, K=K)
    np.testing.assert_array_equal(neg, -base)
    e2 = d["e"].copy()
    e2[3] += 1                                                     # block k in [96, 128) doubles
    moved = oracle.gemm_w4a8_mxfp4(qa, s_a, d["q"], e2, N=N, K=K)
    blk = np.zeros_like(d["q"])
    blk[12:16] = d["q"][12:16]
    e_blk = oracle.gemm_w4a8_mxfp4(qa, s_a, blk, d["e"], N=N, K=K)
    assert rel_err(moved - base, e_blk) < 1e-12


# ---------------------------------------------------------------------------
# W8A8
# ---------------------------------------------------------------------------

def test_w8a8_int_exact_and_epilogue():
    M, N, K = 7, 64, 1024
    d = syn.w8a8_int8(0, M, N, K)
    acc, out = oracle.gemm_w8a8(d["a"], d["s_a"], d["w"], d["s_w"])
    ref = d["a"].astype(np.int64) @ d["w"].astype(np.int64)
    np.testing.assert_array_equal(acc, ref)
    np.testing.assert_array_equal(out, ref * d["s_a"].astype(np.float64)[:, None] * d["s_w"].astype(np.float64)[None, :])


def test_w8a8_extremes_fit_int32_and_e0m7_reading():
    # all codes at +-127: |acc| = 127^2 * K fits in int32 for K = 7168 (e0m7 reads the same -127..127 integers)
    K, N = 7168, 16
    a = np.full((2, K), 127, dtype=np.int8)
    a[1] = -127
    w = np.full((K, N), 127, dtype=np.int8)
    acc, _ = oracle.gemm_w8a8(a, np.ones(2, np.float32), w, np.ones(N, np.float32))
    assert acc[0, 0] == 127 * 127 * K and acc[1, 0] == -127 * 127 * K
    with pytest.raises(OverflowError):
        oracle.gemm_w8a8(np.full((1, 140000), 127, np.int8), np.ones(1, np.float32),
                         np.full((140000, 1), 127, np.int8), np.ones(1, np.float32))


# ---------------------------------------------------------------------------
# MoE
# ---------------------------------------------------------------------------

def test_moe_route_matches_stable_argsort():
    ids = syn.zipf_topk(0, 5, 300, 16, 4)
    counts, offsets, perm = oracle.moe_route(ids, 16)
    flat = ids.reshape(-1)
    np.testing.assert_array_equal(counts, np.bincount(flat, minlength=16))
    np.testing.assert_array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
    np.testing.assert_array_equal(perm, np.argsort(flat, kind="stable"))
    assert all(len(set(r)) == 4 for r in ids)


def test_moe_single_expert_top1_equals_dense_table_matmul():
    T, E, N, K = 5, 1, 32, 256
    d = syn.moe_mxfp4(0, T, E, 1, N, K)
    got = oracle.moe_mxfp4_bf16(d["A"], d["ids"], d["q"], d["e"], N=N, K=K)
    w = e2m1_tab(unpack_k(d["q"][0], K)) * (2.0 ** (np.repeat(d["e"][0].astype(np.int64), 32, axis=0) - 127))
    ref = torch16(d["A"], torch.bfloat16) @ w
    assert rel_err(got, ref) < 1e-13


def test_moe_pairs_are_per_expert_dense_and_indexed_grouped_agree():
    T, E, top_k, N, K = 7, 6, 3, 32, 128
    d = syn.moe_mxfp4(1, T, E, top_k, N, K)
    full = oracle.moe_mxfp4_bf16(d["A"], d["ids"], d["q"], d["e"], N=N, K=K)
    a = torch16(d["A"], torch.bfloat16)
    for p in range(T * top_k):
        t, e = p // top_k, d["ids"].reshape(-1)[p]
        w = e2m1_tab(unpack_k(d["q"][e], K)) * (2.0 ** (np.repeat(d["e"][e].astype(np.int64), 32, axis=0) - 127))
        assert rel_err(full[p], a[t] @ w) < 1e-13
    _, _, perm = oracle.moe_route(d["ids"], E)
    grouped = oracle.moe_mxfp4_bf16(d["A"], d["ids"], d["q"], d["e"], N=N, K=K, pairs=perm)
    np.testing.assert_array_equal(grouped, full[perm])


# ---------------------------------------------------------------------------
# SwiGLU between the MoE projections: bf16 rounding and silu
# ---------------------------------------------------------------------------

def test_bf16_encode_special_cases():
    cases = {
        1.0: 0x3F80, -2.5: 0xC020, 0.0: 0x0000,
        1 + 2 ** -8: 0x3F80,                 # halfway between 1 and 1 + 2^-7: to the even 1
        1 + 3 * 2 ** -8: 0x3F82,             # halfway between 1 + 2^-7 and 1 + 2^-6: to the even upper
        2.0 ** -133: 0x0001,                 # smallest subnormal
        2.0 ** -134: 0x0000,                 # halfway between 0 and it: to the even 0
        1.5 * 2.0 ** -134: 0x0001,
        (2 - 2 ** -7) * 2.0 ** 127: 0x7F7F,  # largest finite
        3.4e38: 0x7F80,                      # rounds past it: inf
    }
    for x, bits in cases.items():
        assert oracle.bf16_encode(x) == bits, (x, hex(oracle.bf16_encode(x)))
    assert oracle.bf16_encode(-0.0) == 0x8000            # (a separate key: -0.0 == 0.0 in a dict)
    assert oracle.bf16_encode(float("nan")) & 0x7FC0 == 0x7FC0


def test_bf16_encode_matches_torch_on_float32():
    """On float32 inputs (normal, subnormal, huge) the encoder equals torch's RNE cast."""
    rng = np.random.default_rng(11)
    f = np.concatenate([rng.standard_normal(20000).astype(np.float32) * np.float32(3),
                        (rng.standard_normal(5000) * 1e-39).astype(np.float32),
                        (rng.standard_normal(5000) * 1e38).astype(np.float32)])
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.bf16_encode(float(v)) for v in f], dtype=np.uint16)
    np.testing.assert_array_equal(got, want)


def test_silu_mul_matches_independent_formula():
    """silu(g) * u with silu written as g (1 + tanh(g / 2)) / 2, gate = first half of
    each row, up = second half, rounded once: any swap of the halves, row-stride
    slip or dropped factor fails here."""
    rows, I = 5, 24
    bits = syn._to16(syn.normal_rows(4, 1, 9, rows, 2 * I, sigma=3.0), torch.bfloat16)
    bits[0, :4] = syn._to16(np.array([0.0, -0.0, 30.0, -30.0], np.float32), torch.bfloat16)
    x = torch16(bits, torch.bfloat16)
    got = oracle.silu_mul_bf16(bits)
    for r in range(rows):
        for i in range(I):
            g, u = x[r, i], x[r, I + i]
            want = oracle.bf16_encode(g * (1.0 + math.tanh(g / 2.0)) / 2.0 * u)
            assert got[r, i] == want, (r, i, g, u)
    assert got[0, 0] in (0, 0x8000) and got[0, 1] in (0, 0x8000)   # silu(+-0) * u is a zero
