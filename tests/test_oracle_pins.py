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


# ---------------------------------------------------------------------------
# MX activations (OCP MX v1.0: E8M0 scale per 32 elements) and MX x MXFP4 GEMMs
# ---------------------------------------------------------------------------

def test_e2m1_encode_round_trip_ties_and_saturation():
    for code, v in golden("e2m1_ocp_mx_v1.txt"):
        assert oracle.e2m1_encode(v) == code, (code, v)
    # midpoints between neighbours go to the even mantissa bit (code & 1 == 0)
    for v, code in [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6),
                    (-0.25, 8), (-0.75, 10), (-5.0, 14)]:
        assert oracle.e2m1_encode(v) == code, (v, code)
    for v in (6.0, 6.5, 7.0, 1e30):
        assert oracle.e2m1_encode(v) == 7 and oracle.e2m1_encode(-v) == 15
    assert oracle.e2m1_encode(-1e-30) == 8 and oracle.e2m1_encode(1e-30) == 0


def test_e2m1_encode_is_nearest_and_monotone():
    vals = np.array([E2M1_TABLE[c] for c in range(8)])
    prev = -1
    for v in np.linspace(0.0, 6.0, 2401):
        c = oracle.e2m1_encode(float(v))
        assert c >= prev
        prev = c
        assert abs(vals[c] - v) <= np.abs(vals - v).min() + 1e-15


@pytest.mark.parametrize("elem,emax,lo,hi", [("e2m1", 2, 4.0, 6.0), ("e4m3", 8, 256.0, 448.0)])
def test_quant_act_mx_scale_rule_and_error_bound(elem, emax, lo, hi):
    x = syn.normal_rows(0, 9, syn.T_A, 17, 256) * np.float32(3.0)
    x[4, 32:64] = 0.0                                     # an all-zero block
    x[5, :32] *= np.float32(1e-30)                        # tiny block
    q, e = oracle.quant_act_mx(x, elem)
    dec = (lambda c: E2M1_TABLE[int(c)]) if elem == "e2m1" else oracle.e4m3
    for m in range(x.shape[0]):
        for b in range(8):
            blk = x[m, 32 * b:32 * b + 32].astype(np.float64)
            amax = np.abs(blk).max()
            E = int(e[m, b])
            codes = [(q[m, (32 * b + i) // 2] >> (4 * (i & 1))) & 15 if elem == "e2m1" else q[m, 32 * b + i]
                     for i in range(32)]
            if amax == 0:
                assert E == 0 and all(c == 0 for c in codes)
                continue
            X = 2.0 ** (E - 127)
            # the scale puts the block maximum in [2^emax, 2^(emax+1)) before rounding
            assert 2.0 ** emax <= amax / X < 2.0 ** (emax + 1)
            im = int(np.abs(blk).argmax())
            assert lo <= abs(dec(codes[im])) <= hi
            for i in range(32):
                r = dec(codes[i]) * X
                # nearest representable: within half the largest grid step (2 for e2m1 at 4..6,
                # 32 for e4m3 at 256..448) times X, or saturated
                step = (2.0 if elem == "e2m1" else 32.0) * X
                assert abs(r - blk[i]) <= step / 2 + 1e-300 or abs(blk[i]) / X > hi


def test_quant_act_mx_hand_worked_block_and_nibble_order():
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, :6] = np.array([6.0, -3.0, 0.5, 0.25, 0.75, 5.0], dtype=np.float32) * np.float32(32.0)
    q, e = oracle.quant_act_mx(x, "e2m1")
    assert e[0, 0] == 127 + 7 - 2                        # amax 192: floor(log2) = 7, E2M1 emax 2
    # codes: 6 -> 7, -3 -> 8|5, 0.5 -> 1, 0.25 -> 0 (tie to even), 0.75 -> 2 (tie to 1.0), 5 -> 6 (tie to 4)
    assert list(q[0, :3]) == [7 | (13 << 4), 1 | (0 << 4), 2 | (6 << 4)]
    assert not q[0, 3:].any()
    q8, e8 = oracle.quant_act_mx(x, "e4m3")
    assert e8[0, 0] == 127 + 7 - 8
    ref = torch.from_numpy(np.ldexp(x.astype(np.float64), 127 - int(e8[0, 0])).astype(np.float32)).to(torch.float8_e4m3fn)
    np.testing.assert_array_equal(q8, ref.view(torch.uint8).numpy())


def test_quant_act_mx_e4m3_matches_torch_cast_in_range_and_saturates():
    x = syn.normal_rows(1, 9, syn.T_A, 9, 512)
    q, e = oracle.quant_act_mx(x, "e4m3")
    v = np.ldexp(x.astype(np.float64), 127 - np.repeat(e.astype(np.int64), 32, axis=1))
    inr = np.abs(v) <= 448.0
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(q[inr], ref[inr])
    assert np.all((q[~inr] & 0x7F) == 0x7E)             # beyond 448 saturates


def test_quant_act_mx_non_finite_block_gets_nan_scale():
    x = syn.normal_rows(2, 9, syn.T_A, 2, 64)
    x[0, 3] = np.nan
    x[1, 40] = -np.inf
    for elem in ("e2m1", "e4m3"):
        q, e = oracle.quant_act_mx(x, elem)
        assert e[0, 0] == 0xFF and e[1, 1] == 0xFF and e[0, 1] != 0xFF and e[1, 0] != 0xFF
        assert math.isnan(oracle.e8m0(int(e[0, 0])))


def mx_a_decode(qa, ea, K, elem):
    if elem == "e2m1":
        codes = np.stack([qa & 15, qa >> 4], axis=-1).reshape(qa.shape[0], K).astype(np.int64)
        v = e2m1_tab(codes)
    else:
        v = np.array([oracle.e4m3(c) for c in range(256)])[qa.astype(np.int64)]
    return v * 2.0 ** (np.repeat(ea.astype(np.int64), 32, axis=1) - 127)


@pytest.mark.parametrize("elem", ["e2m1", "e4m3"])
def test_gemm_mx_mxfp4_exact_rational_tiny(elem):
    M, N, K = 2, 16, 64
    d = syn.w4a8_mxfp4(7, M, N, K)
    qa, ea = oracle.quant_act_mx(d["A0"] * np.float32(50.0), elem)
    got = oracle.gemm_mx_mxfp4(qa, ea, d["q"], d["e"], N=N, K=K, a_elem=elem)
    a = mx_a_decode(qa, ea, K, elem)
    codes = unpack_k(d["q"], K)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += Fraction(float(a[m, k])) * Fraction(E2M1_TABLE[int(codes[k, n])]) * Fraction(2) ** (int(d["e"][k // 32, n]) - 127)
            assert abs(got[m, n] - float(acc)) <= 1e-13 * max(abs(float(acc)), 1e-30)


def test_gemm_mx_with_unit_scales_equals_tokenwise_w4a8():
    """E4M3 activations whose MX scales are all 127 are the tokenwise W4A8 case with s_a = 1."""
    M, N, K = 5, 48, 256
    d = syn.w4a8_mxfp4(8, M, N, K)
    qa, _ = oracle.quant_act_e4m3(d["A0"])
    ones = np.ones(M, dtype=np.float32)
    e127 = np.full((M, K // 32), 127, dtype=np.uint8)
    np.testing.assert_array_equal(oracle.gemm_mx_mxfp4(qa, e127, d["q"], d["e"], N=N, K=K, a_elem="e4m3"),
                                  oracle.gemm_w4a8_mxfp4(qa, ones, d["q"], d["e"], N=N, K=K))


@pytest.mark.parametrize("elem", ["e2m1", "e4m3"])
def test_gemm_mx_block_scale_step_and_sign_flip(elem):
    M, N, K = 3, 32, 256
    d = syn.w4a8_mxfp4(9, M, N, K)
    qa, ea = oracle.quant_act_mx(d["A0"], elem)
    base = oracle.gemm_mx_mxfp4(qa, ea, d["q"], d["e"], N=N, K=K, a_elem=elem)
    flip = qa ^ np.uint8(0x88 if elem == "e2m1" else 0x80)
    np.testing.assert_array_equal(oracle.gemm_mx_mxfp4(flip, ea, d["q"], d["e"], N=N, K=K, a_elem=elem), -base)
    e2 = ea.copy()
    e2[1, 5] += 1                                          # row 1, K block [160, 192) doubles
    moved = oracle.gemm_mx_mxfp4(qa, e2, d["q"], d["e"], N=N, K=K, a_elem=elem)
    assert np.array_equal(moved[[0, 2]], base[[0, 2]])
    a = mx_a_decode(qa, ea, K, elem)
    w = e2m1_tab(unpack_k(d["q"], K)) * (2.0 ** (np.repeat(d["e"].astype(np.int64), 32, axis=0) - 127))
    contrib = a[1, 160:192] @ w[160:192]
    assert rel_err(moved[1] - base[1], contrib) < 1e-12


# ---------------------------------------------------------------------------
# FP8 W8A8 with blockwise scales (1 x 128 activation blocks, 128 x 128 weight blocks)
# ---------------------------------------------------------------------------

E4M3_LUT = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_quant_act_e4m3_blocks_reduces_to_tokenwise_and_per_block():
    x = syn.normal_rows(3, 10, syn.T_A, 9, 512)
    x[2, 128:256] = 0.0
    q1, s1 = oracle.quant_act_e4m3_blocks(x, 512)
    qt, st = oracle.quant_act_e4m3(x)
    np.testing.assert_array_equal(q1, qt)
    np.testing.assert_array_equal(s1[:, 0], st)
    q, s = oracle.quant_act_e4m3_blocks(x, 128)
    for b in range(4):                                    # each block is its own tokenwise problem
        qb, sb = oracle.quant_act_e4m3(x[:, 128 * b:128 * b + 128])
        np.testing.assert_array_equal(q[:, 128 * b:128 * b + 128], qb)
        np.testing.assert_array_equal(s[:, b], sb)
    assert s[2, 1] == 1.0 and not q[2, 128:256].any()


def test_gemm_fp8_blockwise_matches_decoded_matmul_and_exact_rational():
    M, N, K = 5, 200, 384
    d = syn.w8a8_fp8_blockwise(1, M, N, K)
    qa, sa = oracle.quant_act_e4m3_blocks(d["A0"], 128)
    got = oracle.gemm_fp8_blockwise(qa, sa, d["w"], d["s_w"])
    a = E4M3_LUT[qa] * np.repeat(sa.astype(np.float64), 128, axis=1)
    w = E4M3_LUT[d["w"]] * np.repeat(np.repeat(d["s_w"].astype(np.float64), 128, axis=0), 128, axis=1)[:, :N]
    assert rel_err(got, a @ w) < 1e-13
    for m, n in [(0, 0), (4, 199), (2, 128), (3, 127)]:
        acc = Fraction(0)
        for k in range(K):
            acc += (Fraction(float(E4M3_LUT[qa[m, k]])) * Fraction(float(sa[m, k // 128]))
                    * Fraction(float(E4M3_LUT[d["w"][k, n]])) * Fraction(float(d["s_w"][k // 128, n // 128])))
        assert abs(got[m, n] - float(acc)) <= 1e-13 * max(abs(float(acc)), 1e-30)


def test_gemm_fp8_blockwise_scale_indexing():
    """Doubling one activation block scale doubles exactly that row's K block; doubling
    one weight block scale doubles exactly that K block of those 128 columns."""
    M, N, K = 3, 256, 384
    d = syn.w8a8_fp8_blockwise(2, M, N, K)
    qa, sa = oracle.quant_act_e4m3_blocks(d["A0"], 128)
    base = oracle.gemm_fp8_blockwise(qa, sa, d["w"], d["s_w"])
    a = E4M3_LUT[qa] * np.repeat(sa.astype(np.float64), 128, axis=1)
    w = E4M3_LUT[d["w"]] * np.repeat(np.repeat(d["s_w"].astype(np.float64), 128, axis=0), 128, axis=1)[:, :N]
    sa2 = sa.copy()
    sa2[1, 2] *= 2
    got = oracle.gemm_fp8_blockwise(qa, sa2, d["w"], d["s_w"])
    assert np.array_equal(got[[0, 2]], base[[0, 2]])
    assert rel_err(got[1] - base[1], a[1, 256:384] @ w[256:384]) < 1e-12
    sw2 = d["s_w"].copy()
    sw2[0, 1] *= 2
    got = oracle.gemm_fp8_blockwise(qa, sa, d["w"], sw2)
    assert np.array_equal(got[:, :128], base[:, :128])
    assert rel_err(got[:, 128:] - base[:, 128:], a[:, :128] @ w[:128, 128:]) < 1e-12


# ---------------------------------------------------------------------------
# FP4 weights with 16-bit activations: MXFP4 and NVFP4 (second-level scale)
# ---------------------------------------------------------------------------

def test_fp4_a16_mxfp4_equals_single_expert_moe():
    """Dense MXFP4 with bf16 activations is the MoE oracle with one expert and top-1."""
    M, N, K = 6, 48, 256
    d = syn.w4a16_fp4(0, M, N, K, nvfp4=False)
    got = oracle.gemm_fp4_a16(d["A"], d["q"], d["s"], N=N, K=K, a_bf16=True, nvfp4=False)
    moe = oracle.moe_mxfp4_bf16(d["A"], np.zeros((M, 1), np.int32), d["q"][None], d["s"][None], N=N, K=K)
    np.testing.assert_array_equal(got, moe)


def test_fp4_a16_nvfp4_exact_rational_and_second_level_scale():
    M, N, K = 2, 16, 64
    d = syn.w4a16_fp4(1, M, N, K, nvfp4=True)
    got = oracle.gemm_fp4_a16(d["A"], d["q"], d["s"], N=N, K=K, a_bf16=True, nvfp4=True, s2=d["s2"])
    a = torch16(d["A"], torch.bfloat16)
    codes = unpack_k(d["q"], K)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += (Fraction(float(a[m, k])) * Fraction(E2M1_TABLE[int(codes[k, n])])
                        * Fraction(float(E4M3_LUT[d["s"][k // 16, n]])) * Fraction(float(np.float32(d["s2"]))))
            assert abs(got[m, n] - float(acc)) <= 1e-13 * max(abs(float(acc)), 1e-30)
    base = oracle.gemm_fp4_a16(d["A"], d["q"], d["s"], N=N, K=K, a_bf16=True, nvfp4=True)
    np.testing.assert_allclose(got, base * np.float64(np.float32(d["s2"])), rtol=1e-15)


def test_fp4_a16_nvfp4_group_of_16_indexing():
    """Changing one 16-K group scale changes exactly that group's contribution of that column."""
    M, N, K = 3, 32, 128
    d = syn.w4a16_fp4(2, M, N, K, nvfp4=True)
    base = oracle.gemm_fp4_a16(d["A"], d["q"], d["s"], N=N, K=K, a_bf16=False, nvfp4=True)
    s = d["s"].copy()
    s[5, 7] = 0x38                                            # E4M3 1.0 for K in [80, 96), column 7
    got = oracle.gemm_fp4_a16(d["A"], d["q"], s, N=N, K=K, a_bf16=False, nvfp4=True)
    cols = [c for c in range(N) if c != 7]
    assert np.array_equal(got[:, cols], base[:, cols])
    a = torch16(d["A"], torch.float16)
    w = e2m1_tab(unpack_k(d["q"], K))[80:96, 7]
    delta = a[:, 80:96] @ w * (1.0 - E4M3_LUT[d["s"][5, 7]])
    assert rel_err(got[:, 7] - base[:, 7], delta) < 1e-12


# ---------------------------------------------------------------------------
# MXINT4 weights (two's-complement INT4, E8M0 per 32 K) with bf16 activations
# ---------------------------------------------------------------------------

def test_mxint4_a16_exact_rational():
    M, N, K = 2, 16, 64
    d = syn.w4a16_mxint4(0, M, N, K)
    got = oracle.gemm_mxint4_a16(d["A"], d["q"], d["e"], N=N, K=K)
    a = torch16(d["A"], torch.bfloat16)
    codes = unpack_k(d["q"], K)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                c = int(codes[k, n])
                c = c - 16 if c >= 8 else c
                acc += Fraction(float(a[m, k])) * c * Fraction(2) ** (int(d["e"][k // 32, n]) - 127)
            assert abs(got[m, n] - float(acc)) <= 1e-13 * max(abs(float(acc)), 1e-30)


def test_mxint4_a16_unit_scales_equal_symmetric_w4a16():
    """With every E8M0 exponent 127 (scale 1) MXINT4 is symmetric INT4 W4A16 with unit group scales."""
    M, N, K = 5, 40, 256
    d = syn.w4a16_mxint4(1, M, N, K)
    e = np.full((K // 32, N), 127, np.uint8)
    got = oracle.gemm_mxint4_a16(d["A"], d["q"], e, N=N, K=K)
    ones = np.full((K // 128, N), 0x3F80, np.uint16)
    ref = oracle.gemm_wna16(d["A"], d["q"], ones, None, N=N, K=K, G=128, a_bf16=True, w_signed=True)
    np.testing.assert_array_equal(got, ref)


def test_mxint4_a16_single_weight_and_block_step():
    """A lone code 0x8 decodes to -8 at its (k, n); raising one block's exponent by one
    doubles exactly that block's contribution of that column."""
    M, N, K = 3, 16, 128
    d = syn.w4a16_mxint4(2, M, N, K)
    a = torch16(d["A"], torch.bfloat16).astype(np.float64)
    q = np.zeros((K // 8, N), np.uint32)
    k0, n0 = 37, 5
    q[k0 // 8, n0] = np.uint32(0x8) << np.uint32(4 * (k0 % 8))
    e = np.full((K // 32, N), 127, np.uint8)
    got = oracle.gemm_mxint4_a16(d["A"], q, e, N=N, K=K)
    want = np.zeros((M, N))
    want[:, n0] = -8.0 * a[:, k0]
    np.testing.assert_array_equal(got, want)
    base = oracle.gemm_mxint4_a16(d["A"], d["q"], d["e"], N=N, K=K)
    e2 = d["e"].copy()
    e2[2, 7] += 1
    moved = oracle.gemm_mxint4_a16(d["A"], d["q"], e2, N=N, K=K)
    codes = unpack_k(d["q"], K).astype(np.int64)
    codes = np.where(codes >= 8, codes - 16, codes)
    blk = a[:, 64:96] @ (codes[64:96, 7] * 2.0 ** (int(d["e"][2, 7]) - 127))
    np.testing.assert_allclose(moved[:, 7] - base[:, 7], blk, rtol=1e-12, atol=1e-12)
    other = [n for n in range(N) if n != 7]
    np.testing.assert_array_equal(moved[:, other], base[:, other])


# ---------------------------------------------------------------------------
# INT8 weight-only (W8A16): 16-bit activations x INT8 weights, per-column fp32 scale
# ---------------------------------------------------------------------------

def test_w8a16_integer_activations_equal_w8a8():
    """With integer-valued activations in [-127, 127] and unit token scales, W8A16 is the
    (exact, int64) W8A8 oracle: same sums, same per-column epilogue."""
    M, N, K = 5, 24, 192
    d = syn.w8a16_int8(0, M, N, K)
    a8 = syn.int8_uniform(0, 99, 0, (M, K))
    for bf in (True, False):
        dt = torch.bfloat16 if bf else torch.float16
        A = torch.from_numpy(a8.astype(np.float32)).to(dt).view(torch.int16).numpy().view(np.uint16)
        got = oracle.gemm_w8a16(A, d["w"], d["s_w"], a_bf16=bf)
        _, ref = oracle.gemm_w8a8(a8, np.ones(M, np.float32), d["w"], d["s_w"])
        np.testing.assert_array_equal(got, ref)


def test_w8a16_exact_rational_and_column_scale():
    M, N, K = 2, 8, 64
    d = syn.w8a16_int8(1, M, N, K, torch.float16)
    got = oracle.gemm_w8a16(d["A"], d["w"], d["s_w"], a_bf16=False)
    a = torch16(d["A"], torch.float16)
    for m in range(M):
        for n in range(N):
            acc = sum(Fraction(float(a[m, k])) * int(d["w"][k, n]) for k in range(K)) * Fraction(float(d["s_w"][n]))
            assert abs(got[m, n] - float(acc)) <= 1e-13 * max(abs(float(acc)), 1e-30)
    # -128 is a code like any other; a column's scale scales exactly that column
    w = np.zeros((K, N), np.int8)
    w[17, 3] = -128
    s = np.ones(N, np.float32)
    s[3] = 0.5
    got = oracle.gemm_w8a16(d["A"], w, s, a_bf16=False)
    want = np.zeros((M, N))
    want[:, 3] = -64.0 * a[:, 17].astype(np.float64)
    np.testing.assert_array_equal(got, want)


# ---------------------------------------------------------------------------
# FP8 weight-only: 16-bit activations x E4M3 weights, per-column fp32 scale
# ---------------------------------------------------------------------------

def test_fp8w_a16_integer_codes_equal_w8a16():
    """E4M3 codes of the integers -16..16 (every one exactly representable) give the
    INT8 weight-only oracle's result on the same integers, bit for bit."""
    M, N, K = 4, 24, 128
    d = syn.w8a16_fp8(0, M, N, K)
    ints = np.random.default_rng(5).integers(-16, 17, size=(K, N)).astype(np.int8)
    codes = np.array([oracle.e4m3_encode(float(v)) for v in ints.reshape(-1)], np.uint8).reshape(K, N)
    for bf in (True, False):
        dt = torch.bfloat16 if bf else torch.float16
        A = syn.w8a16_fp8(0, M, N, K, dt)["A"]
        got = oracle.gemm_fp8w_a16(A, codes, d["s_w"], a_bf16=bf)
        ref = oracle.gemm_w8a16(A, ints, d["s_w"], a_bf16=bf)
        np.testing.assert_array_equal(got, ref)


def test_fp8w_a16_exact_rational():
    M, N, K = 2, 8, 64
    d = syn.w8a16_fp8(1, M, N, K)
    got = oracle.gemm_fp8w_a16(d["A"], d["w"], d["s_w"], a_bf16=True)
    a = torch16(d["A"], torch.bfloat16)
    for m in range(M):
        for n in range(N):
            acc = sum(Fraction(float(a[m, k])) * Fraction(float(E4M3_LUT[d["w"][k, n]])) for k in range(K))
            acc *= Fraction(float(d["s_w"][n]))
            assert abs(got[m, n] - float(acc)) <= 1e-13 * max(abs(float(acc)), 1e-30)


# ---- low-bit WnA16 (1, 2, 3-bit codes): "Humming wird angekuendigt", section WnA16 ----

def _pack_k_nibbles(codes):
    """One code per byte [K][N] -> the W4A16 4-bit container uint32 [K/8][N] (two's-complement nibbles)."""
    K, N = codes.shape
    nib = (codes.astype(np.int64) & 15).astype(np.uint32)
    q = np.zeros((K // 8, N), np.uint32)
    for i in range(8):
        q |= nib[i::8] << np.uint32(4 * i)
    return q


@pytest.mark.parametrize("bits", [1, 2, 3])
@pytest.mark.parametrize("signed", [True, False])
def test_wnlow_equals_w4a16_on_the_same_codes(bits, signed):
    """A b-bit code is a 4-bit code of the same value: the low-bit oracle equals the
    (separately pinned) W4A16 oracle fed the codes in 4-bit containers, with the same
    zero-points (unsigned) or none (signed, two's complement)."""
    M, N, K, G = 4, 24, 512, 128
    d = syn.wnlow(bits, M, N, K, bits, signed)
    for bf in (False, True):
        A = d["A"]
        got = oracle.gemm_wnlow(A, d["codes"], d["s"], d.get("z"), N=N, K=K, G=G, bits=bits, a_bf16=bf, w_signed=signed)
        ref = oracle.gemm_wna16(A, _pack_k_nibbles(d["codes"]), d["s"], d.get("z"), N=N, K=K, G=G, a_bf16=bf,
                                w_signed=signed)
        np.testing.assert_array_equal(got, ref)


def test_wnlow_exact_rationals():
    """Hand-computable cases against all-ones fp16 activations over one 128-K group:
    INT2 code -2 (the most negative) under scale 0.5, UINT3 code 7 with zero-point 5
    under 0.25 (and code 0 with the same zero-point), INT1 code -1 under 2.0."""
    K, G = 128, 128
    one16 = np.full((1, K), 0x3C00, np.uint16)  # fp16 1.0
    # bits, signed, (code col 0, code col 1), zero-point, fp16 scale bits, expected (col 0, col 1)
    cases = ((2, True, (-2, 0), 0, 0x3800, (-128.0, 0.0)),
             (3, False, (7, 0), 5, 0x3400, (64.0, -160.0)),
             (1, True, (-1, 0), 0, 0x4000, (-256.0, 0.0)))
    for bits, signed, (c0, c1), zero, scale, want in cases:
        codes = np.empty((K, 2), np.int8)
        codes[:, 0], codes[:, 1] = c0, c1
        s = np.full((1, 2), scale, np.uint16)
        z = None if signed else np.array([[zero | (zero << 4)]], np.uint32)
        got = oracle.gemm_wnlow(one16, codes, s, z, N=2, K=K, G=G, bits=bits, a_bf16=False, w_signed=signed)
        assert tuple(got[0]) == want, (bits, signed, got[0], want)


def test_wnlow_rejects_codes_outside_the_width():
    codes = np.zeros((128, 16), np.int8)
    codes[5, 3] = 2          # INT2 holds -2 .. 1
    A = np.full((1, 128), 0x3C00, np.uint16)
    s = np.full((1, 16), 0x3C00, np.uint16)
    with pytest.raises(ValueError):
        oracle.gemm_wnlow(A, codes, s, None, N=16, K=128, G=128, bits=2, a_bf16=False, w_signed=True)
    codes[5, 3] = 8          # UINT3 holds 0 .. 7
    with pytest.raises(ValueError):
        oracle.gemm_wnlow(A, codes, s, np.zeros((1, 2), np.uint32), N=16, K=128, G=128, bits=3, a_bf16=False,
                          w_signed=False)


# ---- MX-scaled float weights (MXFP8 E4M3, MXFP6 E2M3 / E3M2): "Humming wird
# angekuendigt", section WnA16 (float weights of any width), OCP MX v1.0 ----

@pytest.mark.parametrize("fmt", ["e2m3", "e3m2"])
def test_fp6_matches_ocp_table_and_is_symmetric(fmt):
    for code, v in golden(f"fp6_{fmt}_ocp_mx_v1.txt"):
        assert oracle.fp6(code, fmt == "e3m2") == v, (fmt, code)
        assert oracle.fp6(code | 0x20, fmt == "e3m2") == -v, (fmt, code)


@pytest.mark.parametrize("fmt", ["e2m3", "e3m2"])
def test_fp6_subnormals_evenly_spaced_and_codes_monotone(fmt):
    """The subnormal codes run in equal steps from 0 to the table's largest subnormal
    (the step is the smallest subnormal); positive codes increase strictly, and every
    value is an exact E4M3 value (torch's fp8 cast leaves it unchanged)."""
    tab = dict(golden(f"fp6_{fmt}_ocp_mx_v1.txt"))
    e3 = fmt == "e3m2"
    mb = 2 if e3 else 3
    step = tab[0x01]
    for m in range(1 << mb):
        assert oracle.fp6(m, e3) == m * step
    assert oracle.fp6((1 << mb) - 1, e3) == tab[(1 << mb) - 1]
    vals = [oracle.fp6(c, e3) for c in range(32)]
    assert all(b > a for a, b in zip(vals, vals[1:]))
    t = torch.tensor(vals + [-v for v in vals], dtype=torch.float32)
    assert torch.equal(t.to(torch.float8_e4m3fn).to(torch.float32), t)


def test_fp6_normal_codes_are_e2m1_and_e4m3_codes_with_shifted_fields():
    """E2M3 s.ee.mm0 is E2M1 s.ee.m (same bias, golden E2M1 table); every normal
    E2M3 s.ee.mmm is E4M3 s.(ee+6).mmm and every normal E3M2 s.eee.mm is E4M3
    s.(eee+4).mm0 (the biases differ by 6 and 4; E4M3 pinned by its own table
    and torch), so sign, exponent, bias and each mantissa bit are tied down."""
    for s in (0, 1):
        for e in range(4):
            for m in range(8):
                c = (s << 5) | (e << 3) | m
                v = oracle.fp6(c, False)
                if m % 4 == 0:
                    assert v == E2M1_TABLE[(s << 3) | (e << 1) | (m >> 2)] or (v == 0 and m == 0 and e == 0)
                if e:
                    assert v == E4M3_LUT[(s << 7) | ((e + 6) << 3) | m]
        for e in range(1, 8):
            for m in range(4):
                assert oracle.fp6((s << 5) | (e << 2) | m, True) == E4M3_LUT[(s << 7) | ((e + 4) << 3) | (m << 1)]


def _mxf_exact(A, codes, e8, elem, a_dt):
    a = torch16(A, a_dt)
    M, K = A.shape
    N = codes.shape[1]
    dec = (lambda c: E4M3_LUT[c]) if elem == "e4m3" else (lambda c: oracle.fp6(int(c), elem == "e3m2"))
    out = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += Fraction(float(a[m, k])) * Fraction(float(dec(codes[k, n]))) * Fraction(2) ** (int(e8[k // 32, n]) - 127)
            out[m, n] = float(acc)
    return out


@pytest.mark.parametrize("elem", ["e4m3", "e2m3", "e3m2"])
def test_mxf_a16_exact_rational(elem):
    M, N, K = 2, 8, 64
    d = syn.mxf_a16(0, M, N, K, elem)
    got = oracle.gemm_mxf_a16(d["A"], d["codes"], d["e"], elem=elem)
    want = _mxf_exact(d["A"], d["codes"], d["e"], elem, torch.bfloat16)
    assert np.all(np.abs(got - want) <= 1e-13 * np.maximum(np.abs(want), 1e-30))


def test_mxf_a16_e2m3_on_e2m1_values_equals_mxfp4():
    """E2M3 codes whose low two mantissa bits are zero carry exactly the E2M1 values:
    with the same E8M0 blocks the MXFP4 weight-only oracle (another code path, 4-bit
    words) gives the same result bit for bit."""
    M, N, K = 5, 24, 256
    d = syn.w4a16_fp4(3, M, N, K, nvfp4=False)
    nib = unpack_k(d["q"], K)
    codes = (((nib >> 3) & 1) << 5 | ((nib >> 1) & 3) << 3 | (nib & 1) << 2).astype(np.uint8)
    got = oracle.gemm_mxf_a16(d["A"], codes, d["s"], elem="e2m3")
    ref = oracle.gemm_fp4_a16(d["A"], d["q"], d["s"], N=N, K=K, a_bf16=True, nvfp4=False)
    np.testing.assert_array_equal(got, ref)


def test_mxf_a16_e4m3_unit_blocks_equal_fp8_weight_only():
    """MXFP8 with every E8M0 exponent 127 is FP8 weight-only with unit column scales."""
    M, N, K = 4, 40, 128
    d = syn.mxf_a16(1, M, N, K, "e4m3")
    e = np.full((K // 32, N), 127, np.uint8)
    for bf in (True, False):
        A = syn.mxf_a16(1, M, N, K, "e4m3", torch.bfloat16 if bf else torch.float16)["A"]
        got = oracle.gemm_mxf_a16(A, d["codes"], e, elem="e4m3", a_bf16=bf)
        ref = oracle.gemm_fp8w_a16(A, d["codes"], np.ones(N, np.float32), a_bf16=bf)
        np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("elem", ["e2m3", "e3m2"])
def test_mxf_a16_block_step_and_code_range(elem):
    """Raising one 32-K block's exponent by one doubles exactly that block's share of
    that column; a code with bit 6 or 7 set is rejected."""
    M, N, K = 3, 16, 128
    d = syn.mxf_a16(2, M, N, K, elem)
    base = oracle.gemm_mxf_a16(d["A"], d["codes"], d["e"], elem=elem)
    e2 = d["e"].copy()
    e2[2, 7] += 1
    moved = oracle.gemm_mxf_a16(d["A"], d["codes"], e2, elem=elem)
    cols = [c for c in range(N) if c != 7]
    np.testing.assert_array_equal(moved[:, cols], base[:, cols])
    a = torch16(d["A"], torch.bfloat16)
    w = np.array([oracle.fp6(int(c), elem == "e3m2") for c in d["codes"][64:96, 7]]) * 2.0 ** (int(d["e"][2, 7]) - 127)
    assert rel_err(moved[:, 7] - base[:, 7], a[:, 64:96] @ w) < 1e-12
    bad = d["codes"].copy()
    bad[5, 3] |= 0x40
    with pytest.raises(ValueError):
        oracle.gemm_mxf_a16(d["A"], bad, d["e"], elem=elem)


# ---- zero-exponent floats e0mN: "Humming wird angekuendigt", the paragraph on the
# format whose values are the symmetric integers of its width ----

def test_e0m7_values_are_int8_without_minus_128():
    """The pages' own example: e0m7 and INT8 without -128 both represent -127..127."""
    vals = [oracle.e0m(c, 7) for c in range(256)]
    assert sorted(set(vals)) == list(range(-127, 128))
    assert vals.count(0) == 2 and all(vals.count(v) == 1 for v in range(-127, 128) if v)


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6, 7])
def test_e0m_sign_and_magnitude(n):
    """Every magnitude m < 2^n appears once with each sign (the sign bit is bit n,
    the magnitude the low n bits: code m and code 2^n + m negate each other); a
    bit above n is rejected; the values are exactly the symmetric integers of the
    width n + 1 (INT(n+1) without its most negative code)."""
    for m in range(1 << n):
        assert oracle.e0m(m, n) == m and oracle.e0m((1 << n) | m, n) == -m
    with pytest.raises(ValueError):
        oracle.e0m(1 << (n + 1), n)
    lo = -(1 << n)
    assert sorted({oracle.e0m(c, n) for c in range(1 << (n + 1))}) == list(range(lo + 1, -lo))


# ---- WnA16 at 5-8 bits (INT5-INT8, UINT5-UINT8 with 8-bit zero-points):
# "Humming wird angekuendigt", section WnA16 ----

@pytest.mark.parametrize("bits", [5, 6, 7, 8])
def test_wnwide_on_4bit_codes_equals_w4a16(bits):
    """Codes that fit four bits give the W4A16 oracle's result on the same codes in
    the 4-bit container (signed: -8..7, symmetric; unsigned: 0..15 with zero-points
    0..15 in the UINT4 container), bit for bit."""
    M, N, K, G = 4, 24, 256, 128
    rng = np.random.default_rng(bits)
    for signed in (True, False):
        d = syn.wnwide(bits, M, N, K, bits, signed, G=G)
        if signed:
            codes = rng.integers(-8, 8, size=(K, N)).astype(np.int8)
            got = oracle.gemm_wnwide(d["A"], codes, d["s"], N=N, K=K, G=G, bits=bits, a_bf16=False, w_signed=True)
            ref = oracle.gemm_wna16(d["A"], _pack_k_nibbles(codes), d["s"], None, N=N, K=K, G=G, a_bf16=False,
                                    w_signed=True)
        else:
            codes = rng.integers(0, 16, size=(K, N)).astype(np.uint8)
            z8 = rng.integers(0, 16, size=(K // G, N)).astype(np.uint8)
            zw = np.zeros((K // G, (N + 7) // 8), np.uint32)
            for n in range(N):
                zw[:, n // 8] |= z8[:, n].astype(np.uint32) << np.uint32(4 * (n % 8))
            got = oracle.gemm_wnwide(d["A"], codes, d["s"], z8, N=N, K=K, G=G, bits=bits, a_bf16=False,
                                     w_signed=False)
            ref = oracle.gemm_wna16(d["A"], _pack_k_nibbles(codes.astype(np.int8)), d["s"], zw, N=N, K=K, G=G,
                                    a_bf16=False, w_signed=False)
        np.testing.assert_array_equal(got, ref)


def test_wnwide_uint8_with_zero_128_is_int8():
    """UINT8 codes q with every zero-point 128 equal INT8 codes q - 128, bit for bit."""
    M, N, K, G = 3, 16, 256, 128
    d = syn.wnwide(1, M, N, K, 8, False, G=G)
    z = np.full((K // G, N), 128, np.uint8)
    got = oracle.gemm_wnwide(d["A"], d["codes"], d["s"], z, N=N, K=K, G=G, bits=8, a_bf16=False, w_signed=False)
    q = (d["codes"].astype(np.int16) - 128).astype(np.int8)
    ref = oracle.gemm_wnwide(d["A"], q, d["s"], N=N, K=K, G=G, bits=8, a_bf16=False, w_signed=True)
    np.testing.assert_array_equal(got, ref)


def test_wnwide_int8_one_group_per_column_is_int8_weight_only():
    """INT8 with one group spanning K (G = K) is INT8 weight-only with the group
    scale as the column scale (the other oracle scales the sum, this one each term)."""
    M, N, K = 4, 32, 256
    d = syn.wnwide(2, M, N, K, 8, True, G=K, dtype=torch.bfloat16)
    got = oracle.gemm_wnwide(d["A"], d["codes"], d["s"], N=N, K=K, G=K, bits=8, a_bf16=True, w_signed=True)
    sw = torch16(d["s"], torch.bfloat16)[0].astype(np.float32)
    ref = oracle.gemm_w8a16(d["A"], d["codes"], sw, a_bf16=True)
    assert rel_err(got, ref) < 1e-13


@pytest.mark.parametrize("bits", [5, 8])
@pytest.mark.parametrize("signed", [True, False])
def test_wnwide_exact_rationals_and_range(bits, signed):
    M, N, K, G = 2, 8, 256, 128
    d = syn.wnwide(3, M, N, K, bits, signed, G=G)
    lo, hi = (-(1 << (bits - 1)), (1 << (bits - 1)) - 1) if signed else (0, (1 << bits) - 1)
    codes = d["codes"].copy()
    codes[0, :] = lo
    codes[1, :] = hi
    got = oracle.gemm_wnwide(d["A"], codes, d["s"], d.get("z"), N=N, K=K, G=G, bits=bits, a_bf16=False,
                             w_signed=signed)
    a = torch16(d["A"], torch.float16)
    s = torch16(d["s"], torch.float16)
    cv = codes.astype(np.int64)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                z = 0 if signed else int(d["z"][k // G, n])
                acc += Fraction(float(a[m, k])) * (int(cv[k, n]) - z) * Fraction(float(s[k // G, n]))
            assert abs(got[m, n] - float(acc)) <= 1e-13 * max(abs(float(acc)), 1e-30)
    for bad in ((hi + 1, lo - 1) if signed else (hi + 1,)):
        if bits == 8 and (bad > 255 or bad < -128 or (signed and bad > 127)):
            continue   # (an 8-bit byte cannot hold the value)
        c = codes.copy()
        c[5, 3] = bad
        with pytest.raises(ValueError):
            oracle.gemm_wnwide(d["A"], c, d["s"], d.get("z"), N=N, K=K, G=G, bits=bits, a_bf16=False, w_signed=signed)
