"""Seeded synthetic inputs for the quantized-GEMM workloads.

This module only draws random numbers and lays them out in the documented
logical ("export") form.  It holds none of the GEMM's arithmetic: no decoding,
no dequantisation, no quantisation of activations.  Both the CPU oracle and
the HIP path consume exactly the arrays produced here.

Logical layouts (shared by both sides):

* activations ``A``: row-major ``[M, K]``; bf16/fp16 are returned as their raw
  16-bit patterns (``uint16``); fp32 as ``float32``; int8 as ``int8``.
* 4-bit codes (INT4, UINT4, FP4 e2m1): ``uint32 [K/8, N]``; code ``k = 8*j + i``
  of column ``n`` sits in bits ``[4i, 4i+4)`` of word ``[j, n]``.  Codes drawn
  uniformly over all 16 nibble values are the same thing as uniformly random
  32-bit words, which is how they are drawn.
* INT8 weights: ``int8 [K, N]``.
* group scales: ``[K/G, N]`` in the scale dtype (raw bits for bf16/fp16).
* zero-points (UINT4): ``uint32 [K/G, N/8]``; column ``n = 8*j + i`` in bits
  ``[4i, 4i+4)`` of word ``[g, j]``.
* E8M0 block exponents: ``uint8 [K/32, N]``.
* MoE routing: ``int32 [T, top_k]`` expert ids, distinct within a token.

Every tensor has its own stream ``numpy.random.default_rng([seed, cfg, tensor,
...])`` so tensors do not depend on generation order.  Row-blocked tensors
(activations, routing) draw each block of 64 rows from its own stream, so the
first M rows are the same whatever M is asked for.
"""
from __future__ import annotations

import numpy as np
import torch

ROW_BLOCK = 64

# tensor ids (part of every stream key)
T_A, T_Q, T_S, T_Z, T_E8, T_SA, T_SW, T_IDS = 1, 2, 3, 4, 5, 6, 7, 8

# workload ids
C1, C2, C3, C4, C5 = 1, 2, 3, 4, 5


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng([int(k) for k in key])


def _to16(x: np.ndarray, dtype: torch.dtype) -> np.ndarray:
    """fp32 draws rounded (RNE, torch's cast) to bf16/fp16; returns raw bits."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dtype)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def normal_rows(seed, cfg, tensor, M, K, sigma=1.0) -> np.ndarray:
    """fp32 N(0, sigma^2) rows, drawn per 64-row block (prefix-stable in M)."""
    out = np.empty((M, K), dtype=np.float32)
    for b in range(0, M, ROW_BLOCK):
        r = min(ROW_BLOCK, M - b)
        blk = _rng(seed, cfg, tensor, b // ROW_BLOCK).standard_normal((ROW_BLOCK, K), dtype=np.float32)
        out[b:b + r] = blk[:r] * np.float32(sigma)
    return out


def activations(seed, cfg, M, K, dtype: torch.dtype) -> np.ndarray:
    """A ~ N(0,1) as raw bf16/fp16 bits [M, K]."""
    return _to16(normal_rows(seed, cfg, T_A, M, K), dtype)


def random_words(seed, cfg, tensor, shape, *extra) -> np.ndarray:
    """Uniform uint32 words = 8 independent uniform nibbles each."""
    return _rng(seed, cfg, tensor, *extra).integers(0, 2**32, size=shape, dtype=np.uint64).astype(np.uint32)


def abs_normal_scales(seed, cfg, tensor, shape, sigma, offset, dtype, *extra) -> np.ndarray:
    """|N(0, sigma^2)| + offset, rounded to ``dtype`` (the rounded value is the truth)."""
    x = np.abs(_rng(seed, cfg, tensor, *extra).standard_normal(shape, dtype=np.float32) * np.float32(sigma)) + np.float32(offset)
    if dtype is torch.float32:
        return x.astype(np.float32)
    return _to16(x, dtype)


def e8m0_exponents(seed, cfg, shape, lo=118, hi=127, *extra) -> np.ndarray:
    return _rng(seed, cfg, T_E8, *extra).integers(lo, hi + 1, size=shape, dtype=np.int64).astype(np.uint8)


def int8_uniform(seed, cfg, tensor, shape, lo=-127, hi=127, *extra) -> np.ndarray:
    return _rng(seed, cfg, tensor, *extra).integers(lo, hi + 1, size=shape, dtype=np.int64).astype(np.int8)


def int8_rows(seed, cfg, tensor, M, K) -> np.ndarray:
    out = np.empty((M, K), dtype=np.int8)
    for b in range(0, M, ROW_BLOCK):
        r = min(ROW_BLOCK, M - b)
        out[b:b + r] = int8_uniform(seed, cfg, tensor, (ROW_BLOCK, K), -127, 127, b // ROW_BLOCK)[:r]
    return out


def per_token_scales(seed, cfg, M, sigma=0.01, offset=1e-4) -> np.ndarray:
    out = np.empty((M,), dtype=np.float32)
    for b in range(0, M, ROW_BLOCK):
        r = min(ROW_BLOCK, M - b)
        blk = np.abs(_rng(seed, cfg, T_SA, b // ROW_BLOCK).standard_normal(ROW_BLOCK, dtype=np.float32) * np.float32(sigma)) + np.float32(offset)
        out[b:b + r] = blk[:r]
    return out


# ---------------------------------------------------------------------------
# routing: Zipf(s) over experts, distinct experts per token
# ---------------------------------------------------------------------------

def zipf_topk(seed, cfg, T, E, top_k, s=1.1) -> np.ndarray:
    """Expert ids [T, top_k] (int32), expert e drawn with p ∝ (e+1)^-s, no repeats.

    Sequential draws without replacement (renormalising after each draw) are
    sampled with the Gumbel-top-k identity: the indices of the top_k largest
    ``log p + Gumbel`` values, in decreasing order, have exactly the
    distribution of the successive draws.  Slot j is the j-th draw.
    """
    logp = -s * np.log(np.arange(1, E + 1, dtype=np.float64))
    out = np.empty((T, top_k), dtype=np.int32)
    for b in range(0, T, ROW_BLOCK):
        r = min(ROW_BLOCK, T - b)
        g = _rng(seed, cfg, T_IDS, b // ROW_BLOCK).gumbel(size=(ROW_BLOCK, E))
        key = logp[None, :] + g
        idx = np.argsort(-key, axis=1, kind="stable")[:, :top_k]
        out[b:b + r] = idx[:r].astype(np.int32)
    return out


# ---------------------------------------------------------------------------
# the five workloads (logical/export form)
# ---------------------------------------------------------------------------

def w4a16_sym(seed, M, N, K, G=128, dtype=torch.bfloat16, cfg=C1):
    """Dense W4A16, symmetric INT4 codes uniform in [-8, 7], scales |N(0,0.02)|+1e-3."""
    return dict(
        A=activations(seed, cfg, M, K, dtype),
        q=random_words(seed, cfg, T_Q, (K // 8, N)),
        s=abs_normal_scales(seed, cfg, T_S, (K // G, N), 0.02, 1e-3, dtype),
    )


def w4a16_zp(seed, M, N, K, G=128, dtype=torch.float16, cfg=C2):
    """Dense W4A16 asymmetric: UINT4 codes and UINT4 zero-points uniform in [0, 15]."""
    return dict(
        A=activations(seed, cfg, M, K, dtype),
        q=random_words(seed, cfg, T_Q, (K // 8, N)),
        s=abs_normal_scales(seed, cfg, T_S, (K // G, N), 0.02, 1e-3, dtype),
        z=random_words(seed, cfg, T_Z, (K // G, (N + 7) // 8)),
    )


def w4a8_mxfp4(seed, M, N, K, cfg=C3):
    """Dense W4A8-MXFP4: fp32 activations (quantised tokenwise to e4m3 by the
    consumer), e2m1 codes uniform over all 16 values, E8M0 exponents in [118, 127]."""
    return dict(
        A0=normal_rows(seed, cfg, T_A, M, K),
        q=random_words(seed, cfg, T_Q, (K // 8, N)),
        e=e8m0_exponents(seed, cfg, (K // 32, N)),
    )


def w8a8_int8(seed, M, N, K, cfg=C4):
    """Dense W8A8: int8 uniform [-127, 127] both sides, fp32 |N(0,0.01)|+1e-4 scales."""
    return dict(
        a=int8_rows(seed, cfg, T_A, M, K),
        s_a=per_token_scales(seed, cfg, M),
        w=int8_uniform(seed, cfg, T_Q, (K, N)),
        s_w=abs_normal_scales(seed, cfg, T_SW, (N,), 0.01, 1e-4, torch.float32),
    )


C6 = 6  # FP8 W8A8 with blockwise scales


def fp8_codes(seed, cfg, tensor, shape) -> np.ndarray:
    """E4M3 codes drawn uniformly over the finite codes (0x7F / 0xFF, the NaNs, excluded)."""
    c = _rng(seed, cfg, tensor).integers(0, 254, size=shape, dtype=np.int64)
    c = c + (c >= 0x7F) # skip 0x7F
    return c.astype(np.uint8)


def w8a8_fp8_blockwise(seed, M, N, K, cfg=C6):
    """FP8 W8A8 with blockwise scales: fp32 activations (quantised per 1 x 128 block
    by the consumer), E4M3 weight codes [K, N] uniform over the finite codes, fp32
    weight scales |N(0, 0.01)| + 1e-4 per 128 x 128 block [K/128, ceil(N/128)]."""
    return dict(
        A0=normal_rows(seed, cfg, T_A, M, K),
        w=fp8_codes(seed, cfg, T_Q, (K, N)),
        s_w=abs_normal_scales(seed, cfg, T_SW, (K // 128, (N + 127) // 128), 0.01, 1e-4, torch.float32),
    )


C7 = 7  # FP4 weights with 16-bit activations (MXFP4 / NVFP4 WnA16)


def w4a16_fp4(seed, M, N, K, nvfp4: bool, dtype=torch.bfloat16, cfg=C7):
    """FP4 WnA16: N(0,1) activations rounded to bf16/fp16, e2m1 codes uniform over all 16,
    MXFP4: E8M0 exponents in [118, 127] per 32 K; NVFP4: E4M3 scales per 16 K drawn as
    |N(0, 0.1)| + 0.01 rounded to E4M3 (torch's cast) and a per-tensor fp32 scale."""
    out = dict(A=activations(seed, cfg, M, K, dtype), q=random_words(seed, cfg, T_Q, (K // 8, N)))
    if nvfp4:
        v = np.abs(_rng(seed, cfg, T_S).standard_normal((K // 16, N), dtype=np.float32)) * np.float32(0.1) + np.float32(0.01)
        out["s"] = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
        out["s2"] = float(np.float32(np.abs(_rng(seed, cfg, T_Z).standard_normal()) * 0.5 + 0.25))
    else:
        out["s"] = e8m0_exponents(seed, cfg, (K // 32, N))
    return out


C8 = 8  # MXINT4 weights with 16-bit activations


def w4a16_mxint4(seed, M, N, K, dtype=torch.bfloat16, cfg=C8):
    """MXINT4 WnA16: N(0,1) activations rounded to bf16, INT4 codes uniform over all 16
    (two's complement -8..7), E8M0 exponents in [118, 127] per 32 K."""
    return dict(A=activations(seed, cfg, M, K, dtype), q=random_words(seed, cfg, T_Q, (K // 8, N)),
                e=e8m0_exponents(seed, cfg, (K // 32, N)))


C9 = 9  # INT8 weight-only (W8A16)


def w8a16_int8(seed, M, N, K, dtype=torch.bfloat16, cfg=C9):
    """INT8 weight-only: N(0,1) activations rounded to bf16/fp16, INT8 weights uniform
    over the full two's-complement range [-128, 127], fp32 per-column scales |N(0,0.01)|+1e-4."""
    return dict(A=activations(seed, cfg, M, K, dtype), w=int8_uniform(seed, cfg, T_Q, (K, N), lo=-128, hi=127),
                s_w=abs_normal_scales(seed, cfg, T_SW, (N,), 0.01, 1e-4, torch.float32))


C10 = 10  # FP8 weight-only


def w8a16_fp8(seed, M, N, K, dtype=torch.bfloat16, cfg=C10):
    """FP8 weight-only: N(0,1) activations rounded to bf16/fp16, E4M3 weight codes uniform
    over the finite codes, fp32 per-column scales |N(0,0.01)|+1e-4."""
    return dict(A=activations(seed, cfg, M, K, dtype), w=fp8_codes(seed, cfg, T_Q, (K, N)),
                s_w=abs_normal_scales(seed, cfg, T_SW, (N,), 0.01, 1e-4, torch.float32))


def moe_expert_mxfp4(seed, e, N, K, cfg=C5):
    """One expert's MXFP4 weights (codes + E8M0), drawn from the expert's own stream."""
    return (random_words(seed, cfg, T_Q, (K // 8, N), e),
            e8m0_exponents(seed, cfg, (K // 32, N), 118, 127, e))


def moe_mxfp4(seed, T, E, top_k, N, K, cfg=C5, experts=None):
    """MoE W4A16-MXFP4: bf16 tokens, Zipf(1.1) routing, expert-stacked weights.

    ``experts`` (optional) limits which experts' weights are materialised
    (others are left as zeros); ``None`` means all.
    """
    q = np.zeros((E, K // 8, N), dtype=np.uint32)
    ex = np.full((E, K // 32, N), 127, dtype=np.uint8)
    for e in (range(E) if experts is None else experts):
        q[e], ex[e] = moe_expert_mxfp4(seed, e, N, K, cfg)
    return dict(
        A=activations(seed, cfg, T, K, torch.bfloat16),
        ids=zipf_topk(seed, cfg, T, E, top_k),
        q=q, e=ex,
    )


C11 = 11  # low-bit WnA16 (1, 2 or 3-bit codes)


def wnlow(seed, M, N, K, bits, signed, G=128, dtype=torch.float16, cfg=C11):
    """Low-bit WnA16: one code per byte [K][N], uniform over the width (two's
    complement for signed widths, 0 .. 2^bits - 1 otherwise); 16-bit group scales
    |N(0, 0.02)| + 1e-3 (wider steps for narrower codes do not change the test's
    character); unsigned widths take UINT4-container zero-points uniform in
    [0, 2^bits - 1]."""
    lo, hi = (-(1 << (bits - 1)), (1 << (bits - 1)) - 1) if signed else (0, (1 << bits) - 1)
    codes = _rng(seed, cfg, T_Q, bits).integers(lo, hi + 1, size=(K, N), dtype=np.int64).astype(np.int8)
    out = dict(A=activations(seed, cfg, M, K, dtype), codes=codes,
               s=abs_normal_scales(seed, cfg, T_S, (K // G, N), 0.02, 1e-3, dtype))
    if not signed:
        zn = _rng(seed, cfg, T_Z, bits).integers(0, 1 << bits, size=(K // G, (N + 7) // 8 * 8), dtype=np.int64)
        words = np.zeros((K // G, (N + 7) // 8), dtype=np.uint32)
        for i in range(8):
            words |= (zn[:, i::8].astype(np.uint32) << np.uint32(4 * i))
        out["z"] = words
    return out


C12 = 12  # MX-scaled float weights (MXFP8 E4M3, MXFP6 E2M3 / E3M2) with 16-bit activations


def mxf_a16(seed, M, N, K, elem, dtype=torch.bfloat16, cfg=C12):
    """MX float WnA16: N(0,1) activations rounded to bf16, one code per byte [K][N]
    (E4M3 uniform over the finite codes; FP6 uniform over all 64 six-bit codes),
    E8M0 exponents in [118, 127] per 32 K."""
    if elem == "e4m3":
        codes = fp8_codes(seed, cfg, T_Q, (K, N))
    else:
        codes = _rng(seed, cfg, T_Q, {"e2m3": 1, "e3m2": 2}[elem]).integers(0, 64, size=(K, N)).astype(np.uint8)
    return dict(A=activations(seed, cfg, M, K, dtype), codes=codes, e=e8m0_exponents(seed, cfg, (K // 32, N)))


C13 = 13  # WnA16 at 5-8 bits


def wnwide(seed, M, N, K, bits, signed, G=128, dtype=torch.float16, cfg=C13):
    """WnA16 at 5-8 bits: one code per byte [K][N] uniform over the width (int8 two's
    complement for signed widths, uint8 0 .. 2^bits - 1 otherwise), 16-bit group scales
    |N(0, 0.002)| + 1e-4 (the finer steps of a wider code), 8-bit zero-points uniform
    over the width for unsigned widths."""
    lo, hi = (-(1 << (bits - 1)), (1 << (bits - 1)) - 1) if signed else (0, (1 << bits) - 1)
    v = _rng(seed, cfg, T_Q, bits).integers(lo, hi + 1, size=(K, N), dtype=np.int64)
    codes = v.astype(np.int8) if signed else v.astype(np.uint8)
    out = dict(A=activations(seed, cfg, M, K, dtype), codes=codes,
               s=abs_normal_scales(seed, cfg, T_S, (K // G, N), 0.002, 1e-4, dtype))
    if not signed:
        out["z"] = _rng(seed, cfg, T_Z, bits).integers(0, 1 << bits, size=(K // G, N), dtype=np.int64).astype(np.uint8)
    return out

