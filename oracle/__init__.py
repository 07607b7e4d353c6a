"""CPU oracle for the quantized GEMM (test infrastructure only).

Only the test-suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The library never does.  It shares no
code with the HIP path: the arithmetic lives in ``hq_oracle.c`` (plain C,
fp64 accumulation) and this module only marshals numpy arrays into it.

Functions mirror the C entry points; each returns fp64 outputs for the
requested rows (all rows when ``rows`` is None).  Functions that the pages
and the mathematics pin are listed with their pins in the test-suite
(``tests/test_oracle_pins.py``).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hq_oracle.c")
# HQ_ORACLE_LIB_PATH names another build of the oracle (the host-sanitizer build)
_LIB = os.environ.get("HQ_ORACLE_LIB_PATH") or os.path.join(_HERE, "liboracle.so")


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no FP contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                               "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = C.CDLL(_LIB)
        d, i64, p = C.c_double, C.c_int64, C.c_void_p
        L.hq_oracle_e2m1.restype = d
        L.hq_oracle_e2m1.argtypes = [C.c_uint]
        L.hq_oracle_e8m0.restype = d
        L.hq_oracle_e8m0.argtypes = [C.c_uint]
        L.hq_oracle_e4m3.restype = d
        L.hq_oracle_e4m3.argtypes = [C.c_uint]
        L.hq_oracle_e4m3_encode.restype = C.c_uint
        L.hq_oracle_e4m3_encode.argtypes = [C.c_float]
        L.hq_oracle_bf16.restype = d
        L.hq_oracle_bf16.argtypes = [C.c_uint16]
        L.hq_oracle_fp16.restype = d
        L.hq_oracle_fp16.argtypes = [C.c_uint16]
        L.hq_oracle_quant_act_e4m3.restype = None
        L.hq_oracle_quant_act_e4m3.argtypes = [i64, i64, p, p, p]
        L.hq_oracle_gemm_wna16.restype = C.c_int
        L.hq_oracle_gemm_wna16.argtypes = [i64, i64, i64, i64, C.c_int, p, C.c_int, p, p, p, p, i64, p]
        L.hq_oracle_gemm_wnlow.restype = C.c_int
        L.hq_oracle_gemm_wnlow.argtypes = [i64, i64, i64, i64, C.c_int, C.c_int, C.c_int, p, p, p, p, p, i64, p]
        L.hq_oracle_gemm_w4a8_mxfp4.restype = C.c_int
        L.hq_oracle_gemm_wnwide.restype = C.c_int
        L.hq_oracle_gemm_wnwide.argtypes = [i64, i64, i64, i64, C.c_int, C.c_int, C.c_int, p, p, p, p, p, i64, p]
        L.hq_oracle_gemm_w4a8_mxfp4.argtypes = [i64, i64, i64, p, p, p, p, p, i64, p]
        L.hq_oracle_e2m1_encode.restype = C.c_uint
        L.hq_oracle_e2m1_encode.argtypes = [d]
        L.hq_oracle_quant_act_mx.restype = C.c_int
        L.hq_oracle_quant_act_mx.argtypes = [i64, i64, C.c_int, p, p, p]
        L.hq_oracle_gemm_mx_mxfp4.restype = C.c_int
        L.hq_oracle_gemm_mx_mxfp4.argtypes = [i64, i64, i64, C.c_int, p, p, p, p, p, i64, p]
        L.hq_oracle_quant_act_e4m3_blocks.restype = C.c_int
        L.hq_oracle_quant_act_e4m3_blocks.argtypes = [i64, i64, i64, p, p, p]
        L.hq_oracle_gemm_fp8_blockwise.restype = C.c_int
        L.hq_oracle_gemm_fp8_blockwise.argtypes = [i64, i64, i64, p, p, p, p, p, i64, p]
        L.hq_oracle_gemm_fp4_a16.restype = C.c_int
        L.hq_oracle_gemm_fp4_a16.argtypes = [i64, i64, i64, C.c_int, p, p, C.c_int, p, p, p, i64, p]
        L.hq_oracle_e0m.restype = C.c_double
        L.hq_oracle_e0m.argtypes = [C.c_uint, C.c_int, p]
        L.hq_oracle_fp6.restype = C.c_double
        L.hq_oracle_fp6.argtypes = [C.c_uint, C.c_int]
        L.hq_oracle_gemm_mxf_a16.restype = C.c_int
        L.hq_oracle_gemm_mxf_a16.argtypes = [i64, i64, i64, C.c_int, p, C.c_int, p, p, p, i64, p]
        L.hq_oracle_gemm_fp8w_a16.restype = C.c_int
        L.hq_oracle_gemm_fp8w_a16.argtypes = [i64, i64, i64, C.c_int, p, p, p, p, i64, p]
        L.hq_oracle_gemm_w8a16.restype = C.c_int
        L.hq_oracle_gemm_w8a16.argtypes = [i64, i64, i64, C.c_int, p, p, p, p, i64, p]
        L.hq_oracle_gemm_mxint4_a16.restype = C.c_int
        L.hq_oracle_gemm_mxint4_a16.argtypes = [i64, i64, i64, C.c_int, p, p, p, p, i64, p]
        L.hq_oracle_gemm_w8a8.restype = C.c_int
        L.hq_oracle_gemm_w8a8.argtypes = [i64, i64, i64, p, p, p, p, p, i64, p, p]
        L.hq_oracle_moe_route.restype = C.c_int
        L.hq_oracle_moe_route.argtypes = [i64, i64, i64, p, p, p, p]
        L.hq_oracle_bf16_encode.restype = C.c_uint16
        L.hq_oracle_bf16_encode.argtypes = [d]
        L.hq_oracle_silu_mul_bf16.restype = None
        L.hq_oracle_silu_mul_bf16.argtypes = [i64, i64, p, p]
        L.hq_oracle_moe_mxfp4_bf16.restype = C.c_int
        L.hq_oracle_moe_mxfp4_bf16.argtypes = [i64, i64, i64, i64, i64, p, p, p, p, p, i64, p]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _rows(rows, M):
    if rows is None:
        return None, M
    r = np.ascontiguousarray(rows, dtype=np.int64)
    assert r.ndim == 1 and (r.size == 0 or (r.min() >= 0 and r.max() < M))
    return r, r.size


# scalar decoders ---------------------------------------------------------

def e2m1(code: int) -> float:
    return lib().hq_oracle_e2m1(code)


def e8m0(e: int) -> float:
    return lib().hq_oracle_e8m0(e)


def e4m3(code: int) -> float:
    return lib().hq_oracle_e4m3(code)


def e0m(code: int, n: int) -> float:
    """Zero-exponent float e0mN: sign bit n, integer magnitude in bits 0..n-1."""
    ok = C.c_int(0)
    v = lib().hq_oracle_e0m(code, n, C.byref(ok))
    if not ok.value:
        raise ValueError(f"e0m{n} code 0x{code:x} has bits above bit {n}")
    return v


def e0m_to_int(codes, n: int) -> np.ndarray:
    """Array of e0mN codes -> their integer values (int8), through the scalar decode."""
    codes = np.asarray(codes)
    lut = np.array([e0m(c, n) for c in range(1 << (n + 1))], dtype=np.int64)
    if codes.size and int(codes.max()) >= (1 << (n + 1)):
        raise ValueError(f"e0m{n} codes above {(1 << (n + 1)) - 1}")
    return lut[codes.astype(np.int64)].astype(np.int8)


def fp6(code: int, e3m2: bool) -> float:
    """OCP MX FP6 decode: E2M3 (e3m2 False) or E3M2 (e3m2 True), 6-bit code."""
    return lib().hq_oracle_fp6(code, int(e3m2))


def e4m3_encode(x: float) -> int:
    return lib().hq_oracle_e4m3_encode(x)


def bf16(bits: int) -> float:
    return lib().hq_oracle_bf16(bits)


def fp16(bits: int) -> float:
    return lib().hq_oracle_fp16(bits)


# activation quantisation -------------------------------------------------

def quant_act_e4m3(x: np.ndarray):
    """Tokenwise E4M3: returns (codes uint8 [M,K], scales fp32 [M])."""
    x = _c(x, np.float32)
    M, K = x.shape
    q = np.empty((M, K), dtype=np.uint8)
    s = np.empty((M,), dtype=np.float32)
    lib().hq_oracle_quant_act_e4m3(M, K, _ptr(x), _ptr(q), _ptr(s))
    return q, s


def quant_act_e4m3_blocks(x: np.ndarray, block: int):
    """E4M3 activations with one fp32 scale per (row, block of `block` along K):
    returns (codes uint8 [M,K], scales fp32 [M,K/block]); block == K is tokenwise."""
    x = _c(x, np.float32)
    M, K = x.shape
    q = np.empty((M, K), dtype=np.uint8)
    s = np.empty((M, K // block), dtype=np.float32)
    if lib().hq_oracle_quant_act_e4m3_blocks(M, K, block, _ptr(x), _ptr(q), _ptr(s)):
        raise ValueError("K must be a multiple of the block")
    return q, s


def e2m1_encode(x: float) -> int:
    """E2M1 code of x: nearest, ties to even, saturating at +-6 (sign kept)."""
    return int(lib().hq_oracle_e2m1_encode(float(x)))


def quant_act_mx(x: np.ndarray, elem: str):
    """MX activations (OCP MX v1.0, one E8M0 scale per 32 along K): elem 'e4m3'
    -> (codes uint8 [M,K], scales uint8 [M,K/32]); elem 'e2m1' -> (codes
    uint8 [M,K/2] two per byte, low nibble first, scales uint8 [M,K/32])."""
    x = _c(x, np.float32)
    M, K = x.shape
    fp4 = elem == "e2m1"
    assert fp4 or elem == "e4m3"
    q = np.zeros((M, K // 2 if fp4 else K), dtype=np.uint8)
    e = np.empty((M, K // 32), dtype=np.uint8)
    if lib().hq_oracle_quant_act_mx(M, K, int(fp4), _ptr(x), _ptr(q), _ptr(e)):
        raise ValueError("K must be a multiple of 32")
    return q, e


# GEMMs -----------------------------------------------------------------

def gemm_wna16(A, q, s, z=None, *, N, K, G, a_bf16: bool, w_signed: bool, rows=None):
    A = _c(A, np.uint16)
    M = A.shape[0]
    r, R = _rows(rows, M)
    out = np.empty((R, N), dtype=np.float64)
    rc = lib().hq_oracle_gemm_wna16(M, N, K, G, int(a_bf16), _ptr(A), int(w_signed), _ptr(_c(q, np.uint32)),
                                    _ptr(_c(s, np.uint16)), _ptr(_c(z, np.uint32)), _ptr(r), R, _ptr(out))
    if rc:
        raise ValueError(f"oracle gemm_wna16 failed ({rc})")
    return out


def gemm_wnlow(A, codes, s, z=None, *, N, K, G, bits: int, a_bf16: bool, w_signed: bool, rows=None):
    """Low-bit WnA16 (1, 2 or 3-bit codes, one per byte [K][N]; signed, or unsigned
    with UINT4-container zero-points), fp64."""
    A = _c(A, np.uint16)
    M = A.shape[0]
    r, R = _rows(rows, M)
    out = np.empty((R, N), dtype=np.float64)
    rc = lib().hq_oracle_gemm_wnlow(M, N, K, G, int(a_bf16), int(bits), int(w_signed), _ptr(A),
                                    _ptr(_c(codes, np.int8)), _ptr(_c(s, np.uint16)), _ptr(_c(z, np.uint32)),
                                    _ptr(r), R, _ptr(out))
    if rc:
        raise ValueError(f"oracle gemm_wnlow failed ({rc})")
    return out


def gemm_w4a8_mxfp4(qa, s_a, q, e, *, N, K, rows=None):
    qa = _c(qa, np.uint8)
    M = qa.shape[0]
    r, R = _rows(rows, M)
    out = np.empty((R, N), dtype=np.float64)
    rc = lib().hq_oracle_gemm_w4a8_mxfp4(M, N, K, _ptr(qa), _ptr(_c(s_a, np.float32)), _ptr(_c(q, np.uint32)),
                                         _ptr(_c(e, np.uint8)), _ptr(r), R, _ptr(out))
    if rc:
        raise ValueError(f"oracle gemm_w4a8_mxfp4 failed ({rc})")
    return out


def gemm_mx_mxfp4(qa, ea, q, e, *, N, K, a_elem: str, rows=None):
    """MX activations (E4M3 or E2M1 codes + E8M0 per 32) x MXFP4 weights, fp64."""
    qa = _c(qa, np.uint8)
    M = qa.shape[0]
    r, R = _rows(rows, M)
    out = np.empty((R, N), dtype=np.float64)
    rc = lib().hq_oracle_gemm_mx_mxfp4(M, N, K, int(a_elem == "e2m1"), _ptr(qa), _ptr(_c(ea, np.uint8)),
                                       _ptr(_c(q, np.uint32)), _ptr(_c(e, np.uint8)), _ptr(r), R, _ptr(out))
    if rc:
        raise ValueError(f"oracle gemm_mx_mxfp4 failed ({rc})")
    return out


def gemm_fp4_a16(A, q, scales, *, N, K, a_bf16: bool, nvfp4: bool, s2=None, rows=None):
    """FP4 (e2m1) weights with 16-bit activations: MXFP4 (E8M0 per 32 K) or NVFP4
    (E4M3 per 16 K, times the per-tensor fp32 second-level scale s2), fp64."""
    A = _c(A, np.uint16)
    M = A.shape[0]
    r, R = _rows(rows, M)
    out = np.empty((R, N), dtype=np.float64)
    s2a = None if s2 is None else np.array([s2], dtype=np.float32)
    rc = lib().hq_oracle_gemm_fp4_a16(M, N, K, int(a_bf16), _ptr(A), _ptr(_c(q, np.uint32)), int(nvfp4),
                                      _ptr(_c(scales, np.uint8)), _ptr(s2a), _ptr(r), R, _ptr(out))
    if rc:
        raise ValueError(f"oracle gemm_fp4_a16 failed ({rc})")
    return out


def gemm_mxint4_a16(A, q, e8, *, N, K, a_bf16: bool = True, rows=None):
    """MXINT4 weights (two's-complement INT4, E8M0 per 32 K) with 16-bit activations, fp64."""
    A = _c(A, np.uint16)
    M = A.shape[0]
    r, R = _rows(rows, M)
    out = np.empty((R, N), dtype=np.float64)
    rc = lib().hq_oracle_gemm_mxint4_a16(M, N, K, int(a_bf16), _ptr(A), _ptr(_c(q, np.uint32)),
                                         _ptr(_c(e8, np.uint8)), _ptr(r), R, _ptr(out))
    if rc:
        raise ValueError(f"oracle gemm_mxint4_a16 failed ({rc})")
    return out


def gemm_w8a16(A, w, s_w, *, a_bf16: bool, rows=None):
    """INT8 weight-only: 16-bit activations x INT8 weights [K][N], fp32 per-column scales, fp64."""
    A = _c(A, np.uint16)
    w = _c(w, np.int8)
    M, K = A.shape
    N = w.shape[1]
    r, R = _rows(rows, M)
    out = np.empty((R, N), dtype=np.float64)
    rc = lib().hq_oracle_gemm_w8a16(M, N, K, int(a_bf16), _ptr(A), _ptr(w), _ptr(_c(s_w, np.float32)), _ptr(r), R,
                                    _ptr(out))
    if rc:
        raise ValueError(f"oracle gemm_w8a16 failed ({rc})")
    return out


def gemm_fp8w_a16(A, w, s_w, *, a_bf16: bool, rows=None):
    """FP8 weight-only: 16-bit activations x E4M3 weight codes [K][N], fp32 per-column scales, fp64."""
    A = _c(A, np.uint16)
    w = _c(w, np.uint8)
    M, K = A.shape
    N = w.shape[1]
    r, R = _rows(rows, M)
    out = np.empty((R, N), dtype=np.float64)
    rc = lib().hq_oracle_gemm_fp8w_a16(M, N, K, int(a_bf16), _ptr(A), _ptr(w), _ptr(_c(s_w, np.float32)), _ptr(r),
                                       R, _ptr(out))
    if rc:
        raise ValueError(f"oracle gemm_fp8w_a16 failed ({rc})")
    return out


MXF_ELEMS = {"e4m3": 0, "e2m3": 1, "e3m2": 2}


def gemm_mxf_a16(A, codes, e8, *, elem: str, a_bf16: bool = True, rows=None):
    """MX-scaled float weights (MXFP8 E4M3, MXFP6 E2M3 / E3M2: one code per byte
    [K][N], E8M0 per 32 K [K/32][N]) with 16-bit activations, fp64."""
    A = _c(A, np.uint16)
    codes = _c(codes, np.uint8)
    M, K = A.shape
    N = codes.shape[1]
    r, R = _rows(rows, M)
    out = np.empty((R, N), dtype=np.float64)
    rc = lib().hq_oracle_gemm_mxf_a16(M, N, K, int(a_bf16), _ptr(A), MXF_ELEMS[elem], _ptr(codes),
                                      _ptr(_c(e8, np.uint8)), _ptr(r), R, _ptr(out))
    if rc:
        raise ValueError(f"oracle gemm_mxf_a16 failed ({rc})")
    return out


def gemm_wnwide(A, codes, s, z8=None, *, N, K, G, bits: int, a_bf16: bool, w_signed: bool, rows=None):
    """WnA16 at 5-8 bits: one code per byte [K][N] (int8 for signed widths, uint8
    otherwise), 16-bit group scales [K/G][N], 8-bit zero-points [K/G][N] for
    unsigned widths; fp64."""
    A = _c(A, np.uint16)
    M = A.shape[0]
    r, R = _rows(rows, M)
    out = np.empty((R, N), dtype=np.float64)
    rc = lib().hq_oracle_gemm_wnwide(M, N, K, G, int(a_bf16), bits, int(w_signed), _ptr(A),
                                     _ptr(np.ascontiguousarray(codes).view(np.uint8)), _ptr(_c(s, np.uint16)),
                                     _ptr(_c(z8, np.uint8)), _ptr(r), R, _ptr(out))
    if rc:
        raise ValueError(f"oracle gemm_wnwide failed ({rc})")
    return out


def gemm_fp8_blockwise(qa, sa, w, sw, *, rows=None):
    """FP8 W8A8 with blockwise scales (1 x 128 activation blocks, 128 x 128 weight blocks), fp64."""
    qa = _c(qa, np.uint8)
    w = _c(w, np.uint8)
    M, K = qa.shape
    N = w.shape[1]
    r, R = _rows(rows, M)
    out = np.empty((R, N), dtype=np.float64)
    rc = lib().hq_oracle_gemm_fp8_blockwise(M, N, K, _ptr(qa), _ptr(_c(sa, np.float32)), _ptr(w),
                                            _ptr(_c(sw, np.float32)), _ptr(r), R, _ptr(out))
    if rc:
        raise ValueError(f"oracle gemm_fp8_blockwise failed ({rc})")
    return out


def gemm_w8a8(a, s_a, w, s_w, *, rows=None):
    a = _c(a, np.int8)
    w = _c(w, np.int8)
    M, K = a.shape
    N = w.shape[1]
    r, R = _rows(rows, M)
    acc = np.empty((R, N), dtype=np.int64)
    out = np.empty((R, N), dtype=np.float64)
    rc = lib().hq_oracle_gemm_w8a8(M, N, K, _ptr(a), _ptr(_c(s_a, np.float32)), _ptr(w), _ptr(_c(s_w, np.float32)),
                                   _ptr(r), R, _ptr(acc), _ptr(out))
    if rc == 3:
        raise OverflowError("int32 accumulator overflow")
    if rc:
        raise ValueError(f"oracle gemm_w8a8 failed ({rc})")
    return acc, out


def bf16_encode(x: float) -> int:
    """bf16 bits of x, round to nearest even."""
    return int(lib().hq_oracle_bf16_encode(float(x)))


def silu_mul_bf16(x: np.ndarray) -> np.ndarray:
    """SwiGLU between the MoE projections ("Humming wird angekuendigt", section
    "Leistung"): x [rows][2I] bf16 bits (gate | up) -> bf16 bits [rows][I] of
    silu(gate) * up in double, rounded once to nearest even."""
    rows, two_i = x.shape
    I = two_i // 2
    src = _c(x, np.uint16)
    out = np.empty((rows, I), dtype=np.uint16)
    lib().hq_oracle_silu_mul_bf16(rows, I, _ptr(src), _ptr(out))
    return out


def moe_route(ids: np.ndarray, E: int):
    """Returns (counts [E], offsets [E+1], perm [T*top_k]) as int64."""
    ids = _c(ids, np.int32)
    T, top_k = ids.shape
    counts = np.empty(E, dtype=np.int64)
    offsets = np.empty(E + 1, dtype=np.int64)
    perm = np.empty(T * top_k, dtype=np.int64)
    if lib().hq_oracle_moe_route(T, top_k, E, _ptr(ids), _ptr(counts), _ptr(offsets), _ptr(perm)):
        raise ValueError("bad expert id")
    return counts, offsets, perm


def moe_mxfp4_bf16(A, ids, q, e, *, N, K, pairs=None):
    """Rows of the Indexed output ``[T*top_k, N]`` for the listed pairs (all when None)."""
    A = _c(A, np.uint16)
    ids = _c(ids, np.int32)
    T, top_k = ids.shape
    E = q.shape[0]
    p = np.arange(T * top_k, dtype=np.int64) if pairs is None else np.ascontiguousarray(pairs, dtype=np.int64)
    out = np.empty((p.size, N), dtype=np.float64)
    rc = lib().hq_oracle_moe_mxfp4_bf16(T, top_k, E, N, K, _ptr(A), _ptr(ids), _ptr(_c(q, np.uint32)),
                                        _ptr(_c(e, np.uint8)), _ptr(p), p.size, _ptr(out))
    if rc:
        raise ValueError(f"oracle moe failed ({rc})")
    return out
