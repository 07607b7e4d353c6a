"""ctypes binding of libhq (include/hq.h).  Argument marshalling only.

Every function here has the name of the C entry point it wraps and calls it
directly; all arithmetic runs in the library's HIP kernels (device entry
points) or its C++ repack (host).  PyTorch is used only to hold device memory
and to name the current HIP stream.  A missing library raises at import of
the first call: there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# HQ_LIB_PATH names another build of the same library (the host-sanitizer build)
LIB_PATH = os.environ.get("HQ_LIB_PATH") or os.path.join(_HERE, "libhq.so")

HQ_ABI_VERSION = 1

# hq_status
HQ_OK, HQ_ERR_INVALID_ARG, HQ_ERR_UNSUPPORTED, HQ_ERR_ALIGNMENT, HQ_ERR_WORKSPACE, HQ_ERR_ABI, HQ_ERR_HIP = range(7)
# hq_dtype
(HQ_DT_NONE, HQ_DT_BF16, HQ_DT_FP16, HQ_DT_FP32, HQ_DT_FP8_E4M3, HQ_DT_INT8, HQ_DT_INT4, HQ_DT_UINT4,
 HQ_DT_FP4_E2M1, HQ_DT_E8M0, HQ_DT_INT32, HQ_DT_INT1, HQ_DT_UINT1, HQ_DT_INT2, HQ_DT_UINT2, HQ_DT_INT3,
 HQ_DT_UINT3, HQ_DT_FP6_E2M3, HQ_DT_FP6_E3M2, HQ_DT_E0M1, HQ_DT_E0M2, HQ_DT_E0M3, HQ_DT_E0M7, HQ_DT_INT5, HQ_DT_UINT5,
 HQ_DT_INT6, HQ_DT_UINT6, HQ_DT_INT7, HQ_DT_UINT7, HQ_DT_UINT8, HQ_DT_E0M4, HQ_DT_E0M5, HQ_DT_E0M6) = range(33)
HQ_GRAN_NONE, HQ_GRAN_PER_GROUP_K, HQ_GRAN_PER_CHANNEL, HQ_GRAN_BLOCK_128x128 = range(4)
HQ_ASCALE_NONE, HQ_ASCALE_PER_TOKEN_F32, HQ_ASCALE_MX_E8M0, HQ_ASCALE_PER_BLOCK128_F32 = range(4)
HQ_S2_NONE, HQ_S2_PER_TENSOR_F32 = 0, 1
HQ_MOE_INDEXED, HQ_MOE_GROUPED = 1, 2
HQ_FLAG_BATCH_INVARIANT = 1
HQ_TUNE_STREAM, HQ_TUNE_T128, HQ_TUNE_T256, HQ_TUNE_W128, HQ_TUNE_W256, HQ_TUNE_STREAM8 = 1, 2, 3, 4, 5, 6


def HQ_TUNE(path: int, splits: int = 0) -> int:
    return int(path) | (int(splits) << 8)


class HQError(RuntimeError):
    def __init__(self, status: int, where: str, msg: str):
        super().__init__(f"{where}: status {status}: {msg}")
        self.status = status


class hq_layer_desc(C.Structure):
    _fields_ = [
        ("abi_version", C.c_int32), ("num_experts", C.c_int32),
        ("N", C.c_int64), ("K", C.c_int64),
        ("a_dtype", C.c_int32), ("a_scale", C.c_int32), ("w_dtype", C.c_int32),
        ("w_scale_dtype", C.c_int32), ("w_scale_gran", C.c_int32), ("group_size", C.c_int32),
        ("zp_dtype", C.c_int32), ("scale2", C.c_int32), ("out_dtype", C.c_int32),
        ("flags", C.c_int32), ("tune", C.c_int32), ("reserved", C.c_int32),
    ]


_lib = None

_P = C.c_void_p
_SIGS = {
    "hq_abi_version": (C.c_int32, []),
    "hq_status_str": (C.c_char_p, [C.c_int]),
    "hq_last_error": (C.c_char_p, []),
    "hq_desc_validate": (C.c_int, [_P]),
    "hq_repacked_bytes": (C.c_int, [_P, _P, _P, _P, _P]),
    "hq_repack": (C.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "hq_workspace_bytes": (C.c_int, [_P, C.c_int64, C.c_int32, _P]),
    "hq_workspace_init": (C.c_int, [_P, C.c_size_t, _P]),
    "hq_gemm": (C.c_int, [_P, C.c_int64, _P, _P, _P, _P, _P, _P, _P, _P, C.c_size_t, _P]),
    "hq_gemm_plan": (C.c_int, [_P, C.c_int64, C.c_char_p, C.c_size_t]),
    "hq_gemm_noalloc": (C.c_int, [_P, C.c_int64, _P, _P, _P, _P, _P, _P, _P, _P]),
    "hq_moe_gemm": (C.c_int, [_P, C.c_int32, C.c_int64, C.c_int32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                              C.c_size_t, _P]),
    "hq_quantize_act": (C.c_int, [C.c_int32, C.c_int64, C.c_int64, _P, _P, _P, _P]),
    "hq_quantize_act_mx": (C.c_int, [C.c_int32, C.c_int64, C.c_int64, _P, _P, _P, _P]),
    "hq_quantize_act_blocks": (C.c_int, [C.c_int32, C.c_int64, C.c_int64, C.c_int64, _P, _P, _P, _P]),
    "hq_moe_align": (C.c_int, [C.c_int64, C.c_int32, C.c_int32, _P, _P, _P, _P, C.c_size_t, _P]),
    "hq_moe_gather": (C.c_int, [C.c_int32, C.c_int64, C.c_int32, C.c_int64, _P, _P, _P, _P]),
    "hq_silu_mul": (C.c_int, [C.c_int32, C.c_int64, C.c_int64, _P, _P, _P]),
    "hq_probe_stream": (C.c_int, [_P, C.c_size_t, _P, C.c_int32, _P]),
    "hq_probe_mfma": (C.c_int, [C.c_int32, C.c_int64, C.c_int32, _P, _P]),
}


def lib() -> C.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libhq.so not built at {LIB_PATH}: run python -m bit_quantized_gemm_w4a16_amd.build")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        if L.hq_abi_version() != HQ_ABI_VERSION:
            raise ImportError("libhq ABI version mismatch")
        _lib = L
    return _lib


def _check(status: int, where: str):
    if status != HQ_OK:
        raise HQError(status, where, lib().hq_last_error().decode())


def _dp(t):
    """Device (or host numpy) pointer of a tensor/array; None -> NULL."""
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ---------------------------------------------------------------------------
# descriptors
# ---------------------------------------------------------------------------

def make_desc(N, K, a_dtype, w_dtype, w_scale_dtype, w_scale_gran, group_size, out_dtype,
              zp_dtype=HQ_DT_NONE, a_scale=HQ_ASCALE_NONE, num_experts=0) -> hq_layer_desc:
    d = hq_layer_desc()
    d.abi_version = HQ_ABI_VERSION
    d.num_experts = num_experts
    d.N, d.K = N, K
    d.a_dtype, d.a_scale, d.w_dtype = a_dtype, a_scale, w_dtype
    d.w_scale_dtype, d.w_scale_gran, d.group_size = w_scale_dtype, w_scale_gran, group_size
    d.zp_dtype, d.scale2, d.out_dtype = zp_dtype, HQ_S2_NONE, out_dtype
    return d


def desc_w4a16(N, K, group_size=128, bf16=True, zp=False) -> hq_layer_desc:
    a = HQ_DT_BF16 if bf16 else HQ_DT_FP16
    return make_desc(N, K, a, HQ_DT_UINT4 if zp else HQ_DT_INT4, a, HQ_GRAN_PER_GROUP_K, group_size, a,
                     zp_dtype=HQ_DT_UINT4 if zp else HQ_DT_NONE)


def desc_mxf_a16(N, K, elem, bf16: bool = True) -> hq_layer_desc:
    """16-bit activations x MX float weights: elem "e4m3" (MXFP8), "e2m3" or "e3m2"
    (MXFP6), one E8M0 scale per 32 K."""
    a = HQ_DT_BF16 if bf16 else HQ_DT_FP16
    w = {"e4m3": HQ_DT_FP8_E4M3, "e2m3": HQ_DT_FP6_E2M3, "e3m2": HQ_DT_FP6_E3M2}[elem]
    return make_desc(N, K, a, w, HQ_DT_E8M0, HQ_GRAN_PER_GROUP_K, 32, a)


def desc_e0m(N, K, n, group_size=128, bf16=True) -> hq_layer_desc:
    """Zero-exponent float weights e0mN: n = 1..6 with 16-bit group scales (the
    WnA16 kernels of width n + 1), n = 7 with fp32 per-channel scales (INT8 weight-only)."""
    a = HQ_DT_BF16 if bf16 else HQ_DT_FP16
    w = {1: HQ_DT_E0M1, 2: HQ_DT_E0M2, 3: HQ_DT_E0M3, 4: HQ_DT_E0M4, 5: HQ_DT_E0M5, 6: HQ_DT_E0M6, 7: HQ_DT_E0M7}[n]
    if n == 7:
        return make_desc(N, K, a, w, HQ_DT_FP32, HQ_GRAN_PER_CHANNEL, K, a)
    return make_desc(N, K, a, w, a, HQ_GRAN_PER_GROUP_K, group_size, a)


def desc_wnwide(N, K, bits, signed, group_size=128, bf16=True) -> hq_layer_desc:
    """WnA16 at 5-8 bits: 16-bit group scales; unsigned widths take UINT8 zero-points."""
    a = HQ_DT_BF16 if bf16 else HQ_DT_FP16
    w = {(5, True): HQ_DT_INT5, (5, False): HQ_DT_UINT5, (6, True): HQ_DT_INT6, (6, False): HQ_DT_UINT6,
         (7, True): HQ_DT_INT7, (7, False): HQ_DT_UINT7, (8, True): HQ_DT_INT8, (8, False): HQ_DT_UINT8}[(bits, signed)]
    return make_desc(N, K, a, w, a, HQ_GRAN_PER_GROUP_K, group_size, a,
                     zp_dtype=HQ_DT_NONE if signed else HQ_DT_UINT8)


def desc_wnlow(N, K, bits, signed, group_size=128, bf16=True) -> hq_layer_desc:
    """Low-bit WnA16: 1-3-bit codes; unsigned widths take UINT4 zero-points."""
    a = HQ_DT_BF16 if bf16 else HQ_DT_FP16
    w = {(1, True): HQ_DT_INT1, (1, False): HQ_DT_UINT1, (2, True): HQ_DT_INT2, (2, False): HQ_DT_UINT2,
         (3, True): HQ_DT_INT3, (3, False): HQ_DT_UINT3}[(bits, signed)]
    return make_desc(N, K, a, w, a, HQ_GRAN_PER_GROUP_K, group_size, a,
                     zp_dtype=HQ_DT_NONE if signed else HQ_DT_UINT4)


def desc_w4a8_mxfp4(N, K) -> hq_layer_desc:
    return make_desc(N, K, HQ_DT_FP8_E4M3, HQ_DT_FP4_E2M1, HQ_DT_E8M0, HQ_GRAN_PER_GROUP_K, 32, HQ_DT_BF16,
                     a_scale=HQ_ASCALE_PER_TOKEN_F32)


def desc_mx_act_mxfp4(N, K, fp4_act: bool) -> hq_layer_desc:
    """MX activations (E2M1 for W4A4, E4M3 for MXFP8 x MXFP4), E8M0 per 32 K, x MXFP4 weights."""
    return make_desc(N, K, HQ_DT_FP4_E2M1 if fp4_act else HQ_DT_FP8_E4M3, HQ_DT_FP4_E2M1, HQ_DT_E8M0,
                     HQ_GRAN_PER_GROUP_K, 32, HQ_DT_BF16, a_scale=HQ_ASCALE_MX_E8M0)


def desc_fp8_blockwise(N, K) -> hq_layer_desc:
    """FP8 W8A8 with blockwise scales: E4M3 activations with fp32 scales per 128-K block,
    E4M3 weights with fp32 scales per 128 x 128 block, bf16 output."""
    return make_desc(N, K, HQ_DT_FP8_E4M3, HQ_DT_FP8_E4M3, HQ_DT_FP32, HQ_GRAN_BLOCK_128x128, 128, HQ_DT_BF16,
                     a_scale=HQ_ASCALE_PER_BLOCK128_F32)


def desc_fp4_a16(N, K, nvfp4: bool, bf16: bool = True) -> hq_layer_desc:
    """16-bit activations (bf16, or fp16) x FP4 (e2m1) weights: MXFP4 (E8M0 per 32 K) or
    NVFP4 (E4M3 per 16 K and a per-tensor fp32 second-level scale)."""
    a = HQ_DT_BF16 if bf16 else HQ_DT_FP16
    d = make_desc(N, K, a, HQ_DT_FP4_E2M1, HQ_DT_FP8_E4M3 if nvfp4 else HQ_DT_E8M0, HQ_GRAN_PER_GROUP_K,
                  16 if nvfp4 else 32, a)
    if nvfp4:
        d.scale2 = HQ_S2_PER_TENSOR_F32
    return d


def desc_mxint4_a16(N, K, bf16: bool = True) -> hq_layer_desc:
    """16-bit activations x MXINT4 weights (two's-complement INT4, E8M0 scale per 32 K)."""
    a = HQ_DT_BF16 if bf16 else HQ_DT_FP16
    return make_desc(N, K, a, HQ_DT_INT4, HQ_DT_E8M0, HQ_GRAN_PER_GROUP_K, 32, a)


def desc_w8a16(N, K, bf16=True) -> hq_layer_desc:
    """bf16 / fp16 activations x INT8 weights with fp32 per-channel scales (INT8 weight-only)."""
    a = HQ_DT_BF16 if bf16 else HQ_DT_FP16
    return make_desc(N, K, a, HQ_DT_INT8, HQ_DT_FP32, HQ_GRAN_PER_CHANNEL, K, a)


def desc_fp8w_a16(N, K, bf16=True) -> hq_layer_desc:
    """bf16 / fp16 activations x FP8 (E4M3) weights with fp32 per-channel scales (FP8 weight-only)."""
    a = HQ_DT_BF16 if bf16 else HQ_DT_FP16
    return make_desc(N, K, a, HQ_DT_FP8_E4M3, HQ_DT_FP32, HQ_GRAN_PER_CHANNEL, K, a)


def desc_w8a8(N, K, raw_int32=False) -> hq_layer_desc:
    return make_desc(N, K, HQ_DT_INT8, HQ_DT_INT8, HQ_DT_FP32, HQ_GRAN_PER_CHANNEL, K,
                     HQ_DT_INT32 if raw_int32 else HQ_DT_BF16, a_scale=HQ_ASCALE_PER_TOKEN_F32)


def desc_moe_mxfp4(E, N, K) -> hq_layer_desc:
    return make_desc(N, K, HQ_DT_BF16, HQ_DT_FP4_E2M1, HQ_DT_E8M0, HQ_GRAN_PER_GROUP_K, 32, HQ_DT_BF16,
                     num_experts=E)


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def hq_desc_validate(desc: hq_layer_desc) -> None:
    _check(lib().hq_desc_validate(C.byref(desc)), "hq_desc_validate")


def hq_repacked_bytes(desc: hq_layer_desc):
    w, s, z, s2 = C.c_size_t(), C.c_size_t(), C.c_size_t(), C.c_size_t()
    _check(lib().hq_repacked_bytes(C.byref(desc), C.byref(w), C.byref(s), C.byref(z), C.byref(s2)),
           "hq_repacked_bytes")
    return w.value, s.value, z.value, s2.value


def hq_repack(desc: hq_layer_desc, w: np.ndarray, scale: np.ndarray, zp: np.ndarray | None = None, scale2=None):
    """Host repack; returns the packed (w, s, z) as uint8 numpy arrays (z None if unused),
    plus the packed second-level scale as a fourth item when `scale2` is given."""
    wb, sb, zb, s2b = hq_repacked_bytes(desc)
    w = np.ascontiguousarray(w)
    scale = np.ascontiguousarray(scale)
    zp = None if zp is None else np.ascontiguousarray(zp)
    s2 = None if scale2 is None else np.ascontiguousarray(np.atleast_1d(np.asarray(scale2, dtype=np.float32)))
    wo = np.empty(wb, dtype=np.uint8)
    so = np.empty(sb, dtype=np.uint8)
    zo = np.empty(zb, dtype=np.uint8) if zb else None
    s2o = np.empty(s2b, dtype=np.uint8) if s2b else None
    _check(lib().hq_repack(C.byref(desc), _dp(w), _dp(scale), _dp(zp), _dp(s2), _dp(wo), _dp(so), _dp(zo), _dp(s2o)),
           "hq_repack")
    return (wo, so, zo) if scale2 is None else (wo, so, zo, s2o)


def hq_workspace_bytes(desc: hq_layer_desc, M_or_T: int, top_k: int = 0) -> int:
    b = C.c_size_t()
    _check(lib().hq_workspace_bytes(C.byref(desc), M_or_T, top_k, C.byref(b)), "hq_workspace_bytes")
    return b.value


def hq_workspace_init(workspace, nbytes: int, stream=None) -> None:
    _check(lib().hq_workspace_init(_dp(workspace), nbytes, _stream(stream)), "hq_workspace_init")


def hq_gemm(desc, M, A, a_scale, w, s, z, D, workspace=None, ws_bytes=0, stream=None, s2=None) -> None:
    _check(lib().hq_gemm(C.byref(desc), M, _dp(A), _dp(a_scale), _dp(w), _dp(s), _dp(z), _dp(s2), _dp(D),
                         _dp(workspace), ws_bytes, _stream(stream)), "hq_gemm")


HQ_NOALLOC_SCRATCH_BYTES = 32 << 20


def hq_gemm_noalloc(desc, M, A, a_scale, w, s, z, D, stream=None) -> None:
    _check(lib().hq_gemm_noalloc(C.byref(desc), M, _dp(A), _dp(a_scale), _dp(w), _dp(s), _dp(z), None, _dp(D),
                                 _stream(stream)), "hq_gemm_noalloc")


def hq_gemm_plan(desc, M) -> list:
    """The kernel launches hq_gemm would enqueue for (desc, M), one string each (host only)."""
    buf = C.create_string_buffer(4096)
    _check(lib().hq_gemm_plan(C.byref(desc), M, buf, len(buf)), "hq_gemm_plan")
    txt = buf.value.decode()
    return txt.split(";") if txt else []


def hq_moe_gemm(desc, mode, T, top_k, A, a_scale, topk_ids, expert_offsets, w, s, z, D, workspace=None,
                ws_bytes=0, stream=None) -> None:
    _check(lib().hq_moe_gemm(C.byref(desc), mode, T, top_k, _dp(A), _dp(a_scale), _dp(topk_ids),
                             _dp(expert_offsets), _dp(w), _dp(s), _dp(z), None, _dp(D), _dp(workspace),
                             ws_bytes, _stream(stream)), "hq_moe_gemm")


def hq_quantize_act(out_dtype, M, K, x, q, s, stream=None) -> None:
    _check(lib().hq_quantize_act(out_dtype, M, K, _dp(x), _dp(q), _dp(s), _stream(stream)), "hq_quantize_act")


def hq_quantize_act_blocks(out_dtype, M, K, block, x, q, s, stream=None) -> None:
    _check(lib().hq_quantize_act_blocks(out_dtype, M, K, block, _dp(x), _dp(q), _dp(s), _stream(stream)),
           "hq_quantize_act_blocks")


def hq_quantize_act_mx(out_dtype, M, K, x, q, e, stream=None) -> None:
    _check(lib().hq_quantize_act_mx(out_dtype, M, K, _dp(x), _dp(q), _dp(e), _stream(stream)), "hq_quantize_act_mx")


def hq_moe_align(T, top_k, num_experts, topk_ids, expert_offsets, sorted_pairs, workspace=None, ws_bytes=0,
                 stream=None) -> None:
    _check(lib().hq_moe_align(T, top_k, num_experts, _dp(topk_ids), _dp(expert_offsets), _dp(sorted_pairs),
                              _dp(workspace), ws_bytes, _stream(stream)), "hq_moe_align")


def hq_moe_gather(dtype, T, top_k, K, A, sorted_pairs, A_sorted, stream=None) -> None:
    _check(lib().hq_moe_gather(dtype, T, top_k, K, _dp(A), _dp(sorted_pairs), _dp(A_sorted), _stream(stream)),
           "hq_moe_gather")


def hq_probe_stream(src, nbytes, sink, reps=1, stream=None) -> None:
    """Read nbytes of src `reps` times (a measurement of the attainable HBM read rate)."""
    _check(lib().hq_probe_stream(_dp(src), nbytes, _dp(sink), reps, _stream(stream)), "hq_probe_stream")


# flops (int8: ops) of one MFMA of each probed type
PROBE_MFMA_FLOPS = {HQ_DT_FP16: 16384, HQ_DT_BF16: 16384, HQ_DT_FP8_E4M3: 65536, HQ_DT_FP4_E2M1: 65536,
                    HQ_DT_INT8: 32768}


def hq_probe_mfma(dtype, workgroups, iters, sink, stream=None) -> float:
    """Run the dense MFMA probe; returns the flops (int8: ops) the call performs."""
    _check(lib().hq_probe_mfma(dtype, workgroups, iters, _dp(sink), _stream(stream)), "hq_probe_mfma")
    return float(workgroups) * 4 * iters * 8 * PROBE_MFMA_FLOPS[dtype]


def hq_silu_mul(dtype, rows, I, gate_up, out, stream=None) -> None:
    _check(lib().hq_silu_mul(dtype, rows, I, _dp(gate_up), _dp(out), _stream(stream)), "hq_silu_mul")
