"""Host-only check (no GPU) that the GPU parity suite reaches every kernel
configuration the benchmark times.

hq_gemm_plan runs the library's own dispatch without launching and names the
kernels a call would enqueue.  For each dense workload of the benchmark and
each M of its sweep, every launched kernel -- template arguments plus whether
its K is split (partial tiles and a finalize pass) or not (direct epilogue) --
must also be launched by at least one case of the GPU suite (tests/cases.py).
"""
import re

import pytest

import cases
from bit_quantized_gemm_w4a16_amd import hq


def desc_of(fmt, N, K, G, flags):
    if fmt == "wna16":
        return hq.desc_w4a16(N, K, G, bf16=flags["bf16"], zp=flags["zp"])
    if fmt == "wnlow":
        return hq.desc_wnlow(N, K, flags["bits"], flags["signed"], G, bf16=flags["bf16"])
    if fmt == "wnwide":
        return hq.desc_wnwide(N, K, flags["bits"], flags["signed"], G, bf16=flags["bf16"])
    if fmt == "mxf":
        return hq.desc_mxf_a16(N, K, flags["elem"])
    if fmt == "w4a8":
        return hq.desc_w4a8_mxfp4(N, K)
    if fmt == "mxa":
        return hq.desc_mx_act_mxfp4(N, K, fp4_act=flags["elem"] == "e2m1")
    if fmt == "fp8b":
        return hq.desc_fp8_blockwise(N, K)
    if fmt == "w8a16":
        return hq.desc_w8a16(N, K, bf16=flags["bf16"])
    if fmt == "fp8w":
        return hq.desc_fp8w_a16(N, K, bf16=flags["bf16"])
    if fmt == "mxint4":
        return hq.desc_mxint4_a16(N, K)
    if fmt == "fp4a16":
        return hq.desc_fp4_a16(N, K, nvfp4=flags["kind"] == "nvfp4")
    return hq.desc_w8a8(N, K, raw_int32=flags["raw"])


def keys(desc, M):
    out = set()
    for item in hq.hq_gemm_plan(desc, M):
        name = item.split(" ")[0]
        m = re.search(r"splits=(\d+)", item)
        if m:
            name += " split" if int(m.group(1)) > 1 else " direct"
        out.add(name)
    return out


def covered():
    cov = set()
    for fmt, M, N, K, G, flags in cases.all_dense_cases():
        cov |= keys(desc_of(fmt, N, K, G, flags), M)
    return cov


BENCH = {
    "c2": ("wna16", cases.C2["N"], cases.C2["K"], cases.C2["G"], dict(bf16=False, zp=True)),
    "c3": ("w4a8", cases.C3["N"], cases.C3["K"], 32, {}),
    "c4": ("w8a8", cases.C4["N"], cases.C4["K"], cases.C4["K"], dict(raw=False)),
    "c4raw": ("w8a8", cases.C4["N"], cases.C4["K"], cases.C4["K"], dict(raw=True)),
    "w4a4": ("mxa", cases.C3["N"], cases.C3["K"], 32, dict(elem="e2m1")),
    "w4a8mx": ("mxa", cases.C3["N"], cases.C3["K"], 32, dict(elem="e4m3")),
    "fp8b": ("fp8b", 7168, 7168, 128, {}),
    "mxfp4a16": ("fp4a16", 4096, 7168, 32, dict(kind="mxfp4")),
    "nvfp4a16": ("fp4a16", 4096, 7168, 16, dict(kind="nvfp4")),
    "mxint4a16": ("mxint4", 4096, 7168, 32, {}),
    "w8a16bf": ("w8a16", 4096, 7168, 7168, dict(bf16=True)),
    "w8a16fp": ("w8a16", 4096, 7168, 7168, dict(bf16=False)),
    "fp8wbf": ("fp8w", 4096, 7168, 7168, dict(bf16=True)),
    "fp8wfp": ("fp8w", 4096, 7168, 7168, dict(bf16=False)),
    "w3a16": ("wnlow", cases.C2["N"], cases.C2["K"], cases.C2["G"], dict(bits=3, signed=False, bf16=False)),
    "w2a16": ("wnlow", cases.C2["N"], cases.C2["K"], cases.C2["G"], dict(bits=2, signed=True, bf16=True)),
    "w8a16g": ("wnwide", cases.C2["N"], cases.C2["K"], cases.C2["G"], dict(bits=8, signed=False, bf16=False)),
    "w5a16": ("wnwide", cases.C2["N"], cases.C2["K"], cases.C2["G"], dict(bits=5, signed=True, bf16=True)),
    "mxfp8a16": ("mxf", cases.C2["N"], cases.C2["K"], 32, dict(elem="e4m3")),
    "mxfp6a16": ("mxf", cases.C2["N"], cases.C2["K"], 32, dict(elem="e2m3")),
}


def test_plan_names_kernels_without_launching():
    d = hq.desc_w4a16(4096, 7168, 128, bf16=False, zp=True)
    assert hq.hq_gemm_plan(d, 0) == []
    p1 = hq.hq_gemm_plan(d, 1)
    assert len(p1) == 1 and p1[0].startswith("skinny_kernel<WNA16_F16,") and "splits=1" in p1[0]
    p8k = hq.hq_gemm_plan(d, 8192)
    assert len(p8k) == 1 and p8k[0].startswith("tile_gemm_kernel<WNA16_F16,")
    with pytest.raises(hq.HQError):
        hq.hq_gemm_plan(hq.desc_moe_mxfp4(8, 128, 128), 4)


@pytest.mark.parametrize("cfg", sorted(BENCH))
def test_every_bench_sweep_kernel_has_a_gpu_parity_case(cfg):
    fmt, N, K, G, flags = BENCH[cfg]
    d = desc_of(fmt, N, K, G, flags)
    cov = covered()
    missing = {}
    for M in cases.SWEEP:
        for k in keys(d, M) - cov:
            missing.setdefault(k, []).append(M)
    assert not missing, missing
