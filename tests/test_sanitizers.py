"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Builds the library's host translation units (descriptor validation, planning,
weight repacking: hq_api.cpp, hq_repack.cpp) and the C oracle with ASan and
UBSan on the host side, links the former with the ordinary kernel objects, and
runs the host-side suites (the C-ABI checks, the oracle pins and the planner
coverage) in a child process against those builds, with the sanitizer runtime
preloaded and every report fatal.  Device code is compiled as usual: only
`-Xarch_host` carries the sanitizer flags.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_quantized_gemm_w4a16_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
SAN = ["address", "undefined"]
SUITES = ["tests/test_abi.py", "tests/test_oracle_pins.py", "tests/test_plan_coverage.py"]


def _asan_runtime() -> str | None:
    if not os.path.exists(CLANG):
        return None
    r = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if os.path.isabs(path) and os.path.exists(path):
        return path
    hits = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    return hits[0] if hits else None


def _run(cmd: list[str]) -> None:
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}")


def _host_flags() -> list[str]:
    flags = []
    for s in SAN:
        flags += ["-Xarch_host", f"-fsanitize={s}"]
    return flags + ["-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _build_libhq() -> str:
    from bit_quantized_gemm_w4a16_amd import build as B

    os.makedirs(OUT, exist_ok=True)
    host_objs = []
    for src in ("hq_api.cpp", "hq_repack.cpp"):
        obj = os.path.join(OUT, src + ".o")
        _run([HIPCC, "-x", "hip", *B.COMMON, "-O1", "-g", *_host_flags(), "-c", os.path.join(CSRC, src),
              "-o", obj])
        host_objs.append(obj)
    kernels = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    kobjs = [os.path.join(B.BUILD, os.path.basename(k) + ".o") for k in kernels]
    if not all(os.path.exists(o) and os.path.getmtime(o) >= os.path.getmtime(k) for k, o in zip(kernels, kobjs)):
        os.makedirs(B.BUILD, exist_ok=True)
        kobjs = [B._compile(k) for k in kernels]
    lib = os.path.join(OUT, "libhq.so")
    _run([HIPCC, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", *_host_flags(), "-shared-libasan",
          *host_objs, *kobjs, "-o", lib])
    return lib


def _build_oracle() -> str:
    os.makedirs(OUT, exist_ok=True)
    lib = os.path.join(OUT, "liboracle.so")
    # serial (no OpenMP): the pins are small, and the sanitizer runtime is clang's
    _run([CLANG, "-O1", "-g", "-std=c11", "-ffp-contract=off", "-Wno-unknown-pragmas",
          "-Wno-source-uses-openmp", f"-fsanitize={','.join(SAN)}", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", "-shared-libasan", "-shared", "-fPIC",
          os.path.join(ROOT, "oracle", "hq_oracle.c"), "-o", lib, "-lm"])
    return lib


@pytest.mark.timeout(900)
def test_host_code_under_asan_ubsan():
    runtime = _asan_runtime()
    if runtime is None or not os.path.exists(HIPCC):
        pytest.skip("clang's sanitizer runtime or hipcc not available")
    libhq = _build_libhq()
    liboracle = _build_oracle()
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": runtime,
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:detect_odr_violation=0:alloc_dealloc_mismatch=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "HQ_LIB_PATH": libhq,
        "HQ_ORACLE_LIB_PATH": liboracle,
    })
    r = subprocess.run([sys.executable, "-m", "pytest", *SUITES, "-m", "not gpu", "-q", "-x", "-p",
                        "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=800)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-6000:]
    assert r.returncode == 0, out[-6000:]
    assert " passed" in r.stdout, out[-3000:]
