"""GPU parity of the weight-only formats of the scaled converts (MXFP4, NVFP4,
MXINT4, MXFP8, MXFP6 E2M3 / E3M2) with fp16 activations: the codes become fp16
operands under the lane's scale, fp16 MFMA, fp16 output; against the CPU oracle
(the same oracle functions with fp16 A) through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from bit_quantized_gemm_w4a16_amd import hq
from gpu_util import GATE, dev, empty, gate_error, note, sample_rows, sweep_rows, to_f64

pytestmark = pytest.mark.gpu

FORMATS = ["mxfp4", "nvfp4", "mxint4", "e4m3", "e2m3", "e3m2"]
SHAPES = [(1, 272, 1024), (16, 272, 1024), (64, 272, 1024), (300, 1000, 512), (2000, 4100, 384), (4096, 4096, 7168)]


def layer(fmt, M, N, K, seed):
    dt = torch.float16
    if fmt in ("mxfp4", "nvfp4"):
        nv = fmt == "nvfp4"
        d = syn.w4a16_fp4(seed, M, N, K, nvfp4=nv, dtype=dt)
        desc = hq.desc_fp4_a16(N, K, nv, bf16=False)
        if nv:
            wp, sp, _, s2 = hq.hq_repack(desc, d["q"], d["s"], None, d["s2"])
        else:
            (wp, sp, _), s2 = hq.hq_repack(desc, d["q"], d["s"]), None
        ref = lambda r: oracle.gemm_fp4_a16(d["A"], d["q"], d["s"], N=N, K=K, a_bf16=False, nvfp4=nv,
                                            s2=d.get("s2"), rows=r)
    elif fmt == "mxint4":
        d = syn.w4a16_mxint4(seed, M, N, K, dt)
        desc = hq.desc_mxint4_a16(N, K, bf16=False)
        (wp, sp, _), s2 = hq.hq_repack(desc, d["q"], d["e"]), None
        ref = lambda r: oracle.gemm_mxint4_a16(d["A"], d["q"], d["e"], N=N, K=K, a_bf16=False, rows=r)
    else:
        d = syn.mxf_a16(seed, M, N, K, fmt, dt)
        desc = hq.desc_mxf_a16(N, K, fmt, bf16=False)
        (wp, sp, _), s2 = hq.hq_repack(desc, d["codes"], d["e"]), None
        ref = lambda r: oracle.gemm_mxf_a16(d["A"], d["codes"], d["e"], elem=fmt, a_bf16=False, rows=r)
    return d["A"], desc, wp, sp, s2, ref


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("fmt", FORMATS)
def test_fp16_activations_match_the_oracle(fmt, M, N, K):
    A, desc, wp, sp, s2, ref = layer(fmt, M, N, K, seed=M + 3)
    note(f"fp16-A {fmt} M={M} N={N} K={K} {hq.hq_gemm_plan(desc, M)}")
    D = empty(M * N * 2)
    nb = hq.hq_workspace_bytes(desc, M)
    ws = torch.zeros(max(nb, 16), dtype=torch.uint8, device="cuda") if nb else None
    hq.hq_gemm(desc, M, dev(A), None, dev(wp), dev(sp), None, D, ws, nb, s2=dev(s2) if s2 is not None else None)
    torch.cuda.synchronize()
    Dh = to_f64(D[: M * N * 2].cpu().numpy().view(np.uint16).reshape(M, N), torch.float16)
    rows = sweep_rows(M) if M >= 4096 else sample_rows(M)
    O = ref(rows)
    err = gate_error(Dh[rows], O)
    assert np.all(np.isfinite(Dh[rows])) and err <= GATE and err <= 3e-3, err
