"""Seeded dense layers of every format on the device, run through the C ABI and
checked against the oracle (shared by the GPU tests of the kernel choice)."""
import numpy as np
import torch

import oracle
import synthetic as syn
from bit_quantized_gemm_w4a16_amd import hq
from gpu_util import GATE, dev, empty, gate_error, to_f64

FORMATS = ["wna16_f16_zp", "wna16_bf16_sym", "w4a8_mxfp4", "w8a8_bf16", "w8a8_raw", "w4a4_mx", "mxfp8_mx",
           "fp8_blockwise", "mxfp4_a16", "nvfp4_a16", "mxint4_a16", "w8a16_bf16", "w8a16_f16", "fp8w_bf16", "fp8w_f16",
           "mxfp8_a16", "mxfp6e2_a16", "mxfp6e3_a16", "w3a16_uint3", "w2a16_int2", "w1a16_int1",
           "mxfp4_a16_f16", "mxfp6e2_a16_f16"]
# formats with 16-bit activations that every small-M schedule takes (the low-bit
# widths have no eight-wave stream)
A16_FORMATS = ["wna16_f16_zp", "wna16_bf16_sym", "mxfp4_a16", "nvfp4_a16", "mxint4_a16", "w8a16_bf16", "w8a16_f16",
               "fp8w_bf16", "fp8w_f16", "mxfp8_a16", "mxfp6e2_a16", "mxfp6e3_a16", "mxfp4_a16_f16", "mxfp6e2_a16_f16"]
MXF_ELEM = {"mxfp8_a16": "e4m3", "mxfp6e2_a16": "e2m3", "mxfp6e3_a16": "e3m2", "mxfp6e2_a16_f16": "e2m3"}
LOWBIT = {"w3a16_uint3": (3, False), "w2a16_int2": (2, True), "w1a16_int1": (1, True)}
# 5-8-bit WnA16: (bits, signed, bf16 activations)
WIDE = {"wn5_int5_bf16": (5, True, True), "wn5_uint5_f16": (5, False, False), "wn6_int6_f16": (6, True, False),
        "wn6_uint6_bf16": (6, False, True), "wn7_int7_f16": (7, True, False), "wn7_uint7_bf16": (7, False, True),
        "wn8_int8_bf16": (8, True, True), "wn8_uint8_f16": (8, False, False)}


class Layer:
    """One dense layer of a format with seeded inputs on the device; `run` calls
    hq_gemm on rows r0 .. r0+M-1 of the activations."""

    def __init__(self, fmt, M, N, K, seed, G=128):
        self.fmt, self.M, self.N, self.K = fmt, M, N, K
        f16 = fmt.endswith("_a16_f16")   # a weight-only format of the scaled converts with fp16 activations
        self.raw = fmt == "w8a8_raw"
        self.out_dt = torch.float16 if fmt == "wna16_f16_zp" else torch.bfloat16
        s2 = None
        if fmt.startswith("wna16"):
            zp = fmt.endswith("zp")
            dt = torch.float16 if zp else torch.bfloat16
            d = syn.w4a16_zp(seed, M, N, K, 128, dt) if zp else syn.w4a16_sym(seed, M, N, K, 128, dt)
            self.desc = hq.desc_w4a16(N, K, 128, bf16=not zp, zp=zp)
            packed = hq.hq_repack(self.desc, d["q"], d["s"], d.get("z") if zp else None)
            A, sa, arow, srow = d["A"], None, K * 2, 0
            self.ref = lambda r: oracle.gemm_wna16(d["A"], d["q"], d["s"], d.get("z") if zp else None, N=N, K=K,
                                                   G=128, a_bf16=not zp, w_signed=not zp, rows=r)
        elif fmt == "w4a8_mxfp4":
            d = syn.w4a8_mxfp4(seed, M, N, K)
            qa, s_a = oracle.quant_act_e4m3(d["A0"])
            self.desc = hq.desc_w4a8_mxfp4(N, K)
            packed = hq.hq_repack(self.desc, d["q"], d["e"])
            A, sa, arow, srow = qa, s_a, K, 4
            self.ref = lambda r: oracle.gemm_w4a8_mxfp4(qa, s_a, d["q"], d["e"], N=N, K=K, rows=r)
        elif fmt.startswith("w8a8"):
            d = syn.w8a8_int8(seed, M, N, K)
            self.desc = hq.desc_w8a8(N, K, raw_int32=self.raw)
            packed = hq.hq_repack(self.desc, d["w"], d["s_w"])
            A, sa, arow, srow = d["a"], d["s_a"], K, 4
            self.ref = lambda r: oracle.gemm_w8a8(d["a"], d["s_a"], d["w"], d["s_w"], rows=r)[0 if self.raw else 1]
        elif fmt in ("w4a4_mx", "mxfp8_mx"):
            elem = "e2m1" if fmt == "w4a4_mx" else "e4m3"
            d = syn.w4a8_mxfp4(seed, M, N, K)
            qa, ea = oracle.quant_act_mx(d["A0"], elem)
            self.desc = hq.desc_mx_act_mxfp4(N, K, fp4_act=elem == "e2m1")
            packed = hq.hq_repack(self.desc, d["q"], d["e"])
            A, sa, arow, srow = qa, ea, qa.shape[1], K // 32
            self.ref = lambda r: oracle.gemm_mx_mxfp4(qa, ea, d["q"], d["e"], N=N, K=K, a_elem=elem, rows=r)
        elif fmt == "fp8_blockwise":
            d = syn.w8a8_fp8_blockwise(seed, M, N, K)
            qa, s_a = oracle.quant_act_e4m3_blocks(d["A0"], 128)
            self.desc = hq.desc_fp8_blockwise(N, K)
            packed = hq.hq_repack(self.desc, d["w"], d["s_w"])
            A, sa, arow, srow = qa, s_a, K, (K // 128) * 4
            self.ref = lambda r: oracle.gemm_fp8_blockwise(qa, s_a, d["w"], d["s_w"], rows=r)
        elif fmt.startswith("w8a16") or fmt.startswith("fp8w"):
            bf = fmt.endswith("bf16")
            fp8 = fmt.startswith("fp8w")
            self.out_dt = torch.bfloat16 if bf else torch.float16
            d = (syn.w8a16_fp8 if fp8 else syn.w8a16_int8)(seed, M, N, K, self.out_dt)
            self.desc = (hq.desc_fp8w_a16 if fp8 else hq.desc_w8a16)(N, K, bf16=bf)
            packed = hq.hq_repack(self.desc, d["w"], d["s_w"])
            A, sa, arow, srow = d["A"], None, K * 2, 0
            ref = oracle.gemm_fp8w_a16 if fp8 else oracle.gemm_w8a16
            self.ref = lambda r: ref(d["A"], d["w"], d["s_w"], a_bf16=bf, rows=r)
        elif fmt in MXF_ELEM:
            elem = MXF_ELEM[fmt]
            if f16:
                self.out_dt = torch.float16
            d = syn.mxf_a16(seed, M, N, K, elem, dtype=self.out_dt)
            self.desc = hq.desc_mxf_a16(N, K, elem, bf16=not f16)
            packed = hq.hq_repack(self.desc, d["codes"], d["e"])
            A, sa, arow, srow = d["A"], None, K * 2, 0
            self.ref = lambda r: oracle.gemm_mxf_a16(d["A"], d["codes"], d["e"], elem=elem, a_bf16=not f16, rows=r)
        elif fmt in LOWBIT:
            bits, signed = LOWBIT[fmt]
            self.out_dt = torch.bfloat16 if signed else torch.float16
            d = syn.wnlow(seed, M, N, K, bits, signed, dtype=self.out_dt)
            self.desc = hq.desc_wnlow(N, K, bits, signed, bf16=signed)
            packed = hq.hq_repack(self.desc, d["codes"], d["s"], d.get("z"))
            A, sa, arow, srow = d["A"], None, K * 2, 0
            self.ref = lambda r: oracle.gemm_wnlow(d["A"], d["codes"], d["s"], d.get("z"), N=N, K=K, G=128, bits=bits,
                                                   a_bf16=signed, w_signed=signed, rows=r)
        elif fmt in WIDE:
            bits, signed, bf = WIDE[fmt]
            self.out_dt = torch.bfloat16 if bf else torch.float16
            d = syn.wnwide(seed, M, N, K, bits, signed, G=G, dtype=self.out_dt)
            self.desc = hq.desc_wnwide(N, K, bits, signed, group_size=G, bf16=bf)
            packed = hq.hq_repack(self.desc, d["codes"], d["s"], d.get("z"))
            A, sa, arow, srow = d["A"], None, K * 2, 0
            self.ref = lambda r: oracle.gemm_wnwide(d["A"], d["codes"], d["s"], d.get("z"), N=N, K=K, G=G, bits=bits,
                                                    a_bf16=bf, w_signed=signed, rows=r)
        elif fmt == "mxint4_a16":
            d = syn.w4a16_mxint4(seed, M, N, K)
            self.desc = hq.desc_mxint4_a16(N, K)
            packed = hq.hq_repack(self.desc, d["q"], d["e"])
            A, sa, arow, srow = d["A"], None, K * 2, 0
            self.ref = lambda r: oracle.gemm_mxint4_a16(d["A"], d["q"], d["e"], N=N, K=K, rows=r)
        else:
            nv = fmt == "nvfp4_a16"
            if f16:
                self.out_dt = torch.float16
            d = syn.w4a16_fp4(seed, M, N, K, nvfp4=nv, dtype=self.out_dt)
            self.desc = hq.desc_fp4_a16(N, K, nv, bf16=not f16)
            if nv:
                wp, sp, _, s2p = hq.hq_repack(self.desc, d["q"], d["s"], None, d["s2"])
                packed, s2 = (wp, sp, None), s2p
            else:
                packed = hq.hq_repack(self.desc, d["q"], d["s"])
            A, sa, arow, srow = d["A"], None, K * 2, 0
            self.ref = lambda r: oracle.gemm_fp4_a16(d["A"], d["q"], d["s"], N=N, K=K, a_bf16=not f16, nvfp4=nv,
                                                     s2=d.get("s2"), rows=r)
        self.A = dev(A)
        self.sa = dev(sa) if sa is not None else None
        self.arow, self.srow = arow, srow
        self.w, self.s = dev(packed[0]), dev(packed[1])
        self.z = dev(packed[2]) if packed[2] is not None else None
        self.s2 = dev(s2) if s2 is not None else None
        self.ob = 4 if self.raw else 2

    def run(self, desc, M, r0=0):
        """Output rows for activation rows r0 .. r0+M-1, as raw bits [M, N]."""
        N = self.N
        D = empty(M * N * self.ob)
        nb = hq.hq_workspace_bytes(desc, M)
        ws = torch.zeros(max(nb, 16), dtype=torch.uint8, device="cuda") if nb else None
        A = self.A[r0 * self.arow:]
        sa = self.sa[r0 * self.srow:] if self.sa is not None else None
        hq.hq_gemm(desc, M, A, sa, self.w, self.s, self.z, D, ws, nb, s2=self.s2)
        torch.cuda.synchronize()
        bits = D[: M * N * self.ob].cpu().numpy()
        return bits.view(np.int32 if self.raw else np.uint16).reshape(M, N)

    def values(self, bits):
        return bits.astype(np.int64) if self.raw else to_f64(bits, self.out_dt)

    def check(self, bits, rows):
        key = tuple(rows.tolist())
        if getattr(self, "_want_key", None) != key:     # one oracle run per row set
            self._want_key, self._want = key, self.ref(rows)
        got, want = self.values(bits), self._want
        if self.raw:
            np.testing.assert_array_equal(got, want)
            return 0.0
        assert np.all(np.isfinite(got))
        err = gate_error(got, want)
        assert err <= min(GATE, 3e-3 if self.out_dt == torch.float16 else 8e-3), err
        return err
