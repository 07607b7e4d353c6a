"""GPU checks of the two controls on the dense kernel choice, through the C ABI:

* batch-invariant mode (HQ_FLAG_BATCH_INVARIANT): a row's output must not
  depend on the batch it is computed in.  One large batch is run, then windows
  of it (other row offsets, other M, so other tile shapes) are run on their own
  and must reproduce the large batch's rows bit for bit; the large batch is
  checked against the oracle as well.
* tuning overrides (the descriptor's tune field, HQ_TUNE(path, splits)): every
  candidate the autotuner would time must give the oracle's result, to the
  format's parity bound (bit-exact for the raw INT32 output).
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from bit_quantized_gemm_w4a16_amd import autotune, hq
from gpu_util import GATE, dev, empty, gate_error, note, to_f64

pytestmark = pytest.mark.gpu

FORMATS = ["wna16_f16_zp", "wna16_bf16_sym", "w4a8_mxfp4", "w8a8_bf16", "w8a8_raw", "w4a4_mx", "mxfp8_mx",
           "fp8_blockwise", "mxfp4_a16", "nvfp4_a16", "mxint4_a16", "w8a16_bf16", "w8a16_f16", "fp8w_bf16", "fp8w_f16"]


class Layer:
    """One dense layer of a format with seeded inputs on the device; `run` calls
    hq_gemm on rows r0 .. r0+M-1 of the activations."""

    def __init__(self, fmt, M, N, K, seed):
        self.fmt, self.M, self.N, self.K = fmt, M, N, K
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
        elif fmt == "mxint4_a16":
            d = syn.w4a16_mxint4(seed, M, N, K)
            self.desc = hq.desc_mxint4_a16(N, K)
            packed = hq.hq_repack(self.desc, d["q"], d["e"])
            A, sa, arow, srow = d["A"], None, K * 2, 0
            self.ref = lambda r: oracle.gemm_mxint4_a16(d["A"], d["q"], d["e"], N=N, K=K, rows=r)
        else:
            nv = fmt == "nvfp4_a16"
            d = syn.w4a16_fp4(seed, M, N, K, nvfp4=nv)
            self.desc = hq.desc_fp4_a16(N, K, nv)
            if nv:
                wp, sp, _, s2p = hq.hq_repack(self.desc, d["q"], d["s"], None, d["s2"])
                packed, s2 = (wp, sp, None), s2p
            else:
                packed = hq.hq_repack(self.desc, d["q"], d["s"])
            A, sa, arow, srow = d["A"], None, K * 2, 0
            self.ref = lambda r: oracle.gemm_fp4_a16(d["A"], d["q"], d["s"], N=N, K=K, a_bf16=True, nvfp4=nv,
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


def invariant(desc):
    d = hq.hq_layer_desc.from_buffer_copy(desc)
    d.flags = hq.HQ_FLAG_BATCH_INVARIANT
    return d


BIG = 4096
# row offsets are multiples of 4: per-row fp32 activation scales must stay 16-byte aligned
WINDOWS = [(1, 0), (4, 4092), (5, 1000), (130, 8), (1024, 512), (2048, 1024), (3000, 1096)]


@pytest.mark.parametrize("fmt", FORMATS)
def test_batch_invariant_rows_do_not_depend_on_the_batch(fmt):
    N, K = 4096, 512
    note(f"batch invariance {fmt} M={BIG} N={N} K={K}")
    L = Layer(fmt, BIG, N, K, seed=11)
    d = invariant(L.desc)
    shapes = {hq.hq_gemm_plan(d, M)[0].split(" ")[0] for M, _ in WINDOWS + [(BIG, 0)]}
    assert all("splits=1" in hq.hq_gemm_plan(d, M)[0] and len(hq.hq_gemm_plan(d, M)) == 1 for M, _ in WINDOWS)
    big = L.run(d, BIG)
    rows = np.array([0, 1, 777, 2047, 2048, 4094, 4095])
    L.check(big[rows], rows)
    for M, r0 in WINDOWS:
        note(f"batch invariance {fmt} window M={M} r0={r0} {hq.hq_gemm_plan(d, M)[0]}")
        sub = L.run(d, M, r0)
        bad = np.argwhere(sub != big[r0:r0 + M])
        assert bad.size == 0, f"M={M} r0={r0}: {len(bad)} outputs differ, first at {bad[0].tolist()}"
    # the formats with several tile classes reach more than one of them
    if fmt != "wna16_bf16_sym":
        assert len(shapes) >= 2, shapes


@pytest.mark.parametrize("M", [8, 24, 300])
@pytest.mark.parametrize("fmt", FORMATS)
def test_every_tuning_candidate_matches_the_oracle(fmt, M):
    N, K = 1000, 1024
    L = Layer(fmt, M, N, K, seed=M + 3)
    rows = np.arange(M)
    cands = autotune.candidates(L.desc, M)
    assert len(cands) >= 2
    for t in cands:
        d = autotune.with_tune(L.desc, t)
        note(f"tune {fmt} M={M} N={N} K={K} tune=0x{t:x} {hq.hq_gemm_plan(d, M)}")
        L.check(L.run(d, M), rows)
