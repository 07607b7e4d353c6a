"""GPU parity of the 5-8-bit WnA16 weights (INT5-INT8, UINT5-UINT8 with 8-bit
zero-points, 16-bit group scales; bf16 and fp16 activations) against the CPU
oracle, through the C ABI.

Small M runs the weight stream on the packed codes (the 4-bit word set plus the
high bits); larger M first rewrites the codes as bytes in the
workspace (u = q, or q + 128 for signed codes, in the INT8 weight-only layout)
and runs the INT8 weight-only tiles on them, which subtract the zero-points
exactly in the decode and apply the group scales to each step's fp32 partials.  N = 1000 and 4100 end in a partial 16-column strip."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from bit_quantized_gemm_w4a16_amd import autotune, hq
import cases
from gpu_util import GATE, dev, empty, gate_error, note, sample_rows, sweep_rows, to_f64

pytestmark = pytest.mark.gpu


class Wide:
    """One seeded 5-8-bit layer on the device."""

    def __init__(self, M, N, K, G, bits, signed, bf16, seed=0, codes=None):
        self.M, self.N, self.K, self.G, self.bits, self.signed, self.bf16 = M, N, K, G, bits, signed, bf16
        self.dt = torch.bfloat16 if bf16 else torch.float16
        self.d = syn.wnwide(seed, M, N, K, bits, signed, G=G, dtype=self.dt)
        if codes is not None:
            self.d["codes"] = codes
        self.desc = hq.desc_wnwide(N, K, bits, signed, G, bf16=bf16)
        wp, sp, zp = hq.hq_repack(self.desc, self.d["codes"], self.d["s"], self.d.get("z"))
        self.A, self.w, self.s = dev(self.d["A"]), dev(wp), dev(sp)
        self.z = dev(zp) if zp is not None else None

    def run(self, desc=None, M=None, r0=0):
        desc = desc or self.desc
        M = M or self.M
        N = self.N
        D = empty(M * N * 2)
        nb = hq.hq_workspace_bytes(desc, M)
        ws = torch.zeros(max(nb, 16), dtype=torch.uint8, device="cuda") if nb else None
        hq.hq_gemm(desc, M, self.A[r0 * self.K * 2:], None, self.w, self.s, self.z, D, ws, nb)
        torch.cuda.synchronize()
        return to_f64(D[: M * N * 2].cpu().numpy().view(np.uint16).reshape(M, N), self.dt)

    def oracle(self, rows):
        d = self.d
        return oracle.gemm_wnwide(d["A"], d["codes"], d["s"], d.get("z"), N=self.N, K=self.K, G=self.G,
                                  bits=self.bits, a_bf16=self.bf16, w_signed=self.signed, rows=rows)

    def check(self, Dh, rows, out_rows=None):
        O = self.oracle(rows)
        Dr = Dh[rows if out_rows is None else out_rows]
        assert np.all(np.isfinite(Dr))
        err = gate_error(Dr, O)
        assert err <= GATE, err
        assert err <= (8e-3 if self.bf16 else 3e-3), err
        return err


def case(M, N, K, G, bits, signed, bf16, seed, rows=None):
    L = Wide(M, N, K, G, bits, signed, bf16, seed)
    note(f"wnwide M={M} N={N} K={K} G={G} bits={bits} signed={signed} bf16={bf16} seed={seed} "
         f"{hq.hq_gemm_plan(L.desc, M)}")
    L.check(L.run(), sample_rows(M) if rows is None else rows)


@pytest.mark.parametrize("M,N,K,G,bits,signed,bf16", cases.WNWIDE_SMALL)
def test_small_m_stream(M, N, K, G, bits, signed, bf16):
    case(M, N, K, G, bits, signed, bf16, seed=M + bits)


@pytest.mark.parametrize("M,N,K,G,bits,signed,bf16", cases.WNWIDE_TILES)
def test_tiles_ragged(M, N, K, G, bits, signed, bf16):
    """Ragged rows and columns on the tiles, groups of one and two chunks."""
    case(M, N, K, G, bits, signed, bf16, seed=M + N + bits)


@pytest.mark.parametrize("M,N,K,G,bits,signed,bf16", cases.WNWIDE_SWEEP)
def test_full_size_sweep(M, N, K, G, bits, signed, bf16):
    """N = 4096, K = 7168, G = 128 at every M of the benchmark sweep, in the
    launch configuration the benchmark times; sampled rows from M = 16 on."""
    case(M, N, K, G, bits, signed, bf16, seed=0, rows=sweep_rows(M))


@pytest.mark.parametrize("bits,signed", cases.WNWIDE_WIDTHS)
def test_extreme_codes(bits, signed):
    """Every code at the bottom, then at the top of its width, on the stream
    (M = 8) and on the tiles (M = 160)."""
    N, K, G = 144, 1024, 128
    lo, hi = (-(1 << (bits - 1)), (1 << (bits - 1)) - 1) if signed else (0, (1 << bits) - 1)
    for M in (8, 160):
        for c in (lo, hi):
            note(f"wnwide extreme bits={bits} signed={signed} M={M} code={c}")
            codes = np.full((K, N), c, dtype=np.int64).astype(np.int8 if signed else np.uint8)
            L = Wide(M, N, K, G, bits, signed, bf16=bits % 2 == 0, seed=bits, codes=codes)
            L.check(L.run(), np.arange(M))


def test_per_channel_scales():
    """One group over K (G = K = 2048) on both paths."""
    for M in (3, 200):
        case(M, 520, 2048, 2048, 7, False, True, seed=M)


@pytest.mark.parametrize("bits,signed,bf16", [(6, False, True), (8, False, False)])
def test_tuned_paths_and_row_offset(bits, signed, bf16):
    """Forced K splits on the 128 x 128 tiles and on the stream, and rows taken
    from an offset into the activations."""
    L = Wide(160, 1000, 3072, 128, bits, signed, bf16, seed=3)
    tunes = [(hq.HQ_TUNE(hq.HQ_TUNE_T128, 3), 150), (hq.HQ_TUNE(hq.HQ_TUNE_T128, 1), 40),
             (hq.HQ_TUNE(hq.HQ_TUNE_STREAM, 2), 9)]
    if not bf16:     # fp16 also has the 128 x 256 tiles
        tunes += [(hq.HQ_TUNE(hq.HQ_TUNE_W128, 2), 150), (hq.HQ_TUNE(hq.HQ_TUNE_W128, 1), 20)]
    for tune, M in tunes:
        d = autotune.with_tune(L.desc, tune)
        note(f"wnwide tuned bits={bits} M={M} {hq.hq_gemm_plan(d, M)}")
        L.check(L.run(d, M), np.arange(M))
    note(f"wnwide offset bits={bits}")
    L.check(L.run(M=100, r0=60), np.arange(60, 160), out_rows=np.arange(100))


def test_batch_invariant_mode():
    """Batch-invariant mode: the tiles without K split at every M, each row's
    output independent of the other rows of the call."""
    L = Wide(200, 1000, 2048, 128, 8, False, False, seed=5)
    d = hq.hq_layer_desc.from_buffer_copy(L.desc)
    d.flags |= hq.HQ_FLAG_BATCH_INVARIANT
    full = L.run(d, 200)
    L.check(full, np.arange(200))
    part = L.run(d, 7)
    np.testing.assert_array_equal(part, full[:7])
