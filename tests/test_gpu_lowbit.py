"""GPU parity of the low-bit WnA16 path (INT1/2/3 two's-complement codes,
UINT1/2/3 with 4-bit zero-points, 16-bit group scales) against the CPU oracle,
through the C ABI.  The small-M stream decodes the bit planes in registers; the
tiles read the planes widened to the 4-bit layout in the workspace."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from bit_quantized_gemm_w4a16_amd import autotune, hq
import cases
from gpu_util import GATE, dev, empty, gate_error, note, sample_rows, sweep_rows, to_f64

pytestmark = pytest.mark.gpu


class Low:
    """One seeded low-bit layer on the device."""

    def __init__(self, M, N, K, G, bits, signed, bf16, seed=0, codes=None):
        self.M, self.N, self.K, self.G, self.bits, self.signed, self.bf16 = M, N, K, G, bits, signed, bf16
        self.dt = torch.bfloat16 if bf16 else torch.float16
        self.d = syn.wnlow(seed, M, N, K, bits, signed, G=G, dtype=self.dt)
        if codes is not None:
            self.d["codes"] = codes
        self.desc = hq.desc_wnlow(N, K, bits, signed, G, bf16=bf16)
        wp, sp, zp = hq.hq_repack(self.desc, self.d["codes"], self.d["s"], self.d.get("z"))
        self.A, self.w, self.s = dev(self.d["A"]), dev(wp), dev(sp)
        self.z = dev(zp) if zp is not None else None

    def run(self, desc=None, ws=None, nb=None):
        desc = desc or self.desc
        M, N = self.M, self.N
        D = empty(M * N * 2)
        if ws is None:
            nb = hq.hq_workspace_bytes(desc, M)
            ws = torch.zeros(max(nb, 16), dtype=torch.uint8, device="cuda") if nb else None
        hq.hq_gemm(desc, M, self.A, None, self.w, self.s, self.z, D, ws, nb)
        torch.cuda.synchronize()
        return to_f64(D[: M * N * 2].cpu().numpy().view(np.uint16).reshape(M, N), self.dt)

    def oracle(self, rows):
        d = self.d
        return oracle.gemm_wnlow(d["A"], d["codes"], d["s"], d.get("z"), N=self.N, K=self.K, G=self.G,
                                 bits=self.bits, a_bf16=self.bf16, w_signed=self.signed, rows=rows)

    def check(self, Dh, rows):
        O = self.oracle(rows)
        Dr = Dh[rows]
        assert np.all(np.isfinite(Dr))
        err = gate_error(Dr, O)
        assert err <= GATE, err
        assert err <= (8e-3 if self.bf16 else 3e-3), err
        return err


def case(M, N, K, G, bits, signed, bf16, seed, rows=None):
    note(f"wnlow M={M} N={N} K={K} G={G} bits={bits} signed={signed} bf16={bf16} seed={seed}")
    L = Low(M, N, K, G, bits, signed, bf16, seed)
    L.check(L.run(), sample_rows(M) if rows is None else rows)


@pytest.mark.parametrize("M,N,K,G,bits,signed,bf16", cases.WNLOW_SMALL)
def test_small_m_stream(M, N, K, G, bits, signed, bf16):
    case(M, N, K, G, bits, signed, bf16, seed=M + bits)


@pytest.mark.parametrize("M,N,K,G,bits,signed,bf16", cases.WNLOW_TILES)
def test_widened_tiles_ragged(M, N, K, G, bits, signed, bf16):
    case(M, N, K, G, bits, signed, bf16, seed=M + N + bits)


@pytest.mark.parametrize("M,N,K,G,bits,signed,bf16", cases.WNLOW_SWEEP)
def test_full_size_sweep(M, N, K, G, bits, signed, bf16):
    """N = 4096, K = 7168, G = 128 at every M of the benchmark sweep, in the
    launch configuration the benchmark times; sampled rows from M = 16 on."""
    case(M, N, K, G, bits, signed, bf16, seed=0, rows=sweep_rows(M))


@pytest.mark.parametrize("bits,signed", cases.WNLOW_WIDTHS)
def test_extreme_codes(bits, signed):
    """Every code at the bottom, then at the top of its width, on the stream
    (M = 8) and on the tiles (M = 160)."""
    N, K, G = 144, 1024, 128
    lo, hi = (-(1 << (bits - 1)), (1 << (bits - 1)) - 1) if signed else (0, (1 << bits) - 1)
    for M in (8, 160):
        for c in (lo, hi):
            note(f"wnlow extreme bits={bits} signed={signed} M={M} code={c}")
            L = Low(M, N, K, G, bits, signed, bf16=False, seed=bits, codes=np.full((K, N), c, dtype=np.int8))
            L.check(L.run(), np.arange(M))


@pytest.mark.parametrize("bits,signed", [(3, False), (1, True)])
def test_tile_override_at_small_m_with_split(bits, signed):
    """HQ_TUNE_T128 with a K split at M = 8: the widened weights and the
    partial tiles share the workspace."""
    M, N, K, G = 8, 1000, 2048, 128
    note(f"wnlow tile override bits={bits} signed={signed} M={M}")
    L = Low(M, N, K, G, bits, signed, bf16=True, seed=3)
    d = autotune.with_tune(L.desc, hq.HQ_TUNE(hq.HQ_TUNE_T128, 4))
    plan = hq.hq_gemm_plan(d, M)
    assert plan[0].startswith("widen_lowbit_kernel") and "splits=4" in plan[1]
    L.check(L.run(d), np.arange(M))


def test_workspace_shared_with_4bit_layers_and_sizes():
    """One workspace serves, back to back, a 4-bit tile call, low-bit tile calls
    of two widths and a low-bit split stream call: each call writes what it reads."""
    N, K, G = 1024, 2048, 128
    layers = [Low(300, N, K, G, 3, False, False, seed=1), Low(40, N, K, G, 2, True, False, seed=2),
              Low(700, N, K, G, 1, True, False, seed=3)]
    d4 = syn.w4a16_zp(4, 500, N, K, G, torch.float16)
    desc4 = hq.desc_w4a16(N, K, G, bf16=False, zp=True)
    nb = max([hq.hq_workspace_bytes(L.desc, L.M) for L in layers] + [hq.hq_workspace_bytes(desc4, 500)])
    ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    wp, sp, zp = hq.hq_repack(desc4, d4["q"], d4["s"], d4["z"])
    for L in layers:
        note(f"wnlow shared workspace 4-bit then bits={L.bits} M={L.M}")
        D = empty(500 * N * 2)
        hq.hq_gemm(desc4, 500, dev(d4["A"]), None, dev(wp), dev(sp), dev(zp), D, ws, nb)
        L.check(L.run(ws=ws, nb=nb), sample_rows(L.M))
