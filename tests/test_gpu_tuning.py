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

from bit_quantized_gemm_w4a16_amd import autotune, hq
from gpu_layers import FORMATS, Layer
from gpu_util import note

pytestmark = pytest.mark.gpu


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
    # (low-bit and FP6 weights are widened by a kernel of their own before the tile)
    tile = lambda M: [x for x in hq.hq_gemm_plan(d, M) if x.startswith("tile_gemm")]
    shapes = {tile(M)[0].split(" ")[0] for M, _ in WINDOWS + [(BIG, 0)]}
    assert all(len(tile(M)) == 1 and "splits=1" in tile(M)[0] and not any("finalize" in x for x in hq.hq_gemm_plan(d, M))
               for M, _ in WINDOWS)
    big = L.run(d, BIG)
    rows = np.array([0, 1, 777, 2047, 2048, 4094, 4095])
    L.check(big[rows], rows)
    for M, r0 in WINDOWS:
        note(f"batch invariance {fmt} window M={M} r0={r0} {hq.hq_gemm_plan(d, M)[0]}")
        sub = L.run(d, M, r0)
        bad = np.argwhere(sub != big[r0:r0 + M])
        assert bad.size == 0, f"M={M} r0={r0}: {len(bad)} outputs differ, first at {bad[0].tolist()}"
    # the formats with several tile classes reach more than one of them (bf16
    # W4A16 and its low-bit widths have one)
    if fmt not in ("wna16_bf16_sym", "w2a16_int2", "w1a16_int1"):
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
