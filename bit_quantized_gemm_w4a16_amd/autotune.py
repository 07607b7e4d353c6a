"""Autotuning of the dense kernel choice per M bucket.

The library picks a kernel, tile shape and K split for every (layer, M) from
fixed rules.  This module times the alternatives on the device and returns,
per M, the tuning override (the descriptor's ``tune`` field, ``HQ_TUNE(path,
splits)``) that ran fastest -- the autotune of the per-M-bucket table that the
Humming pages plan ("Humming wird angekuendigt", section "Zukuenftige Plaene":
benchmark candidate configurations on the target device to find better
execution parameters per workload).

Candidates are the tuning paths the layer's format has (small-M weight
stream on four waves, or on eight with direct A loads; 128 x 128 / 256-row /
128 x 256 / 256 x 256 tiles) with a range of K splits; ``hq_gemm_plan`` filters out the ones that do not apply.  Every timing
runs the library's own kernels through ``hq_gemm``; nothing is computed here.
"""
from __future__ import annotations

from typing import Callable, Dict, Iterable, List, Tuple

from . import hq

STREAM_SPLITS = (0, 1, 2, 3, 4, 6, 8, 12, 16)
TILE_SPLITS = {hq.HQ_TUNE_T128: (1, 2, 3, 4, 6, 8, 12, 16), hq.HQ_TUNE_T256: (1, 2, 4),
               hq.HQ_TUNE_W128: (1, 2, 4, 8), hq.HQ_TUNE_W256: (1, 2)}


def with_tune(desc: hq.hq_layer_desc, tune: int) -> hq.hq_layer_desc:
    """A copy of the descriptor carrying a tuning override."""
    d = hq.hq_layer_desc.from_buffer_copy(desc)
    d.tune = tune
    return d


def candidates(desc: hq.hq_layer_desc, M: int) -> List[int]:
    """Tuning values that apply to (desc, M): 0 (the library's own choice) first."""
    out = [0]
    tunes = [hq.HQ_TUNE(hq.HQ_TUNE_STREAM, s) for s in STREAM_SPLITS]
    tunes.append(hq.HQ_TUNE(hq.HQ_TUNE_STREAM8, 0))
    for path, splits in TILE_SPLITS.items():
        tunes += [hq.HQ_TUNE(path, s) for s in splits]
    seen = {tuple(hq.hq_gemm_plan(desc, M))}
    for t in tunes:
        try:
            plan = tuple(hq.hq_gemm_plan(with_tune(desc, t), M))
        except hq.HQError:
            continue
        if plan and plan not in seen:       # distinct launches only
            seen.add(plan)
            out.append(t)
    return out


def autotune(desc: hq.hq_layer_desc, sweep: Iterable[int], time_us: Callable[[hq.hq_layer_desc, int], float],
             verbose: Callable[[str], None] | None = None) -> Dict[int, Tuple[int, float, float]]:
    """For each M: (best tune, its time in us, the library's own choice's time in us).

    ``time_us(desc, M)`` runs the layer with the given descriptor (carrying the
    candidate's tune value) and returns its time per call; the caller owns the
    buffers, the cold-cache protocol and the clock."""
    table = {}
    for M in sweep:
        base = time_us(desc, M)
        best, best_t = 0, base
        for t in candidates(desc, M)[1:]:
            us = time_us(with_tune(desc, t), M)
            if verbose:
                verbose(f"[autotune] M={M} tune=0x{t:x} {us:.2f} us {hq.hq_gemm_plan(with_tune(desc, t), M)}")
            if us < best_t:
                best, best_t = t, us
        table[M] = (best, best_t, base)
        if verbose:
            verbose(f"[autotune] M={M}: best 0x{best:x} {best_t:.2f} us (library's choice {base:.2f} us)")
    return table


def plan_name(desc: hq.hq_layer_desc, tune: int, M: int) -> str:
    return "; ".join(hq.hq_gemm_plan(with_tune(desc, tune), M))
