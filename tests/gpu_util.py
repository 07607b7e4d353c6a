"""Shared helpers for the GPU parity tests (imported by tests/test_gpu_*.py).

The HIP path is always driven through the C ABI (bit_quantized_gemm_w4a16_amd.hq);
expected values always come from the CPU oracle on the same seeded inputs.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

from bit_quantized_gemm_w4a16_amd import hq

# The gate for floating outputs: max |D - O| / max(|O|, rms(O)) <= 1e-2, with
# rms over every compared output of the case ("parity").
GATE = 1e-2


def note(msg: str) -> None:
    """Name the case on stdout before it touches the GPU (kept if a run dies)."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    """Host numpy -> device tensor holding the same bytes."""
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.uint8).reshape(-1).copy())
    return t.to("cuda")


def empty(nbytes: int) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device="cuda")


def workspace(desc, M, top_k=0):
    nb = hq.hq_workspace_bytes(desc, M, top_k)
    if nb == 0:
        return None, 0
    ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    return ws, nb


def to_f64(bits: np.ndarray, dt: torch.dtype) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(dt).to(torch.float64).numpy()


def gate_error(D: np.ndarray, O: np.ndarray) -> float:
    rms = float(np.sqrt(np.mean(O * O))) if O.size else 0.0
    den = np.maximum(np.abs(O), rms)
    den = np.where(den > 0, den, 1.0)
    return float(np.max(np.abs(D - O) / den)) if O.size else 0.0


def sample_rows(M: int, seed: int = 0, tile: int = 128, extra: int = 64) -> np.ndarray:
    """Rows to compare at sizes where the oracle cannot do every row: first and
    last row of every 128-row tile plus `extra` seeded random rows."""
    if M <= 256:
        return np.arange(M)
    rows = set()
    for t0 in range(0, M, tile):
        rows.add(t0)
        rows.add(min(M, t0 + tile) - 1)
    rows.update(np.random.default_rng([seed, M]).choice(M, size=min(extra, M), replace=False).tolist())
    return np.array(sorted(rows), dtype=np.int64)


def sweep_rows(M: int, seed: int = 1, extra: int = 12) -> np.ndarray:
    """Rows to compare at full-size sweep points: every row up to M = 8, else the
    first two, the last two and `extra` seeded random rows."""
    if M <= 8:
        return np.arange(M)
    rows = {0, 1, M - 2, M - 1}
    rows.update(np.random.default_rng([seed, M]).choice(M, size=min(extra, M), replace=False).tolist())
    return np.array(sorted(rows), dtype=np.int64)
