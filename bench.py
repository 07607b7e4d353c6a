#!/usr/bin/env python3
"""Benchmark of the hq quantized GEMM on one MI355X.

A step is one pass of the hot path over the workload's M sweep: for every
M in {1, 2, 4, ..., 8192} one library call (host dispatch -> HIP kernels ->
output) on inputs already resident in HBM.  The default workload is the
dense W4A16 asymmetric layer (fp16 activations, UINT4 weights with UINT4
zero-points and fp16 scales per 128 K, N=4096, K=7168), the configuration
the metric is quoted on.  --config c1|c3|c4|c5|c5g|c5l|all measures the other
workloads (one JSON line each); c5 is the MoE gate-up on the Indexed path, c5g
the same on the Grouped path, c5l the whole MoE layer the pages time (gate-up
GEMM, SwiGLU, down-projection GEMM).

Cold cache: the packed weights are replicated into enough device copies
(> 512 MiB in total, more than the 256 MiB Infinity Cache plus every L2) and
successive calls rotate through them, so every call streams its weights from
HBM, as in the pages' cold-L2 protocol ("Humming wird angekuendigt", section
"Leistung").

Timing: the calls are captured into HIP graphs, so host launch overhead does
not starve the GPU.  Per M: a graph of back-to-back calls (one per weight
copy) is replayed between HIP events on the capturing stream.  Per step: a
graph of the whole sweep is replayed, K replays bracketed by
torch.cuda.synchronize(); `value` = total algorithmic flops of one step /
step wall time.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synthetic as syn  # noqa: E402
from bit_quantized_gemm_w4a16_amd import hq  # noqa: E402

PEAK_HBM = 8.0e12          # B/s, MI355X HBM3E
PEAK = {"fp16": 2.5e15, "bf16": 2.5e15, "fp8": 5.0e15, "int8": 5.0e15}
SWEEP = [1 << i for i in range(14)]
COLD_BYTES = 512 << 20
METRIC = "quant GEMM TFLOP/s + HBM GB/s vs roofline, M=1..8192, W4A16/W4A8/MoE"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.uint8).reshape(-1).copy()).to("cuda")


def _cores():
    omp = os.environ.get("OMP_NUM_THREADS")
    n = len(os.sched_getaffinity(0))
    return min(n, int(omp)) if omp and omp.isdigit() else n


def _timed_oracle(fn, nrows_for, budget_s):
    """Time fn(rows) on a row sample of about budget_s of CPU work: the sample
    doubles until one run takes at least budget_s / 2 (the oracle's cost per
    row grows once its output leaves the caches, so no linear extrapolation)."""
    n = 2
    while True:
        rows = nrows_for(n)
        t0 = time.perf_counter()
        fn(rows)
        dt = time.perf_counter() - t0
        if dt >= budget_s / 2 or len(nrows_for(2 * n)) == len(rows):
            return len(rows), dt
        n *= 2


def _copies(tensors, nbytes, minimum=2):
    n = max(minimum, -(-COLD_BYTES // max(nbytes, 1)))
    return [tuple(None if t is None else t.clone() for t in tensors) for _ in range(n)]


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------

class DenseW4A16:
    """Dense W4A16 (UINT4 + zero-points fp16, or symmetric INT4 bf16), group 128."""

    def __init__(self, N=4096, K=7168, G=128, Mmax=8192, bf16=False, zp=True, sweep=SWEEP, name=None):
        self.N, self.K, self.G, self.Mmax = N, K, G, Mmax
        self.bf16, self.zp, self.sweep = bf16, zp, sweep
        self.dtype = "bf16" if bf16 else "fp16"
        self.name = name or f"dense_w4a16_{'zp' if zp else 'sym'}_{self.dtype}_N{N}_K{K}"
        t = torch.bfloat16 if bf16 else torch.float16
        log(f"[bench] generating {self.name}")
        d = syn.w4a16_zp(0, Mmax, N, K, G, t) if zp else syn.w4a16_sym(0, Mmax, N, K, G, t, cfg=syn.C1)
        self.host = d
        self.desc = hq.desc_w4a16(N, K, G, bf16=bf16, zp=zp)
        wp, sp, zpk = hq.hq_repack(self.desc, d["q"], d["s"], d.get("z") if zp else None)
        self.wbytes = wp.size + sp.size + (zpk.size if zpk is not None else 0)
        self.copies = _copies((dev(wp), dev(sp), dev(zpk) if zp else None), self.wbytes)
        self.A = dev(d["A"])
        self.D = torch.empty(Mmax * N * 2, dtype=torch.uint8, device="cuda")
        self.ws_bytes = max(hq.hq_workspace_bytes(self.desc, m) for m in sweep)
        self.ws = torch.zeros(max(self.ws_bytes, 16), dtype=torch.uint8, device="cuda")

    def flops(self, M):
        return 2.0 * M * self.N * self.K

    def bytes(self, M):
        return self.wbytes + M * self.K * 2 + M * self.N * 2

    def kernel_of(self, M):
        if M <= 64:
            return (f"skinny_kernel<WNA16_{self.dtype.upper()}> (M<=64)", "hbm")
        return (f"tile_gemm_kernel<WNA16_{self.dtype.upper()}> (M>64)", "mfma" if M >= 128 else "hbm")

    def call(self, M, c):
        w, s, z = self.copies[c]
        hq.hq_gemm(self.desc, M, self.A, None, w, s, z, self.D, self.ws if self.ws_bytes else None, self.ws_bytes)

    def cpu_baseline(self, budget_s=16.0):
        import oracle
        d = self.host
        f = lambda rows: oracle.gemm_wna16(d["A"], d["q"], d["s"], d.get("z"), N=self.N, K=self.K, G=self.G,
                                           a_bf16=self.bf16, w_signed=not self.zp, rows=rows)
        n, dt = _timed_oracle(f, lambda n: np.arange(min(n, self.Mmax)), budget_s)
        return dict(value=round(self.flops(n) / dt / 1e12, 6), unit="TFLOP/s", cores=_cores(), kind="oracle",
                    sample=f"{n} output rows x N={self.N} x K={self.K}, fp64 accumulation, {dt:.1f} s")


class DenseW4A8:
    """Dense W4A8-MXFP4: tokenwise e4m3 activations (quantised on the GPU, untimed)."""

    def __init__(self, N=7168, K=4096, Mmax=8192, sweep=SWEEP):
        self.N, self.K, self.Mmax, self.sweep = N, K, Mmax, sweep
        self.dtype = "fp8"
        self.name = f"dense_w4a8_mxfp4_N{N}_K{K}"
        log(f"[bench] generating {self.name}")
        d = syn.w4a8_mxfp4(0, Mmax, N, K)
        self.host = d
        self.desc = hq.desc_w4a8_mxfp4(N, K)
        wp, ep, _ = hq.hq_repack(self.desc, d["q"], d["e"])
        self.wbytes = wp.size + ep.size
        self.copies = _copies((dev(wp), dev(ep)), self.wbytes)
        x = dev(d["A0"])
        self.A = torch.empty(Mmax * K, dtype=torch.uint8, device="cuda")
        self.s_a = torch.empty(Mmax, dtype=torch.float32, device="cuda")
        hq.hq_quantize_act(hq.HQ_DT_FP8_E4M3, Mmax, K, x, self.A, self.s_a)
        torch.cuda.synchronize()
        del x
        self.D = torch.empty(Mmax * N * 2, dtype=torch.uint8, device="cuda")
        self.ws_bytes = max(hq.hq_workspace_bytes(self.desc, m) for m in sweep)
        self.ws = torch.empty(max(self.ws_bytes, 16), dtype=torch.uint8, device="cuda")

    def flops(self, M):
        return 2.0 * M * self.N * self.K

    def bytes(self, M):
        return self.wbytes + M * self.K + 4 * M + M * self.N * 2

    def kernel_of(self, M):
        if M <= 64:
            return ("skinny_kernel<W4A8_MX> (M<=64)", "hbm")
        return ("tile_gemm_kernel<W4A8_MX> (M>64)", "mfma" if M >= 256 else "hbm")

    def call(self, M, c):
        w, e = self.copies[c]
        hq.hq_gemm(self.desc, M, self.A, self.s_a, w, e, None, self.D, self.ws if self.ws_bytes else None, self.ws_bytes)

    def aux(self, reps=20):
        """The activation quantisation before the GEMM (outside the timed
        sweep): fp32 [Mmax][K] in, e4m3 codes + one fp32 scale per row out,
        timed alone with HIP events on the launching stream; two input copies
        used in turn (268 MB together) so that no call finds its input in the
        Infinity Cache."""
        xs = [dev(self.host["A0"]) for _ in range(2)]
        q = torch.empty_like(self.A)
        s = torch.empty_like(self.s_a)
        f = lambda i: hq.hq_quantize_act(hq.HQ_DT_FP8_E4M3, self.Mmax, self.K, xs[i % 2], q, s)
        for i in range(4):
            f(i)
        st = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for i in range(reps):
            f(i)
        e1.record(st)
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3 / reps
        B = self.Mmax * self.K * 5 + 4 * self.Mmax
        del xs, q, s
        return {"act_quant": dict(kernel="quant_e4m3_rows_kernel", M=self.Mmax, K=self.K, us=round(t * 1e6, 2),
                                  algorithmic_bytes=B, gbps=round(B / t / 1e9, 1),
                                  hbm_frac=round(B / t / PEAK_HBM, 3))}

    def cpu_baseline(self, budget_s=16.0):
        import oracle
        d = self.host
        qa, s_a = oracle.quant_act_e4m3(d["A0"][:64])
        f = lambda rows: oracle.gemm_w4a8_mxfp4(qa, s_a, d["q"], d["e"], N=self.N, K=self.K, rows=rows)
        n, dt = _timed_oracle(f, lambda n: np.arange(min(n, 64)), budget_s)
        return dict(value=round(self.flops(n) / dt / 1e12, 6), unit="TFLOP/s", cores=_cores(), kind="oracle",
                    sample=f"{n} output rows x N={self.N} x K={self.K}, fp64 accumulation, {dt:.1f} s")


class DenseW8A8:
    """Dense W8A8 INT8 with per-token x per-channel epilogue, bf16 output."""

    def __init__(self, N=18432, K=7168, Mmax=8192, sweep=SWEEP):
        self.N, self.K, self.Mmax, self.sweep = N, K, Mmax, sweep
        self.dtype = "int8"
        self.name = f"dense_w8a8_int8_N{N}_K{K}"
        log(f"[bench] generating {self.name}")
        d = syn.w8a8_int8(0, Mmax, N, K)
        self.host = d
        self.desc = hq.desc_w8a8(N, K)
        wp, sp, _ = hq.hq_repack(self.desc, d["w"], d["s_w"])
        self.wbytes = wp.size + sp.size
        self.copies = _copies((dev(wp), dev(sp)), self.wbytes)
        self.A = dev(d["a"])
        self.s_a = dev(d["s_a"])
        self.D = torch.empty(Mmax * N * 2, dtype=torch.uint8, device="cuda")
        self.ws_bytes = max(hq.hq_workspace_bytes(self.desc, m) for m in sweep)
        self.ws = torch.empty(max(self.ws_bytes, 16), dtype=torch.uint8, device="cuda")

    def flops(self, M):
        return 2.0 * M * self.N * self.K

    def bytes(self, M):
        return self.wbytes + M * self.K + 4 * M + M * self.N * 2

    def kernel_of(self, M):
        if M <= 64:
            return ("skinny_kernel<W8A8_I8> (M<=64)", "hbm")
        return ("tile_gemm_kernel<W8A8_I8> (M>64)", "mfma" if M >= 512 else "hbm")

    def call(self, M, c):
        w, s = self.copies[c]
        hq.hq_gemm(self.desc, M, self.A, self.s_a, w, s, None, self.D, self.ws if self.ws_bytes else None, self.ws_bytes)

    def cpu_baseline(self, budget_s=16.0):
        import oracle
        d = self.host
        f = lambda rows: oracle.gemm_w8a8(d["a"], d["s_a"], d["w"], d["s_w"], rows=rows)
        n, dt = _timed_oracle(f, lambda n: np.arange(min(n, self.Mmax)), budget_s)
        return dict(value=round(self.flops(n) / dt / 1e12, 6), unit="TOP/s", cores=_cores(), kind="oracle",
                    sample=f"{n} output rows x N={self.N} x K={self.K}, exact int64 accumulation, {dt:.1f} s")


class MoEMXFP4:
    """MoE W4A16-MXFP4 gate+up: E=256, top-8, N=4096, K=7168, Zipf(1.1) routing; Indexed path
    (each call = routing metadata + expert GEMM)."""

    def __init__(self, E=256, top_k=8, N=4096, K=7168, Tmax=8192, sweep=SWEEP, mode="indexed"):
        self.E, self.top_k, self.N, self.K, self.Tmax, self.sweep = E, top_k, N, K, Tmax, sweep
        self.mode = mode
        self.dtype = "bf16"
        self.name = f"moe_w4a16_mxfp4_{mode}_E{E}_top{top_k}_N{N}_K{K}"
        log(f"[bench] generating {self.name} (all {E} experts)")
        d = syn.moe_mxfp4(0, Tmax, E, top_k, N, K)
        self.host = d
        self.desc = hq.desc_moe_mxfp4(E, N, K)
        wp, ep, _ = hq.hq_repack(self.desc, d["q"], d["e"])
        self.ebytes = (wp.size + ep.size) // E
        n = 3                                     # 3 x 3.8 GB: > 256 MiB between reuses at every T
        w0, e0 = dev(wp), dev(ep)
        self.copies = [(w0, e0)] + [(w0.clone(), e0.clone()) for _ in range(n - 1)]
        del wp, ep
        self.ids = dev(d["ids"].astype(np.int32))
        self.A = dev(d["A"])
        self.D = torch.empty(Tmax * top_k * N * 2, dtype=torch.uint8, device="cuda")
        self.ws_bytes = hq.hq_workspace_bytes(self.desc, Tmax, top_k)
        self.ws = torch.zeros(self.ws_bytes, dtype=torch.uint8, device="cuda")
        flat = d["ids"]
        self.active = {T: len(np.unique(flat[:T])) for T in sweep}

    def flops(self, T):
        return 2.0 * T * self.top_k * self.N * self.K

    def bytes(self, T):
        return self.active[T] * self.ebytes + T * self.K * 2 + T * self.top_k * (self.N * 2 + 4)

    def kernel_of(self, T):
        return ("moe: routing + moe_stream_kernel + tile_gemm_kernel<MOE_MX> tiers", "mfma" if T >= 4096 else "hbm")

    def call(self, T, c):
        w, e = self.copies[c]
        hq.hq_moe_gemm(self.desc, hq.HQ_MOE_INDEXED, T, self.top_k, self.A, None, self.ids, None, w, e, None, self.D,
                       self.ws, self.ws_bytes)

    def cpu_baseline(self, budget_s=16.0):
        import oracle
        d = self.host
        ids = d["ids"][:64]
        sub_e = sorted(set(int(e) for e in ids.reshape(-1)))
        f = lambda pairs: oracle.moe_mxfp4_bf16(d["A"][:64], ids, d["q"], d["e"], N=self.N, K=self.K, pairs=pairs)
        n, dt = _timed_oracle(f, lambda n: np.arange(min(n, 64 * self.top_k)), budget_s)
        return dict(value=round(2.0 * n * self.N * self.K / dt / 1e12, 6), unit="TFLOP/s", cores=_cores(),
                    kind="oracle", sample=f"{n} (token, expert) pairs of 64 tokens x N={self.N} x K={self.K} "
                                          f"({len(sub_e)} experts touched), fp64 accumulation, {dt:.1f} s")


class MoEGroupedMXFP4(MoEMXFP4):
    """The same MoE gate+up on the Grouped path: tokens already sorted by expert
    (the Grouped path's input).  The expert offsets and the sorted rows are built
    once per T with the library's own routing and gather (hq_moe_align,
    hq_moe_gather) before timing; each timed call is the expert GEMM alone."""

    def __init__(self):
        super().__init__(mode="grouped")
        E, k, K = self.E, self.top_k, self.K
        self.rows = {}
        for T in self.sweep:
            P = T * k
            offs = torch.empty(E + 4, dtype=torch.int32, device="cuda")
            srt = torch.empty(max(P, 4), dtype=torch.int32, device="cuda")
            nb = hq.hq_workspace_bytes(self.desc, T, k)
            ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
            hq.hq_moe_align(T, k, E, self.ids, offs, srt, ws, nb)
            As = torch.empty(P * K * 2, dtype=torch.uint8, device="cuda")
            hq.hq_moe_gather(hq.HQ_DT_BF16, T, k, K, self.A, srt, As)
            self.rows[T] = (As, offs)
        torch.cuda.synchronize()

    def bytes(self, T):
        P = T * self.top_k
        return self.active[T] * self.ebytes + P * self.K * 2 + P * self.N * 2 + (self.E + 1) * 4

    def call(self, T, c):
        w, e = self.copies[c]
        As, offs = self.rows[T]
        hq.hq_moe_gemm(self.desc, hq.HQ_MOE_GROUPED, T, self.top_k, As, None, None, offs, w, e, None, self.D,
                       self.ws, self.ws_bytes)


class MoELayerMXFP4(MoEMXFP4):
    """The MoE layer the pages time (gate-up + down): gate-up W4A16-MXFP4 (N=4096, K=7168,
    Indexed), SwiGLU, down projection (N=7168, K=2048, Indexed with one row per pair),
    E=256, top-8, Zipf(1.1) routing; each call = the three steps with their routing."""

    def __init__(self, N2=7168):
        super().__init__()
        self.N2, self.I = N2, self.N // 2
        self.name = f"moe_layer_w4a16_mxfp4_E{self.E}_top{self.top_k}_N{self.N}_K{self.K}_down_N{N2}_K{self.I}"
        log(f"[bench] generating the down projection (all {self.E} experts)")
        d2 = syn.moe_mxfp4(1, 1, self.E, 1, N2, self.I)
        self.desc2 = hq.desc_moe_mxfp4(self.E, N2, self.I)
        wp, ep, _ = hq.hq_repack(self.desc2, d2["q"], d2["e"])
        self.ebytes2 = (wp.size + ep.size) // self.E
        w0, e0 = dev(wp), dev(ep)
        self.copies2 = [(w0, e0)] + [(w0.clone(), e0.clone()) for _ in range(len(self.copies) - 1)]
        del wp, ep, d2
        P = self.Tmax * self.top_k
        self.flat = dev(self.host["ids"].reshape(-1).astype(np.int32))
        self.H = torch.empty(P * self.I * 2, dtype=torch.uint8, device="cuda")
        self.D2 = torch.empty(P * N2 * 2, dtype=torch.uint8, device="cuda")
        self.ws_bytes = max(self.ws_bytes, hq.hq_workspace_bytes(self.desc2, P, 1))
        self.ws = torch.zeros(self.ws_bytes, dtype=torch.uint8, device="cuda")

    def flops(self, T):
        return 2.0 * T * self.top_k * (self.N * self.K + self.N2 * self.I)

    def bytes(self, T):
        P = T * self.top_k
        return (self.active[T] * (self.ebytes + self.ebytes2) + T * self.K * 2 + P * (self.N * 2 + 4) * 2
                + P * self.I * 2 * 2 + P * self.N2 * 2)

    def kernel_of(self, T):
        return ("moe layer: gate-up + silu_mul + down (routing, moe_stream_kernel, tile_gemm_kernel<MOE_MX> tiers)",
                "mfma" if T >= 4096 else "hbm")

    def call(self, T, c):
        super().call(T, c)
        P = T * self.top_k
        hq.hq_silu_mul(hq.HQ_DT_BF16, P, self.I, self.D, self.H)
        w, e = self.copies2[c]
        hq.hq_moe_gemm(self.desc2, hq.HQ_MOE_INDEXED, P, 1, self.H, None, self.flat, None, w, e, None, self.D2,
                       self.ws, self.ws_bytes)

    def cpu_baseline(self, budget_s=16.0):
        b = super().cpu_baseline(budget_s)
        b["sample"] = "gate-up projection only: " + b["sample"]
        return b


WORKLOADS = {
    "c1": lambda: DenseW4A16(N=1024, K=1024, Mmax=16, bf16=True, zp=False, sweep=[16],
                             name="dense_w4a16_sym_bf16_M16_N1024_K1024"),
    "c2": lambda: DenseW4A16(),
    "c3": lambda: DenseW4A8(),
    "c4": lambda: DenseW8A8(),
    "c5": lambda: MoEMXFP4(),
    "c5g": lambda: MoEGroupedMXFP4(),
    "c5l": lambda: MoELayerMXFP4(),
}


# ---------------------------------------------------------------------------

def _capture(fn):
    """Capture fn() (a sequence of hq calls on the current stream) into a HIP graph."""
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                      # eager run on the capture stream
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=side):
        fn()
    torch.cuda.synchronize()
    return g


class _Eager:
    """Stand-in for a captured graph: replay() issues the calls directly (for
    counter-collection runs, which need plain dispatches)."""

    def __init__(self, fn):
        self.fn = fn

    def replay(self):
        self.fn()


def run(work, steps, warmup, eager=False):
    """Per-M timing from graphs of back-to-back calls (each on its own cold weight copy),
    and the step timing from graphs of whole sweeps (rotating copies)."""
    sweep = work.sweep
    ncopy = len(work.copies)
    per = {}
    capture = _Eager if eager else _capture
    for M in sweep:
        def calls(M=M):
            for r in range(ncopy):
                work.call(M, r)
        g = capture(calls)
        g.replay()
        torch.cuda.synchronize()
        reps = 3
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        per[M] = e0.elapsed_time(e1) * 1e-3 / (reps * ncopy)
        del g
    nsw = max(1, ncopy // len(sweep))
    graphs = []
    for j in range(nsw):
        def sweep_calls(j=j):
            for i, M in enumerate(sweep):
                work.call(M, (j * len(sweep) + i) % ncopy)
        graphs.append(capture(sweep_calls))
    for w in range(warmup):
        graphs[w % nsw].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        graphs[k % nsw].replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, per


# The sources the counted kernel (the dense W4A16 tile GEMM and its launch) is
# built from: counter figures taken on other versions of them are stale.
KERNEL_SOURCES = ["bit_quantized_gemm_w4a16_amd/csrc/" + f for f in
                  ("tile_gemm.hpp", "skinny.hpp", "hq_device.hpp", "hq_internal.h", "hq_common.h", "k_wna16.hip")]
KERNEL_SOURCES.append("include/hq.h")


def kernel_source_hash():
    """Hash of the counted kernel's sources; counter figures taken on other sources are stale."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _traffic(workload, M):
    """HBM bytes per launch from the committed counter runs (profiles/traffic.json):
    FETCH_SIZE + WRITE_SIZE per dispatch, each scaled by the factor the same counter
    gives on a plain device copy of known size.  None when absent or stale."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh).get(workload)
    if not rec or rec.get("M") != M or rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def copy_probe(nbytes, reps):
    """A plain device-to-device copy of nbytes (read nbytes, write nbytes), reps times:
    the reference for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "reps": reps}), flush=True)


def report(work, args, wall, per):
    ms_per_step = wall / args.steps * 1e3
    flops_step = sum(work.flops(M) for M in work.sweep)
    peak = PEAK[work.dtype]
    table, kern = [], {}
    for M in work.sweep:
        t = per[M]
        F, B = work.flops(M), work.bytes(M)
        table.append(dict(M=M, us=round(t * 1e6, 2), tflops=round(F / t / 1e12, 2), gbps=round(B / t / 1e9, 1),
                          hbm_frac=round(B / t / PEAK_HBM, 3), mfma_frac=round(F / t / peak, 3),
                          roofline_frac=round(max(B / PEAK_HBM, F / peak) / t, 3)))
        name, bound = work.kernel_of(M)
        k = kern.setdefault(name, dict(F=0.0, B=0.0, t=0.0, n=0, bounds={}))
        k["F"] += F
        k["B"] += B
        k["t"] += t
        k["n"] += 1
        k["bounds"][bound] = k["bounds"].get(bound, 0.0) + t
    # Roofline of the dominant kernel, taken at the sweep's largest M, where one
    # call is one launch of it: achieved = algorithmic flops (or bytes) of that
    # launch / its average duration over back-to-back launches (HIP events on
    # the launching stream).
    dom = max(kern, key=lambda n: kern[n]["t"])
    Mr = max(M for M in work.sweep if work.kernel_of(M)[0] == dom)
    name, bound = work.kernel_of(Mr)
    t, F, B = per[Mr], work.flops(Mr), work.bytes(Mr)
    if bound == "mfma":
        roof = dict(bound="mfma", achieved=round(F / t / 1e12, 1), peak=peak / 1e12,
                    unit="TFLOP/s" if work.dtype != "int8" else "TOP/s", frac=round(F / t / peak, 4))
    else:
        roof = dict(bound="hbm", achieved=round(B / t / 1e9, 1), peak=PEAK_HBM / 1e9, unit="GB/s",
                    frac=round(B / t / PEAK_HBM, 4))
    roof.update(traffic=_traffic(work.name, Mr), kernel=dom, M=Mr, avg_us=round(t * 1e6, 2),
                algorithmic_flops=F, algorithmic_bytes=B,
                per_unit="2*M*N*K flops per launch" if bound == "mfma" else "algorithmic bytes per launch")
    cpu = None if args.no_cpu_baseline else work.cpu_baseline()
    return {
        "metric": METRIC,
        "value": round(flops_step / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s" if work.dtype != "int8" else "TOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": work.dtype,
        "data": "synthetic",
        "config": {"workload": work.name, "M_sweep": work.sweep, "N": work.N, "K": work.K,
                   "cold_weight_copies": len(work.copies)},
        "roofline": roof,
        "cpu_baseline": cpu,
        "per_M": table,
        **({"aux": work.aux()} if hasattr(work, "aux") else {}),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="c2", help="c1|c2|c3|c4|c5|c5g|c5l|all (default c2; c5g = MoE on the Grouped path, c5l = MoE gate-up + SwiGLU + down)")
    ap.add_argument("--sweep", default=None, help="comma-separated M values (default 1..8192 powers of 2)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true", help="issue calls directly instead of replaying HIP graphs "
                    "(for counter-collection runs)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(the sharding design is described in DESIGN.md); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.copy_probe:
        copy_probe(args.copy_probe, args.steps)
        return
    names = list(WORKLOADS) if args.config == "all" else [args.config]
    for nm in names:
        if nm not in WORKLOADS:
            raise SystemExit(f"unknown --config {nm}")
        work = WORKLOADS[nm]()
        if args.sweep and nm != "c1":
            work.sweep = [int(x) for x in args.sweep.split(",")]
            if hasattr(work, "active"):
                flat = work.host["ids"]
                work.active = {T: len(np.unique(flat[:T])) for T in work.sweep}
        wall, per = run(work, args.steps, args.warmup, eager=args.eager)
        print(json.dumps(report(work, args, wall, per)), flush=True)
        del work
        torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
