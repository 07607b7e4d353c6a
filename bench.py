#!/usr/bin/env python3
"""Benchmark of the hq quantized GEMM on one MI355X.

A step is one pass of the hot path over the workload's M sweep: for every
M in {1, 2, 4, ..., 8192} one library call (host dispatch -> HIP kernels ->
output) on inputs already resident in HBM.  The headline workload is the
dense W4A16 asymmetric layer (fp16 activations, UINT4 weights with UINT4
zero-points and fp16 scales per 128 K, N=4096, K=7168), the configuration
the metric is quoted on; its line also carries, under "configs", the same
measurement of every other workload (dense W4A8-MXFP4, W8A8-INT8, the MoE
gate-up on the Indexed path with its routing timed apart, W4A4 MXFP4 x MXFP4,
MXFP8 x MXFP4, FP8 W8A8 with blockwise scales, bf16 x MXFP4, NVFP4 and MXINT4 WnA16, INT8 and FP8 weight-only).
--config NAME measures one workload alone (c5g: the MoE Grouped path, c5l:
the whole MoE layer the pages time, gate-up + SwiGLU + down).

Cold cache: the packed weights are replicated into enough device copies
(> 512 MiB in total, more than the 256 MiB Infinity Cache plus every L2) and
successive calls rotate through them, so every call streams its weights from
HBM, as in the pages' cold-L2 protocol ("Humming wird angekuendigt", section
"Leistung").

Timing: the calls are captured into HIP graphs, so host launch overhead does
not starve the GPU.  Per M: a graph of back-to-back calls (one per weight
copy) is replayed several times, each replay between HIP events on the
capturing stream; per-call time = replay time / calls, reported as the median
with p10 / p90 over the replays.  Per step: a graph of the whole sweep is
replayed, K replays bracketed by torch.cuda.synchronize(); `value` = total
algorithmic flops of one step / step wall time.
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
PEAK = {"fp16": 2.5e15, "bf16": 2.5e15, "fp8": 5.0e15, "int8": 5.0e15, "fp4": 10.1e15}
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

    def call(self, M, c, desc=None):
        w, s, z = self.copies[c]
        hq.hq_gemm(desc or self.desc, M, self.A, None, w, s, z, self.D, self.ws if self.ws_bytes else None, self.ws_bytes)

    def cpu_baseline(self, budget_s=16.0):
        import oracle
        d = self.host
        f = lambda rows: oracle.gemm_wna16(d["A"], d["q"], d["s"], d.get("z"), N=self.N, K=self.K, G=self.G,
                                           a_bf16=self.bf16, w_signed=not self.zp, rows=rows)
        n, dt = _timed_oracle(f, lambda n: np.arange(min(n, self.Mmax)), budget_s)
        return dict(value=round(self.flops(n) / dt / 1e12, 6), unit="TFLOP/s", cores=_cores(), kind="oracle",
                    sample=f"{n} output rows x N={self.N} x K={self.K}, fp64 accumulation, {dt:.1f} s")


class DenseWnLow(DenseW4A16):
    """Low-bit WnA16 at the dense W4A16 layer's shape (N=4096, K=7168, group 128):
    UINT1-3 codes with 4-bit zero-points and fp16, or INT1-3 codes and bf16."""

    def __init__(self, bits, signed, N=4096, K=7168, G=128, Mmax=8192, sweep=SWEEP):
        self.N, self.K, self.G, self.Mmax, self.sweep = N, K, G, Mmax, sweep
        self.bits, self.signed, self.bf16, self.zp = bits, signed, signed, not signed
        self.dtype = "bf16" if self.bf16 else "fp16"
        self.name = f"dense_w{bits}a16_{'int' if signed else 'uint'}{bits}_{self.dtype}_N{N}_K{K}"
        t = torch.bfloat16 if self.bf16 else torch.float16
        log(f"[bench] generating {self.name}")
        d = syn.wnlow(0, Mmax, N, K, bits, signed, G=G, dtype=t)
        self.host = d
        self.desc = hq.desc_wnlow(N, K, bits, signed, G, bf16=self.bf16)
        wp, sp, zpk = hq.hq_repack(self.desc, d["codes"], d["s"], d.get("z"))
        self.wbytes = wp.size + sp.size + (zpk.size if zpk is not None else 0)
        self.copies = _copies((dev(wp), dev(sp), dev(zpk) if zpk is not None else None), self.wbytes)
        self.A = dev(d["A"])
        self.D = torch.empty(Mmax * N * 2, dtype=torch.uint8, device="cuda")
        self.ws_bytes = max(hq.hq_workspace_bytes(self.desc, m) for m in sweep)
        self.ws = torch.zeros(max(self.ws_bytes, 16), dtype=torch.uint8, device="cuda")

    def kernel_of(self, M):
        f = f"WNA16_{self.dtype.upper()}"
        if M <= 64:
            return (f"skinny_kernel<{f},w{self.bits}> (M<=64)", "hbm")
        return (f"widen_lowbit_kernel<{self.bits}> + tile_gemm_kernel<{f}> (M>64)", "mfma" if M >= 128 else "hbm")

    def cpu_baseline(self, budget_s=8.0):
        import oracle
        d = self.host
        f = lambda rows: oracle.gemm_wnlow(d["A"], d["codes"], d["s"], d.get("z"), N=self.N, K=self.K, G=self.G,
                                           bits=self.bits, a_bf16=self.bf16, w_signed=self.signed, rows=rows)
        n, dt = _timed_oracle(f, lambda n: np.arange(min(n, self.Mmax)), budget_s)
        return dict(value=round(self.flops(n) / dt / 1e12, 6), unit="TFLOP/s", cores=_cores(), kind="oracle",
                    sample=f"{n} output rows x N={self.N} x K={self.K}, fp64 accumulation, {dt:.1f} s")


class DenseWnWide(DenseWnLow):
    """5-8-bit WnA16 at the dense W4A16 layer's shape (N=4096, K=7168, group 128):
    UINT5-8 codes with 8-bit zero-points and fp16, or INT5-8 codes and bf16."""

    def __init__(self, bits, signed, N=4096, K=7168, G=128, Mmax=8192, sweep=SWEEP):
        self.N, self.K, self.G, self.Mmax, self.sweep = N, K, G, Mmax, sweep
        self.bits, self.signed, self.bf16, self.zp = bits, signed, signed, not signed
        self.dtype = "bf16" if self.bf16 else "fp16"
        self.name = f"dense_w{bits}a16_{'int' if signed else 'uint'}{bits}_{self.dtype}_N{N}_K{K}"
        t = torch.bfloat16 if self.bf16 else torch.float16
        log(f"[bench] generating {self.name}")
        d = syn.wnwide(0, Mmax, N, K, bits, signed, G=G, dtype=t)
        self.host = d
        self.desc = hq.desc_wnwide(N, K, bits, signed, G, bf16=self.bf16)
        wp, sp, zpk = hq.hq_repack(self.desc, d["codes"], d["s"], d.get("z"))
        self.wbytes = wp.size + sp.size + (zpk.size if zpk is not None else 0)
        self.copies = _copies((dev(wp), dev(sp), dev(zpk) if zpk is not None else None), self.wbytes)
        self.A = dev(d["A"])
        self.D = torch.empty(Mmax * N * 2, dtype=torch.uint8, device="cuda")
        self.ws_bytes = max(hq.hq_workspace_bytes(self.desc, m) for m in sweep)
        self.ws = torch.zeros(max(self.ws_bytes, 16), dtype=torch.uint8, device="cuda")

    def kernel_of(self, M):
        f = f"WNA16_{self.dtype.upper()}"
        if M <= 64:
            return (f"skinny_kernel<{f},w{self.bits}> (M<=64)", "hbm")
        return (f"widen_wide_kernel<{self.bits}> + tile_gemm_kernel<W8G_{self.dtype.upper()}> (M>64)",
                "mfma" if M >= 128 else "hbm")

    def cpu_baseline(self, budget_s=8.0):
        import oracle
        d = self.host
        f = lambda rows: oracle.gemm_wnwide(d["A"], d["codes"], d["s"], d.get("z"), N=self.N, K=self.K, G=self.G,
                                            bits=self.bits, a_bf16=self.bf16, w_signed=self.signed, rows=rows)
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

    def call(self, M, c, desc=None):
        w, e = self.copies[c]
        hq.hq_gemm(desc or self.desc, M, self.A, self.s_a, w, e, None, self.D, self.ws if self.ws_bytes else None,
                   self.ws_bytes)

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

    def call(self, M, c, desc=None):
        w, s = self.copies[c]
        hq.hq_gemm(desc or self.desc, M, self.A, self.s_a, w, s, None, self.D, self.ws if self.ws_bytes else None,
                   self.ws_bytes)

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

    def routing_us(self, T):
        """Median time of the routing step alone at T tokens (hq_moe_align: expert
        counts, offsets and the pairs sorted by expert), which an Indexed call runs
        before its expert GEMM -- except at T * top_k <= 64, where the streaming
        kernel routes by itself (reported as 0)."""
        P = T * self.top_k
        if P <= 64:
            return 0.0
        offs = torch.empty(self.E + 4, dtype=torch.int32, device="cuda")
        srt = torch.empty(max(P, 4), dtype=torch.int32, device="cuda")
        nb = hq.hq_workspace_bytes(self.desc, T, self.top_k)
        ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")

        def calls():
            for _ in range(16):
                hq.hq_moe_align(T, self.top_k, self.E, self.ids, offs, srt, ws, nb)
        return round(statistics.median(_graph_times(calls, 16, reps=3)) * 1e6, 2)

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


class DenseMXAct:
    """MX activations (OCP MX: E8M0 per 32 K; E2M1 for W4A4, E4M3 for MXFP8) x MXFP4
    weights, N=7168, K=4096 (the W4A8 layer's shape); activations quantised on the
    GPU once, untimed."""

    def __init__(self, fp4_act: bool, N=7168, K=4096, Mmax=8192, sweep=SWEEP):
        self.N, self.K, self.Mmax, self.sweep, self.fp4 = N, K, Mmax, sweep, fp4_act
        self.dtype = "fp4" if fp4_act else "fp8"
        self.name = f"dense_{'w4a4_mxfp4' if fp4_act else 'w4a8_mxfp8_mxfp4'}_N{N}_K{K}"
        log(f"[bench] generating {self.name}")
        d = syn.w4a8_mxfp4(0, Mmax, N, K)
        self.host = d
        self.desc = hq.desc_mx_act_mxfp4(N, K, fp4_act=fp4_act)
        wp, ep, _ = hq.hq_repack(self.desc, d["q"], d["e"])
        self.wbytes = wp.size + ep.size
        self.copies = _copies((dev(wp), dev(ep)), self.wbytes)
        x = dev(d["A0"])
        self.abytes = K // 2 if fp4_act else K
        self.A = torch.empty(Mmax * self.abytes, dtype=torch.uint8, device="cuda")
        self.e = torch.empty(Mmax * K // 32, dtype=torch.uint8, device="cuda")
        hq.hq_quantize_act_mx(hq.HQ_DT_FP4_E2M1 if fp4_act else hq.HQ_DT_FP8_E4M3, Mmax, K, x, self.A, self.e)
        torch.cuda.synchronize()
        del x
        self.D = torch.empty(Mmax * N * 2, dtype=torch.uint8, device="cuda")
        self.ws_bytes = max(hq.hq_workspace_bytes(self.desc, m) for m in sweep)
        self.ws = torch.empty(max(self.ws_bytes, 16), dtype=torch.uint8, device="cuda")

    def flops(self, M):
        return 2.0 * M * self.N * self.K

    def bytes(self, M):
        return self.wbytes + M * (self.abytes + self.K // 32) + M * self.N * 2

    def kernel_of(self, M):
        f = "W4A4_MX" if self.fp4 else "W4A8_MXA"
        if M <= 64:
            return (f"skinny_kernel<{f}> (M<=64)", "hbm")
        return (f"tile_gemm_kernel<{f}> (M>64)", "mfma" if M >= 256 else "hbm")

    def call(self, M, c, desc=None):
        w, e = self.copies[c]
        hq.hq_gemm(desc or self.desc, M, self.A, self.e, w, e, None, self.D, self.ws if self.ws_bytes else None,
                   self.ws_bytes)

    def cpu_baseline(self, budget_s=8.0):
        import oracle
        elem = "e2m1" if self.fp4 else "e4m3"
        qa, ea = oracle.quant_act_mx(self.host["A0"][:64], elem)
        f = lambda rows: oracle.gemm_mx_mxfp4(qa, ea, self.host["q"], self.host["e"], N=self.N, K=self.K,
                                              a_elem=elem, rows=rows)
        n, dt = _timed_oracle(f, lambda n: np.arange(min(n, 64)), budget_s)
        return dict(value=round(self.flops(n) / dt / 1e12, 6), unit="TFLOP/s", cores=_cores(), kind="oracle",
                    sample=f"{n} output rows x N={self.N} x K={self.K}, fp64 accumulation, {dt:.1f} s")


class DenseFP8Blockwise:
    """FP8 W8A8 with blockwise scales (1x128 activation blocks quantised on the GPU
    once, untimed; 128x128 weight blocks), N=K=7168 (a DeepSeek-class FP8 layer)."""

    def __init__(self, N=7168, K=7168, Mmax=8192, sweep=SWEEP):
        self.N, self.K, self.Mmax, self.sweep = N, K, Mmax, sweep
        self.dtype = "fp8"
        self.name = f"dense_w8a8_fp8_blockwise_N{N}_K{K}"
        log(f"[bench] generating {self.name}")
        d = syn.w8a8_fp8_blockwise(0, Mmax, N, K)
        self.host = d
        self.desc = hq.desc_fp8_blockwise(N, K)
        wp, sp, _ = hq.hq_repack(self.desc, d["w"], d["s_w"])
        self.wbytes = wp.size + sp.size
        self.copies = _copies((dev(wp), dev(sp)), self.wbytes)
        x = dev(d["A0"])
        self.A = torch.empty(Mmax * K, dtype=torch.uint8, device="cuda")
        self.s_a = torch.empty(Mmax * (K // 128), dtype=torch.float32, device="cuda")
        hq.hq_quantize_act_blocks(hq.HQ_DT_FP8_E4M3, Mmax, K, 128, x, self.A, self.s_a)
        torch.cuda.synchronize()
        del x
        self.D = torch.empty(Mmax * N * 2, dtype=torch.uint8, device="cuda")
        self.ws_bytes = max(hq.hq_workspace_bytes(self.desc, m) for m in sweep)
        self.ws = torch.empty(max(self.ws_bytes, 16), dtype=torch.uint8, device="cuda")

    def flops(self, M):
        return 2.0 * M * self.N * self.K

    def bytes(self, M):
        return self.wbytes + M * self.K + M * (self.K // 128) * 4 + M * self.N * 2

    def kernel_of(self, M):
        if M <= 64:
            return ("skinny_kernel<W8A8_F8B> (M<=64)", "hbm")
        return ("tile_gemm_kernel<W8A8_F8B> (M>64)", "mfma" if M >= 512 else "hbm")

    def call(self, M, c, desc=None):
        w, s = self.copies[c]
        hq.hq_gemm(desc or self.desc, M, self.A, self.s_a, w, s, None, self.D, self.ws if self.ws_bytes else None,
                   self.ws_bytes)

    def cpu_baseline(self, budget_s=8.0):
        import oracle
        qa, sa = oracle.quant_act_e4m3_blocks(self.host["A0"][:64], 128)
        f = lambda rows: oracle.gemm_fp8_blockwise(qa, sa, self.host["w"], self.host["s_w"], rows=rows)
        n, dt = _timed_oracle(f, lambda n: np.arange(min(n, 64)), budget_s)
        return dict(value=round(self.flops(n) / dt / 1e12, 6), unit="TFLOP/s", cores=_cores(), kind="oracle",
                    sample=f"{n} output rows x N={self.N} x K={self.K}, fp64 accumulation, {dt:.1f} s")


class DenseFP4A16:
    """bf16 activations x FP4 weights (MXFP4: E8M0 per 32 K; NVFP4: E4M3 per 16 K and a
    per-tensor second-level scale) at the dense W4A16 layer's shape, N=4096, K=7168."""

    def __init__(self, nvfp4: bool, N=4096, K=7168, Mmax=8192, sweep=SWEEP):
        self.N, self.K, self.Mmax, self.sweep, self.nv = N, K, Mmax, sweep, nvfp4
        self.dtype = "bf16"
        self.name = f"dense_w4a16_{'nvfp4' if nvfp4 else 'mxfp4'}_bf16_N{N}_K{K}"
        log(f"[bench] generating {self.name}")
        d = syn.w4a16_fp4(0, Mmax, N, K, nvfp4=nvfp4)
        self.host = d
        self.desc = hq.desc_fp4_a16(N, K, nvfp4)
        if nvfp4:
            wp, sp, _, s2 = hq.hq_repack(self.desc, d["q"], d["s"], None, d["s2"])
        else:
            (wp, sp, _), s2 = hq.hq_repack(self.desc, d["q"], d["s"]), None
        self.wbytes = wp.size + sp.size + (s2.size if s2 is not None else 0)
        self.copies = _copies((dev(wp), dev(sp), dev(s2) if s2 is not None else None), self.wbytes)
        self.A = dev(d["A"])
        self.D = torch.empty(Mmax * N * 2, dtype=torch.uint8, device="cuda")
        self.ws_bytes = max(hq.hq_workspace_bytes(self.desc, m) for m in sweep)
        self.ws = torch.empty(max(self.ws_bytes, 16), dtype=torch.uint8, device="cuda")

    def flops(self, M):
        return 2.0 * M * self.N * self.K

    def bytes(self, M):
        return self.wbytes + M * self.K * 2 + M * self.N * 2

    def kernel_of(self, M):
        f = "NVFP4_BF16" if self.nv else "MXFP4_BF16"
        if M <= 64:
            return (f"skinny_kernel<{f}> (M<=64)", "hbm")
        return (f"tile_gemm_kernel<{f}> (M>64)", "mfma" if M >= 128 else "hbm")

    def call(self, M, c, desc=None):
        w, s, s2 = self.copies[c]
        hq.hq_gemm(desc or self.desc, M, self.A, None, w, s, None, self.D, self.ws if self.ws_bytes else None,
                   self.ws_bytes, s2=s2)

    def cpu_baseline(self, budget_s=8.0):
        import oracle
        d = self.host
        f = lambda rows: oracle.gemm_fp4_a16(d["A"], d["q"], d["s"], N=self.N, K=self.K, a_bf16=True, nvfp4=self.nv,
                                             s2=d.get("s2"), rows=rows)
        n, dt = _timed_oracle(f, lambda n: np.arange(min(n, self.Mmax)), budget_s)
        return dict(value=round(self.flops(n) / dt / 1e12, 6), unit="TFLOP/s", cores=_cores(), kind="oracle",
                    sample=f"{n} output rows x N={self.N} x K={self.K}, fp64 accumulation, {dt:.1f} s")


class DenseMXINT4A16(DenseFP4A16):
    """bf16 activations x MXINT4 weights (two's-complement INT4, E8M0 per 32 K) at the
    dense W4A16 layer's shape, N=4096, K=7168."""

    def __init__(self, N=4096, K=7168, Mmax=8192, sweep=SWEEP):
        self.N, self.K, self.Mmax, self.sweep, self.nv = N, K, Mmax, sweep, False
        self.dtype = "bf16"
        self.name = f"dense_w4a16_mxint4_bf16_N{N}_K{K}"
        log(f"[bench] generating {self.name}")
        d = syn.w4a16_mxint4(0, Mmax, N, K)
        self.host = d
        self.desc = hq.desc_mxint4_a16(N, K)
        wp, sp, _ = hq.hq_repack(self.desc, d["q"], d["e"])
        self.wbytes = wp.size + sp.size
        self.copies = _copies((dev(wp), dev(sp), None), self.wbytes)
        self.A = dev(d["A"])
        self.D = torch.empty(Mmax * N * 2, dtype=torch.uint8, device="cuda")
        self.ws_bytes = max(hq.hq_workspace_bytes(self.desc, m) for m in sweep)
        self.ws = torch.empty(max(self.ws_bytes, 16), dtype=torch.uint8, device="cuda")

    def kernel_of(self, M):
        if M <= 64:
            return ("skinny_kernel<MXINT4_BF16> (M<=64)", "hbm")
        return ("tile_gemm_kernel<MXINT4_BF16> (M>64)", "mfma" if M >= 128 else "hbm")

    def cpu_baseline(self, budget_s=8.0):
        import oracle
        d = self.host
        f = lambda rows: oracle.gemm_mxint4_a16(d["A"], d["q"], d["e"], N=self.N, K=self.K, rows=rows)
        n, dt = _timed_oracle(f, lambda n: np.arange(min(n, self.Mmax)), budget_s)
        return dict(value=round(self.flops(n) / dt / 1e12, 6), unit="TFLOP/s", cores=_cores(), kind="oracle",
                    sample=f"{n} output rows x N={self.N} x K={self.K}, fp64 accumulation, {dt:.1f} s")


class DenseMXF(DenseFP4A16):
    """bf16 activations x MX float weights (MXFP8 E4M3 or MXFP6 E2M3 codes, E8M0 per
    32 K) at the dense W4A16 layer's shape, N=4096, K=7168."""

    def __init__(self, elem, N=4096, K=7168, Mmax=8192, sweep=SWEEP):
        self.N, self.K, self.Mmax, self.sweep, self.nv, self.elem = N, K, Mmax, sweep, False, elem
        self.dtype = "bf16"
        self.name = f"dense_w{'8' if elem == 'e4m3' else '6'}a16_mx{elem}_bf16_N{N}_K{K}"
        log(f"[bench] generating {self.name}")
        d = syn.mxf_a16(0, Mmax, N, K, elem)
        self.host = d
        self.desc = hq.desc_mxf_a16(N, K, elem)
        wp, sp, _ = hq.hq_repack(self.desc, d["codes"], d["e"])
        self.wbytes = wp.size + sp.size
        self.copies = _copies((dev(wp), dev(sp), None), self.wbytes)
        self.A = dev(d["A"])
        self.D = torch.empty(Mmax * N * 2, dtype=torch.uint8, device="cuda")
        self.ws_bytes = max(hq.hq_workspace_bytes(self.desc, m) for m in sweep)
        self.ws = torch.empty(max(self.ws_bytes, 16), dtype=torch.uint8, device="cuda")

    def kernel_of(self, M):
        f = "MXF8_BF16" if self.elem == "e4m3" else "MXF6E2_BF16"
        if M <= 64:
            return (f"skinny_kernel<{f}> (M<=64)", "hbm")
        pre = "" if self.elem == "e4m3" else "widen_fp6_kernel + "
        return (f"{pre}tile_gemm_kernel<MXF8_BF16> (M>64)", "mfma" if M >= 128 else "hbm")

    def cpu_baseline(self, budget_s=8.0):
        import oracle
        d = self.host
        f = lambda rows: oracle.gemm_mxf_a16(d["A"], d["codes"], d["e"], elem=self.elem, rows=rows)
        n, dt = _timed_oracle(f, lambda n: np.arange(min(n, self.Mmax)), budget_s)
        return dict(value=round(self.flops(n) / dt / 1e12, 6), unit="TFLOP/s", cores=_cores(), kind="oracle",
                    sample=f"{n} output rows x N={self.N} x K={self.K}, fp64 accumulation, {dt:.1f} s")


class DenseW8A16:
    """8-bit weight-only: bf16 activations x INT8 (or FP8-E4M3) weights with fp32 per-channel
    scales at the dense W4A16 layer's shape, N=4096, K=7168."""

    def __init__(self, fp8=False, N=4096, K=7168, Mmax=8192, sweep=SWEEP):
        self.N, self.K, self.Mmax, self.sweep, self.fp8 = N, K, Mmax, sweep, fp8
        self.dtype = "bf16"
        self.name = f"dense_w8a16_{'fp8' if fp8 else 'int8'}_bf16_N{N}_K{K}"
        log(f"[bench] generating {self.name}")
        d = (syn.w8a16_fp8 if fp8 else syn.w8a16_int8)(0, Mmax, N, K)
        self.host = d
        self.desc = (hq.desc_fp8w_a16 if fp8 else hq.desc_w8a16)(N, K, bf16=True)
        wp, sp, _ = hq.hq_repack(self.desc, d["w"], d["s_w"])
        self.wbytes = wp.size + sp.size
        self.copies = _copies((dev(wp), dev(sp)), self.wbytes)
        self.A = dev(d["A"])
        self.D = torch.empty(Mmax * N * 2, dtype=torch.uint8, device="cuda")
        self.ws_bytes = max(hq.hq_workspace_bytes(self.desc, m) for m in sweep)
        self.ws = torch.empty(max(self.ws_bytes, 16), dtype=torch.uint8, device="cuda")

    def flops(self, M):
        return 2.0 * M * self.N * self.K

    def bytes(self, M):
        return self.wbytes + M * self.K * 2 + M * self.N * 2

    def kernel_of(self, M):
        f = "F8W_BF16" if self.fp8 else "W8A16_BF16"
        if M <= 64:
            return (f"skinny_kernel<{f}> (M<=64)", "hbm")
        return (f"tile_gemm_kernel<{f}> (M>64)", "mfma" if M >= 256 else "hbm")

    def call(self, M, c, desc=None):
        w, s = self.copies[c]
        hq.hq_gemm(desc or self.desc, M, self.A, None, w, s, None, self.D, self.ws if self.ws_bytes else None,
                   self.ws_bytes)

    def cpu_baseline(self, budget_s=8.0):
        import oracle
        d = self.host
        ref = oracle.gemm_fp8w_a16 if self.fp8 else oracle.gemm_w8a16
        f = lambda rows: ref(d["A"], d["w"], d["s_w"], a_bf16=True, rows=rows)
        n, dt = _timed_oracle(f, lambda n: np.arange(min(n, self.Mmax)), budget_s)
        return dict(value=round(self.flops(n) / dt / 1e12, 6), unit="TFLOP/s", cores=_cores(), kind="oracle",
                    sample=f"{n} output rows x N={self.N} x K={self.K}, fp64 accumulation, {dt:.1f} s")


WORKLOADS = {
    "c1": lambda: DenseW4A16(N=1024, K=1024, Mmax=16, bf16=True, zp=False, sweep=[16],
                             name="dense_w4a16_sym_bf16_M16_N1024_K1024"),
    "c2": lambda: DenseW4A16(),
    "c3": lambda: DenseW4A8(),
    "c4": lambda: DenseW8A8(),
    "c5": lambda: MoEMXFP4(),
    "c5g": lambda: MoEGroupedMXFP4(),
    "c5l": lambda: MoELayerMXFP4(),
    "w4a4": lambda: DenseMXAct(fp4_act=True),
    "w4a8mx": lambda: DenseMXAct(fp4_act=False),
    "fp8b": lambda: DenseFP8Blockwise(),
    "mxfp4a16": lambda: DenseFP4A16(nvfp4=False),
    "nvfp4a16": lambda: DenseFP4A16(nvfp4=True),
    "mxint4a16": lambda: DenseMXINT4A16(),
    "w8a16": lambda: DenseW8A16(),
    "fp8w": lambda: DenseW8A16(fp8=True),
    "w3a16": lambda: DenseWnLow(3, False),
    "w2a16": lambda: DenseWnLow(2, True),
    "w8a16g": lambda: DenseWnWide(8, False),
    "w5a16": lambda: DenseWnWide(5, True),
    "mxfp8a16": lambda: DenseMXF("e4m3"),
    "mxfp6a16": lambda: DenseMXF("e2m3"),
}
# the workloads the default run measures besides the headline one (c2)
DEFAULT_EXTRA = ["c3", "c4", "c5", "w4a4", "w4a8mx", "fp8b", "mxfp4a16", "nvfp4a16", "mxint4a16", "w8a16", "fp8w",
                 "w3a16", "w2a16", "w8a16g", "w5a16", "mxfp8a16", "mxfp6a16"]


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


REPS = 7        # timed replays per M (median, p10, p90 over them)


def _pct(xs, q):
    return float(np.percentile(np.asarray(xs), q))


def _graph_times(fn, ncalls, eager=False, reps=REPS):
    """Per-call seconds of each of `reps` replays of a graph of fn() (ncalls calls);
    HIP events on the replaying stream."""
    g = (_Eager if eager else _capture)(fn)
    g.replay()
    torch.cuda.synchronize()
    out = []
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    for _ in range(reps):
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) * 1e-3 / ncalls)
    del g
    return out


def time_calls(work, M, desc=None, eager=False, reps=REPS):
    """Per-call seconds over `reps` replays of back-to-back calls at M, one call
    per cold weight copy."""
    ncopy = len(work.copies)

    def calls():
        for r in range(ncopy):
            if desc is None:
                work.call(M, r)
            else:
                work.call(M, r, desc)
    return _graph_times(calls, ncopy, eager, reps)


def run(work, steps, warmup, eager=False):
    """Per-M timings (list of per-call seconds over the replays) and the wall time
    of `steps` replays of the whole sweep (graphs of sweeps over rotating copies)."""
    sweep = work.sweep
    ncopy = len(work.copies)
    per = {M: time_calls(work, M, eager=eager) for M in sweep}
    nsw = max(1, ncopy // len(sweep))
    graphs = []
    capture = _Eager if eager else _capture
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


def tune_table(work, log_fn=log):
    """Autotune the workload's dense layer over its sweep: per M the fastest
    tuning override (HQ_TUNE(path, splits)) and the library's own choice."""
    from bit_quantized_gemm_w4a16_amd import autotune as at

    def time_us(desc, M):
        need = hq.hq_workspace_bytes(desc, M)
        if need > work.ws.numel():
            work.ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        if need > work.ws_bytes:
            work.ws_bytes = need
        # the fastest of 5 replays: the candidates are compared on what they can do,
        # not on the clock and queue noise of one replay
        return min(time_calls(work, M, desc=desc, reps=5)) * 1e6

    table = at.autotune(work.desc, work.sweep, time_us, verbose=log_fn)
    return [dict(M=M, best_tune=t, best_plan=at.plan_name(work.desc, t, M), best_us=round(b, 2),
                 library_plan=at.plan_name(work.desc, 0, M), library_us=round(base, 2),
                 gain=round(base / b, 3)) for M, (t, b, base) in table.items()]


# The library's sources: counter figures taken on other versions of them are stale.
KERNEL_SOURCES = sorted("bit_quantized_gemm_w4a16_amd/csrc/" + f
                        for f in os.listdir(os.path.join(ROOT, "bit_quantized_gemm_w4a16_amd", "csrc"))
                        if f.endswith((".hip", ".hpp", ".h", ".cpp")))
KERNEL_SOURCES += ["include/hq.h", "bit_quantized_gemm_w4a16_amd/build.py"]   # (the build flags shape the code too)


def kernel_source_hash():
    """Hash of the library's sources; counter figures taken on other sources are stale."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _traffic(workload, M):
    """HBM bytes at M from the committed counter runs (profiles/traffic.json):
    FETCH_SIZE + WRITE_SIZE per dispatch, each scaled by the factor the same counter
    gives on a plain device copy of known size; `kernel_bytes` for one launch of the
    call's main kernel, `call_bytes` for all of the call's launches.  None when
    absent or taken on other sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh).get(workload)
    if not rec or rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("per_M", {}).get(str(M))


MEASURED = {}   # on-device peaks from the library's probes (filled by measure_peaks)


def measure_peaks():
    """The device's attainable HBM read rate and dense MFMA rate per type, from
    the library's probes (hq_probe_stream, hq_probe_mfma), timed with HIP events:
    what the kernels' rooflines are also set against, next to the published peaks."""
    nbytes = 2 << 30
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(16, dtype=torch.uint8, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    hq.hq_probe_stream(src, nbytes, sink, 1)
    reps = 8
    e0.record()
    hq.hq_probe_stream(src, nbytes, sink, reps)
    e1.record()
    torch.cuda.synchronize()
    hbm = reps * nbytes / (e0.elapsed_time(e1) * 1e-3)
    del src
    out = {"hbm": hbm}
    wgs, iters = 1024, 4000
    fsink = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
    for name, dt in (("fp16", hq.HQ_DT_FP16), ("bf16", hq.HQ_DT_BF16), ("fp8", hq.HQ_DT_FP8_E4M3),
                     ("fp4", hq.HQ_DT_FP4_E2M1), ("int8", hq.HQ_DT_INT8)):
        hq.hq_probe_mfma(dt, wgs, 100, fsink)
        e0.record()
        flops = hq.hq_probe_mfma(dt, wgs, iters, fsink)
        e1.record()
        torch.cuda.synchronize()
        out[name] = flops / (e0.elapsed_time(e1) * 1e-3)
    MEASURED.update(out)
    spec = {"hbm": PEAK_HBM, **PEAK}
    return {k: {"measured": round(v / (1e9 if k == "hbm" else 1e12), 1),
                "unit": "GB/s" if k == "hbm" else ("TOP/s" if k == "int8" else "TFLOP/s"),
                "spec": round(spec[k] / (1e9 if k == "hbm" else 1e12), 1), "frac_of_spec": round(v / spec[k], 3)}
            for k, v in out.items()}


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


def report(work, args, wall, per, cpu_budget=16.0):
    ms_per_step = wall / args.steps * 1e3 if args.steps else None
    flops_step = sum(work.flops(M) for M in work.sweep)
    peak = PEAK[work.dtype]
    table, kern = [], {}
    for M in work.sweep:
        t = statistics.median(per[M])
        F, B = work.flops(M), work.bytes(M)
        row = dict(M=M, flops=F, bytes=B, us=round(t * 1e6, 2), us_p10=round(_pct(per[M], 10) * 1e6, 2),
                   us_p90=round(_pct(per[M], 90) * 1e6, 2), tflops=round(F / t / 1e12, 2),
                   gbps=round(B / t / 1e9, 1), hbm_frac=round(B / t / PEAK_HBM, 3),
                   mfma_frac=round(F / t / peak, 3), roofline_frac=round(max(B / PEAK_HBM, F / peak) / t, 3))
        if hasattr(work, "routing_us") and not args.eager:   # (eager: counter runs, no extra launches)
            row["routing_us"] = work.routing_us(M)
        tr = _traffic(work.name, M)
        if tr:   # HBM bytes of the whole call from the counter runs, against the algorithmic bytes
            row["traffic_bytes"] = tr["call_bytes"]
            row["traffic_ratio"] = round(tr["call_bytes"] / B, 3)
        table.append(row)
        name, bound = work.kernel_of(M)
        k = kern.setdefault(name, dict(t=0.0))
        k["t"] += t
    # Roofline of the dominant kernel, taken at the sweep's largest M, where one
    # call is one launch of it: achieved = algorithmic flops (or bytes) of that
    # launch / its median duration over back-to-back launches (HIP events on
    # the launching stream).
    dom = max(kern, key=lambda n: kern[n]["t"])
    Mr = max(M for M in work.sweep if work.kernel_of(M)[0] == dom)
    name, bound = work.kernel_of(Mr)
    t, F, B = statistics.median(per[Mr]), work.flops(Mr), work.bytes(Mr)
    unit = "TFLOP/s" if work.dtype != "int8" else "TOP/s"
    if bound == "mfma":
        roof = dict(bound="mfma", achieved=round(F / t / 1e12, 1), peak=peak / 1e12, unit=unit,
                    frac=round(F / t / peak, 4))
    else:
        roof = dict(bound="hbm", achieved=round(B / t / 1e9, 1), peak=PEAK_HBM / 1e9, unit="GB/s",
                    frac=round(B / t / PEAK_HBM, 4))
    key = "hbm" if bound == "hbm" else work.dtype
    if key in MEASURED:   # the same achieved rate against the probe-measured peak
        roof.update(measured_peak=round(MEASURED[key] / (1e9 if key == "hbm" else 1e12), 1),
                    frac_of_measured=round((B if key == "hbm" else F) / t / MEASURED[key], 4))
    tr = _traffic(work.name, Mr)
    roof.update(traffic=tr["kernel_bytes"] if tr else None, kernel=dom, M=Mr, avg_us=round(t * 1e6, 2),
                algorithmic_flops=F, algorithmic_bytes=B,
                per_unit="2*M*N*K flops per launch" if bound == "mfma" else "algorithmic bytes per launch")
    cpu = None if args.no_cpu_baseline else work.cpu_baseline(cpu_budget)
    cfg = {"workload": work.name, "M_sweep": work.sweep, "N": work.N, "K": work.K,
           "cold_weight_copies": len(work.copies)}
    if hasattr(work, "E"):
        cfg.update(E=work.E, top_k=work.top_k)
    out = {
        "metric": METRIC,
        "value": round(flops_step / (ms_per_step * 1e-3) / 1e12, 2) if ms_per_step else None,
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4) if ms_per_step else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": work.dtype,
        "data": "synthetic",
        "config": cfg,
        "roofline": roof,
        "cpu_baseline": cpu,
        "per_M": table,
    }
    if hasattr(work, "aux"):
        out["aux"] = work.aux()
    return out


def _dispatches(csv_path):
    """The dispatches of a rocprofv3 kernel trace or counter collection (CSV), in
    dispatch order: (kernel name, duration in us, {counter: value})."""
    import csv
    by = {}
    with open(csv_path) as fh:
        for r in csv.DictReader(fh):
            d = by.setdefault(int(r["Dispatch_Id"]), [r["Kernel_Name"],
                              (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3, {}])
            if r.get("Counter_Name"):
                d[2][r["Counter_Name"]] = float(r["Counter_Value"])
    return [tuple(by[k]) for k in sorted(by)]


def _base(name):
    return name.split("<")[0].split("(")[0].replace("void ", "").strip().split("::")[-1]


def _median_counters(ds):
    keys = sorted({k for d in ds for k in d})
    return {k: _pct([d.get(k, 0.0) for d in ds], 50) for k in keys}


def kernel_stats(csv_path, config, sweep=None, reps=REPS, eager=False):
    """Kernel-only time (and counters) per M from a rocprofv3 kernel trace or
    counter collection of `bench.py --config <workload> --steps 0 --warmup 0
    --no-cpu-baseline [--eager]`.

    Dense workloads: the CSV lists the dispatches in order; per M the run makes
    (2 + reps) x copies calls (graph capture's eager pass, the warm-up replay, the
    timed replays; with --eager there is no capture pass), each launching the
    kernels hq_gemm_plan names.  Those are matched in order against the CSV (other
    kernels -- torch's, the setup's -- are skipped; a name that does not match the
    plan aborts).  Per M: the summed kernel time of a call (median / p10 / p90 over
    the timed calls), and per planned kernel its median duration and the median of
    each collected counter.  MoE workloads (no plan): per kernel name over every
    dispatch of the library's kernels.  Prints one JSON object."""
    ds = _dispatches(csv_path)
    if config not in _DRY:
        groups = {}
        for name, t, c in ds:
            if not _is_torch_kernel(name):
                groups.setdefault(_base(name), []).append((t, c))
        out = {k: dict(dispatches=len(v), median_us=round(_pct([t for t, _ in v], 50), 2),
                       p10_us=round(_pct([t for t, _ in v], 10), 2), p90_us=round(_pct([t for t, _ in v], 90), 2),
                       counters=_median_counters([c for _, c in v])) for k, v in groups.items()}
        print(json.dumps({"workload": config, "by_kernel": out}))
        return
    desc = _DRY[config]()
    sweep = sweep or SWEEP
    ncopy = _ncopies(desc)
    untimed = (1 if eager else 2) * ncopy
    i, out = 0, []
    # the library's setup launches (activation quantisers) come before the sweep
    first = _base(hq.hq_gemm_plan(desc, sweep[0])[0])
    while i < len(ds) and _base(ds[i][0]) != first:
        i += 1
    if i == len(ds):
        raise SystemExit(f"M={sweep[0]}: expected {first}, the trace has no such dispatch")
    for M in sweep:
        plan = hq.hq_gemm_plan(desc, M)
        calls = []
        for _ in range(untimed + reps * ncopy):
            call = []
            for item in plan:
                k = _base(item)
                while i < len(ds) and _is_torch_kernel(ds[i][0]):
                    i += 1
                if i >= len(ds):
                    raise SystemExit(f"trace ended before M={M}")
                if _base(ds[i][0]) != k:
                    raise SystemExit(f"M={M}: expected {k}, trace has {ds[i][0]}")
                call.append(ds[i])
                i += 1
            calls.append(call)
        timed = calls[untimed:]
        tot = [sum(d[1] for d in c) for c in timed]
        kern = []
        for j, item in enumerate(plan):
            ts = [c[j][1] for c in timed]
            kern.append(dict(kernel=item, median_us=round(_pct(ts, 50), 2),
                             counters=_median_counters([c[j][2] for c in timed])))
        out.append(dict(M=M, calls=len(timed), median_us=round(_pct(tot, 50), 2), p10_us=round(_pct(tot, 10), 2),
                        p90_us=round(_pct(tot, 90), 2), kernels=kern))
    print(json.dumps({"workload": config, "copies": ncopy, "kernel_only_us": out}))


def _is_torch_kernel(name):
    return "at::native" in name or name.startswith("__amd_rocclr") or "at::" in name.split("(")[0]


# descriptors of the dense workloads, for kernel_stats (no device memory needed)
_DRY = {
    "c2": lambda: hq.desc_w4a16(4096, 7168, 128, bf16=False, zp=True),
    "c3": lambda: hq.desc_w4a8_mxfp4(7168, 4096),
    "c4": lambda: hq.desc_w8a8(18432, 7168),
    "w4a4": lambda: hq.desc_mx_act_mxfp4(7168, 4096, fp4_act=True),
    "w4a8mx": lambda: hq.desc_mx_act_mxfp4(7168, 4096, fp4_act=False),
    "fp8b": lambda: hq.desc_fp8_blockwise(7168, 7168),
    "mxfp4a16": lambda: hq.desc_fp4_a16(4096, 7168, False),
    "nvfp4a16": lambda: hq.desc_fp4_a16(4096, 7168, True),
    "mxint4a16": lambda: hq.desc_mxint4_a16(4096, 7168),
    "w8a16": lambda: hq.desc_w8a16(4096, 7168, bf16=True),
    "fp8w": lambda: hq.desc_fp8w_a16(4096, 7168, bf16=True),
    "w3a16": lambda: hq.desc_wnlow(4096, 7168, 3, False, 128, bf16=False),
    "w2a16": lambda: hq.desc_wnlow(4096, 7168, 2, True, 128, bf16=True),
    "w8a16g": lambda: hq.desc_wnwide(4096, 7168, 8, False, 128, bf16=False),
    "w5a16": lambda: hq.desc_wnwide(4096, 7168, 5, True, 128, bf16=True),
    "mxfp8a16": lambda: hq.desc_mxf_a16(4096, 7168, "e4m3"),
    "mxfp6a16": lambda: hq.desc_mxf_a16(4096, 7168, "e2m3"),
}


def _ncopies(desc):
    """The number of cold weight copies a workload makes (as _copies does)."""
    return max(2, -(-COLD_BYTES // sum(hq.hq_repacked_bytes(desc))))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default=None,
                    help=f"one of {', '.join(WORKLOADS)} or all (default: c2 as the headline line, "
                         f"with {', '.join(DEFAULT_EXTRA)} under its 'configs'; c5g = MoE on the Grouped path, "
                         "c5l = MoE gate-up + SwiGLU + down)")
    ap.add_argument("--sweep", default=None, help="comma-separated M values (default 1..8192 powers of 2)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true", help="issue calls directly instead of replaying HIP graphs "
                    "(for counter-collection runs)")
    ap.add_argument("--autotune", action="store_true",
                    help="also time every tuning override per M (dense workloads) and report the fastest")
    ap.add_argument("--no-peaks", action="store_true", help="skip the on-device peak probes")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (counter calibration) and exit")
    ap.add_argument("--kernel-stats", default=None, metavar="CSV",
                    help="no GPU: per-M kernel-only times from a rocprofv3 kernel trace of this script "
                         "(--config <dense workload> --steps 0 --warmup 0)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(the sharding design is described in DESIGN.md); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    sweep = [int(x) for x in args.sweep.split(",")] if args.sweep else None
    if args.kernel_stats:
        kernel_stats(args.kernel_stats, args.config or "c2", sweep, eager=args.eager)
        return
    torch.cuda.set_device(0)
    if args.copy_probe:
        copy_probe(args.copy_probe, args.steps)
        return

    def measure(nm, cpu_budget):
        if nm not in WORKLOADS:
            raise SystemExit(f"unknown --config {nm}")
        work = WORKLOADS[nm]()
        if sweep and nm != "c1":
            work.sweep = sweep
            if hasattr(work, "active"):
                flat = work.host["ids"]
                work.active = {T: len(np.unique(flat[:T])) for T in work.sweep}
        t0 = time.perf_counter()
        wall, per = run(work, args.steps, args.warmup, eager=args.eager)
        rec = report(work, args, wall, per, cpu_budget)
        if args.autotune and hasattr(work, "desc") and not hasattr(work, "E"):
            rec["autotune"] = tune_table(work)
        log(f"[bench] {nm}: {time.perf_counter() - t0:.1f} s")
        del work
        torch.cuda.empty_cache()
        return rec

    peaks = None if args.no_peaks or args.eager else measure_peaks()
    if peaks:
        log("[bench] measured peaks " + json.dumps(peaks))

    if args.config is None:
        head = measure("c2", 16.0)
        head["peaks"] = peaks
        head["configs"] = {}
        for nm in DEFAULT_EXTRA:
            rec = measure(nm, 3.0)
            head["configs"][nm] = {k: rec[k] for k in ("value", "unit", "ms_per_step", "dtype", "config", "roofline",
                                                       "cpu_baseline", "per_M") + (("aux",) if "aux" in rec else ())}
        print(json.dumps(head), flush=True)
        return
    names = list(WORKLOADS) if args.config == "all" else [args.config]
    for nm in names:
        rec = measure(nm, 16.0)
        rec["peaks"] = peaks
        print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
