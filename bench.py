#!/usr/bin/env python3
"""Benchmark of the hq quantized GEMM on one MI355X.

A step is one pass of the hot path over the workload's M sweep: for every
M in {1, 2, 4, ..., 8192} one hq_gemm call (host dispatch -> HIP kernels ->
output) on inputs already resident in HBM.  The default workload is the
dense W4A16 asymmetric layer (fp16 activations, UINT4 weights with UINT4
zero-points and fp16 scales per 128 K, N=4096, K=7168).  Other workloads
(--config c1|c3|c4|c5) print their own line.

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


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.uint8).reshape(-1).copy()).to("cuda")


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------

class DenseW4A16:
    """Dense W4A16 asymmetric: fp16 A, UINT4 codes + UINT4 zero-points, fp16 scales, G=128."""
    name = "dense_w4a16_zp_fp16_N4096_K7168"
    dtype = "fp16"

    def __init__(self, N=4096, K=7168, G=128, Mmax=8192, bf16=False, zp=True, sym_cfg=False):
        self.N, self.K, self.G, self.Mmax = N, K, G, Mmax
        self.bf16, self.zp = bf16, zp
        t = torch.bfloat16 if bf16 else torch.float16
        log(f"[bench] generating {self.name}")
        if zp:
            d = syn.w4a16_zp(0, Mmax, N, K, G, t)
        else:
            d = syn.w4a16_sym(0, Mmax, N, K, G, t)
        self.host = d
        self.desc = hq.desc_w4a16(N, K, G, bf16=bf16, zp=zp)
        wp, sp, zpk = hq.hq_repack(self.desc, d["q"], d["s"], d.get("z") if zp else None)
        self.wbytes = wp.size + sp.size + (zpk.size if zpk is not None else 0)
        ncopy = max(2, -(-COLD_BYTES // self.wbytes))
        w0, s0 = dev(wp), dev(sp)
        z0 = dev(zpk) if zp else None
        self.copies = [(w0.clone(), s0.clone(), None if z0 is None else z0.clone()) for _ in range(ncopy)]
        self.A = dev(d["A"])
        self.D = torch.empty(Mmax * N * 2, dtype=torch.uint8, device="cuda")
        self.ws_bytes = max(hq.hq_workspace_bytes(self.desc, m) for m in SWEEP if m <= Mmax)
        self.ws = torch.zeros(max(self.ws_bytes, 16), dtype=torch.uint8, device="cuda")
        self.i = 0

    def flops(self, M):
        return 2.0 * M * self.N * self.K

    def bytes(self, M):
        # packed weights + scales + zeros (static) + A + D
        return self.wbytes + M * self.K * 2 + M * self.N * 2

    def kernel_of(self, M):
        return "gemv" if M <= 64 else "tile"

    def call(self, M, copy):
        w, s, z = self.copies[copy]
        hq.hq_gemm(self.desc, M, self.A, None, w, s, z, self.D, self.ws if self.ws_bytes else None, self.ws_bytes)

    def cpu_baseline(self, budget_s=15.0):
        import oracle
        d = self.host
        rows = np.arange(2)
        t0 = time.perf_counter()
        oracle.gemm_wna16(d["A"], d["q"], d["s"], d.get("z"), N=self.N, K=self.K, G=self.G,
                          a_bf16=self.bf16, w_signed=not self.zp, rows=rows)
        t1 = time.perf_counter() - t0
        nrows = int(max(2, min(self.Mmax, budget_s / max(t1, 1e-3) * 2)))
        rows = np.arange(nrows)
        t0 = time.perf_counter()
        oracle.gemm_wna16(d["A"], d["q"], d["s"], d.get("z"), N=self.N, K=self.K, G=self.G,
                          a_bf16=self.bf16, w_signed=not self.zp, rows=rows)
        dt = time.perf_counter() - t0
        return dict(value=self.flops(nrows) / dt / 1e12, unit="TFLOP/s", cores=_cores(), kind="oracle",
                    sample=f"{nrows} output rows x N={self.N} x K={self.K} (fp64 accumulation), {dt:.1f} s")


def _cores():
    omp = os.environ.get("OMP_NUM_THREADS")
    n = len(os.sched_getaffinity(0))
    return min(n, int(omp)) if omp and omp.isdigit() else n


# ---------------------------------------------------------------------------

def _capture(fn):
    """Capture fn() (a sequence of hq calls on the current stream) into a HIP graph."""
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                      # eager run on the capture stream (allocator warm-up)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=side):
        fn()
    torch.cuda.synchronize()
    return g


def run(work, sweep, steps, warmup):
    """Per-M timing from graphs of R back-to-back calls (each on its own cold weight copy),
    and the step timing from graphs of whole sweeps (one weight copy per call)."""
    ncopy = len(work.copies)
    per = {}
    for M in sweep:
        def calls(M=M):
            for r in range(ncopy):
                work.call(M, r)
        g = _capture(calls)
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
        per[M] = [e0.elapsed_time(e1) * 1e-3 / (reps * ncopy)]
        del g
    # sweep graphs: graph j uses copies j*len(sweep) + i (mod ncopy), so no copy repeats within ncopy calls
    nsw = max(1, ncopy // len(sweep))
    graphs = []
    for j in range(nsw):
        def sweep_calls(j=j):
            for i, M in enumerate(sweep):
                work.call(M, (j * len(sweep) + i) % ncopy)
        graphs.append(_capture(sweep_calls))
    for w in range(warmup):
        graphs[w % nsw].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        graphs[k % nsw].replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, per


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="c2")
    ap.add_argument("--sweep", default=None, help="comma-separated M values (default 1..8192 powers of 2)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(the sharding design is described in DESIGN.md); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    sweep = [int(x) for x in args.sweep.split(",")] if args.sweep else SWEEP
    if args.config != "c2":
        raise SystemExit(f"unknown --config {args.config}")
    work = DenseW4A16()
    wall, per = run(work, sweep, args.steps, args.warmup)
    ms_per_step = wall / args.steps * 1e3
    flops_step = sum(work.flops(M) for M in sweep)
    table = []
    kern = {}
    for M in sweep:
        t = statistics.median(per[M])
        F, B = work.flops(M), work.bytes(M)
        peak = PEAK[work.dtype]
        table.append(dict(M=M, us=round(t * 1e6, 2), tflops=round(F / t / 1e12, 2), gbps=round(B / t / 1e9, 1),
                          hbm_frac=round(B / t / PEAK_HBM, 3), mfma_frac=round(F / t / peak, 3),
                          roofline_frac=round(max(B / PEAK_HBM, F / peak) / t, 3)))
        k = work.kernel_of(M)
        kern.setdefault(k, [0.0, 0.0, 0.0, 0])
        kern[k][0] += F * len(per[M])
        kern[k][1] += B * len(per[M])
        kern[k][2] += sum(per[M])
        kern[k][3] += len(per[M])
    dom = max(kern, key=lambda k: kern[k][2])
    F_tot, B_tot, t_tot, n = kern[dom]
    if dom == "tile":
        roof = dict(bound="mfma", achieved=round(F_tot / t_tot / 1e12, 1), peak=PEAK[work.dtype] / 1e12,
                    unit="TFLOP/s", frac=round(F_tot / t_tot / PEAK[work.dtype], 4), traffic=None,
                    kernel="tile_gemm_kernel (W4A16 fp16, M>=128)", launches=n, avg_us=round(t_tot / n * 1e6, 2))
    else:
        roof = dict(bound="hbm", achieved=round(B_tot / t_tot / 1e9, 1), peak=PEAK_HBM / 1e9, unit="GB/s",
                    frac=round(B_tot / t_tot / PEAK_HBM, 4), traffic=None,
                    kernel="wna16_gemv_kernel (M<=64)", launches=n, avg_us=round(t_tot / n * 1e6, 2))
    cpu = None if args.no_cpu_baseline else work.cpu_baseline()
    line = {
        "metric": "quant GEMM TFLOP/s + HBM GB/s vs roofline, M=1..8192, W4A16/W4A8/MoE",
        "value": round(flops_step / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": work.dtype,
        "data": "synthetic",
        "config": {"workload": work.name, "M_sweep": sweep, "N": work.N, "K": work.K, "group_size": work.G,
                   "cold_weight_copies": len(work.copies)},
        "roofline": roof,
        "cpu_baseline": cpu,
        "per_M": table,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
