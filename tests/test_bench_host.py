"""Host-only checks of the benchmark's bookkeeping and of the autotuner's
candidate list (no GPU): the kernel-trace attribution, the one-GPU exit, and
that every tuning candidate names a distinct, valid plan."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from bit_quantized_gemm_w4a16_amd import autotune, hq  # noqa: E402


def _write_trace(path, config, sweep, dur_of):
    """A kernel trace as rocprofv3 writes it, for the dispatch sequence a
    `--steps 0 --warmup 0` run of `config` makes, with foreign kernels between."""
    desc = bench._DRY[config]()
    ncopy = bench._ncopies(desc)
    rows, t, did = [], 1000, 1
    rows.append(("void at::native::fill_kernel<float>(int)", 5000))
    rows.append(("void quant_mx_kernel<true>(QuantArgs)", 5000))
    for M in sweep:
        plan = hq.hq_gemm_plan(desc, M)
        for c in range((2 + bench.REPS) * ncopy):
            for k, item in enumerate(plan):
                name = "void " + item.split(" ")[0].replace("WNA16_F16", "(Fmt)0") + "(Args)"
                rows.append((name, dur_of(M, c, k)))
            if c == 3:
                rows.append(("void at::native::copy_kernel(int)", 777000))
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        for name, d in rows:
            w.writerow([did, name, t, t + d])
            did += 1
            t += d + 100
    return ncopy


def test_kernel_stats_attributes_dispatches_per_M(tmp_path):
    sweep = [1, 32, 8192]

    def dur(M, c, k):       # ns; the first two calls per M are untimed warm-ups
        if c < 2 * ncopy_ref[0]:
            return 1_000_000
        return (10_000 if k == 0 else 3_000) + M + (c % 3) * 10

    ncopy_ref = [bench._ncopies(bench._DRY["c2"]())]
    p = tmp_path / "trace.csv"
    _write_trace(p, "c2", sweep, dur)
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--kernel-stats", str(p), "--config", "c2",
                          "--sweep", "1,32,8192"], capture_output=True, text=True, check=True)
    rec = json.loads(out.stdout.strip().splitlines()[-1])
    by = {r["M"]: r for r in rec["kernel_only_us"]}
    assert [k["kernel"].split("<")[0] for k in by[1]["kernels"]] == ["skinny_kernel"]
    assert by[1]["calls"] == bench.REPS * ncopy_ref[0]
    # M=1: one kernel of 10 us + 1 ns + {0,10,20} ns; M=32 (K split): 10 + 3 us + 2*32 ns + 2*{0,10,20} ns
    assert 10.0 <= by[1]["p10_us"] <= by[1]["median_us"] <= by[1]["p90_us"] <= 10.03
    assert 13.06 <= by[32]["median_us"] <= 13.11
    assert [k["kernel"].split("<")[0] for k in by[32]["kernels"]] == ["skinny_kernel", "splitk_finalize_kernel"]
    assert 3.03 <= by[32]["kernels"][1]["median_us"] <= 3.06


def test_kernel_stats_reads_counter_collections(tmp_path):
    """A counter collection has one row per (dispatch, counter); --eager runs
    have no capture pass."""
    desc = bench._DRY["c3"]()
    ncopy = bench._ncopies(desc)
    p = tmp_path / "pmc.csv"
    did, t = 1, 0
    with open(p, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
                    "End_Timestamp"])
        for M in (1, 8192):
            for c in range((1 + bench.REPS) * ncopy):
                for item in hq.hq_gemm_plan(desc, M):
                    for cn, cv in (("FETCH_SIZE", 100.0 * M), ("WRITE_SIZE", 7.0 + (c >= ncopy))):
                        w.writerow([did, "void " + item.split(" ")[0] + "(TileArgs)", cn, cv, t, t + 2000])
                    did += 1
                    t += 3000
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--kernel-stats", str(p), "--config", "c3",
                          "--sweep", "1,8192", "--eager"], capture_output=True, text=True, check=True)
    rec = json.loads(out.stdout.strip().splitlines()[-1])
    big = rec["kernel_only_us"][1]
    assert big["M"] == 8192 and big["kernels"][0]["counters"] == {"FETCH_SIZE": 819200.0, "WRITE_SIZE": 8.0}


def test_kernel_stats_rejects_a_trace_of_another_plan(tmp_path):
    p = tmp_path / "trace.csv"
    _write_trace(p, "c2", [8192], lambda M, c, k: 1000)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--kernel-stats", str(p), "--config", "c2",
                        "--sweep", "1"], capture_output=True, text=True)
    assert r.returncode != 0 and "expected skinny_kernel" in (r.stderr + r.stdout)


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr


@pytest.mark.parametrize("name", sorted(bench._DRY))
def test_autotune_candidates_are_distinct_valid_plans(name):
    desc = bench._DRY[name]()
    for M in (1, 16, 64, 128, 512, 8192):
        cands = autotune.candidates(desc, M)
        assert cands[0] == 0
        plans = [tuple(hq.hq_gemm_plan(autotune.with_tune(desc, t), M)) for t in cands]
        assert len(set(plans)) == len(plans)
        assert all(plans)
        for t in cands:
            assert hq.hq_workspace_bytes(autotune.with_tune(desc, t), M) >= 0
    # small M offers the weight-streaming path with several splits, large M several tiles
    assert len(autotune.candidates(desc, 16)) > 3
    assert len(autotune.candidates(desc, 8192)) > 1


def test_tuning_override_out_of_range_is_rejected():
    desc = hq.desc_w4a16(1000, 1024, 128, bf16=True, zp=False)
    # a weight-streaming override above the streaming path's largest M
    with pytest.raises(hq.HQError):
        hq.hq_gemm_plan(autotune.with_tune(desc, hq.HQ_TUNE(hq.HQ_TUNE_STREAM, 2)), 300)
    # a 256-row tile the bf16 format does not have
    with pytest.raises(hq.HQError):
        hq.hq_gemm_plan(autotune.with_tune(desc, hq.HQ_TUNE(hq.HQ_TUNE_T256, 1)), 300)
    # more K slices than 128-K steps
    with pytest.raises(hq.HQError):
        hq.hq_gemm_plan(autotune.with_tune(desc, hq.HQ_TUNE(hq.HQ_TUNE_T128, 16)), 300)
    # batch-invariant mode: tiled kernels without K split at every M
    d = hq.hq_layer_desc.from_buffer_copy(desc)
    d.flags = hq.HQ_FLAG_BATCH_INVARIANT
    for M in (1, 64, 300, 5000):
        plan = hq.hq_gemm_plan(d, M)
        assert len(plan) == 1 and plan[0].startswith("tile_gemm_kernel<") and "splits=1" in plan[0]
