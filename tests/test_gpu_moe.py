"""GPU parity of the MoE path (W4A16-MXFP4, bf16 tokens): routing metadata,
the Grouped gather, and the Indexed / Grouped expert GEMMs, against the CPU
oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from bit_quantized_gemm_w4a16_amd import hq
from gpu_util import GATE, dev, empty, gate_error, note, to_f64

pytestmark = pytest.mark.gpu


def i32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32).reshape(-1).copy()).to("cuda")


def gpu_align(ids, E):
    T, top_k = ids.shape
    P = T * top_k
    offs = torch.empty(E + 4, dtype=torch.int32, device="cuda")
    srt = torch.empty(max(P, 4), dtype=torch.int32, device="cuda")
    desc = hq.desc_moe_mxfp4(E, 128, 128)
    nb = hq.hq_workspace_bytes(desc, T, top_k)
    ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    hq.hq_moe_align(T, top_k, E, i32(ids), offs, srt, ws, nb)
    torch.cuda.synchronize()
    return offs[: E + 1].cpu().numpy(), srt[:P].cpu().numpy()


@pytest.mark.parametrize("T,E,top_k", [(1, 8, 2), (7, 16, 4), (300, 256, 8), (8192, 256, 8), (2000, 1000, 3)])
def test_align_matches_stable_counting_sort(T, E, top_k):
    note(f"moe_align T={T} E={E} top_k={top_k}")
    ids = syn.zipf_topk(T, 5, T, E, top_k)
    offs, srt = gpu_align(ids, E)
    counts, offsets, perm = oracle.moe_route(ids, E)
    np.testing.assert_array_equal(offs.astype(np.int64), offsets)
    np.testing.assert_array_equal(srt.astype(np.int64), perm)


def run_moe(T, E, top_k, N, K, seed=0, data=None, pairs=None, modes=("indexed", "grouped")):
    d = syn.moe_mxfp4(seed, T, E, top_k, N, K) if data is None else data
    ids = d["ids"]
    P = T * top_k
    desc = hq.desc_moe_mxfp4(E, N, K)
    wp, sp, _ = hq.hq_repack(desc, d["q"], d["e"])
    w, s = dev(wp), dev(sp)
    A = dev(d["A"])
    nb = hq.hq_workspace_bytes(desc, T, top_k)
    ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    pr = np.arange(P) if pairs is None else np.asarray(pairs)
    O = oracle.moe_mxfp4_bf16(d["A"], ids, d["q"], d["e"], N=N, K=K, pairs=pr)
    out = {}
    if "indexed" in modes:
        note(f"moe indexed T={T} E={E} top_k={top_k} N={N} K={K}")
        D = empty(P * N * 2)
        hq.hq_moe_gemm(desc, hq.HQ_MOE_INDEXED, T, top_k, A, None, i32(ids), None, w, s, None, D, ws, nb)
        torch.cuda.synchronize()
        Dh = to_f64(D[: P * N * 2].cpu().numpy().view(np.uint16).reshape(P, N), torch.bfloat16)
        out["indexed"] = (Dh[pr], O)
    if "grouped" in modes:
        note(f"moe grouped T={T} E={E} top_k={top_k} N={N} K={K}")
        counts, offsets, perm = oracle.moe_route(ids, E)
        As = empty(P * K * 2)
        srt = i32(perm)
        hq.hq_moe_gather(hq.HQ_DT_BF16, T, top_k, K, A, srt, As)
        torch.cuda.synchronize()
        # gather is a pure row copy: bit-exact
        ref = d["A"][perm // top_k]
        np.testing.assert_array_equal(As[: P * K * 2].cpu().numpy().view(np.uint16).reshape(P, K), ref)
        D = empty(P * N * 2)
        hq.hq_moe_gemm(desc, hq.HQ_MOE_GROUPED, T, top_k, As, None, None, i32(offsets), w, s, None, D, ws, nb)
        torch.cuda.synchronize()
        Dh = to_f64(D[: P * N * 2].cpu().numpy().view(np.uint16).reshape(P, N), torch.bfloat16)
        inv = np.empty(P, dtype=np.int64)
        inv[perm] = np.arange(P)
        out["grouped"] = (Dh[inv[pr]], O)   # grouped row i holds pair perm[i]
    return out


def check(out):
    for mode, (Dr, O) in out.items():
        err = gate_error(Dr, O)
        assert np.all(np.isfinite(Dr)), mode
        assert err <= min(GATE, 8e-3), (mode, err)


@pytest.mark.parametrize("T", [1, 2, 5, 32, 33, 300])
def test_moe_small(T):
    check(run_moe(T, 8, 2, 272, 512, seed=T))


@pytest.mark.parametrize("T,E,top_k", [(1, 64, 64), (2, 3, 2), (3, 40, 8), (16, 4, 4), (64, 3, 1)])
def test_moe_small_pair_counts(T, E, top_k):
    """At most 64 pairs.  Below 4 tokens the streaming kernel builds its tile
    list itself: 64 one-row tiles (the list's limit), two-row tiles, three-row
    tiles.  From 4 tokens on, every expert still takes the streaming kernel,
    several 4-row tiles per busy expert."""
    check(run_moe(T, E, top_k, 160, 256, seed=T + E))


def test_moe_one_hot_expert_and_empty_experts():
    T, E, top_k, N, K = 400, 16, 3, 128, 256
    d = syn.moe_mxfp4(3, T, E, top_k, N, K)
    d["ids"][:, 0] = 5                                     # expert 5 receives every token (>3 m-tiles)
    d["ids"][:, 1] = np.where(d["ids"][:, 1] == 5, 6, d["ids"][:, 1])
    d["ids"][:, 2] = np.where(np.isin(d["ids"][:, 2], [5, 6]), 7, d["ids"][:, 2])
    d["ids"][:, 1:] = np.where(d["ids"][:, 1:] >= 12, 4, d["ids"][:, 1:])   # experts 12..15 get nothing
    for t in range(T):                                      # keep ids distinct per token
        if len(set(d["ids"][t])) < top_k:
            d["ids"][t] = [5, 6, 7]
    check(run_moe(T, E, top_k, N, K, data=d))


def test_moe_single_expert_top1_equals_dense():
    T, E, N, K = 65, 1, 256, 384
    check(run_moe(T, E, 1, N, K, seed=9))


@pytest.mark.parametrize("T", [1, 8, 64, 8192])
def test_moe_full_size_sampled(T):
    """The MoE workload: E=256, top-8, N=4096, K=7168, Zipf(1.1) routing; sampled pairs."""
    E, top_k, N, K = 256, 8, 4096, 7168
    ids = syn.zipf_topk(0, syn.C5, T, E, top_k)
    P = T * top_k
    rng = np.random.default_rng([T, 1])
    flat = ids.reshape(-1)
    top = np.bincount(flat, minlength=E).argmax()
    pick = list(rng.choice(P, size=min(P, 24), replace=False))
    pick += list(np.flatnonzero(flat == top)[[0, -1]])     # first and last row of the busiest expert
    pairs = np.array(sorted(set(int(p) for p in pick)))
    needed = sorted(set(int(e) for e in flat))             # experts any token uses (the kernel reads these)
    note(f"moe full T={T}: generating {len(needed)} experts")
    d = syn.moe_mxfp4(0, T, E, top_k, N, K, experts=needed)
    check(run_moe(T, E, top_k, N, K, data=d, pairs=pairs))
