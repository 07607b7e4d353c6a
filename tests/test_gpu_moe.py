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
    """At most 64 pairs: the streaming kernel builds its tile list itself, in
    tiles of min(T, 4) rows: 64 one-row tiles (the list's limit), two-row
    tiles, three-row tiles, and from 4 tokens on several 4-row tiles per busy
    expert."""
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


def test_moe_every_small_row_count():
    """Experts holding 0..12 rows in one routed call (78 pairs, above the
    in-kernel routing limit): up to 4 rows they take the streaming kernel, from
    5 rows the 32-row tiled tier."""
    E, N, K = 13, 256, 384
    counts = np.arange(E)
    T = int(counts.sum())
    d = syn.moe_mxfp4(21, T, E, 1, N, K)
    ids = np.repeat(np.arange(E), counts)
    np.random.default_rng(21).shuffle(ids)
    d["ids"] = ids.reshape(T, 1).astype(d["ids"].dtype)
    check(run_moe(T, E, 1, N, K, data=d))


def test_moe_single_expert_top1_equals_dense():
    T, E, N, K = 65, 1, 256, 384
    check(run_moe(T, E, 1, N, K, seed=9))


def moe_sample_pairs(ids, E, tile_rows=256, extra=24, seed=1):
    """Pairs to compare at full size: every active expert's first and last pair,
    the first and last row of every m-tile of the busiest expert (in the sorted
    order the kernels tile), and `extra` seeded random pairs."""
    T, top_k = ids.shape
    P = T * top_k
    counts, offsets, perm = oracle.moe_route(ids, E)
    pick = set(np.random.default_rng([T, seed]).choice(P, size=min(P, extra), replace=False).tolist())
    for e in np.flatnonzero(counts):
        pick.add(int(perm[offsets[e]]))
        pick.add(int(perm[offsets[e + 1] - 1]))
    top = int(counts.argmax())
    for r0 in range(0, int(counts[top]), tile_rows):
        pick.add(int(perm[offsets[top] + r0]))
        pick.add(int(perm[offsets[top] + min(r0 + tile_rows, int(counts[top])) - 1]))
    return np.array(sorted(pick), dtype=np.int64)


@pytest.mark.parametrize("T", [1, 8, 64, 2048, 8192])
def test_moe_full_size_sampled(T):
    """The MoE workload: E=256, top-8, N=4096, K=7168, Zipf(1.1) routing; sampled
    pairs covering every active expert and every tile of the busiest one."""
    E, top_k, N, K = 256, 8, 4096, 7168
    ids = syn.zipf_topk(0, syn.C5, T, E, top_k)
    flat = ids.reshape(-1)
    pairs = moe_sample_pairs(ids, E)
    needed = sorted(set(int(e) for e in flat))             # experts any token uses (the kernel reads these)
    note(f"moe full T={T}: generating {len(needed)} experts")
    d = syn.moe_mxfp4(0, T, E, top_k, N, K, experts=needed)
    check(run_moe(T, E, top_k, N, K, data=d, pairs=pairs))


# ---------------------------------------------------------------------------
# the MoE down projection: SwiGLU between the projections, then the expert GEMM
# on the activated rows (Indexed with one row per pair)
# ---------------------------------------------------------------------------

def ordered16(bits):
    """bf16 bits -> integers ordered like the values (adjacent values differ by 1)."""
    b = bits.astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def gpu_silu_mul(x_bits):
    rows, two_i = x_bits.shape
    out = empty(rows * two_i)
    hq.hq_silu_mul(hq.HQ_DT_BF16, rows, two_i // 2, dev(x_bits), out)
    torch.cuda.synchronize()
    return out[: rows * two_i].cpu().numpy().view(np.uint16).reshape(rows, two_i // 2)


def check_silu(got, x_bits):
    """fp32 arithmetic vs the fp64 oracle: at most one bf16 step where the result is a
    normal bf16; below 2^-126 (where fp32 itself runs out of precision) within 2^-126."""
    want = oracle.silu_mul_bf16(x_bits)
    gv, wv = to_f64(got, torch.bfloat16), to_f64(want, torch.bfloat16)
    steps = np.abs(ordered16(got) - ordered16(want))
    normal = np.abs(wv) >= 2.0 ** -126
    bad = (normal & (steps > 1)) | (~normal & (np.abs(gv - wv) > 2.0 ** -126))
    if bad.any():
        r, i = np.argwhere(bad)[0]
        I = got.shape[1]
        g, u = to_f64(x_bits[r:r + 1, [i, I + i]], torch.bfloat16)[0]
        raise AssertionError(f"row {r} col {i}: gate {g!r} up {u!r} got {gv[r, i]!r} want {wv[r, i]!r}")
    assert (steps > 0).mean() <= 0.01, (steps > 0).mean()


@pytest.mark.parametrize("rows,I", [(1, 8), (7, 2048), (300, 136)])
# gates below about -88.7 overflow e^-g in fp32 (-89.5 x 53.5 must still give -6.5e-36)
def test_silu_mul_matches_oracle(rows, I):
    note(f"silu_mul rows={rows} I={I}")
    x = syn._to16(syn.normal_rows(rows, 5, 9, rows, 2 * I, sigma=3.0), torch.bfloat16)
    x[0, :8] = syn._to16(np.array([0.0, -0.0, 1e-30, -1e-30, 40.0, -80.0, -89.5, -120.0], np.float32), torch.bfloat16)
    check_silu(gpu_silu_mul(x), x)


def test_silu_mul_rejects_bad_shapes():
    x = empty(64)
    with pytest.raises(hq.HQError):
        hq.hq_silu_mul(hq.HQ_DT_BF16, 1, 12, x, x)          # I not a multiple of 8
    with pytest.raises(hq.HQError):
        hq.hq_silu_mul(hq.HQ_DT_FP16, 1, 8, x, x)            # bf16 only


def run_layer(T, E, top_k, I, K1, N2, seed=0, pairs=None, experts=None):
    """Gate-up (N = 2I, K = K1) -> SwiGLU -> down (N = N2, K = I), all through the C ABI;
    the activation and the down projection are each checked against the oracle on the
    GPU's own input to that step."""
    d1 = syn.moe_mxfp4(seed, T, E, top_k, 2 * I, K1, experts=experts)
    d2 = syn.moe_mxfp4(seed + 1, 1, E, 1, N2, I, experts=experts)
    ids = d1["ids"]
    P = T * top_k
    pr = np.arange(P) if pairs is None else np.asarray(pairs)
    note(f"moe layer T={T} E={E} top_k={top_k} I={I} K1={K1} N2={N2}")
    desc1, desc2 = hq.desc_moe_mxfp4(E, 2 * I, K1), hq.desc_moe_mxfp4(E, N2, I)
    w1, s1, _ = hq.hq_repack(desc1, d1["q"], d1["e"])
    w2, s2, _ = hq.hq_repack(desc2, d2["q"], d2["e"])
    nb = max(hq.hq_workspace_bytes(desc1, T, top_k), hq.hq_workspace_bytes(desc2, P, 1))
    ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    D1, H, D2 = empty(P * 2 * I * 2), empty(P * I * 2), empty(P * N2 * 2)
    hq.hq_moe_gemm(desc1, hq.HQ_MOE_INDEXED, T, top_k, dev(d1["A"]), None, i32(ids), None, dev(w1), dev(s1), None,
                   D1, ws, nb)
    hq.hq_silu_mul(hq.HQ_DT_BF16, P, I, D1, H)
    flat = ids.reshape(P, 1)
    hq.hq_moe_gemm(desc2, hq.HQ_MOE_INDEXED, P, 1, H, None, i32(flat), None, dev(w2), dev(s2), None, D2, ws, nb)
    torch.cuda.synchronize()
    d1_bits = D1[: P * 2 * I * 2].cpu().numpy().view(np.uint16).reshape(P, 2 * I)
    h_bits = H[: P * I * 2].cpu().numpy().view(np.uint16).reshape(P, I)
    check_silu(h_bits[pr], d1_bits[pr])
    O = oracle.moe_mxfp4_bf16(h_bits, flat, d2["q"], d2["e"], N=N2, K=I, pairs=pr)
    Dh = to_f64(D2[: P * N2 * 2].cpu().numpy().view(np.uint16).reshape(P, N2), torch.bfloat16)
    err = gate_error(Dh[pr], O)
    assert np.all(np.isfinite(Dh[pr]))
    assert err <= min(GATE, 8e-3), err


@pytest.mark.parametrize("T", [3, 33, 300])
def test_moe_down_projection_small(T):
    """Both streaming paths (in-kernel routing below 4 rows, routed tier-0) and the tiled tiers."""
    run_layer(T, 8, 2, 128, 256, 384, seed=T)


def test_moe_down_projection_full_size():
    """The MoE layer at its real shape: gate-up N=4096 K=7168, down N=7168 K=2048, E=256 top-8."""
    T, E, top_k = 8, 256, 8
    ids = syn.zipf_topk(0, syn.C5, T, E, top_k)
    needed = sorted(set(int(e) for e in ids.reshape(-1)))
    pairs = np.arange(0, T * top_k, 3)
    run_layer(T, E, top_k, 2048, 7168, 7168, seed=0, pairs=pairs, experts=needed)
