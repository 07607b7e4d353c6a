"""Dense GEMM shapes of the GPU parity suite, in one place.

The GPU tests parametrize over these lists, and the host-only coverage test
(tests/test_plan_coverage.py) asks the library's planner (hq_gemm_plan) which
kernels each of them launches, to check that every kernel configuration the
benchmark sweeps time is reached by at least one parity case.  No torch here.
"""
from __future__ import annotations

# the benchmark's M sweep: 1, 2, 4, ..., 8192
SWEEP = [1 << i for i in range(14)]

# the dense workloads at their real shapes
C2 = dict(N=4096, K=7168, G=128)          # W4A16 UINT4 + zero-points, fp16
C3 = dict(N=7168, K=4096)                 # W4A8-MXFP4
C4 = dict(N=18432, K=7168)                # W8A8 INT8

# ---- W4A16: (M, N, K, G, bf16, zp) ----
WNA16_SMALL_M = [1, 2, 3, 5, 8, 15, 16, 17, 24, 31, 33, 48, 63, 64]
WNA16_SMALL = [(M, 272, 1024, 128, bf, zp) for M in WNA16_SMALL_M
               for bf, zp in ((True, False), (False, True), (True, True), (False, False))]
WNA16_LARGER = [(M, 384, 768, 128, False, True) for M in (65, 100, 128, 200, 300)]
WNA16_SHAPES = [(M, N, K, G, False, True) for N, K, G in ((1000, 512, 128), (24, 128, 128), (512, 2048, 256),
                                                          (1024, 7168, 128), (48, 1024, 1024))
                for M in (1, 9, 40)]
# skinny two-m-tile batches (17..32 rows) at a K whose quarter is 14 chunks
WNA16_SKINNY_K7168 = [(24, 304, 7168, 128, bf, True) for bf in (False, True)]
WNA16_WIDE = [(4000, 4100, 512, 128, False, True), (4096, 4096, 1024, 128, False, False),
              (1100, 16000, 256, 128, False, True), (8192, 2056, 384, 128, False, True),
              (2000, 4100, 384, 128, False, True), (2048, 4096, 512, 128, False, False)]
# bf16 activations above the small-M schedule (the 128 x 128 tile with the row-sum MFMA)
WNA16_BF16_LARGE = [(M, N, 7168, 128, True, zp) for M, N in ((65, 4096), (300, 4100), (2048, 4096))
                    for zp in (False, True)]
WNA16_C2_SWEEP = [(M, C2["N"], C2["K"], C2["G"], False, True) for M in SWEEP]

# ---- W4A8-MXFP4: (M, N, K) ----
W4A8_SMALL = [(M, 272, 512) for M in (1, 3, 16, 24, 32, 64, 100, 257)]
W4A8_BIG = [(1100, 7200, 128), (1100, 7168, 640)]
# the two-stage 128 x 128 tile (grids of more than 256 such tiles below the 256 x 256 threshold)
W4A8_MID = [(1024, 7168, 256), (1000, 7000, 384)]
W4A8_C3_SWEEP = [(M, C3["N"], C3["K"]) for M in SWEEP]

# ---- W8A8-INT8: (M, N, K) ----
W8A8_SMALL_RAW = [(M, 304, 640) for M in (1, 7, 24, 64, 130)]
W8A8_SMALL_BF16 = [(M, 304, 640) for M in (1, 33, 200)]
# skinny two-m-tile batches at K = 7168 (14-chunk register batches)
W8A8_SKINNY_K7168 = [(M, 304, 7168) for M in (20, 32)]
W8A8_BIG_RAW = [(2100, 16400, 256), (600, 11000, 384), (600, 11000, 128)]
# the 256 x 128 stage ring: from the 128-row branch (M <= 1024, > 256 tiles of 128 x 128)
# and from the 256-row branch (>= 256 tiles of 256 x 128 that 256 x 256 would not halve into one round)
W8A8_RING = [(200, 20000, 384), (1024, 18432, 256), (256, 18432, 640)]
W8A8_C4_SWEEP = [(M, C4["N"], C4["K"]) for M in SWEEP]


# ---- MX activations x MXFP4 weights: (M, N, K), for E2M1 (W4A4) and E4M3 (MXFP8) activations ----
MXA_SMALL = [(M, 272, 512) for M in (1, 3, 16, 24, 32, 64, 100, 257)]
MXA_MID = [(1024, 7168, 256), (1000, 7000, 384)]
MXA_BIG = [(1100, 7200, 128), (1100, 7168, 640)]
MXA_SWEEP = [(M, C3["N"], C3["K"]) for M in SWEEP]


# ---- FP8 W8A8 with blockwise scales: (M, N, K) ----
FP8B_SMALL = [(M, 304, 640) for M in (1, 3, 16, 24, 33, 64, 100, 200)] + [(M, 300, 7168) for M in (1, 20, 64)]
FP8B_TILES = [(1100, 7200, 384), (600, 4000, 1280), (2100, 16400, 256)]
FP8B_SWEEP = [(M, 7168, 7168) for M in SWEEP]


# ---- FP4 weights with bf16 activations (MXFP4 / NVFP4): (M, N, K) ----
FP4A16_SMALL = [(M, 272, 1024) for M in (1, 3, 16, 24, 33, 64, 100, 300)] + [(M, 304, 7168) for M in (1, 20)]
FP4A16_TILES = [(2000, 4100, 384), (4000, 4100, 512), (1100, 16000, 256)]
FP4A16_SWEEP = [(M, C2["N"], C2["K"]) for M in SWEEP]


# ---- MXINT4 weights with bf16 activations: (M, N, K) ----
MXINT4_SMALL = [(M, 272, 1024) for M in (1, 3, 16, 24, 33, 64, 100, 300)] + [(M, 304, 7168) for M in (1, 20)]
MXINT4_TILES = [(2000, 4100, 384), (4000, 4100, 512), (1100, 16000, 256)]
MXINT4_SWEEP = [(M, C2["N"], C2["K"]) for M in SWEEP]


# ---- INT8 / FP8 weight-only (bf16 / fp16 activations): (M, N, K) ----
W8A16_SMALL = [(M, 272, 1024) for M in (1, 3, 16, 24, 33, 64, 100, 300)] + [(M, 304, 7168) for M in (1, 20)]
W8A16_TILES = [(2000, 4100, 384), (1100, 16000, 256), (700, 4100, 512)]
W8A16_SWEEP = [(M, C2["N"], C2["K"]) for M in SWEEP]

# ---- low-bit WnA16 (INT1/2/3, UINT1/2/3 + zero-points): (M, N, K, G, bits, signed, bf16) ----
WNLOW_WIDTHS = [(b, sg) for b in (1, 2, 3) for sg in (True, False)]
WNLOW_SMALL = [(M, 272, 1024, 128, b, sg, sg) for M in (1, 5, 16, 24, 64) for b, sg in WNLOW_WIDTHS]
WNLOW_TILES = [(M, N, K, G, b, sg, not sg) for M, N, K, G in ((100, 384, 768, 128), (300, 1000, 512, 256),
                                                             (2000, 4100, 384, 128)) for b, sg in WNLOW_WIDTHS]
# the dense W4A16 shape with 3-bit (UINT3 + zero-points, fp16) and 2-bit (INT2, bf16) codes
WNLOW_SWEEP = [(M, C2["N"], C2["K"], C2["G"], b, sg, bf) for b, sg, bf in ((3, False, False), (2, True, True))
               for M in SWEEP]

# ---- 5-8-bit WnA16 (INT5-8, UINT5-8 + 8-bit zero-points): (M, N, K, G, bits, signed, bf16) ----
WNWIDE_WIDTHS = [(b, sg) for b in (5, 6, 7, 8) for sg in (True, False)]
WNWIDE_SMALL = [(M, 1000, 1024, 128, b, sg, (b + sg) % 2 == 0) for M in (1, 5, 16, 33, 64) for b, sg in WNWIDE_WIDTHS]
WNWIDE_TILES = [(M, N, K, G, b, sg, (b + sg) % 2 == 1) for M, N, K, G in ((130, 1000, 1024, 128), (300, 520, 2048, 256),
                                                                         (2000, 4100, 384, 128)) for b, sg in WNWIDE_WIDTHS]
# the dense W4A16 shape with 8-bit (UINT8 + zero-points, fp16) and 5-bit (INT5, bf16) codes
WNWIDE_SWEEP = [(M, C2["N"], C2["K"], C2["G"], b, sg, bf) for b, sg, bf in ((8, False, False), (5, True, True))
                for M in SWEEP]

# ---- MX float weights (MXFP8 E4M3, MXFP6 E2M3 / E3M2), bf16 activations: (M, N, K, elem) ----
MXF_ELEMS = ["e4m3", "e2m3", "e3m2"]
MXF_SMALL = [(M, 272, 1024, e) for M in (1, 5, 16, 33, 64) for e in MXF_ELEMS]
MXF_TILES = [(M, N, K, e) for M, N, K in ((100, 384, 768), (300, 1000, 512), (2000, 4100, 384)) for e in MXF_ELEMS]
# at the dense W4A16 layer's shape, the widths the benchmark times
MXF_SWEEP = [(M, C2["N"], C2["K"], e) for e in ("e4m3", "e2m3") for M in SWEEP]


def all_dense_cases():
    """(format, M, N, K, G, flags) for every dense GPU case, flags a dict."""
    out = []
    for M, N, K, G, bf, zp in (WNA16_SMALL + WNA16_LARGER + WNA16_SHAPES + WNA16_SKINNY_K7168 + WNA16_WIDE
                               + WNA16_BF16_LARGE + WNA16_C2_SWEEP + [(16, 1024, 1024, 128, True, False)]):
        out.append(("wna16", M, N, K, G, dict(bf16=bf, zp=zp)))
    for M, N, K in W4A8_SMALL + W4A8_BIG + W4A8_MID + W4A8_C3_SWEEP + [(20, 1000, 1024)]:
        out.append(("w4a8", M, N, K, 32, {}))
    for M, N, K in W8A8_SMALL_RAW + W8A8_SKINNY_K7168 + W8A8_BIG_RAW + W8A8_RING + W8A8_C4_SWEEP + [(8, 64, 7168)]:
        out.append(("w8a8", M, N, K, K, dict(raw=True)))
    for M, N, K in W8A8_SMALL_BF16 + W8A8_C4_SWEEP:
        out.append(("w8a8", M, N, K, K, dict(raw=False)))
    for elem in ("e2m1", "e4m3"):
        for M, N, K in MXA_SMALL + MXA_MID + MXA_BIG + MXA_SWEEP:
            out.append(("mxa", M, N, K, 32, dict(elem=elem)))
    for M, N, K in FP8B_SMALL + FP8B_TILES + FP8B_SWEEP:
        out.append(("fp8b", M, N, K, 128, {}))
    for kind in ("mxfp4", "nvfp4"):
        for M, N, K in FP4A16_SMALL + FP4A16_TILES + FP4A16_SWEEP:
            out.append(("fp4a16", M, N, K, 16 if kind == "nvfp4" else 32, dict(kind=kind)))
    for M, N, K in MXINT4_SMALL + MXINT4_TILES + MXINT4_SWEEP:
        out.append(("mxint4", M, N, K, 32, {}))
    for M, N, K, G, b, sg, bf in WNLOW_SMALL + WNLOW_TILES + WNLOW_SWEEP:
        out.append(("wnlow", M, N, K, G, dict(bits=b, signed=sg, bf16=bf)))
    for M, N, K, G, b, sg, bf in WNWIDE_SMALL + WNWIDE_TILES + WNWIDE_SWEEP:
        out.append(("wnwide", M, N, K, G, dict(bits=b, signed=sg, bf16=bf)))
    for M, N, K, e in MXF_SMALL + MXF_TILES + MXF_SWEEP:
        out.append(("mxf", M, N, K, 32, dict(elem=e)))
    for wf in ("w8a16", "fp8w"):
        for dt in ("bf16", "fp16"):
            for M, N, K in W8A16_SMALL + W8A16_TILES + W8A16_SWEEP:
                out.append((wf, M, N, K, K, dict(bf16=dt == "bf16")))
    return out
