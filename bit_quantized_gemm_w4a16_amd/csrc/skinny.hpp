// Small-M schedule for every weight format on gfx950: a GEMV-like stream of
// the packed weights.
//
// The pages give the idea, not the code: at small batch the GEMM is bound by
// the weight traffic, so the kernel must keep the memory system busy and split
// the K dimension over the machine when the output alone gives too few
// workgroups ("Humming wird angekuendigt", section "Tuning und JIT-Kompilierung
// fuer jeden Workload", and the Stream-K option for small shapes in section
// "Gemeinsam genutzte CUDA-Komponenten").  The schedule below is our own for
// CDNA4.
//
// Workgroup = 4 waves over NS strips (16 output columns each) and one K slice
// of 128-K chunks.  The waves split the
// workgroup as WS strip-columns x WK K-parts; each wave owns SPW strips.
//   1. Every wave issues the first half of its packed-weight loads (16 bytes
//      per lane = one MFMA B fragment per load), in chunk order.
//   2. The A rows of the slice and the slice's scales (group scales +
//      zero-points, or E8M0 exponents) go to LDS with direct-to-LDS loads,
//      then the second half of the weight loads: the whole weight stream of
//      the chip is in flight at once, the weights (the long pole) first.
//   3. One wait for the LDS copies (memory returns in order, so the first
//      half of the weights has landed too), one barrier, then each chunk is
//      decoded and fed to the MFMA as soon as its own load has landed.
//   4. The K-parts of the workgroup reduce through LDS; K slices of a split
//      launch write fp32 / int32 partial tiles that a finalize pass sums in
//      slice order.  (A last-arriving-slice reduction inside the kernel needs a
//      device-scope release of the partials, which writes back the L2 and was
//      measured to cost far more than the extra launch.)
//
// Per format (one 128-K chunk of one strip):
//   WNA16_F16       4 x v_mfma_f32_16x16x32_f16 on the exact integer (q - z);
//                   the group scale multiplies the fp32 partial of the chunk
//   WNA16_BF16      4 x v_mfma_f32_16x16x32_bf16 on the exact 128 + u, the
//                   -(128 + z) offset from a row-sum MFMA and the group scale
//                   on the fp32 partial of the chunk
//   W4A8_MX         1 x v_mfma_scale_f32_16x16x128_f8f6f4 (fp8 A, fp4 B with
//                   the E8M0 exponent as the B scale)
//   W4A8_MXA        the same with the activations' own E8M0 block scales as
//                   the A scale (MXFP8 activations; copied to LDS with the A slice)
//   W4A4_MX         the same with fp4 e2m1 activations (MXFP4 x MXFP4)
//   W8A8_I8         2 x v_mfma_i32_16x16x64_i8 (exact int32)
//   MXFP4_BF16      4 x v_mfma_f32_16x16x32_bf16 on e2m1 x 2^(E-127) converted
//                   to bf16 (exact) with the lane's E8M0 byte
//   NVFP4_BF16      the same with the lane's two E4M3 group scales (16 K each)
//                   and the per-tensor fp32 second-level scale on the output
//   MXINT4_BF16     the same with two's-complement INT4 codes: sign-extended,
//                   scaled by 2^(E-127) in fp32 and rounded to bf16 (exact)
//   W8A16_F16/_BF16 4 x v_mfma_f32_16x16x32_{f16,bf16} on INT8 codes decoded to
//                   exact 16-bit operands (two 16-byte loads per chunk and lane),
//                   the per-channel fp32 scale in the epilogue
//   F8W_F16/_BF16   the same with E4M3 weight codes (FP8 weight-only)
//   W8A8_F8B        1 x the scaled MFMA on fp8 x fp8 per chunk (one 128-K scale
//                   block), its partial scaled by the row's activation block
//                   scale times the strip's weight block scale (both in LDS)
#pragma once

#include "tile_gemm.hpp"

namespace hq {

constexpr int kSkinnyLds = 150 * 1024;
constexpr int64_t kSkinnyMaxM = 64;  // dense M this schedule can take (tuning overrides)
// The M up to which the library's own choice is this schedule.  8-bit A on
// MFMAs that take whole 128-K steps: above 32 rows (INT8: 16) the tiled ring
// with a K split is faster (at N=7168 K=4096, M=64: 15.4 against 19.2 us; INT8
// at N=18432 K=7168, M=32: 32.9 against 35.7 us).
constexpr int64_t skinny_max_m(Fmt F) {
    return F == Fmt::W8A8_I8 ? 16 : (mx_mfma(F) || F == Fmt::W8A8_F8B) ? 32 : kSkinnyMaxM;
}

struct SkinnyArgs {
    const void* A;          // activations [a_rows][K]
    const float* a_scale;   // per-token fp32 (W4A8 / W8A8), by A row
    const uint8_t* a_e8;    // MX activation scales E8M0 [a_rows][K/32] (W4A8_MXA / W4A4_MX)
    const float* a_blk;     // activation scales per row and 128-K block [a_rows][K/128] (W8A8_F8B)
    const float* s2;        // per-tensor second-level weight scale, fp32 [1] (NVFP4_BF16)
    const void* W;          // packed weights
    const void* S;          // packed group scales / E8M0 / per-channel fp32
    const void* Z;          // packed zero-points (WNA16 with UINT4), or null
    void* D;                // output [rows][N]
    void* part;             // split-K partial tiles [splits][M][Np], or null
    int M, K, N, Np;
    int nc;                 // 128-K chunks in K
    int ngroups, gchunks;   // WNA16: K / G and G / 128
    int splits;
    int cps, cpk;           // chunks per K slice, chunks per wave K-part (host-computed)
    int NS, WS;             // strips per workgroup, wave strip-columns (WK = 4 / WS)
    int a_off, s_off, z_off;  // LDS layout (bytes); MX activation scales share z_off
    int raw_i32;            // W8A8: store the int32 accumulators
    int wbits;              // W4A16 formats: code width (4, or 1-3 for the low-bit planes)
    int part_nt;            // partial tiles stored non-temporally (set by the launcher)
};

template <Fmt F>
struct SkinnyTraits {
    static constexpr bool WNA16 = F == Fmt::WNA16_F16 || F == Fmt::WNA16_BF16;
    static constexpr bool MX = mx_mfma(F);               // E8M0 weight scales per 32 K
    static constexpr bool MXA = mx_act(F);               // E8M0 activation scales per 32 K
    // 4-, 6- or 8-bit codes -> bf16 operands under the lane's scale
    static constexpr bool FP4B = mxfp4w(F) || nvfp4(F) || mxint4w(F) || mxf8(F) || mxf6(F);
    static constexpr int SB = nvfp4(F) ? 128 : 64;  // scale bytes per strip and chunk
    static constexpr int AROW = FmtTraits<F>::AROW;      // bytes of a row per 128-K chunk
    static constexpr int UPC = AROW / 16;                // 16-byte A units per 128-K chunk and row
    static constexpr int NB = FmtTraits<F>::BSTRIP / 1024;  // 16-byte weight loads per chunk and lane
};

// A unit u of LDS row r holds global unit u ^ skinny_swz(r): 16 consecutive
// rows of a fragment read land in distinct bank groups.
template <int UPC>
__device__ __forceinline__ int skinny_swz(int row) {
    return UPC == 16 ? (row & 15) : UPC == 8 ? (row & 7) : (row & 3);
}

// One work item: K slice `split` of the launch.  Every thread of the
// workgroup calls it (it holds barriers).
//
// NW = 4: the A slice goes to LDS, where the waves of different strips share it.
// NW = 8 (16-bit A, one m-tile, one strip per workgroup, no K split): eight
// waves each take an eighth of K and load their A fragments straight from
// global memory into registers (the A rows are read by every workgroup and sit
// in L2), all at once with the weights; no A slice in LDS, so K need not be
// split to fit it (M = 9..16 otherwise splits K four ways and adds a finalize
// launch).
template <Fmt F, int MT, int SPW, int CPW, int NW, int WB>
__device__ __forceinline__ void skinny_item(const SkinnyArgs& p, int split, char* lds) {
    using Tr = SkinnyTraits<F>;
    using Acc = typename FmtTraits<F>::Acc;
    static_assert(F != Fmt::MOE_MX, "MoE experts stream through moe_stream_kernel");
    constexpr bool WNA16 = Tr::WNA16, MX = Tr::MX, MXA = Tr::MXA, FP4B = Tr::FP4B;
    constexpr int SB = Tr::SB;
    constexpr int AROW = Tr::AROW, UPC = Tr::UPC, NB = Tr::NB;
    constexpr int ROWS = 16 * MT;
    // WB < 4 (W4A16 formats): 1-3-bit codes in bit planes, widened to 4-bit words
    // after the load (a 2-bit plane of 8 B and a 1-bit plane of 4 B per lane and chunk)
    static_assert(WB == 4 || Tr::WNA16, "low-bit codes: W4A16 formats");
    // WB > 4 (W4A16 formats): 5-8-bit codes as the 4-bit word set plus the high
    // bits (a second word set for 8 bits, the low-bit planes for 5-7)
    constexpr int LPC = WB == 4 ? NB : WB == 3 ? 2 : WB < 4 ? 1 : WB == 7 ? 3 : 2;  // weight loads per chunk and lane
    constexpr int NLOAD = SPW * CPW * LPC;  // weight loads per wave and batch
    static_assert(NLOAD < 64, "vmcnt counts at most 63 loads");
    constexpr bool ADIR = NW == 8;  // A fragments straight from global memory
    static_assert(NW == 4 || (ADIR && AROW == 256 && MT == 1 && SPW == 1), "direct A: 16-bit A, one m-tile and strip");
    static_assert(!ADIR || NLOAD + CPW * MT * 4 + 4 < 64, "direct A: every load of a wave in flight at once");

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, quad = lane >> 4;
    const int WS = p.WS, wsh = WS >> 1, WK = NW >> wsh;  // WS is 1, 2 or 4 (1 with eight waves)
    const int ws = wave & (WS - 1), wk = wave >> wsh;
    const int nstrips = p.Np / 16;
    const int strip_base = blockIdx.x * p.NS;

    const char* Wb = (const char*)p.W;
    const char* Sb = (const char*)p.S;
    const int rows = p.M;
    // K slice [c0, c1) and this wave's part [cw0, cw1), in 128-K chunks (no division on the device)
    const int c0 = min(split * p.cps, p.nc), c1 = min(c0 + p.cps, p.nc);
    const int cw0 = min(c0 + wk * p.cpk, c1), cw1 = min(cw0 + p.cpk, c1);
    const int nsl = c1 - c0;   // chunks in the slice
    const int U = nsl * UPC;   // A units per LDS row

    // ---- the wave's packed weights, chunk-major, all in flight ----
    // Chunks past the wave's range repeat its last chunk (never used); a wave
    // with an empty range re-reads the slice's first chunk, so every load
    // stays inside the strip.  The first CH chunks go out before the A slice
    // and scales (the weights are the long pole), the rest after them.
    const int wlast = cw1 > cw0 ? cw1 - 1 : c0;
    int wstrip[SPW];
    const v4u* wsrc[SPW];
    const char* wp2[SPW];  // low-bit planes of the strip, at this lane
    const char* wp1[SPW];
    const size_t plane2 = WB >= 2 && WB < 4 ? (size_t)nstrips * p.nc * 512 : 0;  // bytes of the 2-bit plane
    // 5-8 bits: the high planes follow the 4-bit word set
    const size_t lowset = WB > 4 ? (size_t)nstrips * p.nc * 1024 : 0;
    const size_t plane2w = WB == 6 || WB == 7 ? (size_t)nstrips * p.nc * 512 : 0;
    const v4u* wh4[SPW];
    // MXFP6: a 16-byte plane (codes 0-20 of the lane's 32, and two bits of code 21)
    // then an 8-byte plane (the rest) per lane and chunk
    const char* f6b[SPW];
#pragma unroll
    for (int sp = 0; sp < SPW; ++sp) {
        wstrip[sp] = strip_base + ws * SPW + sp;
        const int st = wstrip[sp] < nstrips ? wstrip[sp] : nstrips - 1;
        wsrc[sp] = (const v4u*)(Wb + (size_t)st * p.nc * FmtTraits<F>::BSTRIP) + lane;
        wp2[sp] = Wb + lowset + (size_t)st * p.nc * 512 + lane * 8;
        wp1[sp] = Wb + lowset + (WB > 4 ? plane2w : plane2) + (size_t)st * p.nc * 256 + lane * 4;
        wh4[sp] = (const v4u*)(Wb + lowset + (size_t)st * p.nc * 1024) + lane;
        if constexpr (mxf6(F)) {
            wsrc[sp] = (const v4u*)(Wb + (size_t)st * p.nc * 1024) + lane;
            f6b[sp] = Wb + (size_t)nstrips * p.nc * 1024 + (size_t)st * p.nc * 512 + lane * 8;
        }
    }
    v4u w[CPW][SPW][NB];
    v4u wh[WB > 4 ? CPW : 1][SPW];  // 5-8 bits: the high bits of the chunk
    constexpr int CH = CPW / 2;
    auto issue_w = [&](int i) {
#pragma unroll
        for (int sp = 0; sp < SPW; ++sp) {
            const size_t c = (size_t)min(cw0 + i, wlast);
            if constexpr (mxf6(F)) {
                w[i][sp][0] = ld_nt(wsrc[sp] + c * 64);
                const v2u b = __builtin_nontemporal_load((const v2u*)(f6b[sp] + c * 512));
                w[i][sp][1] = v4u{b[0], b[1], 0u, 0u};
            } else if constexpr (WB == 4) {
#pragma unroll
                for (int h = 0; h < NB; ++h) w[i][sp][h] = ld_nt(wsrc[sp] + (c * NB + h) * 64);
            } else if constexpr (WB > 4) {
                w[i][sp][0] = ld_nt(wsrc[sp] + c * 64);
                if constexpr (WB == 8) {
                    wh[i][sp] = ld_nt(wh4[sp] + c * 64);
                } else {
                    v4u x = v4u{0u, 0u, 0u, 0u};
                    if constexpr (WB == 6 || WB == 7) {
                        const v2u a = __builtin_nontemporal_load((const v2u*)(wp2[sp] + c * 512));
                        x[0] = a[0];
                        x[1] = a[1];
                    }
                    if constexpr (WB != 6) x[2] = __builtin_nontemporal_load((const uint32_t*)(wp1[sp] + c * 256));
                    wh[i][sp] = x;
                }
            } else {
                // 2-bit plane into words 0-1, 1-bit plane into word 2
                v4u x = v4u{0u, 0u, 0u, 0u};
                if constexpr (WB >= 2) {
                    const v2u a = __builtin_nontemporal_load((const v2u*)(wp2[sp] + c * 512));
                    x[0] = a[0];
                    x[1] = a[1];
                }
                if constexpr (WB != 2) x[2] = __builtin_nontemporal_load((const uint32_t*)(wp1[sp] + c * 256));
                w[i][sp][0] = x;
            }
        }
        // keep the issue order = the consumption order, so each chunk waits only for its own loads
        __builtin_amdgcn_sched_barrier(0);
    };
#pragma unroll
    for (int i = 0; i < CH; ++i) issue_w(i);

    // ---- A slice and scales -> LDS (direct loads, issued between the two halves of the weights) ----
    {
        const char* Abase = (const char*)p.A + (size_t)c0 * AROW;
        const int nblk = (U + 63) >> 6;  // 64-unit blocks per row
        int r = 0, blk = wave;
        while (r < rows && blk >= nblk) { blk -= nblk; ++r; }
        while (!ADIR && r < rows) {
            const int pos = blk * 64 + lane;
            const char* arow = Abase + (size_t)r * (p.K / 128) * AROW;
            if (pos < U) lds_dma16(arow + ((pos ^ skinny_swz<UPC>(r)) * 16), lds + p.a_off + (r * U + blk * 64) * 16);
            blk += NW;
            while (r < rows && blk >= nblk) { blk -= nblk; ++r; }
        }
        if constexpr (F == Fmt::W8A8_F8B) {
            // weight block scales [strip j][chunk] at s_off (strip j's 128-column block is
            // its strip index / 8); activation scales [chunk][row, 16-row aligned] at z_off
            const int nbn = (p.Np + 127) / 128, R16 = (rows + 15) & ~15;
            const float* swg = (const float*)Sb;
            for (int w0 = wave * 64; w0 < p.NS * nsl; w0 += 64 * NW) {
                const int w = w0 + lane;
                if (w < p.NS * nsl) {
                    const int j = w / nsl, c = w - j * nsl;
                    const int st = strip_base + j < nstrips ? strip_base + j : nstrips - 1;
                    lds_dma4(swg + (size_t)(c0 + c) * nbn + st / 8, lds + p.s_off + w0 * 4);
                }
            }
            for (int w0 = wave * 64; w0 < nsl * R16; w0 += 64 * NW) {
                const int w = w0 + lane;
                if (w < nsl * R16) {
                    const int c = w / R16, r = w - c * R16;
                    lds_dma4(p.a_blk + (size_t)(r < rows ? r : rows - 1) * (p.K / 128) + c0 + c, lds + p.z_off + w0 * 4);
                }
            }
        }
        if constexpr (WNA16) {
            const int sg0 = c0 / p.gchunks, sgslab = (c1 - 1) / p.gchunks - sg0 + 1;
            for (int j = 0; j < p.NS; ++j) {
                const int st = strip_base + j < nstrips ? strip_base + j : nstrips - 1;
                const char* sg = (const char*)Sb + ((size_t)st * p.ngroups + sg0) * 32;
                constexpr int ZW = WB > 4 ? 4 : 2;  // zero-point words per strip and group (UINT8 or UINT4)
                const char* zg = (const char*)p.Z + ((size_t)st * p.ngroups + sg0) * ZW * 4;
                for (int pos0 = wave * 64; pos0 < sgslab * ZW; pos0 += 64 * NW) {
                    const int pos = pos0 + lane;  // 16-byte scale units / 32-bit zero-point words
                    if (pos < sgslab * 2) lds_dma16(sg + pos * 16, lds + p.s_off + (j * sgslab * 2 + pos0) * 16);
                    if (p.Z && pos < sgslab * ZW) lds_dma4(zg + pos * 4, lds + p.z_off + (j * sgslab * ZW + pos0) * 4);
                }
            }
        } else if constexpr (MX || FP4B) {
            constexpr int UPS = SB / 16;  // 16-byte scale units per chunk and strip
            for (int j = 0; j < p.NS; ++j) {
                const int st = strip_base + j < nstrips ? strip_base + j : nstrips - 1;
                for (int pos0 = wave * 64; pos0 < nsl * UPS; pos0 += 64 * NW) {  // SB bytes per chunk
                    const int pos = pos0 + lane;
                    if (pos < nsl * UPS)
                        lds_dma16((const char*)Sb + ((size_t)st * p.nc + c0) * SB + pos * 16, lds + p.s_off + (j * nsl * UPS + pos0) * 16);
                }
            }
            if constexpr (MXA) {
                // the slice's activation scales: one 4-byte word (4 K blocks) per row and chunk, [row][nsl]
                const int nw = rows * nsl;
                for (int w0 = wave * 64; w0 < nw; w0 += 64 * NW) {
                    const int w = w0 + lane;
                    if (w < nw) {
                        const int r = w / nsl, c = w - r * nsl;
                        lds_dma4(p.a_e8 + (size_t)r * (p.K / 32) + (size_t)(c0 + c) * 4, lds + p.z_off + w0 * 4);
                    }
                }
            }
        }
    }

    // direct A: this wave's A fragments of every chunk of its K-part (lane (row,
    // quad) holds K 32 quad .. 32 quad + 31 of its row and chunk: 64 contiguous
    // bytes, one 16-byte fragment per K sub-step); rows past M read row M - 1
    Frag8 afd[ADIR ? CPW : 1][MT][4];
    if constexpr (ADIR) {
        const char* arow = (const char*)p.A + (size_t)min(col, rows - 1) * (p.K / 128) * AROW + quad * 64;
#pragma unroll
        for (int i = 0; i < CPW; ++i) {
            const int c = min(cw0 + i, wlast);
#pragma unroll
            for (int t = 0; t < 4; ++t) afd[i][0][t].u = *(const v4u*)(arow + (size_t)c * AROW + t * 16);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = CH; i < CPW; ++i) issue_w(i);
    // the LDS copies were issued before the last (CPW - CH) chunks' loads (and,
    // direct A, before the A fragments): once at most that many loads are
    // outstanding, this wave's copies (and its first CH chunks) have landed
    wait_vmcnt<SPW * (CPW - CH) * LPC + (ADIR ? CPW * MT * 4 : 0)>();
    lds_barrier();

    // ---- 3. decode + MFMA ----
    // two independent accumulator sets (alternating by K sub-step or chunk) so
    // consecutive MFMAs do not wait on each other; summed before the reduction
    Acc acc2[2][SPW][MT];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int sp = 0; sp < SPW; ++sp)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc2[q][sp][mt] = Acc{0, 0, 0, 0};
    const char* lA = lds + p.a_off;
    int arow_l[MT];  // this lane's A row in LDS per m-tile (rows past the tile read its last row)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) arow_l[mt] = min(mt * 16 + col, rows - 1);
    Frag8 ones;
    ones.u = v4u{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
    const bool zsel = p.Z != nullptr;
    const uint32_t wx = zsel ? 0u : 0x88888888u;  // symmetric INT4: two's complement -> offset binary
    // low-bit codes: signed ones to offset binary (top bit flipped: the 2-bit
    // plane's high bits for width 2, the 1-bit plane for widths 1 and 3)
    const uint32_t lx2 = !zsel && WB == 2 ? 0xAAAAAAAAu : 0u, lx1 = !zsel && WB != 2 ? 0xFFFFFFFFu : 0u;
    // 5-8 bits: signed codes to offset binary (their top bit: bit 3 of the high
    // nibble for 8 bits, the high bits of the 2-bit fields for 6, the 1-bit plane
    // for 5 and 7)
    const uint32_t hx4 = !zsel && WB == 8 ? 0x88888888u : 0u, hx2 = !zsel && WB == 6 ? 0xAAAAAAAAu : 0u;
    const uint32_t hx1 = !zsel && (WB == 5 || WB == 7) ? 0xFFFFFFFFu : 0u;
    const uint32_t zmask = zsel ? (WB > 4 ? 255u : 15u) : 0u;  // zero-point, or the offset of the symmetric codes
    const uint32_t zdef = zsel ? 0u : WB == 4 ? 8u : 1u << (WB - 1);

    // WNA16: group of each chunk, relative to the slice's first group
    const int g0 = WNA16 ? c0 / p.gchunks : 0, gslab = WNA16 ? (c1 - 1) / p.gchunks - g0 + 1 : 0;
    int gi[CPW];
    {
        int gcur = WNA16 ? cw0 / p.gchunks - g0 : 0, grem = WNA16 ? cw0 % p.gchunks : 0;
#pragma unroll
        for (int i = 0; i < CPW; ++i) {
            gi[i] = min(gcur, gslab - 1);
            if (++grem == p.gchunks) {
                grem = 0;
                ++gcur;
            }
        }
    }
    // 16-bit A formats: the LDS operands of chunk i+1 (A fragments, the strip's
    // scale and zero-point word, or its E8M0 byte) are read while chunk i computes
    constexpr bool A16 = AROW == 256;
    Frag8 afb[2][A16 && !ADIR ? MT : 1][4];
    uint32_t sbb[2][SPW], zwb[2][SPW];
    auto lds_operands = [&](int i, auto slot) {
        constexpr int S = decltype(slot)::value;
        const int cl = min(cw0 + i, c1 - 1) - c0;
        if constexpr (A16 && !ADIR) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int row = arow_l[mt];
                const char* ar = lA + (size_t)row * U * 16;
#pragma unroll
                for (int t = 0; t < 4; ++t) afb[S][mt][t].u = *(const v4u*)(ar + (((cl * 16 + 4 * quad + t) ^ skinny_swz<16>(row)) * 16));
            }
        }
#pragma unroll
        for (int sp = 0; sp < SPW; ++sp) {
            const int j = ws * SPW + sp;
            if constexpr (WNA16) {
                sbb[S][sp] = ((const uint16_t*)(lds + p.s_off))[(j * gslab + gi[i]) * 16 + col];
                if constexpr (WB > 4)  // UINT8 zero-points: four words per strip and group
                    zwb[S][sp] = ((const uint32_t*)(lds + p.z_off))[(j * gslab + gi[i]) * 4 + (col >> 2)];
                else
                    zwb[S][sp] = ((const uint32_t*)(lds + p.z_off))[(j * gslab + gi[i]) * 2 + (col >> 3)];
            }
        }
    };
    using Z0 = std::integral_constant<int, 0>;
    using Z1 = std::integral_constant<int, 1>;
    if constexpr (A16) lds_operands(0, Z0{});
    {  // the plan keeps a wave's K-part within one register batch (cpk <= CPW)
#pragma unroll
        for (int i = 0; i < CPW; ++i) {
            if constexpr (A16) {
                if (i + 1 < CPW) {
                    if (i & 1) lds_operands(i + 1, Z0{});
                    else lds_operands(i + 1, Z1{});
                }
            }
            // Every wave runs all CPW chunk bodies without branches (branches let the
            // compiler merge the bodies and lose the per-load waits); a chunk past the
            // wave's part reads the slice's last chunk and contributes exactly zero.
            const int c = cw0 + i;
            const bool valid = c < cw1;
            const int cl = min(c, c1 - 1) - c0;
            if constexpr (WNA16) {
                constexpr bool BF = F == Fmt::WNA16_BF16;
                const Frag8(&af)[MT][4] = ADIR ? afd[ADIR ? i : 0] : afb[i & 1];
                v4f rs[MT];
                if constexpr (BF && WB <= 4) {
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        rs[mt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int t = 0; t < 4; ++t) rs[mt] = mfma16<true>(af[mt][t], ones, rs[mt]);
                    }
                }
#pragma unroll
                for (int sp = 0; sp < SPW; ++sp) {
                    // the zero-point word was read even without zero-points (no branch
                    // around the LDS read: a branch here costs the per-load waits)
                    const uint32_t sbits = sbb[i & 1][sp], zw = zwb[i & 1][sp];
                    // this chunk's codes: 4-bit words, or the low-bit planes in offset binary
                    v4u wq = w[i][sp][0];
                    if constexpr (WB < 4) {
                        wq[0] ^= lx2;
                        wq[1] ^= lx2;
                        wq[2] ^= lx1;
                    }
                    v4u wk = v4u{0u, 0u, 0u, 0u};  // 5-8 bits: the high bits, in offset binary
                    if constexpr (WB > 4) {
                        wk = wh[i][sp];
                        wk[0] ^= WB == 8 ? hx4 : hx2;
                        wk[1] ^= WB == 8 ? hx4 : hx2;
                        wk[2] ^= WB == 8 ? hx4 : hx1;
                        wk[3] ^= hx4;
                    }
                    const uint32_t z = WB > 4 ? (((zw >> (8 * (col & 3))) & zmask) | zdef)
                                              : (((zw >> (4 * (col & 7))) & zmask) | zdef);
                    if constexpr (BF && WB <= 4) {
                        // bf16: operand 128 + u is exact; the group scale and the
                        // -(128 + z) offset (a row-sum MFMA) act on the fp32 partial
                        const float sc = valid ? bits16_to_f32<true>((uint16_t)sbits) : 0.f;
                        v4f gacc[MT];
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt) gacc[mt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            Frag8 b;
                            if constexpr (WB == 4) b = deq4_bf16_offset(wq[t] ^ wx);
                            else b = deq_low_bf16_offset<WB>(wq, t);
#pragma unroll
                            for (int mt = 0; mt < MT; ++mt) gacc[mt] = mfma16<true>(af[mt][t], b, gacc[mt]);
                        }
                        const float zc = (float)(128u + z);
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt) acc2[0][sp][mt] += sc * (gacc[mt] - zc * rs[mt]);
                    } else {
                        // fp16: the exact integer (q - z) as the operand, the group scale on
                        // the fp32 partial of the chunk (fewer VALU per code than scaling
                        // every operand, and exact); bf16 at 5-8 bits the same, the
                        // difference converted to bf16 (exact: at most 8 significant bits)
                        const float sc = valid ? bits16_to_f32<BF>((uint16_t)sbits) : 0.f;
                        const uint32_t nbw = (0xE400u | z) * 0x10001u;  // 5-8 bits: -(1024 + z)
                        const uint32_t nbz = 0xE400u | z, nhz = 0xD400u | (z << 4);  // -(1024 + z), -(64 + z)
                        const uint32_t nb2 = nbz | (nbz << 16), nh2 = nhz | (nhz << 16);
                        uint32_t nbl[4];  // low-bit widths: -(base_s + z) per pair position
                        if constexpr (WB < 4) low_f16_offsets<WB>(z, nbl);
                        v4f gacc[2][MT];
#pragma unroll
                        for (int q = 0; q < 2; ++q)
#pragma unroll
                            for (int mt = 0; mt < MT; ++mt) gacc[q][mt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            Frag8 b;
                            if constexpr (WB == 4) b = deq4_f16_exact(wq[t] ^ wx, nb2, nh2);
                            else if constexpr (WB > 4) b = deq_wide<WB, BF>(wq, wk, t, nbw);
                            else b = deq_low_f16<WB>(wq, t, nbl);
#pragma unroll
                            for (int mt = 0; mt < MT; ++mt) gacc[t & 1][mt] = mfma16<BF>(af[mt][t], b, gacc[t & 1][mt]);
                        }
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt) acc2[i & 1][sp][mt] += sc * (gacc[0][mt] + gacc[1][mt]);
                    }
                }
            } else if constexpr (w8a16(F)) {
                // INT8 -> exact 16-bit operands (the per-channel scale is applied in the
                // epilogue); a chunk past the wave's part multiplies zeros
                constexpr bool BF = w8bf(F);
                const Frag8(&af)[MT][4] = ADIR ? afd[ADIR ? i : 0] : afb[i & 1];
#pragma unroll
                for (int sp = 0; sp < SPW; ++sp)
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        Frag8 b = deq8<F>(w[i][sp][t >> 1], t & 1);
#pragma unroll
                        for (int e = 0; e < 4; ++e) b.u[e] = valid ? b.u[e] : 0u;
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt) acc2[t & 1][sp][mt] = mfma16<BF>(af[mt][t], b, acc2[t & 1][sp][mt]);
                    }
            } else if constexpr (FP4B) {
                // e2m1 x (2^(E-127) or E4M3 group scale) -> exact 16-bit operands (bf16,
                // or fp16 with fp16 activations), MFMA of that type
                constexpr bool BFO = !f16_operand(F);
                const Frag8(&af)[MT][4] = ADIR ? afd[ADIR ? i : 0] : afb[i & 1];
#pragma unroll
                for (int sp = 0; sp < SPW; ++sp) {
                    const int j = ws * SPW + sp;
                    float sf0, sf1;
                    if constexpr (nvfp4(F)) {
                        const uint32_t two = ((const uint16_t*)(lds + p.s_off))[((j * nsl + cl) * SB) / 2 + lane];
                        sf0 = __builtin_amdgcn_cvt_f32_fp8((int)two, 0);
                        sf1 = __builtin_amdgcn_cvt_f32_fp8((int)two, 1);
                    } else {
                        sf0 = sf1 = e8m0_to_f32(((const uint8_t*)(lds + p.s_off))[(j * nsl + cl) * SB + lane]);
                    }
                    if (!valid) sf0 = sf1 = 0.f;  // a chunk past the wave's part contributes exactly zero
                    v16u y6;  // MXFP6: the chunk's 32 codes at once, 6 bits each (code j at bit 6j)
                    if constexpr (mxf6(F)) {
                        const v6u x6 = v6u{w[i][sp][0][0], w[i][sp][0][1], w[i][sp][0][2], w[i][sp][0][3],
                                           w[i][sp][1][0], w[i][sp][1][1]};
                        if constexpr (!mxf6e3(F) && BFO)
                            y6 = __builtin_bit_cast(v16u, __builtin_amdgcn_cvt_scalef32_pk32_bf16_fp6(x6, sf0));
                        else if constexpr (BFO)
                            y6 = __builtin_bit_cast(v16u, __builtin_amdgcn_cvt_scalef32_pk32_bf16_bf6(x6, sf0));
                        else if constexpr (!mxf6e3(F))
                            y6 = __builtin_bit_cast(v16u, __builtin_amdgcn_cvt_scalef32_pk32_f16_fp6(x6, sf0));
                        else
                            y6 = __builtin_bit_cast(v16u, __builtin_amdgcn_cvt_scalef32_pk32_f16_bf6(x6, sf0));
                    }
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        Frag8 b;
                        if constexpr (nvfp4(F)) b = fp4_to_bf16_mul<BFO>(w[i][sp][0][t], t < 2 ? sf0 : sf1);
                        else if constexpr (mxint4w(F)) b = int4_to_bf16<BFO>(w[i][sp][0][t], sf0);
                        else if constexpr (mxf8(F)) b = fp8_to_bf16_scaled<BFO>(w[i][sp][t >> 1], t & 1, sf0);
                        else if constexpr (mxf6(F)) b.u = v4u{y6[4 * t], y6[4 * t + 1], y6[4 * t + 2], y6[4 * t + 3]};
                        else b = fp4_to_bf16<BFO>(w[i][sp][0][t], sf0);
                        if constexpr (mxf8(F) || mxf6(F)) {
                            // (the scaled converts take only the scale's exponent: a zero scale gives no zeros)
#pragma unroll
                            for (int e = 0; e < 4; ++e) b.u[e] = valid ? b.u[e] : 0u;
                        }
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt) acc2[t & 1][sp][mt] = mfma16<BFO>(af[mt][t], b, acc2[t & 1][sp][mt]);
                    }
                }
            } else if constexpr (MX) {
                v8i af[MT];
                int asc[MT];
                constexpr int CBSZ = F == Fmt::W4A4_MX ? 4 : 0;  // A operand: fp8 e4m3 or fp4 e2m1
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const int row = arow_l[mt];
                    const char* ar = lA + (size_t)row * U * 16;
                    const int sw = skinny_swz<UPC>(row);
                    const v4u lo = *(const v4u*)(ar + (((cl * UPC + quad) ^ sw) * 16));
                    if constexpr (F == Fmt::W4A4_MX) {
                        af[mt] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], 0, 0, 0, 0};
                    } else {
                        const v4u hi = *(const v4u*)(ar + (((cl * 8 + 4 + quad) ^ sw) * 16));
                        af[mt] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                    }
                    // lane (row, quad) supplies the scale of its row's K block `quad` of the chunk
                    asc[mt] = MXA ? (int)((const uint8_t*)(lds + p.z_off))[(row * nsl + cl) * 4 + quad] : 0x7F;
                }
#pragma unroll
                for (int sp = 0; sp < SPW; ++sp) {
                    const int j = ws * SPW + sp;
                    const int bsc = (int)((const uint8_t*)(lds + p.s_off))[(j * nsl + cl) * 64 + lane];
                    const v4u bw = valid ? w[i][sp][0] : v4u{0u, 0u, 0u, 0u};  // e2m1 code 0 is +0
                    const v8i b = v8i{(int)bw[0], (int)bw[1], (int)bw[2], (int)bw[3], 0, 0, 0, 0};
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        acc2[i & 1][sp][mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[mt], b, acc2[i & 1][sp][mt], CBSZ, 4, 0, asc[mt], 0, bsc);
                }
            } else if constexpr (F == Fmt::W8A8_F8B) {
                const int R16 = (rows + 15) & ~15;
                v8i af[MT];
                v4f sa4[MT];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const int row = arow_l[mt];
                    const char* ar = lA + (size_t)row * U * 16;
                    const int sw = skinny_swz<8>(row);
                    const v4u lo = *(const v4u*)(ar + (((cl * 8 + quad) ^ sw) * 16));
                    const v4u hi = *(const v4u*)(ar + (((cl * 8 + 4 + quad) ^ sw) * 16));
                    af[mt] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                    // this lane's output rows mt * 16 + 4 quad .. + 3 (clamped rows are dropped on store)
                    sa4[mt] = *(const v4f*)(lds + p.z_off + (cl * R16 + (mt * 16 + 4 * quad < R16 ? mt * 16 + 4 * quad : R16 - 4)) * 4);
                }
#pragma unroll
                for (int sp = 0; sp < SPW; ++sp) {
                    const float swv = ((const float*)(lds + p.s_off))[(ws * SPW + sp) * nsl + cl];
                    const v4u w0 = valid ? w[i][sp][0] : v4u{0u, 0u, 0u, 0u}, w1 = valid ? w[i][sp][1] : v4u{0u, 0u, 0u, 0u};
                    const v8i b = v8i{(int)w0[0], (int)w0[1], (int)w0[2], (int)w0[3], (int)w1[0], (int)w1[1], (int)w1[2], (int)w1[3]};
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        const v4f part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[mt], b, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0x7F, 0, 0x7F);
                        acc2[i & 1][sp][mt] += part * (sa4[mt] * swv);
                    }
                }
            } else {  // W8A8_I8
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    v4i af[MT];
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        const int row = arow_l[mt];
                        const char* ar = lA + (size_t)row * U * 16;
                        af[mt] = *(const v4i*)(ar + (((cl * 8 + 4 * h + quad) ^ skinny_swz<8>(row)) * 16));
                    }
#pragma unroll
                    for (int sp = 0; sp < SPW; ++sp)
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt)
                            acc2[h][sp][mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[mt], __builtin_bit_cast(v4i, valid ? w[i][sp][h] : v4u{0u, 0u, 0u, 0u}), acc2[h][sp][mt], 0, 0, 0);
                }
            }
        }
    }

    Acc acc[SPW][MT];
#pragma unroll
    for (int sp = 0; sp < SPW; ++sp)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[sp][mt] = acc2[0][sp][mt] + acc2[1][sp][mt];

    // ---- 4. reduce the K-parts of the workgroup through LDS ----
    if (WK > 1) {
        __syncthreads();  // every load has landed; the A slice is no longer needed
        Acc* red = (Acc*)lds;
        if (wk > 0) {
#pragma unroll
            for (int sp = 0; sp < SPW; ++sp)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) red[((((wk - 1) * WS + ws) * SPW + sp) * MT + mt) * 64 + lane] = acc[sp][mt];
        }
        __syncthreads();
        if (wk == 0)
            for (int k2 = 1; k2 < WK; ++k2)
#pragma unroll
                for (int sp = 0; sp < SPW; ++sp)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) acc[sp][mt] += red[((((k2 - 1) * WS + ws) * SPW + sp) * MT + mt) * 64 + lane];
    }
    // ---- 5./6. output (K-part 0): lane (col, quad) holds rows mt*16 + 4*quad + r of column col ----
    // The K slice's fp32 / int32 partial tile (split K, summed in slice order by
    // the finalize pass), or the output with the format's epilogue.  Stores go
    // through a buffer resource over the rows 0 .. M-1 of the output (or of the
    // slice's partial tile): rows past M and columns past N (Np) take an offset
    // outside it and are dropped, so no store sits behind a branch, and the
    // epilogue's scales are loaded before the first store.  The range fits 32
    // bits: M <= 64 rows of at most 2^21 columns of 4 bytes.
    if (wk != 0) return;
    const bool partial = p.splits > 1;
    constexpr bool ASC = F == Fmt::W4A8_MX || F == Fmt::W8A8_I8, WSC = F == Fmt::W8A8_I8 || w8a16(F);
    float asr[ASC ? MT : 1][4], swn[WSC ? SPW : 1];
    if (!partial) {
        if constexpr (ASC) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = mt * 16 + quad * 4 + r;
                    asr[mt][r] = m < rows ? p.a_scale[m] : 0.f;
                }
        }
        if constexpr (WSC) {
#pragma unroll
            for (int sp = 0; sp < SPW; ++sp) {
                const int n = wstrip[sp] * 16 + col;
                swn[sp] = n < p.N ? ((const float*)Sb)[n] : 0.f;
            }
        }
    }
    auto outv = [&](int sp, int mt, int r) -> uint32_t {
        if (partial) return bits32(acc[sp][mt][r]);
        if constexpr (WNA16) return f32_to_16<F == Fmt::WNA16_BF16>(acc[sp][mt][r]);
        else if constexpr (F == Fmt::W8A8_I8)
            return p.raw_i32 ? (uint32_t)acc[sp][mt][r] : f32_to_bf16_bits((float)acc[sp][mt][r] * asr[mt][r] * swn[sp]);
        else if constexpr (F == Fmt::W4A8_MX) return f32_to_bf16_bits(acc[sp][mt][r] * asr[mt][r]);
        else if constexpr (nvfp4(F)) return f32_to_16<!f16_operand(F)>(acc[sp][mt][r] * *p.s2);
        else if constexpr (w8a16(F)) return f32_to_16<w8bf(F)>(acc[sp][mt][r] * swn[sp]);
        else return f32_to_16<!f16_operand(F)>(acc[sp][mt][r]);
    };
    const int es = partial || (F == Fmt::W8A8_I8 && p.raw_i32) ? 4 : 2;
    const int ldo = partial ? p.Np : p.N;
    char* obase = partial ? (char*)p.part + (int64_t)split * p.M * p.Np * 4 : (char*)p.D;
    const rsrc_t rO = make_rsrc(obase, (uint32_t)rows * (uint32_t)ldo * (uint32_t)es);
    constexpr uint32_t DROP = 0xFFFFFFF0u;
    auto store = [&](auto kind) {
        constexpr int K_ = decltype(kind)::value;  // 0: 16-bit, 1: 32-bit, 2: 32-bit non-temporal
#pragma unroll
        for (int sp = 0; sp < SPW; ++sp) {
            const int n = wstrip[sp] * 16 + col;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = mt * 16 + quad * 4 + r;
                    const uint32_t off = m < rows && n < ldo ? ((uint32_t)m * (uint32_t)ldo + (uint32_t)n) * (uint32_t)es : DROP;
                    const uint32_t v = outv(sp, mt, r);
                    if constexpr (K_ == 0) __builtin_amdgcn_raw_buffer_store_b16((uint16_t)v, rO, off, 0, 0);
                    else if constexpr (K_ == 1) __builtin_amdgcn_raw_buffer_store_b32(v, rO, off, 0, 0);
                    else __builtin_amdgcn_raw_buffer_store_b32(v, rO, off, 0, 2);
                }
        }
    };
    if (partial && p.part_nt) store(std::integral_constant<int, 2>{});
    else if (es == 4) store(std::integral_constant<int, 1>{});
    else store(std::integral_constant<int, 0>{});
}

template <Fmt F, int MT, int SPW, int CPW, int NW, int WB>
__global__ __launch_bounds__(64 * NW) void skinny_kernel(SkinnyArgs p) {
    extern __shared__ __attribute__((aligned(1024))) char lds[];  // sized per launch (plan.lds_bytes)
    skinny_item<F, MT, SPW, CPW, NW, WB>(p, blockIdx.y, lds);
}

// ---- host-side plan ----

struct SkinnyPlan {
    bool ok;        // false: a forced K split that the slice's LDS or register batch cannot take
    int NS, WS, SPW, splits, MT, CPW;
    int NW;         // waves per workgroup: 4, or 8 with direct A loads (16-bit A, M <= 16)
    int cps, cpk;   // chunks per slice, per wave K-part
    int a_off, s_off, z_off;
    int lds_bytes;  // dynamic LDS of one workgroup
    int64_t groups_x;
};

inline int skinny_round_cpw(int64_t per, int spw) {
    // 14: a wave's quarter of K = 7168 exactly (16 would add two dead loads per wave)
    if (spw == 1) return per <= 2 ? 2 : per <= 4 ? 4 : per <= 8 ? 8 : per == 14 ? 14 : 16;
    return per <= 2 ? 2 : per <= 4 ? 4 : 8;
}

// LDS layout of one slice of `cmax` chunks for `rows` A rows and NS strips:
// the A rows, then the weight scales (16-bit group scales, or E8M0 bytes),
// then the zero-point words (WNA16) or the activations' E8M0 words (MX
// activations); each region 1 KB aligned.
struct SkinnyLds {
    int64_t a_off, s_off, z_off, bytes;
};
inline int skinny_arow(Fmt F) {
    return F == Fmt::W4A4_MX ? 64 : (F == Fmt::W4A8_MX || F == Fmt::W4A8_MXA || F == Fmt::W8A8_I8 || F == Fmt::W8A8_F8B) ? 128 : 256;
}
inline SkinnyLds skinny_lds(Fmt F, int64_t rows, int64_t cmax, int NS, int gch, int zb = 8) {
    auto al = [](int64_t b) { return (b + 1023) / 1024 * 1024; };
    int64_t s = 0, z = 0;
    if (F == Fmt::WNA16_F16 || F == Fmt::WNA16_BF16) {
        const int64_t gmax = cmax / gch + 2;
        s = al(NS * gmax * 32);
        z = al(NS * gmax * zb);  // zero-point bytes per strip and group: 8 (UINT4) or 16 (UINT8)
    } else if (mx_mfma(F)) {
        s = al(NS * cmax * 64);
        if (mx_act(F)) z = al(rows * cmax * 4);
    } else if (mxfp4w(F) || nvfp4(F) || mxint4w(F) || mxf8(F) || mxf6(F)) {
        s = al(NS * cmax * (nvfp4(F) ? 128 : 64));
    } else if (F == Fmt::W8A8_F8B) {
        s = al(NS * cmax * 4);
        z = al(((rows + 15) / 16 * 16) * cmax * 4);
    }
    SkinnyLds L;
    L.a_off = 0;
    L.s_off = al(rows * cmax * skinny_arow(F));
    L.z_off = L.s_off + s;
    L.bytes = L.z_off + z;
    return L;
}
inline int64_t skinny_lds_need(Fmt F, int64_t rows, int64_t cmax, int NS, int gch, int zb = 8) {
    return skinny_lds(F, rows, cmax, NS, gch, zb).bytes;
}

constexpr bool skinny_a16(Fmt F) {
    return F == Fmt::WNA16_F16 || F == Fmt::WNA16_BF16 || mxfp4w(F) || nvfp4(F) || mxint4w(F) || w8a16(F) || mxf8(F) ||
           mxf6(F);
}

// The eight-wave schedule with direct A loads: one strip per workgroup, K in
// eighths, no split.  It applies to 16-bit A at M <= 16 where a wave's eighth
// of K fits one register batch with its A fragments.
inline bool skinny_direct_fits(Fmt F, int64_t M, int64_t K) {
    const int64_t nc = K / 128, cpk = (nc + 7) / 8;
    return skinny_a16(F) && M >= 1 && M <= 16 && nc >= 8 && cpk <= 8;
}
inline int skinny_direct_cpw(int64_t cpk) { return cpk <= 2 ? 2 : cpk <= 4 ? 4 : cpk == 7 ? 7 : 8; }

// Dense plan: strips per workgroup grow with M so the A slice is re-read about
// nstrips / NS times; K slices until the grid covers the chip and the slice
// fits in LDS.  mode 0: the library's choice; 1: four waves with the A slice in
// LDS (force_splits K slices, 0 = planned); 2: eight waves with direct A loads.
inline SkinnyPlan plan_skinny(Fmt F, int64_t M, int64_t Np, int64_t K, int G, int force_splits = 0, int mode = 0,
                              int wbits = 4) {
    const int64_t nstrips = Np / 16, nc = K / 128;
    const int gch = G >= 128 ? G / 128 : 1;
    const int zb = wbits > 4 ? 16 : 8;  // zero-point bytes per strip and group
    SkinnyPlan p{};
    p.NW = 4;
    // The formats with the longer decodes (NVFP4, MXINT4, 8-bit weights) at up to
    // 8 rows on a strip per CU or more: eight waves hide it better (N=4096,
    // K=7168, M=1: INT8 9.8 -> 9.0 us, FP8 8.8 -> 8.6, MXINT4 9.3 -> 8.6, NVFP4
    // 10.2 -> 9.7).  UINT4 and MXFP4 measured slower that way at 1..4 rows, and
    // every format at 9..16 rows (more A read from L2 than the split's partials
    // and finalize cost: fp16 UINT4 M=16 11.6 against 11.1 us).
    const bool heavy = nvfp4(F) || mxint4w(F) || w8a16(F) || mxf8(F) || mxf6(F);
    const bool direct = mode == 2 || (mode == 0 && heavy && M <= 8 && nstrips >= 192 && skinny_direct_fits(F, M, K));
    if (direct) {
        p.ok = skinny_direct_fits(F, M, K) && force_splits <= 1;
        p.NW = 8;
        p.NS = p.SPW = p.WS = 1;
        p.MT = 1;
        p.groups_x = nstrips;
        p.splits = 1;
        p.cps = (int)nc;
        p.cpk = (int)cdiv(nc, 8);
        p.CPW = skinny_direct_cpw(p.cpk);
        const SkinnyLds L = skinny_lds(F, 0, nc, 1, gch, zb);  // scales only
        p.a_off = (int)L.a_off;
        p.s_off = (int)L.s_off;
        p.z_off = (int)L.z_off;
        const int64_t red = 7 * 1024;  // seven K-parts' 16 x 16 fp32 tiles
        p.lds_bytes = (int)(L.bytes > red ? L.bytes : red);
        if (p.lds_bytes < 1024) p.lds_bytes = 1024;
        if (p.lds_bytes > kSkinnyLds) p.ok = false;
        return p;
    }
    p.NS = M <= 8 ? 1 : M <= 16 ? 2 : M <= 32 ? 4 : 8;
    // W4A8 at M <= 32: two strips per workgroup keep 224 workgroups at N = 7168
    // and the whole 8-bit A slice in LDS, so no K split (and no finalize pass)
    if (mx_mfma(F) && M <= 32 && skinny_lds_need(F, M, K / 128, 2, 1) <= kSkinnyLds) p.NS = M <= 8 ? 1 : 2;
    while (p.NS > 1 && p.NS > nstrips) p.NS /= 2;
    p.SPW = p.NS <= 4 ? 1 : p.NS / 4;
    p.WS = p.NS / p.SPW;
    const int WK = 4 / p.WS;
    p.groups_x = cdiv(nstrips, p.NS);
    // a K split costs partial tiles and a finalize launch (~3 us): only when the
    // strips alone leave a quarter of the chip idle (or the slice must shrink)
    // 16-bit A at 9..16 rows (two strips per workgroup): two workgroups per CU
    // (four slices at N=4096: 11.2 against 11.9 us with two)
    const bool a16 = skinny_a16(F);
    const int64_t target = a16 && p.NS == 2 ? 512 : 256;
    int64_t S = p.groups_x >= 192 ? 1 : cdiv(target, p.groups_x);
    const int64_t smax = nc / WK > 0 ? nc / WK : 1;
    // weight loads per chunk (two 16-byte halves; or the two planes of 3-bit codes)
    const int nb = wbits == 7 ? 3
                 : (F == Fmt::W8A8_I8 || F == Fmt::W8A8_F8B || w8a16(F) || mxf8(F) || mxf6(F) || wbits == 3 || wbits > 4) ? 2
                                                                                                                     : 1;
    const int64_t cap = p.SPW * 16 * nb < 64 ? 16 : 8;  // largest register batch instantiated
    while (S < smax && (skinny_lds_need(F, M, cdiv(nc, S), p.NS, gch, zb) > kSkinnyLds || cdiv(cdiv(nc, S), WK) > cap)) ++S;
    if (S > smax) S = smax;
    p.ok = true;
    if (force_splits > 0) {  // tuning override: the slice must still fit LDS and one register batch
        S = force_splits;
        if (S > nc || skinny_lds_need(F, M, cdiv(nc, S), p.NS, gch, zb) > kSkinnyLds || cdiv(cdiv(nc, S), WK) > cap) p.ok = false;
    }
    p.splits = (int)(S < 1 ? 1 : S);
    p.cps = (int)cdiv(nc, p.splits);
    p.splits = (int)cdiv(nc, p.cps);  // no empty slice
    p.cpk = (int)cdiv(p.cps, WK);
    const int64_t cmax = p.cps;
    const SkinnyLds L = skinny_lds(F, M, cmax, p.NS, gch, zb);
    p.a_off = (int)L.a_off;
    p.s_off = (int)L.s_off;
    p.z_off = (int)L.z_off;
    p.MT = M <= 16 ? 1 : M <= 32 ? 2 : 4;
    p.CPW = skinny_round_cpw(p.cpk, p.SPW);
    const int64_t need = L.bytes;
    const int64_t red = (int64_t)(WK - 1) * p.WS * p.SPW * p.MT * 1024;  // K-part reduction buffer
    p.lds_bytes = (int)(need > red ? need : red);
    return p;
}

template <Fmt F, int MT, int SPW, int CPW, int NW = 4, int WB = 4>
hipError_t launch_skinny_k(dim3 grid, int lds_bytes, const SkinnyArgs& a, hipStream_t st) {
    if (plan_recorder()) {
        if (NW == 8)
            plan_record("skinny_kernel<%s,%d,%d,%d,direct> grid=%ux%u splits=%d", fmt_name(F), MT, SPW, CPW, grid.x, grid.y, a.splits);
        else if (WB != 4)
            plan_record("skinny_kernel<%s,%d,%d,%d,w%d> grid=%ux%u splits=%d", fmt_name(F), MT, SPW, CPW, WB, grid.x, grid.y,
                        a.splits);
        else
            plan_record("skinny_kernel<%s,%d,%d,%d> grid=%ux%u splits=%d", fmt_name(F), MT, SPW, CPW, grid.x, grid.y, a.splits);
        if (a.splits > 1) plan_workspace((size_t)a.splits * (size_t)a.M * (size_t)a.Np * 4);
        return hipSuccess;
    }
    // allow dynamic LDS beyond the 64 KB default, once per instantiation
    static const hipError_t attr = hipFuncSetAttribute((const void*)skinny_kernel<F, MT, SPW, CPW, NW, WB>,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, kSkinnyLds);
    if (attr != hipSuccess) return attr;
    if (lds_bytes < 1024 || lds_bytes > kSkinnyLds) return hipErrorInvalidValue;
    hipLaunchKernelGGL((skinny_kernel<F, MT, SPW, CPW, NW, WB>), grid, dim3(64 * NW), (size_t)lds_bytes, st, a);
    return hipGetLastError();
}

// eight waves, direct A loads (16-bit A formats only)
template <Fmt F>
hipError_t launch_skinny_direct(int cpw, dim3 grid, int lds_bytes, const SkinnyArgs& a, hipStream_t st) {
    if constexpr (skinny_a16(F)) {
        switch (cpw) {
            case 2: return launch_skinny_k<F, 1, 1, 2, 8>(grid, lds_bytes, a, st);
            case 4: return launch_skinny_k<F, 1, 1, 4, 8>(grid, lds_bytes, a, st);
            case 7: return launch_skinny_k<F, 1, 1, 7, 8>(grid, lds_bytes, a, st);
            case 8: return launch_skinny_k<F, 1, 1, 8, 8>(grid, lds_bytes, a, st);
            default: return hipErrorInvalidValue;
        }
    } else {
        return hipErrorNotSupported;
    }
}

template <Fmt F, int MT, int SPW, int WB = 4>
hipError_t launch_skinny_cpw(int cpw, dim3 grid, int lds_bytes, const SkinnyArgs& a, hipStream_t st) {
    constexpr int LPC = WB == 4 ? FmtTraits<F>::BSTRIP / 1024 : WB == 3 ? 2 : WB < 4 ? 1 : WB == 7 ? 3 : 2;  // loads per chunk
    switch (cpw) {
        case 2: return launch_skinny_k<F, MT, SPW, 2, 4, WB>(grid, lds_bytes, a, st);
        case 4: return launch_skinny_k<F, MT, SPW, 4, 4, WB>(grid, lds_bytes, a, st);
        case 8: return launch_skinny_k<F, MT, SPW, 8, 4, WB>(grid, lds_bytes, a, st);
        case 14:
            if constexpr (SPW == 1) return launch_skinny_k<F, MT, SPW, 14, 4, WB>(grid, lds_bytes, a, st);
            else return hipErrorInvalidValue;
        default:
            if constexpr (SPW * 16 * LPC < 64) return launch_skinny_k<F, MT, SPW, 16, 4, WB>(grid, lds_bytes, a, st);
            else return launch_skinny_k<F, MT, SPW, 8, 4, WB>(grid, lds_bytes, a, st);
    }
}

// Dense launch: the weight stream, then the finalize pass when K is split.
template <Fmt F>
hipError_t launch_skinny_dense(const SkinnyPlan& pl, SkinnyArgs s, hipStream_t st) {
    s.splits = pl.splits;
    s.part_nt = part_nontemporal(pl.splits, s.M, s.Np);
    s.cps = pl.cps;
    s.cpk = pl.cpk;
    s.NS = pl.NS;
    s.WS = pl.WS;
    s.a_off = pl.a_off;
    s.s_off = pl.s_off;
    s.z_off = pl.z_off;
    const dim3 grid((unsigned)pl.groups_x, (unsigned)pl.splits);
    if (pl.cpk > pl.CPW) return hipErrorInvalidValue;  // K-part beyond one register batch (planned out)
    if (pl.NW == 8) return pl.splits == 1 ? launch_skinny_direct<F>(pl.CPW, grid, pl.lds_bytes, s, st) : hipErrorInvalidValue;
    auto by_shape = [&](auto wbc) -> hipError_t {
        constexpr int WB = decltype(wbc)::value;
        if (pl.SPW == 2) return launch_skinny_cpw<F, 4, 2, WB>(pl.CPW, grid, pl.lds_bytes, s, st);
        if (pl.MT == 1) return launch_skinny_cpw<F, 1, 1, WB>(pl.CPW, grid, pl.lds_bytes, s, st);
        if (pl.MT == 2) return launch_skinny_cpw<F, 2, 1, WB>(pl.CPW, grid, pl.lds_bytes, s, st);
        return launch_skinny_cpw<F, 4, 1, WB>(pl.CPW, grid, pl.lds_bytes, s, st);
    };
    hipError_t e;
    if constexpr (F == Fmt::WNA16_F16 || F == Fmt::WNA16_BF16) {
        switch (s.wbits) {
            case 1: e = by_shape(std::integral_constant<int, 1>{}); break;
            case 2: e = by_shape(std::integral_constant<int, 2>{}); break;
            case 3: e = by_shape(std::integral_constant<int, 3>{}); break;
            case 5: e = by_shape(std::integral_constant<int, 5>{}); break;
            case 6: e = by_shape(std::integral_constant<int, 6>{}); break;
            case 7: e = by_shape(std::integral_constant<int, 7>{}); break;
            case 8: e = by_shape(std::integral_constant<int, 8>{}); break;
            default: e = by_shape(std::integral_constant<int, 4>{}); break;
        }
    } else {
        e = by_shape(std::integral_constant<int, 4>{});
    }
    if (e != hipSuccess || pl.splits == 1) return e;
    return launch_finalize<F>(FinalizeArgs{s.part, s.D, s.a_scale, (const float*)s.S, s.s2, s.M, s.N, s.Np, s.splits, s.raw_i32,
                                           s.part_nt},
                              st);
}


// Low-bit planes -> the 4-bit W4A16 layout (one 16-byte word set per strip,
// chunk and lane), for the tiled kernels.
template <int WB>
__global__ __launch_bounds__(256) void widen_lowbit_kernel(const char* __restrict__ planes, v4u* __restrict__ out,
                                                           int64_t slots, uint32_t smask) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // slot = (strip * chunks + chunk) * 64 + lane
    if (i >= slots) return;
    const size_t plane2 = WB >= 2 ? (size_t)slots * 8 : 0;
    v4u x = v4u{0u, 0u, 0u, 0u};
    if constexpr (WB >= 2) {
        const v2u a = __builtin_nontemporal_load((const v2u*)(planes + i * 8));
        x[0] = a[0];
        x[1] = a[1];
    }
    if constexpr (WB != 2) x[2] = __builtin_nontemporal_load((const uint32_t*)(planes + plane2 + i * 4));
    v4u o;
#pragma unroll
    for (int t = 0; t < 4; ++t) o[t] = widen_lowbit_word<WB>(x, t, smask);
    out[i] = o;
}

inline hipError_t launch_widen_lowbit(const void* planes, void* out, int wbits, bool is_signed, int64_t Np, int64_t K,
                                      hipStream_t st) {
    const int64_t slots = (Np / 16) * (K / 128) * 64, blocks = (slots + 255) / 256;
    if (plan_recorder()) {
        plan_record("widen_lowbit_kernel<%d> grid=%lld", wbits, (long long)blocks);
        return hipSuccess;
    }
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    const uint32_t smask = is_signed ? 0xFFFFFFFFu : 0u;
    const dim3 g((unsigned)blocks), b(256);
    switch (wbits) {
        case 1: hipLaunchKernelGGL(widen_lowbit_kernel<1>, g, b, 0, st, (const char*)planes, (v4u*)out, slots, smask); break;
        case 2: hipLaunchKernelGGL(widen_lowbit_kernel<2>, g, b, 0, st, (const char*)planes, (v4u*)out, slots, smask); break;
        case 3: hipLaunchKernelGGL(widen_lowbit_kernel<3>, g, b, 0, st, (const char*)planes, (v4u*)out, slots, smask); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// 5- to 8-bit WnA16 codes -> one byte per code, u = q (unsigned) or q + 128
// (signed), in the INT8 weight-only layout, for the tiled kernels (which
// subtract the zero-point, 128 for signed codes, and apply the group scales to
// their fp32 partials): per strip and chunk two 1 KB halves of 64 lanes x 16 B,
// half h of lane l holding K = 32 (l >> 4) + 16 h + 0..15.  One thread per lane slot.
template <int WB>
__global__ __launch_bounds__(256) void widen_wide_kernel(const char* __restrict__ planes, v4u* __restrict__ out,
                                                         int64_t slots, bool sgn) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // slot = (strip * chunks + chunk) * 64 + lane
    if (i >= slots) return;
    const v4u wl = __builtin_nontemporal_load((const v4u*)planes + i);
    const char* hp = planes + (size_t)slots * 16;
    v4u wh = v4u{0u, 0u, 0u, 0u};
    if constexpr (WB == 8) {
        wh = __builtin_nontemporal_load((const v4u*)hp + i);
    } else {
        if constexpr (WB == 6 || WB == 7) {
            const v2u a = __builtin_nontemporal_load((const v2u*)hp + i);
            wh[0] = a[0];
            wh[1] = a[1];
        }
        if constexpr (WB != 6) wh[2] = __builtin_nontemporal_load((const uint32_t*)(hp + (WB == 7 ? (size_t)slots * 8 : 0)) + i);
    }
    // signed codes: the two's-complement code plus 2^(WB-1) (top bit flipped) is
    // the offset-binary value; plus 128 - 2^(WB-1) more makes q + 128
    const uint32_t add = sgn ? 128u - (1u << (WB - 1)) : 0u;
    if (sgn) {
        const uint32_t m4 = WB == 8 ? 0x88888888u : 0u, m2 = WB == 6 ? 0xAAAAAAAAu : m4;
        const uint32_t m1 = WB == 5 || WB == 7 ? 0xFFFFFFFFu : m4;
        wh[0] ^= m2;
        wh[1] ^= m2;
        wh[2] ^= m1;
        wh[3] ^= m4;
    }
    v4u o[2];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        // the code values 0..255 as exact fp16 integers (1024 + code - 1024)
        const Frag8 d = deq_wide<WB, false>(wl, wh, t, 0xE400E400u);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            uint32_t w = 0;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const uint32_t x = d.u[2 * h + e];
                const uint32_t lo = (uint32_t)bits16_to_f32<false>((uint16_t)(x & 0xFFFFu)) + add;
                const uint32_t hi = (uint32_t)bits16_to_f32<false>((uint16_t)(x >> 16)) + add;
                w |= (lo | (hi << 8)) << (16 * e);
            }
            o[t >> 1][2 * (t & 1) + h] = w;
        }
    }
    v4u* dst = out + (i >> 6) * 128 + (i & 63);
    dst[0] = o[0];
    dst[64] = o[1];
}

inline hipError_t launch_widen_wide(const void* planes, void* out, int wbits, bool is_signed, int64_t Np, int64_t K,
                                    hipStream_t st) {
    const int64_t slots = (Np / 16) * (K / 128) * 64, blocks = (slots + 255) / 256;
    if (plan_recorder()) {
        plan_record("widen_wide_kernel<%d> grid=%lld", wbits, (long long)blocks);
        return hipSuccess;
    }
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    const dim3 g((unsigned)blocks), b(256);
    const char* w = (const char*)planes;
    v4u* o = (v4u*)out;
    switch (wbits) {
        case 5: hipLaunchKernelGGL(widen_wide_kernel<5>, g, b, 0, st, w, o, slots, is_signed); break;
        case 6: hipLaunchKernelGGL(widen_wide_kernel<6>, g, b, 0, st, w, o, slots, is_signed); break;
        case 7: hipLaunchKernelGGL(widen_wide_kernel<7>, g, b, 0, st, w, o, slots, is_signed); break;
        case 8: hipLaunchKernelGGL(widen_wide_kernel<8>, g, b, 0, st, w, o, slots, is_signed); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// MXFP6 planes -> MXFP8 codes (exact: every E2M3 and E3M2 value is an E4M3
// value) in the 8-bit weight-only layout, for the tiled kernels: one thread per
// lane and chunk, 24 bytes in, two 16-byte halves out; the packed FP6 convert
// turns the 32 codes into bf16, the fp8 converts those into E4M3 (no rounding
// happens: each value is representable).
template <bool E3M2>
__global__ __launch_bounds__(256) void widen_fp6_kernel(const char* __restrict__ planes, v4u* __restrict__ out,
                                                        int64_t slots) {
    typedef short v2s __attribute__((ext_vector_type(2)));
    typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // slot = (strip * nc + chunk) * 64 + lane
    if (i >= slots) return;
    const v4u a = __builtin_nontemporal_load((const v4u*)(planes + i * 16));
    const v2u b = __builtin_nontemporal_load((const v2u*)(planes + (size_t)slots * 16 + i * 8));
    const v6u x6 = v6u{a[0], a[1], a[2], a[3], b[0], b[1]};
    v16u y;
    if constexpr (E3M2) y = __builtin_bit_cast(v16u, __builtin_amdgcn_cvt_scalef32_pk32_bf16_bf6(x6, 1.0f));
    else y = __builtin_bit_cast(v16u, __builtin_amdgcn_cvt_scalef32_pk32_bf16_fp6(x6, 1.0f));
    uint32_t o[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {  // bf16 pairs 2q, 2q+1 (codes 4q .. 4q+3) -> one word of E4M3 bytes
        const uint32_t lo = y[2 * q], hi = y[2 * q + 1];
        v2s w = v2s{0, 0};
        w = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(w, __builtin_bit_cast(v2bf, lo), 1.0f, false);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(w, __builtin_bit_cast(v2bf, hi), 1.0f, true);
        o[q] = __builtin_bit_cast(uint32_t, w);
    }
    const int64_t sc = i >> 6, lane = i & 63;  // (strip * nc + chunk), lane
    out[(sc * 2) * 64 + lane] = v4u{o[0], o[1], o[2], o[3]};
    out[(sc * 2 + 1) * 64 + lane] = v4u{o[4], o[5], o[6], o[7]};
}

inline hipError_t launch_widen_fp6(const void* planes, void* out, bool e3m2, int64_t Np, int64_t K, hipStream_t st) {
    const int64_t slots = (Np / 16) * (K / 128) * 64, blocks = (slots + 255) / 256;
    if (plan_recorder()) {
        plan_record("widen_fp6_kernel<%s> grid=%lld", e3m2 ? "e3m2" : "e2m3", (long long)blocks);
        return hipSuccess;
    }
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    const dim3 g((unsigned)blocks), b(256);
    if (e3m2) hipLaunchKernelGGL(widen_fp6_kernel<true>, g, b, 0, st, (const char*)planes, (v4u*)out, slots);
    else hipLaunchKernelGGL(widen_fp6_kernel<false>, g, b, 0, st, (const char*)planes, (v4u*)out, slots);
    return hipGetLastError();
}

// Dense dispatch shared by the format launchers: the small-M weight stream up
// to kSkinnyMaxM rows, the tiled kernels above; a tuning override (TunePath and
// K split) or batch-invariant mode (tiled kernels without K split at every M:
// every tile shape of a format accumulates an output in the same order, so a
// row's result does not depend on M) changes the choice.
template <Fmt F>
hipError_t dense_dispatch(const DenseArgs& a, SkinnyArgs s, TileArgs p, int G) {
    const bool tile_forced = a.tune_path >= TUNE_T128 && a.tune_path <= TUNE_W256;
    const bool stream_forced = a.tune_path == TUNE_STREAM || a.tune_path == TUNE_STREAM8;
    if (!a.invariant && !tile_forced && (stream_forced || a.M <= skinny_max_m(F))) {
        if (a.M > kSkinnyMaxM) return hipErrorNotSupported;
        const int mode = a.tune_path == TUNE_STREAM8 ? 2 : a.tune_path == TUNE_STREAM ? 1 : 0;
        if (mode == 2 && a.wbits != 4) return hipErrorNotSupported;  // the direct stream reads 4-bit words only
        s.wbits = a.wbits;
        const SkinnyPlan pl = plan_skinny(F, a.M, a.Np, a.K, G, a.tune_splits, mode, a.wbits);
        if (!pl.ok) return hipErrorNotSupported;
        return launch_skinny_dense<F>(pl, s, a.stream);
    }
    TilePlan pl = plan_tile(a.M, a.Np, a.K, has_big_tile(F), has_wide256_tile(F), has_wide_tile(F), wide256_min_tiles(F));
    if (tile_forced) {
        pl.forced = a.tune_path;
        pl.splits = a.tune_splits;
        if (pl.splits > a.K / 128) return hipErrorNotSupported;
    }
    if (a.invariant) p.max_splits = 1;
    if constexpr (mxf6(F)) {
        // MXFP6 on the tiles: the planes widen to MXFP8 codes (8-bit weight-only
        // layout) at the front of the workspace, the MXFP8 tiles read them with the
        // E8M0 scales as they are, partial tiles follow
        const size_t wide = (size_t)(a.Np / 16) * (size_t)(a.K / 128) * 2048, off = (wide + 255) & ~(size_t)255;
        hipError_t e = launch_widen_fp6(a.w, a.ws, mxf6e3(F), a.Np, a.K, a.stream);
        if (e != hipSuccess) return e;
        plan_workspace(wide);
        plan_workspace_base(off);
        p.W = a.ws;
        p.part = (char*)a.ws + off;
        e = launch_dense_plan<f16_operand(F) ? Fmt::MXF8_F16 : Fmt::MXF8_BF16>(pl, p, a.stream);
        plan_workspace_base(0);
        return e;
    } else {
    if constexpr (F == Fmt::WNA16_F16 || F == Fmt::WNA16_BF16) {
        if (a.wbits < 4) {
            // low-bit widths on the tiles: the planes widen to the 4-bit layout at the
            // front of the workspace, the tiles read that, partial tiles follow it
            const size_t wide = (size_t)(a.Np / 16) * (size_t)(a.K / 128) * 1024, off = (wide + 255) & ~(size_t)255;
            hipError_t e = launch_widen_lowbit(a.w, a.ws, a.wbits, a.z == nullptr, a.Np, a.K, a.stream);
            if (e != hipSuccess) return e;
            plan_workspace(wide);
            plan_workspace_base(off);
            p.W = a.ws;
            p.part = (char*)a.ws + off;
            e = launch_dense_plan<F>(pl, p, a.stream);
            plan_workspace_base(0);
            return e;
        }
        if (a.wbits > 4) {
            // 5-8-bit widths on the tiles: the codes widen to one byte each in the
            // INT8 weight-only layout at the front of the workspace, the INT8
            // weight-only tiles read them with the group scales and UINT8
            // zero-points as they are, partial tiles follow
            constexpr Fmt W = F == Fmt::WNA16_BF16 ? Fmt::W8G_BF16 : Fmt::W8G_F16;
            const size_t wide = (size_t)(a.Np / 16) * (size_t)(a.K / 128) * 2048, off = (wide + 255) & ~(size_t)255;
            TilePlan wp = plan_tile(a.M, a.Np, a.K, has_big_tile(W), has_wide256_tile(W), has_wide_tile(W), wide256_min_tiles(W));
            wp.forced = pl.forced;
            wp.splits = tile_forced ? pl.splits : wp.splits;
            hipError_t e = launch_widen_wide(a.w, a.ws, a.wbits, a.z == nullptr, a.Np, a.K, a.stream);
            if (e != hipSuccess) return e;
            plan_workspace(wide);
            plan_workspace_base(off);
            p.W = a.ws;
            p.part = (char*)a.ws + off;
            e = launch_dense_plan<W>(wp, p, a.stream);
            plan_workspace_base(0);
            return e;
        }
    }
    return launch_dense_plan<F>(pl, p, a.stream);
    }
}

}  // namespace hq
