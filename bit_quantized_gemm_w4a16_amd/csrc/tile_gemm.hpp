// LDS-tiled MFMA GEMM template for gfx950, shared by every weight format.
//
// One workgroup of WM x WN waves computes a BM x BN tile of D (optionally
// over one K slice of a split-K launch).  Each K step covers 128 input
// features: the A tile (BM rows x 128 K, 16- or 8-bit), the packed weight tile
// (BN/16 strips x one step) and the step's scales.  Two pipelines:
//   PD = 0      16-byte direct HBM->LDS loads (buffer_load ... lds) of step s+1
//               into the other of two LDS stages while step s computes; no
//               staging registers (the 4-bit formats);
//   PD = 1, 2   16-byte loads into PD register sets, written to the other LDS
//               stage one step ahead (INT8, whose tiles are twice as large);
//   PD = 3      as PD = 0 with two A stages but ONE weight stage: every wave
//               copies its weight fragments of the step into registers first,
//               so after one barrier the weight stage takes the next step's
//               tile.  That leaves room for 256-row x 256-column tiles of
//               8 waves of 256 x 32, whose dequantised weight fragment feeds
//               16 MFMAs (8 in a 128-row wave).
// The scale block of a step always travels through registers into an LDS
// array of its own (see dma below).
// A rows are XOR-swizzled in LDS with a row permutation measured to be
// bank-conflict free on gfx950 for the fragment reads below.  The packed
// weight chunk of a strip is, lane for lane, the MFMA B fragment, so it is
// copied unchanged.  Workgroups are remapped so that consecutive ids land on
// one XCD's L2 and tiles sharing A rows run close together.
//
// Formats (the decode runs in registers between the LDS read and the MFMA):
//   WNA16_F16   fp16 A; INT4/UINT4 -> (q - z) * s folded into the fp16 operand
//   WNA16_BF16  bf16 A; operand 128 + u (exact), the -(128 + z) offset via a
//               row-sum MFMA, group scale applied to the fp32 accumulator
//   W4A8_MX     fp8-e4m3 A x e2m1 B on the scaled MFMA (E8M0 B scale per
//               32 K), per-token scale in the epilogue
//   W4A8_MXA    fp8-e4m3 A with its own E8M0 scale per 32 K (MXFP8) x e2m1 B,
//               both scales fed to the scaled MFMA (lane l's A scale applies
//               to row l & 15 and K block l >> 4 of the instruction)
//   W4A4_MX     fp4-e2m1 A with E8M0 per 32 K (MXFP4) x e2m1 B on the same
//               scaled MFMA (A lane l holds row l & 15, K = 32 (l >> 4) + i)
//   W8A8_F8B    fp8-e4m3 A (fp32 scale per row and 128-K block) x fp8-e4m3 B
//               (fp32 scale per 128 x 128 block, INT8 packing): each 128-K
//               step's fp8 MFMA partial is scaled by sa[row] * sw and added
//               to the fp32 accumulator
//   W8A8_I8     int8 x int8 -> int32 (exact), per-token x per-channel epilogue
//   MOE_MX      bf16 A x e2m1 B converted to bf16 with the E8M0 scale (exact)
//   MXFP4_BF16  the same decode for dense layers (FP4 WnA16)
//   NVFP4_BF16  bf16 A x e2m1 B with an E4M3 scale per 16 K (e2m1 x e4m3 has
//               at most 5 significant bits: the product is exact in bf16) and
//               the per-tensor fp32 second-level scale in the epilogue
//   MXINT4_BF16 bf16 A x two's-complement INT4 B with E8M0 per 32 K (MXINT4):
//               q x 2^(E-127) in fp32, rounded to bf16 (exact: 3 significant bits)
//   W8A16_*     fp16 / bf16 A x INT8 B (a lane's 32 consecutive K per chunk in two
//               16-byte halves) decoded to exact 16-bit operands; per-channel fp32
//               scale in the epilogue
//   F8W_*       the same with E4M3 weight codes (FP8 weight-only), converted to
//               the 16-bit operand type by the scaled converts (exact)
#pragma once

#include <type_traits>

#include "hq_device.hpp"
#include "hq_internal.h"

namespace hq {

enum class Fmt { WNA16_F16, WNA16_BF16, W4A8_MX, W8A8_I8, MOE_MX, W4A8_MXA, W4A4_MX, W8A8_F8B, MXFP4_BF16, NVFP4_BF16,
                 MXINT4_BF16, W8A16_F16, W8A16_BF16, F8W_F16, F8W_BF16, MXF8_BF16, MXF6E2_BF16, MXF6E3_BF16,
                 MXFP4_F16, NVFP4_F16, MXINT4_F16, MXF8_F16, MXF6E2_F16, MXF6E3_F16, W8G_F16, W8G_BF16 };

constexpr const char* fmt_name(Fmt F) {
    return F == Fmt::WNA16_F16 ? "WNA16_F16" : F == Fmt::WNA16_BF16 ? "WNA16_BF16" : F == Fmt::W4A8_MX ? "W4A8_MX"
         : F == Fmt::W8A8_I8 ? "W8A8_I8" : F == Fmt::MOE_MX ? "MOE_MX" : F == Fmt::W4A8_MXA ? "W4A8_MXA"
         : F == Fmt::W4A4_MX ? "W4A4_MX" : F == Fmt::W8A8_F8B ? "W8A8_F8B" : F == Fmt::MXFP4_BF16 ? "MXFP4_BF16"
         : F == Fmt::NVFP4_BF16 ? "NVFP4_BF16" : F == Fmt::MXINT4_BF16 ? "MXINT4_BF16"
         : F == Fmt::W8A16_F16 ? "W8A16_F16" : F == Fmt::W8A16_BF16 ? "W8A16_BF16" : F == Fmt::F8W_F16 ? "F8W_F16"
         : F == Fmt::F8W_BF16 ? "F8W_BF16" : F == Fmt::MXF8_BF16 ? "MXF8_BF16" : F == Fmt::MXF6E2_BF16 ? "MXF6E2_BF16"
         : F == Fmt::MXF6E3_BF16 ? "MXF6E3_BF16" : F == Fmt::MXFP4_F16 ? "MXFP4_F16" : F == Fmt::NVFP4_F16 ? "NVFP4_F16"
         : F == Fmt::MXINT4_F16 ? "MXINT4_F16" : F == Fmt::MXF8_F16 ? "MXF8_F16" : F == Fmt::MXF6E2_F16 ? "MXF6E2_F16"
         : F == Fmt::MXF6E3_F16 ? "MXF6E3_F16" : F == Fmt::W8G_F16 ? "W8G_F16" : "W8G_BF16";
}
// Formats whose activations carry OCP MX scales (E8M0 per 32 K, [rows][K/32]).
constexpr bool mx_act(Fmt F) { return F == Fmt::W4A8_MXA || F == Fmt::W4A4_MX; }
// fp8 x fp4 or fp4 x fp4 on the scaled MFMA (B always e2m1 + E8M0).
constexpr bool mx_mfma(Fmt F) { return F == Fmt::W4A8_MX || mx_act(F); }

// AROW: bytes of one activation row per 128-K step; BSTRIP: packed weight
// bytes per 16-column strip and step.
template <Fmt F> struct FmtTraits;
template <> struct FmtTraits<Fmt::WNA16_F16> { static constexpr int AROW = 256, BSTRIP = 1024; using Acc = v4f; };
template <> struct FmtTraits<Fmt::WNA16_BF16> { static constexpr int AROW = 256, BSTRIP = 1024; using Acc = v4f; };
template <> struct FmtTraits<Fmt::W4A8_MX> { static constexpr int AROW = 128, BSTRIP = 1024; using Acc = v4f; };
template <> struct FmtTraits<Fmt::W8A8_I8> { static constexpr int AROW = 128, BSTRIP = 2048; using Acc = v4i; };
template <> struct FmtTraits<Fmt::MOE_MX> { static constexpr int AROW = 256, BSTRIP = 1024; using Acc = v4f; };
template <> struct FmtTraits<Fmt::W4A8_MXA> { static constexpr int AROW = 128, BSTRIP = 1024; using Acc = v4f; };
template <> struct FmtTraits<Fmt::W4A4_MX> { static constexpr int AROW = 64, BSTRIP = 1024; using Acc = v4f; };
template <> struct FmtTraits<Fmt::W8A8_F8B> { static constexpr int AROW = 128, BSTRIP = 2048; using Acc = v4f; };
template <> struct FmtTraits<Fmt::MXFP4_BF16> { static constexpr int AROW = 256, BSTRIP = 1024; using Acc = v4f; };
template <> struct FmtTraits<Fmt::NVFP4_BF16> { static constexpr int AROW = 256, BSTRIP = 1024; using Acc = v4f; };
template <> struct FmtTraits<Fmt::MXINT4_BF16> { static constexpr int AROW = 256, BSTRIP = 1024; using Acc = v4f; };
// INT8 weight-only: a lane's 32 consecutive K of its column per 128-K chunk, as two 16-byte halves
template <> struct FmtTraits<Fmt::W8A16_F16> { static constexpr int AROW = 256, BSTRIP = 2048; using Acc = v4f; };
template <> struct FmtTraits<Fmt::W8A16_BF16> { static constexpr int AROW = 256, BSTRIP = 2048; using Acc = v4f; };
template <> struct FmtTraits<Fmt::F8W_F16> { static constexpr int AROW = 256, BSTRIP = 2048; using Acc = v4f; };
template <> struct FmtTraits<Fmt::F8W_BF16> { static constexpr int AROW = 256, BSTRIP = 2048; using Acc = v4f; };
// MXFP8 weight-only: E4M3 codes in the INT8 weight-only layout, E8M0 per lane and chunk
template <> struct FmtTraits<Fmt::MXF8_BF16> { static constexpr int AROW = 256, BSTRIP = 2048; using Acc = v4f; };
// MXFP6 weight-only (the small-M stream; the tiles read it widened to MXFP8): a
// 16-byte and an 8-byte plane per lane and chunk, two loads
template <> struct FmtTraits<Fmt::MXF6E2_BF16> { static constexpr int AROW = 256, BSTRIP = 2048; using Acc = v4f; };
template <> struct FmtTraits<Fmt::MXF6E3_BF16> { static constexpr int AROW = 256, BSTRIP = 2048; using Acc = v4f; };
// the same weight formats with fp16 activations (fp16 operands and output)
template <> struct FmtTraits<Fmt::MXFP4_F16> { static constexpr int AROW = 256, BSTRIP = 1024; using Acc = v4f; };
template <> struct FmtTraits<Fmt::NVFP4_F16> { static constexpr int AROW = 256, BSTRIP = 1024; using Acc = v4f; };
template <> struct FmtTraits<Fmt::MXINT4_F16> { static constexpr int AROW = 256, BSTRIP = 1024; using Acc = v4f; };
template <> struct FmtTraits<Fmt::MXF8_F16> { static constexpr int AROW = 256, BSTRIP = 2048; using Acc = v4f; };
template <> struct FmtTraits<Fmt::MXF6E2_F16> { static constexpr int AROW = 256, BSTRIP = 2048; using Acc = v4f; };
template <> struct FmtTraits<Fmt::MXF6E3_F16> { static constexpr int AROW = 256, BSTRIP = 2048; using Acc = v4f; };
// 5- to 8-bit WnA16 codes rewritten as bytes u (q, or q + 128 for signed codes)
// in the INT8 weight-only layout; the group scales in the W4A16 layout and, for
// unsigned codes, the UINT8 zero-points [Np/16][K/group][16]
template <> struct FmtTraits<Fmt::W8G_F16> { static constexpr int AROW = 256, BSTRIP = 2048; using Acc = v4f; };
template <> struct FmtTraits<Fmt::W8G_BF16> { static constexpr int AROW = 256, BSTRIP = 2048; using Acc = v4f; };
// 8-bit weight-only formats: INT8 or FP8 (E4M3) codes in the same layout, per-channel fp32 scale
constexpr bool f8w(Fmt F) { return F == Fmt::F8W_F16 || F == Fmt::F8W_BF16; }
constexpr bool w8a16(Fmt F) { return F == Fmt::W8A16_F16 || F == Fmt::W8A16_BF16 || f8w(F); }
constexpr bool w8bf(Fmt F) { return F == Fmt::W8A16_BF16 || F == Fmt::F8W_BF16; }
// MX-scaled float weights with bf16 activations: E4M3 (MXFP8), E2M3 / E3M2 (MXFP6)
constexpr bool mxf8(Fmt F) { return F == Fmt::MXF8_BF16 || F == Fmt::MXF8_F16; }
constexpr bool mxf6e3(Fmt F) { return F == Fmt::MXF6E3_BF16 || F == Fmt::MXF6E3_F16; }
constexpr bool mxf6(Fmt F) { return F == Fmt::MXF6E2_BF16 || F == Fmt::MXF6E2_F16 || mxf6e3(F); }
// FP4 / INT4 weight-only with a per-lane byte scale, bf16 or fp16 activations
constexpr bool nvfp4(Fmt F) { return F == Fmt::NVFP4_BF16 || F == Fmt::NVFP4_F16; }
constexpr bool mxfp4w(Fmt F) { return F == Fmt::MXFP4_BF16 || F == Fmt::MXFP4_F16; }
constexpr bool mxint4w(Fmt F) { return F == Fmt::MXINT4_BF16 || F == Fmt::MXINT4_F16; }
// the weight-only formats of the scaled converts taken with fp16 activations (fp16
// operands, fp16 MFMA and output; the others of these families are bf16)
constexpr bool f16_operand(Fmt F) {
    return F == Fmt::MXFP4_F16 || F == Fmt::NVFP4_F16 || F == Fmt::MXINT4_F16 || F == Fmt::MXF8_F16 ||
           F == Fmt::MXF6E2_F16 || F == Fmt::MXF6E3_F16 || F == Fmt::W8G_F16;
}
// byte codes with group scales and zero-points (group scales on the fp32 partials)
constexpr bool w8g(Fmt F) { return F == Fmt::W8G_F16 || F == Fmt::W8G_BF16; }
// 8-bit weight codes in the INT8 weight-only layout (two 16-byte halves per lane and chunk)
constexpr bool w8load(Fmt F) { return w8a16(F) || mxf8(F) || w8g(F); }
// e2m1 weights converted to bf16 operands with a per-lane scale (bf16 MFMA)
constexpr bool fp4w(Fmt F) { return F == Fmt::MOE_MX || mxfp4w(F) || nvfp4(F) || mxint4w(F); }

// Work description of one launch.  Dense launches leave the MoE fields null.
struct TileArgs {
    const void* A;          // activations, row-major [rows][K]
    const float* a_scale;   // per-token fp32 (W4A8 / W8A8), indexed by A row
    const uint8_t* a_e8;    // MX activation scales, E8M0 [rows][K/32] (W4A8_MXA / W4A4_MX)
    const float* a_blk;     // fp32 activation scales per row and 128-K block [rows][K/128] (W8A8_F8B)
    const float* s2;        // second-level weight scale, fp32 [1] per tensor (NVFP4_BF16)
    const void* W;          // packed weights (expert 0)
    const void* S;          // packed scales (expert 0)
    const void* Z;          // packed zero-points (WNA16 + UINT4)
    void* D;                // output, row-major [rows][N]
    void* part;             // split-K partial tiles [splits][M][Np] (fp32 / int32), or null
    int64_t w_estride, s_estride;  // bytes between experts' packed W / scales
    int M, N, K, Np;
    int a_rows;             // rows of A (bounds the buffer loads; A bytes < 2^32)
    int ngroups, gsteps;    // WNA16: K / G and G / 128
    int tiles_m, tiles_n, splits;
    int max_splits;         // upper bound on splits (0: none; 1 in batch-invariant mode)
    int raw_i32;            // W8A8: store int32 accumulators
    int part_nt;            // partial tiles stored non-temporally (set by the launcher)
    // MoE (tiles_m is an upper bound; the real count is *ntiles)
    const int* tile_info;   // per m-tile: expert, first sorted row, row count
    const int* ntiles;      // device count of valid m-tiles
    const int* sorted;      // sorted pair ids (Indexed) or null (Grouped)
    int top_k;
};

// A-tile swizzle: the 16-byte unit u of row r is stored at u ^ swz(r).  Rows
// of 4 units (fp4 A, 64 bytes) need none: a wave's fragment read covers 1 KB
// of consecutive bytes.
// Split-K partial tiles of 4..24 MB are stored and re-read non-temporally.
// Measured on fp16 W4A16 at N=4096, K=7168 (graph replays, cold weights):
// M = 64 (8 slices, 8.4 MB) 21.2 -> 19.0 us, M = 128 (8 slices, 16.8 MB)
// 26.6 -> 21.4 us, W4A8 M = 64 / 128 (7.3 MB) 16.3 / 19.8 -> 14.8 / 18.4 us;
// smaller sets gain nothing (INT8 at M = 16, 2.4 MB: 30.4 -> 31.8 us) and
// larger ones lose (33.5 MB at M = 512: 44.4 -> 46.6 us).
inline int part_nontemporal(int64_t splits, int64_t M, int64_t Np) {
    const int64_t bytes = splits * M * Np * 4;
    return splits > 1 && bytes >= (int64_t)4 << 20 && bytes <= (int64_t)24 << 20;
}
// The non-temporal path uses buffer stores / loads with the NT bit (a plain
// access of the same address in the other branch would be merged with it and
// the hint lost).  rP covers the partial tiles when nt is set (they are then
// under 24 MB).
// The 32 bits of an fp32 / int32 accumulator element.  The element is taken
// by value: a bit cast of the vector element expression itself read element 0
// of the vector (every row of a partial tile came out as row 0).
template <typename T>
__device__ __forceinline__ uint32_t bits32(T v) {
    static_assert(sizeof(T) == 4, "32-bit element");
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ rsrc_t part_rsrc(void* part, int nt, int64_t splits, int64_t M, int64_t Np) {
    return make_rsrc(part, nt ? (uint32_t)(splits * M * Np * 4) : 0u);
}

__device__ __forceinline__ int swz(int row, int units) {
    return units == 16 ? (((row & 3) << 2) | ((row >> 2) & 3)) : units == 8 ? ((row >> 1) & 7) : 0;
}

// A value the compiler keeps in a VGPR and cannot fold (an empty asm: no
// instruction is emitted).
__device__ __forceinline__ uint32_t opaque_vgpr(uint32_t v) {
    asm("" : "+v"(v));
    return v;
}
// (a & m) | c as one v_and_or_b32 (or v_bitop3_b32): with the two constants
// opaque VGPR values the compiler selects the three-operand form (a gfx9 VOP3
// instruction takes no literal, so with literals it would emit an AND and an
// OR) and, emitting the instruction itself, keeps its MFMA hazard waits.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
    return (a & opaque_vgpr(m)) | opaque_vgpr(c);
}

// fp16 (q - z) * s for eight codes of one pair-ordered word.  A nibble in bits
// 0-3 of a half under exponent 0x6400 reads 1024 + u; a nibble in bits 4-7
// under 0x5400 reads 64 + u (fp16 has 10 mantissa bits), so one shift serves
// the upper two pairs.  nb_lo = -(1024 + z), nb_hi = -(64 + z) in both halves;
// both differences are exact, one rounding comes from the scale.
__device__ __forceinline__ Frag8 deq4_f16_scaled(uint32_t w, uint32_t nb_lo, uint32_t nb_hi, uint32_t s2) {
    const uint32_t w8 = w >> 8;
    const v2h lo = __builtin_bit_cast(v2h, nb_lo), hi = __builtin_bit_cast(v2h, nb_hi), sc = __builtin_bit_cast(v2h, s2);
    Frag8 f;
    f.u[0] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(v2h, and_or(w, 0x000F000Fu, 0x64006400u)) + lo) * sc);
    f.u[1] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(v2h, and_or(w, 0x00F000F0u, 0x54005400u)) + hi) * sc);
    f.u[2] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(v2h, and_or(w8, 0x000F000Fu, 0x64006400u)) + lo) * sc);
    f.u[3] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(v2h, and_or(w8, 0x00F000F0u, 0x54005400u)) + hi) * sc);
    return f;
}

// fp16 u - z (exact) for eight codes of one pair-ordered word: the unpack of
// deq4_f16_scaled without the scale (9 VALU per 8 codes).
__device__ __forceinline__ Frag8 deq4_f16_exact(uint32_t w, uint32_t nb_lo, uint32_t nb_hi) {
    const uint32_t w8 = w >> 8;
    const v2h lo = __builtin_bit_cast(v2h, nb_lo), hi = __builtin_bit_cast(v2h, nb_hi);
    Frag8 f;
    f.u[0] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, and_or(w, 0x000F000Fu, 0x64006400u)) + lo);
    f.u[1] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, and_or(w, 0x00F000F0u, 0x54005400u)) + hi);
    f.u[2] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, and_or(w8, 0x000F000Fu, 0x64006400u)) + lo);
    f.u[3] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, and_or(w8, 0x00F000F0u, 0x54005400u)) + hi);
    return f;
}

// Low-bit weight codes (widths 1-3) of one lane and 128-K chunk, as loaded:
// r[0..1] = the 2-bit plane, r[2] = the 1-bit plane.  Code j (0..7) of K
// sub-step t (0..3) keeps its low two bits at bit 16*(j&1) + 8*(t&1) + 2*(j>>1)
// of r[t>>1], and its only bit (width 1) or third bit (width 3) at bit
// 16*(j&1) + 4*t + (j>>1) of r[2]: the codes 2s and 2s+1 of a sub-step sit at
// the same offset of the two 16-bit halves, so one and-or lifts the pair.
//
// Widening to the 4-bit pair-order word of sub-step t (nibble p = code
// {0,2,4,6,1,3,5,7}[p]; signed codes, smask all ones, sign-extended to 4-bit
// two's complement, unsigned ones, smask 0, kept), for the tiled kernels.
__device__ __forceinline__ uint32_t spread2x4(uint32_t v) {  // 4 two-bit fields per half -> nibbles
    v &= 0x00FF00FFu;
    v = (v | (v << 4)) & 0x0F0F0F0Fu;
    return (v | (v << 2)) & 0x33333333u;
}
__device__ __forceinline__ uint32_t spread1x4(uint32_t v) {  // 4 bits per half -> bit 0 of nibbles
    v &= 0x000F000Fu;
    v = (v | (v << 6)) & 0x03030303u;
    return (v | (v << 3)) & 0x11111111u;
}
template <int WB>
__device__ __forceinline__ uint32_t widen_lowbit_word(const v4u& r, int t, uint32_t smask) {
    uint32_t y;
    if constexpr (WB == 1) {
        y = spread1x4(r[2] >> (4 * t));
        y |= ((y << 1) | (y << 2) | (y << 3)) & smask;  // -1 -> 0xF
    } else if constexpr (WB == 2) {
        y = spread2x4(r[t >> 1] >> (8 * (t & 1)));
        const uint32_t sg = y & 0x22222222u;
        y |= ((sg << 1) | (sg << 2)) & smask;
    } else {
        y = spread2x4(r[t >> 1] >> (8 * (t & 1))) | (spread1x4(r[2] >> (4 * t)) << 2);
        y |= ((y & 0x44444444u) << 1) & smask;
    }
    return y;
}

// Low-bit fp16 operands, exact: pair s of sub-step t as base_s + u (the field
// at its own bit offset under an fp16 exponent whose unit is that offset's
// weight), plus nb[s] = -(base_s + z).  r is in offset binary (signed codes
// with their top bit flipped, z = 2^(width-1)).  base_s = 1024 >> 2s for the
// 2-bit plane (and width 3), 1024 >> s for width 1.
template <int WB>
__device__ __forceinline__ Frag8 deq_low_f16(const v4u& r, int t, const uint32_t (&nb)[4]) {
    Frag8 f;
    if constexpr (WB == 1) {
        const uint32_t y = r[2] >> (4 * t);
#pragma unroll
        for (int s = 0; s < 4; ++s)
            f.u[s] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, and_or(y, 0x00010001u << s, (0x6400u - 0x400u * s) * 0x10001u)) +
                                                      __builtin_bit_cast(v2h, nb[s]));
    } else {
        const uint32_t x = r[t >> 1] >> (8 * (t & 1));
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            uint32_t c = (0x6400u - 0x800u * s) * 0x10001u;  // 1024, 256, 64, 16
            if constexpr (WB == 3) {
                // the third bit from bit 4t + s of the 1-bit plane up to bit 2s + 2
                const int sh = s + 2 - 4 * t;
                const uint32_t y = sh >= 0 ? r[2] << sh : r[2] >> -sh;
                c = and_or(y, 0x00040004u << (2 * s), c);
            }
            f.u[s] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, and_or(x, 0x00030003u << (2 * s), c)) +
                                                      __builtin_bit_cast(v2h, nb[s]));
        }
    }
    return f;
}

// The nb[] constants of deq_low_f16 for a zero-point (or the signed offset) z.
template <int WB>
__device__ __forceinline__ void low_f16_offsets(uint32_t z, uint32_t (&nb)[4]) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        // -(base_s + z): the fp16 of -base_s with z in the mantissa at base_s's unit
        const uint32_t h = WB == 1 ? ((0xE400u - 0x400u * s) | (z << s)) : ((0xE400u - 0x800u * s) | (z << (2 * s)));
        nb[s] = h * 0x10001u;
    }
}

// 5-8-bit codes: the low nibble from the 4-bit pair-order word wl[t] and the
// high bits from wh (width 8: a second pair-order word set, wh[t]; 6 and 7: the
// 2-bit plane in wh[0..1]; 5 and 7: the 1-bit plane in wh[2], the bit above the
// 2-bit field for width 7), placed as bits 4.. of each 16-bit half under the
// exponent of 1024: the half reads 1024 + code (code < 256), and nb = -(1024 + z)
// leaves code - z exactly (offset binary for signed codes, z = 2^(width-1)).
// bf16 operands take that exact difference through fp32 (at most 8 significant
// bits, exact in bf16).
__device__ __forceinline__ uint32_t shl_signed(uint32_t x, int sh) { return sh >= 0 ? x << sh : x >> -sh; }
template <int WB, bool BF>
__device__ __forceinline__ Frag8 deq_wide(const v4u& wl, const v4u& wh, int t, uint32_t nb) {
    Frag8 f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        uint32_t c = 0x64006400u;
        if constexpr (WB == 8) {
            c = and_or(shl_signed(wh[t], 4 - 4 * s), 0x00F000F0u, c);
        } else {
            if constexpr (WB == 6 || WB == 7)  // 2-bit field at 2s + 8 (t & 1) -> bits 4-5
                c = and_or(shl_signed(wh[t >> 1], 4 - 2 * s - 8 * (t & 1)), 0x00300030u, c);
            if constexpr (WB == 5)  // 1-bit field at 4t + s -> bit 4
                c = and_or(shl_signed(wh[2], 4 - 4 * t - s), 0x00100010u, c);
            if constexpr (WB == 7)  // -> bit 6
                c = and_or(shl_signed(wh[2], 6 - 4 * t - s), 0x00400040u, c);
        }
        const uint32_t v = and_or(wl[t] >> (4 * s), 0x000F000Fu, c);
        const v2h d = __builtin_bit_cast(v2h, v) + __builtin_bit_cast(v2h, nb);
        if constexpr (BF) {
            typedef float f2v __attribute__((ext_vector_type(2)));
            typedef __bf16 b2v __attribute__((ext_vector_type(2)));
            const f2v x = f2v{(float)d[0], (float)d[1]};
            f.u[s] = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, b2v));
        } else {
            f.u[s] = __builtin_bit_cast(uint32_t, d);
        }
    }
    return f;
}

// Low-bit bf16 operands 128 + u (exact; offset binary as above), pair s of sub-step t.
template <int WB>
__device__ __forceinline__ Frag8 deq_low_bf16_offset(const v4u& r, int t) {
    Frag8 f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        if constexpr (WB == 1) {
            f.u[s] = and_or(r[2] >> (4 * t + s), 0x00010001u, 0x43004300u);
        } else {
            uint32_t c = 0x43004300u;
            if constexpr (WB == 3) {
                const int sh = 4 * t + s - 2;
                const uint32_t y = sh >= 0 ? r[2] >> sh : r[2] << -sh;
                c = and_or(y, 0x00040004u, c);
            }
            f.u[s] = and_or(r[t >> 1] >> (8 * (t & 1) + 2 * s), 0x00030003u, c);
        }
    }
    return f;
}

// bf16 128 + u (exact) for eight codes of one pair-ordered word.
__device__ __forceinline__ Frag8 deq4_bf16_offset(uint32_t w) {
    const uint32_t m = 0x000F000Fu, c = 0x43004300u;
    Frag8 f;
#pragma unroll
    for (int s = 0; s < 4; ++s) f.u[s] = ((w >> (4 * s)) & m) | c;
    return f;
}

// e2m1 x 2^(e-127) -> bf16 (exact) or fp16 (exact inside fp16's range); 8
// natural-order codes of one word.
template <bool BF = true>
__device__ __forceinline__ Frag8 fp4_to_bf16(uint32_t w, float scale) {
    Frag8 f;
    if constexpr (BF) {
        f.u[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0));
        f.u[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1));
        f.u[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2));
        f.u[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3));
    } else {
        f.u[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, 0));
        f.u[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, 1));
        f.u[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, 2));
        f.u[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, 3));
    }
    return f;
}

// e2m1 x s -> bf16 for a scale s that is not a power of two (an E4M3 group
// scale): the scaled convert applies only the exponent of its scale operand, so
// the codes are converted unscaled (exact) and each value is multiplied by s
// in fp32; e2m1 x e4m3 has at most 5 significant bits, so the RNE conversion
// back to bf16 is exact (fp16 too: the products lie in [2^-10, 2688]).
template <bool BF = true>
__device__ __forceinline__ Frag8 fp4_to_bf16_mul(uint32_t w, float s) {
    Frag8 f = fp4_to_bf16<true>(w, 1.0f);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float lo = __uint_as_float(f.u[i] << 16) * s, hi = __uint_as_float(f.u[i] & 0xFFFF0000u) * s;
        f.u[i] = (uint32_t)f32_to_16<BF>(lo) | ((uint32_t)f32_to_16<BF>(hi) << 16);
    }
    return f;
}

// two's-complement INT4 x 2^(e-127) -> bf16, exact (at most 3 significant bits);
// 8 natural-order codes of one word, in the element order of fp4_to_bf16
template <bool BF = true>
__device__ __forceinline__ Frag8 int4_to_bf16(uint32_t w, float scale) {
    typedef float f2v __attribute__((ext_vector_type(2)));
    typedef __bf16 b2v __attribute__((ext_vector_type(2)));
    typedef _Float16 h2v __attribute__((ext_vector_type(2)));
    Frag8 f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int lo = (int)(w << (28 - 8 * i)) >> 28, hi = (int)(w << (24 - 8 * i)) >> 28;
        const f2v v = f2v{(float)lo * scale, (float)hi * scale};
        if constexpr (BF) f.u[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, b2v));
        else f.u[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, h2v));
    }
    return f;
}

// INT8 -> fp16, exact: byte q + 128 placed under the exponent of 1024 (fp16 has 10
// mantissa bits) reads 1024 + q + 128; adding -1152 leaves q.  8 codes, two words.
__device__ __forceinline__ Frag8 deq8_f16(uint32_t w0, uint32_t w1) {
    const v2h nb = __builtin_bit_cast(v2h, 0xE480E480u);  // -1152, -1152
    const uint32_t x0 = w0 ^ 0x80808080u, x1 = w1 ^ 0x80808080u;
    Frag8 f;
    f.u[0] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, __builtin_amdgcn_perm(0x64646464u, x0, 0x04010400u)) + nb);
    f.u[1] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, __builtin_amdgcn_perm(0x64646464u, x0, 0x04030402u)) + nb);
    f.u[2] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, __builtin_amdgcn_perm(0x64646464u, x1, 0x04010400u)) + nb);
    f.u[3] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, __builtin_amdgcn_perm(0x64646464u, x1, 0x04030402u)) + nb);
    return f;
}

// INT8 -> bf16, exact (|q| <= 128 needs at most 8 significant bits).
__device__ __forceinline__ Frag8 deq8_bf16(uint32_t w0, uint32_t w1) {
    typedef float f2v __attribute__((ext_vector_type(2)));
    typedef __bf16 b2v __attribute__((ext_vector_type(2)));
    Frag8 f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t w = i < 2 ? w0 : w1;
        const int lo = (int)(w << (24 - 16 * (i & 1))) >> 24, hi = (int)(w << (16 - 16 * (i & 1))) >> 24;
        f.u[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2v{(float)lo, (float)hi}, b2v));
    }
    return f;
}

// E4M3 -> bf16 / fp16, exact (4 significant bits, exponents 2^-9..2^8 inside both
// formats' normal ranges): the scaled converts with a unit scale.
template <bool BF>
__device__ __forceinline__ Frag8 deq8_fp8(uint32_t w0, uint32_t w1) {
    Frag8 f;
    if constexpr (BF) {
        f.u[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false));
        f.u[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true));
        f.u[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false));
        f.u[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true));
    } else {
        f.u[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false));
        f.u[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true));
        f.u[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false));
        f.u[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true));
    }
    return f;
}

// E4M3 x 2^(E-127) -> bf16, exact for the E8M0 range the format reaches (4
// significant bits); 8 codes (one K sub-step) of a lane's 16-byte half.
template <bool BF = true>
__device__ __forceinline__ Frag8 fp8_to_bf16_scaled(const v4u& half, int pair, float scale) {
    const uint32_t w0 = half[2 * pair], w1 = half[2 * pair + 1];
    Frag8 f;
    if constexpr (BF) {
        f.u[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, scale, false));
        f.u[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, scale, true));
        f.u[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, scale, false));
        f.u[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, scale, true));
    } else {
        f.u[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, scale, false));
        f.u[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, scale, true));
        f.u[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, scale, false));
        f.u[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, scale, true));
    }
    return f;
}

// Bytes u -> u - z, exact (|u - z| < 256): fp16 by u under the exponent of 1024
// and one packed add of -(1024 + z) (nbz, both halves); bf16 through fp32.  8
// codes (one K sub-step) of a lane's 16-byte half.
template <bool BF>
__device__ __forceinline__ Frag8 deq8_zp(const v4u& half, int pair, uint32_t nbz, float zf) {
    const uint32_t w0 = half[2 * pair], w1 = half[2 * pair + 1];
    Frag8 f;
    if constexpr (BF) {
        typedef float f2v __attribute__((ext_vector_type(2)));
        typedef __bf16 b2v __attribute__((ext_vector_type(2)));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t w = i < 2 ? w0 : w1;
            const float lo = (float)((w >> (16 * (i & 1))) & 0xFFu) - zf;
            const float hi = (float)((w >> (16 * (i & 1) + 8)) & 0xFFu) - zf;
            f.u[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2v{lo, hi}, b2v));
        }
    } else {
        const v2h nb = __builtin_bit_cast(v2h, nbz);
        f.u[0] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, __builtin_amdgcn_perm(0x64646464u, w0, 0x04010400u)) + nb);
        f.u[1] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, __builtin_amdgcn_perm(0x64646464u, w0, 0x04030402u)) + nb);
        f.u[2] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, __builtin_amdgcn_perm(0x64646464u, w1, 0x04010400u)) + nb);
        f.u[3] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, __builtin_amdgcn_perm(0x64646464u, w1, 0x04030402u)) + nb);
    }
    return f;
}

// 8 codes (one K sub-step) of a lane's 16-byte half: INT8 or E4M3
template <Fmt F>
__device__ __forceinline__ Frag8 deq8(const v4u& half, int pair) {
    constexpr bool BF = w8bf(F);
    if constexpr (f8w(F)) return deq8_fp8<BF>(half[2 * pair], half[2 * pair + 1]);
    else if constexpr (BF) return deq8_bf16(half[2 * pair], half[2 * pair + 1]);
    else return deq8_f16(half[2 * pair], half[2 * pair + 1]);
}

__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
    e &= 0xFFu;
    return __uint_as_float(e == 0 ? 0x00400000u : e == 255u ? 0x7FC00000u : (e << 23));
}

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for the direct-to-LDS pipelines.  Their only LDS writes are
// the direct loads, whose completion each wave has already waited for with an
// explicit vmcnt; __syncthreads() would add a release fence, which makes the
// compiler wait for every load in flight (vmcnt(0)) and so drain the prefetch.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// This wave's LDS writes complete (lgkmcnt(0), other counters untouched), then
// the workgroup barrier.
__device__ __forceinline__ void lds_sync() {
    __builtin_amdgcn_s_waitcnt(0xC07F);
    lds_barrier();
}

// The 128- and 256-row tiles run one workgroup per CU (their LDS footprint
// admits no second one): 8-wave tiles two waves per SIMD, so the compiler may
// spend up to 256 VGPRs on fragments read ahead instead of aiming for a third
// wave; 4-wave tiles one wave per SIMD with the whole 512-entry register file.
template <Fmt F, int BM, int BN, int WM, int WN, int PD>
__global__ __launch_bounds__(64 * WM * WN, 1)
__attribute__((amdgpu_waves_per_eu(1, BM < 128 ? 4 : WM * WN <= 4 ? 1 : 2)))
void tile_gemm_kernel(TileArgs p) {
    using T = FmtTraits<F>;
    using Acc = typename T::Acc;
    // group scales and zero-points staged per step (UINT4 words, or the byte
    // codes' UINT8 zero-points: 16 bytes per strip)
    constexpr bool WNA16 = F == Fmt::WNA16_F16 || F == Fmt::WNA16_BF16 || w8g(F);
    constexpr int ZB = w8g(F) ? 16 : 8;  // zero-point bytes per strip and group
    constexpr bool NV = nvfp4(F);                         // E4M3 weight scales per 16 K
    constexpr bool MX = mx_mfma(F) || fp4w(F) || mxf8(F);  // byte scales per lane
    static_assert(!mxf6(F), "MXFP6 reaches the tiles widened to MXFP8");
    constexpr bool MXA = mx_act(F);
    constexpr bool F8B = F == Fmt::W8A8_F8B;
    static_assert(!F8B || BN == 128, "blockwise fp8: one 128-column weight block per tile");
    constexpr int NTH = 64 * WM * WN;
    constexpr int BK = 128;
    constexpr int AROW = T::AROW, AUNITS = AROW / 16;
    constexpr int A_STAGE = BM * AROW;
    constexpr int NSTRIP = BN / 16;
    constexpr int B_STAGE = NSTRIP * T::BSTRIP;
    // per-step scale block: WNA16 16 fp16 scales + one zero-point word per strip;
    // MXFP4 one E8M0 byte per lane per strip; INT8 none (per-channel, epilogue)
    constexpr int SC_Z = NSTRIP * 32;                     // zero-point words start (WNA16)
    constexpr int SC_B = WNA16 ? NSTRIP * 48 : NV ? NSTRIP * 128 : MX ? NSTRIP * 64 : 0;
    // MX activations: one E8M0 word (4 K blocks) per row; blockwise fp8: one fp32
    // activation scale per row, then the tile's weight block scale
    constexpr int SC_STAGE = SC_B + (MXA ? BM * 4 : 0) + (F8B ? BM * 4 + 16 : 0);
    constexpr int SC_UNITS = SC_B / 16;
    // a stage holds the A and weight tiles of one step; the step's scale block
    // sits in an LDS array of its own (it is loaded through registers, and its
    // reads take immediate offsets)
    constexpr int SC_PAD = SC_STAGE > 0 ? (SC_STAGE + 15) / 16 * 16 : 16;
    constexpr bool B1 = PD == 3;  // single weight stage
    // MX MFMA formats on the stage ring: the step's scale block (weight E8M0
    // bytes, and the activations' E8M0 words) loads straight into its stage like
    // the tiles.  Through registers it needs one register set per ring stage,
    // which the 256 x 256 tiles cannot hold beside their accumulators (the
    // compiler spills them, and every spill waits for all loads in flight).
    constexpr bool SC_DMA = PD == 4 && mx_mfma(F);
    constexpr int STAGE = A_STAGE + (B1 ? 0 : B_STAGE) + (SC_DMA ? SC_PAD : 0);
    // LDS stages: a ring of four where they fit, else three (PD = 4), else two
    constexpr int NRING = 4 * STAGE <= 150 * 1024 ? 4 : 3;
    constexpr int NST = PD == 4 ? NRING : 2;
    static_assert(PD != 4 || 3 * STAGE <= 150 * 1024, "a ring needs three stages");
    constexpr int NIA = A_STAGE / 16 / NTH;  // 16-byte loads per thread per step (A)
    constexpr int NIB = B_STAGE / 16 / NTH;  // (B)
    constexpr int MT = BM / WM / 16, NT = BN / WN / 16;  // 16x16 tiles per wave
    static_assert(A_STAGE % (16 * NTH) == 0 && B_STAGE % (16 * NTH) == 0, "stage must split evenly over threads");
    static_assert(SC_UNITS <= NTH, "one 16-byte scale unit per fetching thread");
    static_assert(NTH >= 128, "zero-point words are fetched by wave 1");

    // Two LDS stages as distinct objects: the compiler can then tell a direct
    // global->LDS load into one stage from fragment reads of the other and does
    // not make the reads wait for the load.
    __shared__ __attribute__((aligned(1024))) char stage0[STAGE];
    __shared__ __attribute__((aligned(1024))) char stage1[STAGE];
    __shared__ __attribute__((aligned(1024))) char stage2[NST > 2 ? STAGE : 16];
    __shared__ __attribute__((aligned(1024))) char stage3[NST > 3 ? STAGE : 16];
    __shared__ __attribute__((aligned(1024))) char bstage[B1 ? B_STAGE : 16];
    __shared__ __attribute__((aligned(16))) char scst[SC_DMA ? 1 : NST][SC_DMA ? 16 : SC_PAD];
    __shared__ int rowinfo[2 * BM];  // [0,BM): A row per local row; [BM,2BM): D row (-1 = none)

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int col = lane & 15, quad = lane >> 4;

    // ---- tile coordinates: K slice, XCD-aware remap, grouped raster along M ----
    // MoE grids are sized by an upper bound of the m-tile count; the valid
    // tiles take the lowest workgroup ids and the remap below spans only them,
    // so every XCD gets its share of real work
    int tiles_m = p.tiles_m;
    if constexpr (F == Fmt::MOE_MX) {
        tiles_m = min(*p.ntiles, p.tiles_m);
        if ((int)blockIdx.x >= tiles_m * p.tiles_n) return;
    }
    const int ntile = tiles_m * p.tiles_n;
    int bid = blockIdx.x % ntile;
    const int split = blockIdx.x / ntile;
    if ((ntile & 7) == 0) bid = (bid & 7) * (ntile >> 3) + (bid >> 3);
    constexpr int GROUP_M = 4;
    const int tiles_n = p.tiles_n;
    const int group_size = GROUP_M * tiles_n;
    const int first_m = (bid / group_size) * GROUP_M;
    const int gm = min(tiles_m - first_m, GROUP_M);
    const int pid_m = first_m + (bid % group_size) % gm;
    const int pid_n = (bid % group_size) / gm;

    const char* Wbase = (const char*)p.W;
    const char* Sbase = (const char*)p.S;
    int m0 = pid_m * BM, mrows = BM;
    if constexpr (F == Fmt::MOE_MX) {
        const int e = p.tile_info[3 * pid_m], first = p.tile_info[3 * pid_m + 1];
        mrows = p.tile_info[3 * pid_m + 2];
        Wbase += (int64_t)e * p.w_estride;
        Sbase += (int64_t)e * p.s_estride;
        for (int r = tid; r < BM; r += NTH) {
            const int rr = r < mrows ? r : mrows - 1;
            const int pos = first + rr;
            const int pair = p.sorted ? p.sorted[pos] : pos;
            rowinfo[r] = p.sorted ? pair / p.top_k : pos;
            rowinfo[BM + r] = r < mrows ? pair : -1;
        }
    } else {
        mrows = min(BM, p.M - m0);
        for (int r = tid; r < BM; r += NTH) {
            rowinfo[r] = m0 + (r < mrows ? r : mrows - 1);
            rowinfo[BM + r] = r < mrows ? m0 + r : -1;
        }
    }
    __syncthreads();

    const int K = p.K, nsteps = K / BK;
    const int k0 = (int)((int64_t)split * nsteps / p.splits), k1 = (int)((int64_t)(split + 1) * nsteps / p.splits);
    const int strip0 = pid_n * NSTRIP, nstrips_total = p.Np / 16;
    auto clamp_strip = [&](int s) { return s < nstrips_total ? s : nstrips_total - 1; };

    // buffer resources (base + size; wave-uniform K-step offsets go in SGPRs)
    const uint32_t nstr = (uint32_t)(p.Np / 16);
    const uint32_t arow_bytes = (uint32_t)(K / BK) * AROW;  // bytes of one A row
    const rsrc_t rA = make_rsrc(p.A, (uint32_t)p.a_rows * arow_bytes);
    const rsrc_t rAS = MXA ? make_rsrc(p.a_e8, (uint32_t)p.a_rows * (uint32_t)(K / 32))
                     : make_rsrc(p.a_blk, F8B ? (uint32_t)p.a_rows * (uint32_t)(K / 128) * 4u : 0u);
    const rsrc_t rW = make_rsrc(Wbase, nstr * (uint32_t)nsteps * T::BSTRIP);
    const uint32_t nbn = (uint32_t)((p.Np + 127) / 128);  // weight column blocks (blockwise fp8)
    const rsrc_t rS = make_rsrc(Sbase, WNA16 ? nstr * (uint32_t)p.ngroups * 32u : MX ? nstr * (uint32_t)nsteps * (NV ? 128u : 64u)
                                       : F8B ? (uint32_t)nsteps * nbn * 4u : 0u);
    const rsrc_t rZ = make_rsrc(p.Z, WNA16 && p.Z ? nstr * (uint32_t)p.ngroups * (uint32_t)ZB : 0u);

    // per-thread byte offsets of the staged loads (fixed across K steps).  Dense
    // A rows are consecutive: one lane offset serves every load, load i adding
    // a wave-uniform i * (NTH / AUNITS) rows (the swizzle repeats every 16 rows);
    // rows past M fall outside the buffer resource and read zeros (their
    // outputs are dropped).  MoE rows are gathered: one offset per load.
    constexpr bool AFLAT = F != Fmt::MOE_MX && (NTH / AUNITS) % 16 == 0;
    const uint32_t arow_stride = (uint32_t)(NTH / AUNITS) * arow_bytes;
    uint32_t aoff[AFLAT ? 1 : NIA];
#pragma unroll
    for (int i = 0; i < (AFLAT ? 1 : NIA); ++i) {
        const int s = i * NTH + tid;
        const int row = s / AUNITS, pos = s % AUNITS;
        const int unit = pos ^ swz(row, AUNITS);
        aoff[i] = (AFLAT ? (uint32_t)(m0 + row) : (uint32_t)rowinfo[row]) * arow_bytes + unit * 16;
    }
    auto a_voff = [&](int i) -> uint32_t { return AFLAT ? aoff[0] : aoff[i]; };
    auto a_soff = [&](int i, int ks) -> uint32_t { return (AFLAT ? (uint32_t)i * arow_stride : 0u) + (uint32_t)ks * AROW; };
    // weight loads: one lane offset, load i adding i * NTH / UPS strips as a
    // wave-uniform offset.  Strips past the packed width (a ragged last column
    // tile) fall outside the buffer resource and read zeros: the range check
    // covers the scalar offset too (checked on gfx950), and those columns are
    // never stored.
    constexpr int UPS = T::BSTRIP / 16;  // 16-byte units per strip and step
    static_assert(NTH % UPS == 0, "a load instruction covers whole strips");
    const uint32_t boff0 = (uint32_t)(strip0 + tid / UPS) * (uint32_t)nsteps * T::BSTRIP + (uint32_t)(tid % UPS) * 16u;
    const uint32_t bstride = (uint32_t)(NTH / UPS) * (uint32_t)nsteps * T::BSTRIP;
    // scale block fetchers: 16 bytes per thread; MXFP4 4 threads per strip (64 B),
    // NVFP4 8 threads per strip (128 B: two E4M3 bytes per lane)
    constexpr int SPT = NV ? 8 : 4;
    constexpr uint32_t SBYTES = NV ? 128u : 64u;  // scale bytes per strip and step
    const uint32_t sc_strip = (uint32_t)clamp_strip(strip0 + (WNA16 ? (tid < 2 * NSTRIP ? tid / 2 : tid - 2 * NSTRIP) : tid / SPT));
    const uint32_t soff = WNA16 ? (tid < 2 * NSTRIP ? sc_strip * p.ngroups * 32u + (tid & 1) * 16u : sc_strip * p.ngroups * (uint32_t)ZB)
                                : sc_strip * (uint32_t)nsteps * SBYTES + (tid % SPT) * 16u;

    auto stage_lds = [&](auto stc) -> lds_char* {
        constexpr int S = decltype(stc)::value;
        if constexpr (S == 0) return (lds_char*)stage0;
        else if constexpr (S == 1) return (lds_char*)stage1;
        else if constexpr (S == 2) return (lds_char*)stage2;
        else return (lds_char*)stage3;
    };
    auto stage_ptr = [&](auto stc) -> char* {
        constexpr int S = decltype(stc)::value;
        if constexpr (S == 0) return stage0;
        else if constexpr (S == 1) return stage1;
        else if constexpr (S == 2) return stage2;
        else return stage3;
    };
    auto sc_ptr = [&](auto stc) -> char* {
        if constexpr (SC_DMA) return stage_ptr(stc) + A_STAGE + B_STAGE;
        else return scst[decltype(stc)::value];
    };

    // PD = 0: loads go straight from HBM into the next LDS stage (no staging
    // registers).  PD = 1, 2: register sets; the loads of step s+PD fly while
    // step s computes.
    static_assert(PD >= 0 && PD <= 4, "prefetch: direct to LDS, one or two register steps, single weight stage, stage ring");
    constexpr bool RSTAGE = PD == 1 || PD == 2;  // A and B staged through registers
    constexpr int NSET = RSTAGE ? PD : PD == 4 ? NST : 1;  // register sets (the ring: one scale block per stage)
    v4u ra[NSET][RSTAGE ? NIA : 1], rb[NSET][RSTAGE ? NIB : 1], rs[NSET];
    uint32_t rsa[NSET];  // MX activations: this thread's row's E8M0 word of the step (threads < BM)
    const uint32_t as_voff = (uint32_t)(m0 + (tid < BM ? tid : 0)) * (uint32_t)(F8B ? (K / 128) * 4 : K / 32);
    // Direct loads of one step's A and weight tiles into a stage (NIA + NIB
    // unconditional loads per thread).  The scale block goes through registers
    // (sc_load, then sc_write into its own LDS array once landed): the compiler
    // cannot tell direct loads into the scale block of one stage from reads of
    // another stage's, and would make every LDS read wait for them.
    const int wbase = __builtin_amdgcn_readfirstlane((tid & ~63) * 16);  // this wave's first 16-byte slot
    auto dma_a = [&](int ks, auto stc) {
        lds_char* sA = stage_lds(stc);
#pragma unroll
        for (int i = 0; i < NIA; ++i)
            dma16(rA, sA + i * NTH * 16 + wbase, a_voff(i), a_soff(i, ks));
    };
    auto dma_b = [&](int ks, auto stc) {
        lds_char* sB = B1 ? (lds_char*)bstage : stage_lds(stc) + A_STAGE;
#pragma unroll
        for (int i = 0; i < NIB; ++i)
            dma16_nt(rW, sB + i * NTH * 16 + wbase, boff0, (uint32_t)i * bstride + (uint32_t)ks * T::BSTRIP);
    };
    auto dma = [&](int ks, auto stc) {
        dma_a(ks, stc);
        dma_b(ks, stc);
    };
    // the step's scale block: WNA16 threads [0, 2 NSTRIP) fetch 16 scale bytes
    // each, threads [2 NSTRIP, 3 NSTRIP) a strip's zero-point word; MXFP4
    // threads [0, SC_UNITS) 16 E8M0 bytes each
    auto sc_load = [&](int ks, auto setc) {
        constexpr int st = decltype(setc)::value % NSET;
        if constexpr (WNA16) {
            const uint32_t g = (uint32_t)(ks / p.gsteps);
            if (tid < 2 * NSTRIP) {
                rs[st] = buf16(rS, soff, g * 32u);
            } else if (tid < 3 * NSTRIP) {
                // unconditional, straight into the register set (a select after
                // the load would make the wave wait for it at once); without
                // zero-points the buffer range is empty and the load reads zeros,
                // which the symmetric decode ignores
                if constexpr (ZB == 16) {
                    rs[st] = buf16(rZ, soff, g * 16u);
                } else {
                    const uint64_t z = buf8(rZ, soff, g * 8u);
                    rs[st][0] = (uint32_t)z;
                    rs[st][1] = (uint32_t)(z >> 32);
                }
            }
        } else if constexpr (SC_DMA) {
            lds_char* sc = stage_lds(setc) + A_STAGE + B_STAGE;
            if (tid < SC_UNITS) dma16(rS, sc + wbase, soff, (uint32_t)ks * SBYTES);
            // one E8M0 word per row: lane l of wave w writes row 64 w + l
            if constexpr (MXA)
                if (tid < BM) dma4(rAS, sc + SC_B + wbase / 4, as_voff, (uint32_t)ks * 4u);
        } else if constexpr (MX) {
            if (tid < SC_UNITS) rs[st] = buf16(rS, soff, (uint32_t)ks * SBYTES);
            // rows past M fall outside the buffer resource and read zeros (outputs dropped)
            if constexpr (MXA)
                if (tid < BM) rsa[st] = buf4(rAS, as_voff, (uint32_t)ks * 4u);
        } else if constexpr (F8B) {
            if (tid < BM) rsa[st] = buf4(rAS, as_voff, (uint32_t)ks * 4u);
            else if (tid == BM) rsa[st] = buf4(rS, 0u, ((uint32_t)ks * nbn + (uint32_t)(strip0 / 8)) * 4u);
        }
    };
    auto sc_write = [&](auto stc, auto setc) {
        constexpr int st = decltype(setc)::value % NSET;
        char* sS = sc_ptr(stc);
        if constexpr (SC_STAGE > 0 && !SC_DMA) {
            if constexpr (WNA16) {
                if (tid < 2 * NSTRIP) *(v4u*)(sS + tid * 16) = rs[st];
                else if (tid < 3 * NSTRIP) {
                    if constexpr (ZB == 16) *(v4u*)(sS + SC_Z + (tid - 2 * NSTRIP) * 16) = rs[st];
                    else *(uint64_t*)(sS + SC_Z + (tid - 2 * NSTRIP) * 8) = ((uint64_t)rs[st][1] << 32) | rs[st][0];
                }
            } else if constexpr (F8B) {
                if (tid <= BM) *(uint32_t*)(sS + tid * 4) = rsa[st];
            } else {
                if (tid < SC_UNITS) *(v4u*)(sS + tid * 16) = rs[st];
                if constexpr (MXA)
                    if (tid < BM) *(uint32_t*)(sS + SC_B + tid * 4) = rsa[st];
            }
        }
    };
    auto gload = [&](int ks, auto setc) {
        constexpr int st = decltype(setc)::value % NSET;
#pragma unroll
        for (int i = 0; i < NIA; ++i) ra[st][i] = buf16(rA, a_voff(i), a_soff(i, ks));
#pragma unroll
        for (int i = 0; i < NIB; ++i) rb[st][i] = buf16<true>(rW, boff0, (uint32_t)i * bstride + (uint32_t)ks * T::BSTRIP);
        sc_load(ks, setc);
    };
    auto swrite = [&](auto stc, auto setc) {
        constexpr int st = decltype(setc)::value % NSET;
        char* sA = stage_ptr(stc);
        char* sB = sA + A_STAGE;
#pragma unroll
        for (int i = 0; i < NIA; ++i) *(v4u*)(sA + (i * NTH + tid) * 16) = ra[st][i];
#pragma unroll
        for (int i = 0; i < NIB; ++i) *(v4u*)(sB + (i * NTH + tid) * 16) = rb[st][i];
        sc_write(stc, setc);
    };

    Acc acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = Acc{0, 0, 0, 0};

    // LDS offset of this lane's A fragment for K sub-step t of a 128-K step: the
    // rows of a wave's 16-row tiles differ by multiples of 16, so the swizzle
    // depends on the lane's column only and tile i adds i * 16 rows (an
    // immediate offset)
    uint32_t a_frag[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
        a_frag[t] = (uint32_t)((wm * (BM / WM) + col) * AROW + (((4 * quad + t) ^ swz(col, AUNITS)) * 16));
    const uint32_t wx = p.Z ? 0u : 0x88888888u;  // symmetric INT4: two's complement -> offset binary
    // scale block of a step: this lane's column in the wave's first strip
    const uint32_t sc_lane = (uint32_t)(wn * NT * 32 + col * 2), z_lane = (uint32_t)(wn * NT * 8 + (col >> 3) * 4);
    const uint32_t zshift = 4u * (uint32_t)(col & 7), zmask = p.Z ? 15u : 0u, zsym = p.Z ? 0u : 8u;
    const uint32_t zsym8 = p.Z ? 0u : 128u;  // byte codes: signed ones are stored as q + 128
    constexpr int NBH = T::BSTRIP / 1024;  // 16-byte fragments per strip and step (two for INT8)
    // compute(stage, hook): hook(t) runs at the start of K sub-step t = 0..3,
    // after the step's scale block has been read from LDS; the pipelines issue
    // the next steps' loads there (all at t = 0: spreading them over the step
    // measured slower)
    auto nohook = [](int) {};
    auto compute = [&](auto stc, auto hook) {
        const char* sS = sc_ptr(stc);
        const char* sA = stage_ptr(stc);
        const char* sB = B1 ? bstage : sA + A_STAGE;
        // this wave's packed weight words: one 16-byte fragment per strip (per 64-K half for INT8)
        v4u bw[NT][NBH];
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int h = 0; h < NBH; ++h) bw[j][h] = *(const v4u*)(sB + (wn * NT + j) * T::BSTRIP + h * 1024 + lane * 16);

        if constexpr (F == Fmt::WNA16_F16 || fp4w(F) || w8load(F)) {
            // 16-bit A with 4-bit weights decoded into the operand: fp16 (q - z) * s,
            // or e2m1 x (2^(E-127) or an E4M3 value) -> bf16 (exact)
            constexpr bool MOE = fp4w(F) || mxf8(F);  // 16-bit operands under the lane's E8M0 or E4M3 scale
            constexpr bool BFA = (MOE && !f16_operand(F)) || w8bf(F) || F == Fmt::W8G_BF16;  // bf16 MFMA (else fp16)
            // bf16 byte codes with group scales: each step's MFMA partials (st) take
            // the column's group scale at the end of the step (a step lies inside one
            // group); fp16 ones take it in the decode, (q - z) * s rounded once to
            // fp16 as for the 4-bit codes (no second accumulator set, so the 128 x 256
            // tile fits its registers)
            constexpr bool GS = F == Fmt::W8G_BF16;
            Acc st[GS ? MT : 1][GS ? NT : 1];
            if constexpr (GS) {
#pragma unroll
                for (int i = 0; i < MT; ++i)
#pragma unroll
                    for (int j = 0; j < NT; ++j) st[i][j] = Acc{0.f, 0.f, 0.f, 0.f};
            }
            auto mma = [&](int i, int j, const Frag8& a, const Frag8& b) {
                if constexpr (GS) st[i][j] = mfma16<BFA>(a, b, st[i][j]);
                else acc[i][j] = mfma16<BFA>(a, b, acc[i][j]);
            };
            float zf[GS ? NT : 1];
            // A fragments read ahead (software pipeline): a whole sub-step, or
            // a ring of three for tall / wide wave tiles
            Frag8 afr[(NT >= 4 || MT > 8) ? 1 : 2][(NT >= 4 || MT > 8) ? 3 : MT];
            Frag8 bq[2][NT];                  // decoded weights of two sub-steps
            uint32_t s2[NT], nb2[NT], nh2[NT];
            float sf[NT][NV ? 2 : 1];
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                if constexpr (NV) {
                    // this lane's 16-K groups 2 quad and 2 quad + 1 of the step (sub-steps 0-1, 2-3)
                    const uint32_t two = *(const uint16_t*)(sS + (wn * NT + j) * 128 + lane * 2);
                    sf[j][0] = __builtin_amdgcn_cvt_f32_fp8((int)two, 0);
                    sf[j][1] = __builtin_amdgcn_cvt_f32_fp8((int)two, 1);
                } else if constexpr (MOE) {
                    sf[j][0] = e8m0_to_f32(((const uint8_t*)sS)[(wn * NT + j) * 64 + lane]);
                } else if constexpr (w8a16(F)) {
                    // per-channel scale in the epilogue: nothing per step
                } else if constexpr (w8g(F)) {
                    // the column's group scale and zero-point (128 for signed codes,
                    // whose zero-point buffer is null and reads zeros)
                    const uint32_t sc = *(const uint16_t*)(sS + sc_lane + j * 32);
                    sf[j][0] = bits16_to_f32<BFA>((uint16_t)sc);
                    s2[j] = sc | (sc << 16);
                    const uint32_t z = (uint32_t)((const uint8_t*)(sS + SC_Z))[(wn * NT + j) * 16 + col] | zsym8;
                    if constexpr (GS) zf[j] = (float)z;
                    nb2[j] = (0xE400u | z) * 0x10001u;  // -(1024 + z), both halves
                } else {
                    // one lane offset for every strip (strips are immediate offsets); the
                    // zero-point select is branch-free (symmetric INT4: z = 8)
                    const uint32_t sc = *(const uint16_t*)(sS + sc_lane + j * 32);
                    const uint32_t zw = *(const uint32_t*)(sS + SC_Z + z_lane + j * 8);
                    const uint32_t z = ((zw >> zshift) & zmask) | zsym;
                    s2[j] = sc | (sc << 16);
                    const uint32_t nbz = 0xE400u | z, nhz = 0xD400u | (z << 4);  // -(1024 + z), -(64 + z)
                    nb2[j] = nbz | (nbz << 16);
                    nh2[j] = nhz | (nhz << 16);
                }
            }
            // weight operand of strip j for K sub-step t
            auto mkb = [&](int j, int tt) -> Frag8 {
                if constexpr (NV) return fp4_to_bf16_mul<BFA>(bw[j][0][tt], sf[j][tt >> 1]);
                else if constexpr (mxint4w(F)) return int4_to_bf16<BFA>(bw[j][0][tt], sf[j][0]);
                else if constexpr (mxf8(F)) return fp8_to_bf16_scaled<BFA>(bw[j][tt >> 1], tt & 1, sf[j][0]);
                else if constexpr (GS) return deq8_zp<true>(bw[j][tt >> 1], tt & 1, nb2[j], zf[j]);
                else if constexpr (w8g(F)) {
                    Frag8 f = deq8_zp<false>(bw[j][tt >> 1], tt & 1, nb2[j], 0.f);
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const uint32_t x = f.u[u];  // (a bit cast of a vector element reads element 0)
                        f.u[u] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, x) * __builtin_bit_cast(v2h, s2[j]));
                    }
                    return f;
                }
                else if constexpr (w8a16(F)) return deq8<F>(bw[j][tt >> 1], tt & 1);
                else if constexpr (MOE) return fp4_to_bf16<BFA>(bw[j][0][tt], sf[j][0]);
                else return deq4_f16_scaled(bw[j][0][tt] ^ wx, nb2[j], nh2[j], s2[j]);
            };
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                hook(t);
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (NT >= 4 || MT > 8) {
                    // tall or wide wave tiles: A fragments stream through a ring of
                    // three register sets, each read two fragments ahead of its
                    // MFMAs; the weights of sub-step t + 1 are dequantised one
                    // strip per A fragment between the MFMAs of sub-step t
                    constexpr int NQ = 4 * MT;
                    if (t == 0) {
                        afr[0][0].u = *(const v4u*)(sA + a_frag[0]);
                        afr[0][1].u = *(const v4u*)(sA + a_frag[0] + 16 * AROW);
#pragma unroll
                        for (int j = 0; j < NT; ++j) bq[0][j] = mkb(j, 0);
                    }
#pragma unroll
                    for (int i = 0; i < MT; ++i) {
                        const int q = t * MT + i;
                        if (q + 2 < NQ)
                            afr[0][(q + 2) % 3].u = *(const v4u*)(sA + a_frag[(q + 2) / MT] + ((q + 2) % MT) * 16 * AROW);
                        if (t < 3 && i < NT)
                            bq[(t + 1) & 1][i] = mkb(i, t + 1);
                        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                        for (int j = 0; j < NT; ++j) mma(i, j, afr[0][q % 3], bq[t & 1][j]);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                } else {
                    // Software pipeline over the four K sub-steps: the A fragments
                    // and dequantised weights of sub-step t + 1 are produced
                    // between the MFMAs of sub-step t, so one wave's VALU and LDS
                    // work fills the gaps of its own MFMA stream
                    if (t == 0) {
#pragma unroll
                        for (int i = 0; i < MT; ++i) afr[0][i].u = *(const v4u*)(sA + a_frag[0] + i * 16 * AROW);
#pragma unroll
                        for (int j = 0; j < NT; ++j) bq[0][j] = mkb(j, 0);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    if (t < 3) {
#pragma unroll
                        for (int i = 0; i < MT; ++i) afr[(t + 1) & 1][i].u = *(const v4u*)(sA + a_frag[t + 1] + i * 16 * AROW);
#pragma unroll
                        for (int j = 0; j < NT; ++j)
                            bq[(t + 1) & 1][j] = mkb(j, t + 1);
                    }
#pragma unroll
                    for (int i = 0; i < MT; ++i)
#pragma unroll
                        for (int j = 0; j < NT; ++j) mma(i, j, afr[t & 1][i], bq[t & 1][j]);
                    if (t < 3) {
                        // per A fragment: its read, the MFMAs of one fragment of
                        // this sub-step, a share of the next sub-step's dequant
#pragma unroll
                        for (int i = 0; i < MT; ++i) {
                            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);        // DS read
                            __builtin_amdgcn_sched_group_barrier(0x008, NT, 0);       // MFMA
                            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);        // VALU
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            if constexpr (GS) {
#pragma unroll
                for (int i = 0; i < MT; ++i)
#pragma unroll
                    for (int j = 0; j < NT; ++j) acc[i][j] += sf[j][0] * st[i][j];
            }
        } else if constexpr (F == Fmt::WNA16_BF16) {
#pragma unroll
            for (int t = 0; t < 4; ++t) hook(t);
            float sc[NT], zc[NT];
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const int sl = wn * NT + j;
                sc[j] = bits16_to_f32<true>(((const uint16_t*)sS)[sl * 16 + col]);
                const uint32_t z = p.Z ? (((const uint32_t*)(sS + SC_Z))[sl * 2 + (col >> 3)] >> (4 * (col & 7))) & 15u : 8u;
                zc[j] = (float)(128u + z);
            }
            v4f st[MT][NT], rsum[MT];
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                rsum[i] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < NT; ++j) st[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
            }
            Frag8 ones;
            ones.u = v4u{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                Frag8 b[NT];
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    uint32_t w = bw[j][0][t];
                    w ^= wx;
                    b[j] = deq4_bf16_offset(w);
                }
#pragma unroll
                for (int i = 0; i < MT; ++i) {
                    const int row = wm * (BM / WM) + i * 16 + col;
                    Frag8 a;
                    a.u = *(const v4u*)(sA + row * AROW + (((4 * quad + t) ^ swz(row, AUNITS)) * 16));
                    rsum[i] = mfma16<true>(a, ones, rsum[i]);
#pragma unroll
                    for (int j = 0; j < NT; ++j) st[i][j] = mfma16<true>(a, b[j], st[i][j]);
                }
            }
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int j = 0; j < NT; ++j) acc[i][j] += sc[j] * (st[i][j] - zc[j] * rsum[i]);
        } else if constexpr (mx_mfma(F)) {
#pragma unroll
            for (int t = 0; t < 4; ++t) hook(t);
            int bsc[NT];
#pragma unroll
            for (int j = 0; j < NT; ++j) bsc[j] = (int)((const uint8_t*)sS)[(wn * NT + j) * 64 + lane];
            constexpr int CBSZ = F == Fmt::W4A4_MX ? 4 : 0;  // A operand format: fp8 e4m3 or fp4 e2m1
            // A fragment of m-tile i (and, for MX activations, its E8M0 scale
            // byte).  The lane's row is r0 + 16 i; the swizzle depends on the
            // row's low four bits only, so on the lane's column: the offsets of
            // the m-tiles differ by constants (immediate offsets of the LDS reads
            // instead of one address register per m-tile and stage)
            const int r0 = wm * (BM / WM) + col;
            const int swc = swz(col, AUNITS);
            const int a_lo = r0 * AROW + ((quad ^ swc) * 16);
            const int a_hi = r0 * AROW + (((4 + quad) ^ swc) * 16);
            const uint32_t* a_sc = (const uint32_t*)(sS + SC_B + r0 * 4);
            auto rdA = [&](int i, v8i& a, int& asc) {
                const v4u lo = *(const v4u*)(sA + a_lo + i * 16 * AROW);
                if constexpr (F == Fmt::W4A4_MX) {
                    a = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], 0, 0, 0, 0};
                } else {
                    const v4u hi = *(const v4u*)(sA + a_hi + i * 16 * AROW);
                    a = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                }
                // the row's E8M0 word of the step, byte `quad` (a whole-word read: the
                // compiler waits for every load in flight before a byte read of
                // a word that a direct load writes)
                asc = MXA ? (int)((a_sc[i * 16] >> (8 * quad)) & 0xFFu) : 0x7F;
            };
            auto mm = [&](int i, const v8i& a, int asc) {
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    const v8i b = v8i{(int)bw[j][0][0], (int)bw[j][0][1], (int)bw[j][0][2], (int)bw[j][0][3], 0, 0, 0, 0};
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[i][j], CBSZ, 4, 0, asc, 0, bsc[j]);
                }
            };
            if constexpr (MT >= 8 && (MXA || F == Fmt::W4A4_MX)) {
                // tall wave tiles with MX activations: the A fragments stream through
                // two register sets, each read one m-tile ahead of its MFMAs (all of
                // them in flight at once spill the 256-register budget of two waves
                // per SIMD)
                v8i ar[2];
                int as[2];
                rdA(0, ar[0], as[0]);
#pragma unroll
                for (int i = 0; i < MT; ++i) {
                    if (i + 1 < MT) rdA(i + 1, ar[(i + 1) & 1], as[(i + 1) & 1]);
                    __builtin_amdgcn_sched_barrier(0);
                    mm(i, ar[i & 1], as[i & 1]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else {
#pragma unroll
                for (int i = 0; i < MT; ++i) {
                    v8i a;
                    int asc;
                    rdA(i, a, asc);
                    mm(i, a, asc);
                }
            }
        } else if constexpr (F8B) {
#pragma unroll
            for (int t = 0; t < 4; ++t) hook(t);
            // one fp8 x fp8 MFMA per 16 x 16 tile covers the whole 128-K step (A bytes
            // 0-15: K 16 quad + [0,16), bytes 16-31: K 64 + 16 quad + [0,16); the INT8
            // weight packing holds the same K in its two 64-K halves)
            const float swv = ((const float*)sS)[BM];
            const int sw8 = swz(col, AUNITS);
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                const int row = wm * (BM / WM) + i * 16 + col;
                const v4u lo = *(const v4u*)(sA + row * AROW + ((quad ^ sw8) * 16));
                const v4u hi = *(const v4u*)(sA + row * AROW + (((4 + quad) ^ sw8) * 16));
                const v8i a = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                // this lane's output rows 4 quad .. 4 quad + 3 of tile i
                const v4f sa4 = *(const v4f*)(sS + (wm * (BM / WM) + i * 16 + 4 * quad) * 4) * swv;
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    const v8i b = v8i{(int)bw[j][0][0], (int)bw[j][0][1], (int)bw[j][0][2], (int)bw[j][0][3],
                                      (int)bw[j][1][0], (int)bw[j][1][1], (int)bw[j][1][2], (int)bw[j][1][3]};
                    const v4f part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0x7F, 0, 0x7F);
                    acc[i][j] += part * sa4;
                }
            }
        } else if constexpr (F == Fmt::W8A8_I8) {
            // A fragment (h, i): 16 bytes per lane, unit 4h + quad of the lane's row
            // (rows of a wave's tiles differ by multiples of 16, so the swizzle
            // depends on the lane's column only), streamed through a ring of four,
            // three fragments ahead of its MFMAs
            const int sw8 = swz(col, AUNITS);
            const uint32_t a_h[2] = {(uint32_t)((wm * (BM / WM) + col) * AROW + ((quad ^ sw8) * 16)),
                                     (uint32_t)((wm * (BM / WM) + col) * AROW + (((4 + quad) ^ sw8) * 16))};
            constexpr int NQ = 2 * MT;
            auto rdA = [&](int q) -> v4u { return *(const v4u*)(sA + a_h[q / MT] + (q % MT) * 16 * AROW); };
            v4u ar[4];
#pragma unroll
            for (int q = 0; q < 3 && q < NQ; ++q) ar[q] = rdA(q);
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const int h = q / MT, i = q % MT;
                if (q == 0) {
#pragma unroll
                    for (int t = 0; t < 4; ++t) hook(t);
                }
                if (q + 3 < NQ) ar[(q + 3) % 4] = rdA(q + 3);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int j = 0; j < NT; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(v4i, ar[q % 4]), __builtin_bit_cast(v4i, bw[j][h]), acc[i][j], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    // ---- pipeline: LDS holds steps s and s+1; registers (PD > 0) hold s+1 .. s+PD ----
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    if constexpr (PD == 0) {
        // two stages: the A / weight tiles of step s+1 load while step s
        // computes; the scale block of s+1 lands in registers and is written to
        // its LDS array after the step's wait.  The builtin waits (unlike inline
        // asm) tell the compiler which loads have landed, so it adds none of its
        // own that would drain the prefetch.
        if (k0 < k1) {
            sc_load(k0, S0{});
            dma(k0, S0{});
            wait_vmcnt<0>();
            sc_write(S0{}, S0{});
            lds_sync();
        }
        // whole pairs of steps (one loop exit keeps the accumulators in place),
        // then an odd last step; step ks is always in stage 0 at the loop top
        int ks = k0;
        for (; ks + 1 < k1; ks += 2) {
            compute(S0{}, [&](int t) {
                if (t != 0) return;
                sc_load(ks + 1, S0{});
                dma(ks + 1, S1{});
            });
            wait_vmcnt<0>();
            sc_write(S1{}, S0{});
            lds_sync();
            const bool more = ks + 2 < k1;
            compute(S1{}, [&](int t) {
                if (!more || t != 0) return;
                sc_load(ks + 2, S0{});
                dma(ks + 2, S0{});
            });
            wait_vmcnt<0>();
            if (more) sc_write(S0{}, S0{});
            lds_sync();
        }
        if (ks < k1) compute(S0{}, nohook);
    } else if constexpr (PD == 4) {
        // a ring of NST = 3 or 4 stages: the loads of steps s+1 .. s+NST-1 fly
        // while step s computes (INT8 tiles at mid M, whose steps are short
        // next to the load latency; W4A8 256x256 tiles, whose loads take
        // longer than one step of MFMAs).  Unrolled by the stage count, with an
        // unconditional refill: steps past the slice load bytes that are never
        // computed (other rows' data or zeros, always inside the buffer
        // resources), so every point of the loop has the same loads
        // outstanding on every path and the explicit waits hold for the
        // compiler too.
        // A step's scale block comes with its loads: straight into the stage
        // (MX MFMA formats), or into the stage's register set and on to the
        // stage's LDS array once landed (blockwise fp8).  The block's fetching
        // threads issue one or two loads more per step than the others;
        // counting only the tile loads makes their wait stricter, never looser.
        constexpr int NL = NIA + NIB;  // direct loads per thread and step
        using S2 = std::integral_constant<int, 2>;
        using S3 = std::integral_constant<int, 3>;
        auto fetch = [&](int s, auto stc) {
            sc_load(s, stc);
            dma(s, stc);
        };
        fetch(k0, S0{});
        fetch(k0 + 1, S1{});
        if constexpr (NST == 4) fetch(k0 + 2, S2{});
        auto step = [&](int s, auto cur, auto refill) {
            wait_vmcnt<(NST - 2) * NL>();  // step s has landed (the later ones may fly)
            if constexpr (SC_STAGE > 0 && !SC_DMA) {
                sc_write(cur, cur);
                lds_sync();  // the scale block written, and every wave done with step s-1's stage
            } else {
                lds_barrier();  // every wave's loads of step s landed, and every wave done with step s-1's stage
            }
            fetch(s + NST - 1, refill);
            if (s < k1) compute(cur, nohook);
        };
        for (int ks = k0; ks < k1; ks += NST) {
            if constexpr (NST == 4) {
                step(ks, S0{}, S3{});
                step(ks + 1, S1{}, S0{});
                step(ks + 2, S2{}, S1{});
                step(ks + 3, S3{}, S2{});
            } else {
                step(ks, S0{}, S2{});
                step(ks + 1, S1{}, S0{});
                step(ks + 2, S2{}, S1{});
            }
        }
        wait_vmcnt<0>();  // the steps past the loop (never computed)
    } else if constexpr (PD == 3) {
        // as PD = 0; the single weight stage is refilled once every wave holds
        // its fragments of the current step (the barrier in the hook at t = 0)
        if (k0 < k1) {
            sc_load(k0, S0{});
            dma(k0, S0{});
            wait_vmcnt<0>();
            sc_write(S0{}, S0{});
            lds_sync();
        }
        int ks = k0;
        for (; ks + 1 < k1; ks += 2) {
            compute(S0{}, [&](int t) {
                if (t != 0) return;
                lds_sync();
                sc_load(ks + 1, S0{});
                dma(ks + 1, S1{});
            });
            wait_vmcnt<0>();
            sc_write(S1{}, S0{});
            lds_sync();
            const bool more = ks + 2 < k1;
            compute(S1{}, [&](int t) {
                if (!more || t != 0) return;
                lds_sync();
                sc_load(ks + 2, S0{});
                dma(ks + 2, S0{});
            });
            wait_vmcnt<0>();
            if (more) sc_write(S0{}, S0{});
            lds_sync();
        }
        if (ks < k1) compute(S0{}, nohook);
    } else {
        if (k0 < k1) {
            gload(k0, S0{});
            if constexpr (PD == 2)
                if (k0 + 1 < k1) gload(k0 + 1, S1{});
            swrite(S0{}, S0{});
            __syncthreads();
        }
        for (int ks = k0; ks < k1; ks += 2) {
            // step ks from stage 0
            if (ks + PD < k1) gload(ks + PD, S0{});
            compute(S0{}, nohook);
            if (ks + 1 < k1) swrite(S1{}, S1{});
            __syncthreads();
            if (ks + 1 >= k1) break;
            // step ks+1 from stage 1
            if (ks + 1 + PD < k1) gload(ks + 1 + PD, S1{});
            compute(S1{}, nohook);
            if (ks + 2 < k1) swrite(S0{}, S0{});
            __syncthreads();
        }
    }

    // ---- epilogue: lane (col, quad) holds rows 4*quad + r of column col in each 16x16 tile ----
    // The epilogue's scales are loaded before the first store (stores and loads
    // share one counter: a load between stores waits for every store before it).
    constexpr bool ASC = F == Fmt::W4A8_MX || F == Fmt::W8A8_I8, WSC = F == Fmt::W8A8_I8 || w8a16(F);
    const bool partial = p.splits > 1;
    float asr[ASC ? MT : 1][4], swn[WSC ? NT : 1];
    if (!partial) {
        if constexpr (ASC) {
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int lrow = wm * (BM / WM) + i * 16 + quad * 4 + r;
                    asr[i][r] = rowinfo[BM + lrow] >= 0 ? p.a_scale[rowinfo[lrow]] : 0.f;
                }
        }
        if constexpr (WSC) {
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const int n = (pid_n * NSTRIP + wn * NT + j) * 16 + col;
                swn[j] = n < p.N ? ((const float*)Sbase)[n] : 0.f;
            }
        }
    }
    // the output value of accumulator (i, j, r): fp32 partial or int32 bits, or the format's epilogue
    auto outv = [&](int i, int j, int r) -> uint32_t {
        if (partial) return bits32(acc[i][j][r]);
        if constexpr (F == Fmt::WNA16_F16) return f32_to_16<false>(acc[i][j][r]);
        else if constexpr (F == Fmt::W8A8_I8)
            return p.raw_i32 ? (uint32_t)acc[i][j][r] : f32_to_bf16_bits((float)acc[i][j][r] * asr[i][r] * swn[j]);
        else if constexpr (F == Fmt::W4A8_MX) return f32_to_bf16_bits(acc[i][j][r] * asr[i][r]);
        else if constexpr (nvfp4(F)) return f32_to_16<!f16_operand(F)>(acc[i][j][r] * *p.s2);
        else if constexpr (w8a16(F)) return f32_to_16<w8bf(F)>(acc[i][j][r] * swn[j]);
        else return f32_to_16<!f16_operand(F)>(acc[i][j][r]);
    };
    if constexpr (F != Fmt::MOE_MX) {
        // dense: the tile's rows m0 .. m0 + mrows - 1 of the output, or of this K
        // slice's fp32 / int32 partial tile, through a buffer resource that starts
        // at the tile's first row.  Columns past N (Np for partials) and rows past
        // M take an offset outside it and the store is dropped, so no store sits
        // behind a branch (a branch per store makes the compiler wait for every
        // store before it).  The range fits 32 bits: N <= 2^21 (checked at the call).
        const int es = partial || (F == Fmt::W8A8_I8 && p.raw_i32) ? 4 : 2;  // bytes per output element
        const int ld = partial ? p.Np : p.N;                                  // elements per row
        char* base = partial ? (char*)p.part + (((int64_t)split * p.M + m0) * p.Np) * 4 : (char*)p.D + (int64_t)m0 * p.N * es;
        const rsrc_t rO = make_rsrc(base, (uint32_t)mrows * (uint32_t)ld * (uint32_t)es);
        constexpr uint32_t DROP = 0xFFFFFFF0u;  // beyond any range here (at most 2^31 bytes)
        auto store = [&](auto kind) {
            constexpr int K_ = decltype(kind)::value;  // 0: 16-bit, 1: 32-bit, 2: 32-bit non-temporal
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int lr = wm * (BM / WM) + i * 16 + quad * 4 + r;
#pragma unroll
                    for (int j = 0; j < NT; ++j) {
                        const int n = (pid_n * NSTRIP + wn * NT + j) * 16 + col;
                        const uint32_t off = lr < mrows && n < ld ? ((uint32_t)lr * (uint32_t)ld + (uint32_t)n) * (uint32_t)es : DROP;
                        const uint32_t v = outv(i, j, r);
                        if constexpr (K_ == 0) __builtin_amdgcn_raw_buffer_store_b16((uint16_t)v, rO, off, 0, 0);
                        else if constexpr (K_ == 1) __builtin_amdgcn_raw_buffer_store_b32(v, rO, off, 0, 0);
                        else __builtin_amdgcn_raw_buffer_store_b32(v, rO, off, 0, 2);
                    }
                }
        };
        if (partial && p.part_nt) store(std::integral_constant<int, 2>{});
        else if (es == 4) store(std::integral_constant<int, 1>{});
        else store(std::integral_constant<int, 0>{});
    } else {
        // MoE: scattered output rows (a row's pair index), no K split
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int drow = rowinfo[BM + wm * (BM / WM) + i * 16 + quad * 4 + r];
                if (drow < 0) continue;
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    const int n = (pid_n * NSTRIP + wn * NT + j) * 16 + col;
                    if (n >= p.N) continue;
                    ((uint16_t*)p.D)[(int64_t)drow * p.N + n] = (uint16_t)outv(i, j, r);
                }
            }
    }
}

// Split-K finalize shared by the dense launchers: sums the fp32 / int32
// partial tiles [splits][M][Np] in slice order and applies the format's
// epilogue.  One thread per 4 columns of one row; the loads of up to 8 slices
// are issued together (independent 16-byte loads), then added in order.
struct FinalizeArgs {
    const void* part;
    void* D;
    const float* a_scale;  // per-token scale (W4A8 / W8A8)
    const float* s_w;      // per-channel scale (W8A8)
    const float* s2;       // per-tensor second-level scale (NVFP4)
    int M, N, Np, splits, raw_i32;
    int part_nt;           // the partial tiles were stored non-temporally: read them so too
};

template <Fmt F>
__global__ __launch_bounds__(256) void splitk_finalize_kernel(FinalizeArgs p) {
    const int m = blockIdx.y;
    const int n = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (n >= p.N) return;
    const int64_t stride = (int64_t)p.M * p.Np, base = (int64_t)m * p.Np + n, o = (int64_t)m * p.N + n;
    constexpr bool I32 = F == Fmt::W8A8_I8;
    using V = typename std::conditional<I32, v4i, v4f>::type;
    const V* src = (const V*)((const char*)p.part + base * 4);
    const int64_t vstride = stride / 4;  // Np is a multiple of 16
    // non-temporal partial tiles are read with the NT bit (buffer loads; see
    // store_part); one loop per kind, so each keeps its eight loads in flight
    const rsrc_t rP = part_rsrc(const_cast<void*>(p.part), p.part_nt, p.splits, p.M, p.Np);
    auto sum = [&](auto ntc) -> V {
        constexpr bool NT = decltype(ntc)::value;
        auto ld = [&](int s) -> V {
            if constexpr (NT) return __builtin_bit_cast(V, buf16<true>(rP, (uint32_t)((base + (int64_t)s * stride) * 4), 0u));
            else return src[s * vstride];
        };
        V a{};
        for (int s0 = 0; s0 < p.splits; s0 += 8) {  // up to eight slices' loads at once, summed in slice order
            V v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (s0 + j < p.splits) v[j] = ld(s0 + j);
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (s0 + j < p.splits) a = s0 + j == 0 ? v[j] : a + v[j];
        }
        return a;
    };
    V acc = p.part_nt ? sum(std::true_type{}) : sum(std::false_type{});
    const int cnt = p.N - n < 4 ? p.N - n : 4;
    if constexpr (I32) {
        if (p.raw_i32) {
            for (int j = 0; j < cnt; ++j) ((int*)p.D)[o + j] = acc[j];
        } else {
            const float as = p.a_scale[m];
            for (int j = 0; j < cnt; ++j) ((uint16_t*)p.D)[o + j] = f32_to_bf16_bits((float)acc[j] * as * p.s_w[n + j]);
        }
    } else {
        if constexpr (F == Fmt::W4A8_MX) acc *= p.a_scale[m];
        if constexpr (nvfp4(F)) acc *= *p.s2;
        if constexpr (w8a16(F)) acc *= *(const v4f*)(p.s_w + n);  // (s_w padded to a multiple of 16)
        constexpr bool BF = F != Fmt::WNA16_F16 && F != Fmt::W8A16_F16 && F != Fmt::F8W_F16 && !f16_operand(F);
        for (int j = 0; j < cnt; ++j) ((uint16_t*)p.D)[o + j] = f32_to_16<BF>(acc[j]);
    }
}

template <Fmt F>
hipError_t launch_finalize(const FinalizeArgs& f, hipStream_t st) {
    if (plan_recorder()) {
        plan_record("splitk_finalize_kernel<%s>", fmt_name(F));
        return hipSuccess;
    }
    const dim3 grid((unsigned)((f.N + 1023) / 1024), (unsigned)f.M);
    hipLaunchKernelGGL((splitk_finalize_kernel<F>), grid, dim3(256), 0, st, f);
    return hipGetLastError();
}

}  // namespace hq

namespace hq {

// ---- host-side plan shared by the dense launchers ----
struct TilePlan {
    int BM, splits;
    bool wide;  // 256-column tiles: 256 x 256 if BM == 256, else 128 x 256
    int forced; // 0: the heuristic below; else a tuning override (TunePath) with `splits` K slices
};

// Tuning overrides of the kernel choice (the descriptor's tune field).
enum TunePath { TUNE_AUTO = 0, TUNE_STREAM = 1, TUNE_T128 = 2, TUNE_T256 = 3, TUNE_W128 = 4, TUNE_W256 = 5, TUNE_STREAM8 = 6 };

// The largest grids use 256-column tiles where the format has them (256 x 256,
// else 128 x 256), then 256 x 128 tiles on 8 waves; smaller ones 128 x 128
// tiles with K split across workgroups until the grid covers the chip.
inline TilePlan plan_tile(int64_t M, int64_t Np, int64_t K, bool allow256, bool wide256 = false, bool wide128 = false,
                          int64_t wide256_min = 256) {
    const int64_t tn = (Np + 127) / 128, nsteps = K / 128, tn2 = (Np + 255) / 256;
    TilePlan pl{128, 1, false, 0};
    if (wide256 && ((M + 255) / 256) * tn2 >= wide256_min) {
        pl.BM = 256;
        pl.wide = true;
        return pl;
    }
    if (wide128 && ((M + 127) / 128) * tn2 >= 256) {
        pl.wide = true;
        return pl;
    }
    if (allow256 && ((M + 255) / 256) * tn >= 256) {
        pl.BM = 256;
        return pl;
    }
    const int64_t tiles = ((M + 127) / 128) * tn;
    int64_t s = (256 + tiles - 1) / tiles;
    if (s > 8) s = 8;
    if (s > nsteps / 2) s = nsteps / 2;
    pl.splits = (int)(s < 1 ? 1 : s);
    return pl;
}

template <Fmt F, int BM, int BN, int WM, int WN, int PD>
hipError_t launch_tile_kernel(TileArgs p, hipStream_t st) {
    if (p.max_splits > 0 && p.splits > p.max_splits) p.splits = p.max_splits;
    p.tiles_m = (int)((p.M + BM - 1) / BM);
    p.tiles_n = (int)((p.Np + BN - 1) / BN);
    p.part_nt = part_nontemporal(p.splits, p.M, p.Np);
    const int64_t grid = (int64_t)p.tiles_m * p.tiles_n * p.splits;
    if (plan_recorder()) {
        plan_record("tile_gemm_kernel<%s,%d,%d,%d,%d,%d> grid=%lld splits=%d", fmt_name(F), BM, BN, WM, WN, PD,
                    (long long)grid, p.splits);
        if (p.splits > 1) plan_workspace((size_t)p.splits * (size_t)p.M * (size_t)p.Np * 4);
    } else {
        hipLaunchKernelGGL((tile_gemm_kernel<F, BM, BN, WM, WN, PD>), dim3((unsigned)grid), dim3(64 * WM * WN), 0, st, p);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (p.splits == 1) return hipSuccess;
    return launch_finalize<F>(FinalizeArgs{p.part, p.D, p.a_scale, (const float*)p.S, p.s2, p.M, p.N, p.Np, p.splits, p.raw_i32,
                                           p.part_nt},
                              st);
}

// Formats with a 256-row tile.  4-bit weights with 16-bit A: 256 x 128 on 8
// waves of 128 x 32 (two per SIMD, so one wave's LDS reads and dequantisation
// overlap the other's MFMAs), loads straight into LDS (no staging registers).
// W4A8 (8-bit A, no dequantisation): 256 x 256 on 8 waves of 128 x 64, which
// halves the A traffic per flop and still fits two LDS stages.  bf16 A has no
// 256-row variant (its row-sum MFMA needs a second accumulator set).
// INT8 weight-only: 256-row tiles do not fit two stages of its 2 KB weight strips
constexpr bool has_big_tile(Fmt F) { return F != Fmt::WNA16_BF16 && !w8load(F) && !mxf6(F); }
// fp16 A with 4-bit weights: 8 waves side by side, each dequantising its own
// weight strips once: 256 x 256 tiles of 256 x 32 waves with a single weight
// stage (each dequantised fragment feeds 16 MFMAs; 13 % faster than 128 x 256
// at M = 8192), or 128 x 256 tiles of 128 x 32 waves where 256 x 256 would not
// cover the chip (a K step loads 48 KB instead of the 80 KB of 256 x 128).
// (Not the bf16 byte codes with group scales: the 128 x 256 tile's second set
// of per-step accumulators spills, 172 bytes per lane, and ran 1.34x slower
// than 128 x 128 tiles at M = 8192.)
constexpr bool has_wide_tile(Fmt F) {
    return F == Fmt::WNA16_F16 || mxfp4w(F) || nvfp4(F) || mxint4w(F) || (w8load(F) && F != Fmt::W8G_BF16) || mxf6(F);
}
// INT8: 256 x 256 on 8 waves of 128 x 64, direct loads into two full stages
// (M = 8192: 1126 us vs 1569 us for 256 x 128 with register-staged loads); the
// 256 x 128 tile also loads directly (1498 us).
constexpr bool has_wide256_tile(Fmt F) { return (has_wide_tile(F) && !w8load(F) && !mxf6(F)) || F == Fmt::W8A8_I8; }
// 256x256 tiles from this many on: INT8 keeps the 256x128 three-stage ring
// until the wide tiles fill two rounds of the chip (measured: the ring is
// faster at M=1024 and level at M=2048 for N=18432, K=7168)
constexpr int64_t wide256_min_tiles(Fmt F) { return F == Fmt::W8A8_I8 ? 512 : 256; }

// A tuning override: the format's kernel of the requested class with the
// requested K split (hipErrorNotSupported where the format has no such tile).
template <Fmt F>
hipError_t launch_forced(const TilePlan& pl, TileArgs p, hipStream_t st) {
    p.splits = pl.splits < 1 ? 1 : pl.splits;
    constexpr bool RING8 = F == Fmt::W8A8_I8 || F == Fmt::W8A8_F8B;  // tiles on stage rings
    switch (pl.forced) {
        case TUNE_T128:
            if constexpr (RING8 || mx_mfma(F)) return launch_tile_kernel<F, 128, 128, 2, 4, 4>(p, st);
            else return launch_tile_kernel<F, 128, 128, 2, 4, 0>(p, st);
        case TUNE_T256:
            if constexpr (RING8) return launch_tile_kernel<F, 256, 128, 2, 4, 4>(p, st);
            else if constexpr (mx_mfma(F)) return launch_tile_kernel<F, 256, 256, 2, 4, 4>(p, st);
            else if constexpr (has_big_tile(F)) return launch_tile_kernel<F, 256, 128, 2, 4, 0>(p, st);
            else return hipErrorNotSupported;
        case TUNE_W128:
            if constexpr (has_wide_tile(F)) return launch_tile_kernel<F, 128, 256, 1, 8, 0>(p, st);
            else return hipErrorNotSupported;
        case TUNE_W256:
            if constexpr (has_wide_tile(F) && !w8load(F)) return launch_tile_kernel<F, 256, 256, 1, 8, 3>(p, st);
            else if constexpr (F == Fmt::W8A8_I8) return launch_tile_kernel<F, 256, 256, 2, 4, 0>(p, st);
            else if constexpr (mx_mfma(F)) return launch_tile_kernel<F, 256, 256, 2, 4, 4>(p, st);
            else return hipErrorNotSupported;
        default: return hipErrorNotSupported;
    }
}

template <Fmt F>
hipError_t launch_dense_plan(const TilePlan& pl, TileArgs p, hipStream_t st) {
    if (pl.forced) return launch_forced<F>(pl, p, st);
    p.splits = pl.splits;
    if constexpr (F == Fmt::W8A8_I8) {
        if (pl.wide && pl.BM == 256) return launch_tile_kernel<F, 256, 256, 2, 4, 0>(p, st);
        if (pl.BM == 256) {
            // where 256 x 128 ring tiles need two rounds and 256 x 256 tiles fit one
            if (((p.M + 255) / 256) * ((p.Np + 127) / 128) > 256 && ((p.M + 255) / 256) * ((p.Np + 255) / 256) <= 256)
                return launch_tile_kernel<F, 256, 256, 2, 4, 0>(p, st);
            return launch_tile_kernel<F, 256, 128, 2, 4, 4>(p, st);
        }
        // the rings run one workgroup per CU: keep the grid to one round, with
        // 256-row tiles where 128-row ones would need two, and the K split
        // rounded down
        const int64_t tiles = ((p.M + 127) / 128) * ((p.Np + 127) / 128);
        if (tiles > 256 && ((p.M + 255) / 256) * ((p.Np + 127) / 128) <= 256) {
            p.splits = 1;
            return launch_tile_kernel<F, 256, 128, 2, 4, 4>(p, st);
        }
        if (tiles <= 256) {
            const int64_t s = 256 / tiles;
            p.splits = (int)(s < 1 ? 1 : s < pl.splits ? s : pl.splits);
        }
        return launch_tile_kernel<F, 128, 128, 2, 4, 4>(p, st);
    } else {
        if constexpr (F == Fmt::W8A8_F8B) {
            // 128-column tiles (one weight scale block) on stage rings, one round of
            // the chip: 256 rows where that fills it, else 128 rows with K split
            // (from 192 such tiles: at M=1024 N=K=7168, 224 of them take 89.8 us,
            // 448 tiles of 128 x 128 99.0 us)
            if (((p.M + 255) / 256) * ((p.Np + 127) / 128) >= 192) {
                p.splits = 1;
                return launch_tile_kernel<F, 256, 128, 2, 4, 4>(p, st);
            }
            const int64_t tiles = ((p.M + 127) / 128) * ((p.Np + 127) / 128), nsteps = p.K / 128;
            int64_t s = tiles < 256 ? 256 / tiles : 1;
            if (s > 8) s = 8;
            if (s > nsteps / 2) s = nsteps / 2;
            p.splits = (int)(s < 1 ? 1 : s);
            return launch_tile_kernel<F, 128, 128, 2, 4, 4>(p, st);
        }
        if constexpr (mx_mfma(F)) {
            // 8-bit A: a 256-column tile on a three-stage ring (4-bit A: four stages)
            if (pl.BM == 256) return launch_tile_kernel<F, 256, 256, 2, 4, 4>(p, st);
            // mid M: a 128 x 128 step is 8 MFMAs per wave, short next to the load
            // latency.  While the tiles fit one workgroup per CU, a four-stage ring
            // (96 KB) with the K split rounded down to keep one round beats two
            // workgroups per CU on two stages (fewer slices, so the partials and
            // the finalize pass shrink or vanish too)
            // Above 64 rows the K split targets half the chip: a slice's MFMA
            // work grows with M while its loads do not (N=7168 K=4096: M=128 on
            // 2 slices 19.8 against 20.7 us on 4, M=256 unsplit 21.5 against 24.1)
            const int64_t tiles = ((p.M + 127) / 128) * ((p.Np + 127) / 128);
            if (tiles <= 256) {
                const int64_t s = (p.M <= 64 ? 256 : 128) / tiles;
                p.splits = (int)(s < 1 ? 1 : s < pl.splits ? s : pl.splits);
                return launch_tile_kernel<F, 128, 128, 2, 4, 4>(p, st);
            }
        }
        if constexpr (has_wide_tile(F)) {
            if constexpr (!w8load(F))
                if (pl.wide && pl.BM == 256) return launch_tile_kernel<F, 256, 256, 1, 8, 3>(p, st);
            if (pl.wide) return launch_tile_kernel<F, 128, 256, 1, 8, 0>(p, st);
            // from 512 rows, 128 x 256 tiles with the K split filling the chip
            // beat 128 x 128 tiles (each wave dequantises its weights once instead
            // of twice): N=4096 K=7168 fp16, M=512 45.6 against 49.2 us, M=1024
            // 71.9 against 77.0; NVFP4 48.7 against 58.9 and 77.9 against 96.3
            if (p.M >= 512) {
                const int64_t tiles = ((p.M + 127) / 128) * ((p.Np + 255) / 256), nsteps = p.K / 128;
                int64_t s = tiles < 256 ? 256 / tiles : 1;
                if (s > 8) s = 8;
                if (s > nsteps / 2) s = nsteps / 2;
                p.splits = (int)(s < 1 ? 1 : s);
                return launch_tile_kernel<F, 128, 256, 1, 8, 0>(p, st);
            }
        }
        if constexpr (F == Fmt::W8A8_F8B) {
            return hipErrorNotSupported;  // (returned above: no two-stage tiles are built for it)
        } else {
            if constexpr (has_big_tile(F))
                if (pl.BM == 256) return launch_tile_kernel<F, 256, 128, 2, 4, 0>(p, st);
            return launch_tile_kernel<F, 128, 128, 2, 4, 0>(p, st);
        }
    }
}

}  // namespace hq
