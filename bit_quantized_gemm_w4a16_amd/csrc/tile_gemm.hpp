// LDS-tiled MFMA GEMM template for gfx950, shared by every weight format.
//
// One workgroup (4 waves, 2 x 2) computes a BM x BN tile of D.  Each K step
// covers 128 input features: the A tile (BM rows x 128 K, 16- or 8-bit) and
// the packed weight tile (BN/16 strips x one K step) are fetched with 16-byte
// global loads into registers while step s-1 computes, then written to the
// other half of a double-buffered LDS stage, so the copy of step s+1 overlaps
// the MFMAs of step s.  A rows are XOR-swizzled in LDS so that the 16 rows a
// fragment read touches fall in distinct banks.  The packed weight chunk of a
// strip is, lane for lane, the MFMA B fragment, so it is copied unchanged.
//
// Formats (the decode runs in registers between the LDS read and the MFMA):
//   WNA16_F16   fp16 A; INT4/UINT4 -> (q - z) * s folded into the fp16 operand
//   WNA16_BF16  bf16 A; operand 128 + u (exact), the -(128 + z) offset via a
//               row-sum MFMA, group scale applied to the fp32 accumulator
//   W4A8_MX     fp8-e4m3 A x e2m1 B on the scaled MFMA (E8M0 B scale per
//               32 K), per-token scale in the epilogue
//   W8A8_I8     int8 x int8 -> int32 (exact), per-token x per-channel epilogue
//   MOE_MX      bf16 A x e2m1 B converted to bf16 with the E8M0 scale (exact)
#pragma once

#include "hq_device.hpp"

namespace hq {

enum class Fmt { WNA16_F16, WNA16_BF16, W4A8_MX, W8A8_I8, MOE_MX };

template <Fmt F> struct FmtTraits;
template <> struct FmtTraits<Fmt::WNA16_F16> { static constexpr int AB = 2, BSTRIP = 1024; using Acc = v4f; };
template <> struct FmtTraits<Fmt::WNA16_BF16> { static constexpr int AB = 2, BSTRIP = 1024; using Acc = v4f; };
template <> struct FmtTraits<Fmt::W4A8_MX> { static constexpr int AB = 1, BSTRIP = 1024; using Acc = v4f; };
template <> struct FmtTraits<Fmt::W8A8_I8> { static constexpr int AB = 1, BSTRIP = 2048; using Acc = v4i; };
template <> struct FmtTraits<Fmt::MOE_MX> { static constexpr int AB = 2, BSTRIP = 1024; using Acc = v4f; };

// Work description of one launch.  Dense launches leave the MoE fields null.
struct TileArgs {
    const void* A;          // activations, row-major [rows][K]
    const float* a_scale;   // per-token fp32 (W4A8 / W8A8), indexed by A row
    const void* W;          // packed weights (expert 0)
    const void* S;          // packed scales (expert 0)
    const void* Z;          // packed zero-points (WNA16 + UINT4)
    void* D;                // output, row-major [rows][N]
    int64_t w_estride, s_estride;  // bytes between experts' packed W / scales
    int M, N, K, Np;
    int ngroups, gsteps;    // WNA16: K / G and G / 128
    int tiles_m, tiles_n;
    int raw_i32;            // W8A8: store int32 accumulators
    // MoE (tiles_m is an upper bound; the real count is *ntiles)
    const int* tile_info;   // per m-tile: expert, first sorted row, row count
    const int* ntiles;      // device count of valid m-tiles
    const int* sorted;      // sorted pair ids (Indexed) or null (Grouped)
    int top_k;
};

__device__ __forceinline__ int swz(int row, int units) {
    return units == 16 ? (row & 15) : ((row >> 1) & 7);
}

// fp16 (q - z) * s for eight codes of one pair-ordered word.
__device__ __forceinline__ Frag8 deq4_f16_scaled(uint32_t w, uint32_t nbias2, uint32_t s2) {
    const uint32_t m = 0x000F000Fu, c = 0x64006400u;
    const v2h nb = __builtin_bit_cast(v2h, nbias2), sc = __builtin_bit_cast(v2h, s2);
    Frag8 f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        v2h x = __builtin_bit_cast(v2h, ((w >> (4 * s)) & m) | c) + nb;
        f.u[s] = __builtin_bit_cast(uint32_t, x * sc);
    }
    return f;
}

__device__ __forceinline__ Frag8 deq4_bf16_offset(uint32_t w) {
    const uint32_t m = 0x000F000Fu, c = 0x43004300u;
    Frag8 f;
#pragma unroll
    for (int s = 0; s < 4; ++s) f.u[s] = ((w >> (4 * s)) & m) | c;
    return f;
}

// e2m1 x 2^(e-127) -> bf16, exact; 8 natural-order codes of one word.
__device__ __forceinline__ Frag8 fp4_to_bf16(uint32_t w, float scale) {
    Frag8 f;
    f.u[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0));
    f.u[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1));
    f.u[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2));
    f.u[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3));
    return f;
}

__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
    e &= 0xFFu;
    return __uint_as_float(e == 0 ? 0x00400000u : e == 255u ? 0x7FC00000u : (e << 23));
}

template <Fmt F, int BM, int BN>
__global__ __launch_bounds__(256, 1) void tile_gemm_kernel(TileArgs p) {
    using T = FmtTraits<F>;
    using Acc = typename T::Acc;
    constexpr bool WNA16 = F == Fmt::WNA16_F16 || F == Fmt::WNA16_BF16;
    constexpr bool MX = F == Fmt::W4A8_MX || F == Fmt::MOE_MX;
    constexpr int AB = T::AB, BK = 128;
    constexpr int AROW = BK * AB, AUNITS = AROW / 16;
    constexpr int A_STAGE = BM * AROW;
    constexpr int NSTRIP = BN / 16;
    constexpr int B_STAGE = NSTRIP * T::BSTRIP;
    // per-step scale block: WNA16 16 fp16 scales + one zero-point word per strip;
    // MXFP4 one E8M0 byte per lane per strip; INT8 none (per-channel, epilogue)
    constexpr int SC_Z = NSTRIP * 32;                     // zero-point words start (WNA16)
    constexpr int SC_STAGE = WNA16 ? NSTRIP * 48 : MX ? NSTRIP * 64 : 0;
    constexpr int SC_UNITS = SC_STAGE / 16;              // 16-byte units (WNA16: 2 scale + 1 zero per strip)
    constexpr int STAGE = A_STAGE + B_STAGE + SC_STAGE;
    constexpr int NIA = A_STAGE / 4096;  // 16-byte loads per lane per stage (A)
    constexpr int NIB = B_STAGE / 4096;  // (B)
    constexpr int MT = BM / 32, NT = BN / 32;  // 16x16 tiles per wave (2 x 2 waves)
    static_assert(A_STAGE % 4096 == 0 && B_STAGE % 4096 == 0, "stage must split evenly over 4 waves");
    static_assert(SC_UNITS <= 256, "one scale unit per thread at most");

    __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];
    __shared__ int rowinfo[2 * BM];  // [0,BM): A row per local row; [BM,2BM): D row (-1 = none)

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int col = lane & 15, quad = lane >> 4;

    // ---- tile coordinates: XCD-aware remap, then grouped raster along M ----
    int bid = blockIdx.x;
    const int nb = gridDim.x;
    if ((nb & 7) == 0) bid = (bid & 7) * (nb >> 3) + (bid >> 3);
    constexpr int GROUP_M = 4;
    const int tiles_n = p.tiles_n;
    const int group_size = GROUP_M * tiles_n;
    const int first_m = (bid / group_size) * GROUP_M;
    const int gm = min(p.tiles_m - first_m, GROUP_M);
    const int pid_m = first_m + (bid % group_size) % gm;
    const int pid_n = (bid % group_size) / gm;

    const char* Wbase = (const char*)p.W;
    const char* Sbase = (const char*)p.S;
    int m0 = pid_m * BM, mrows = BM;
    if constexpr (F == Fmt::MOE_MX) {
        if (pid_m >= *p.ntiles) return;
        const int e = p.tile_info[3 * pid_m], first = p.tile_info[3 * pid_m + 1];
        mrows = p.tile_info[3 * pid_m + 2];
        Wbase += (int64_t)e * p.w_estride;
        Sbase += (int64_t)e * p.s_estride;
        for (int r = tid; r < BM; r += 256) {
            const int rr = r < mrows ? r : mrows - 1;
            const int pos = first + rr;
            const int pair = p.sorted ? p.sorted[pos] : pos;
            rowinfo[r] = p.sorted ? pair / p.top_k : pos;
            rowinfo[BM + r] = r < mrows ? pair : -1;
        }
    } else {
        mrows = min(BM, p.M - m0);
        for (int r = tid; r < BM; r += 256) {
            rowinfo[r] = m0 + (r < mrows ? r : mrows - 1);
            rowinfo[BM + r] = r < mrows ? m0 + r : -1;
        }
    }
    __syncthreads();

    const int K = p.K, nsteps = K / BK;
    const int strip0 = pid_n * NSTRIP, nstrips_total = p.Np / 16;
    auto clamp_strip = [&](int s) { return s < nstrips_total ? s : nstrips_total - 1; };

    // per-lane source offsets of the staged loads (fixed across K steps)
    uint32_t aoff[NIA];
#pragma unroll
    for (int i = 0; i < NIA; ++i) {
        const int s = (wave * NIA + i) * 64 + lane;
        const int row = s / AUNITS, pos = s % AUNITS;
        const int unit = pos ^ swz(row, AUNITS);
        aoff[i] = (uint32_t)((int64_t)rowinfo[row] * K * AB + unit * 16);
    }
    const char* Abase = (const char*)p.A;
    int64_t boff[NIB];
#pragma unroll
    for (int i = 0; i < NIB; ++i) {
        const int s = (wave * NIB + i) * 64 + lane;
        constexpr int UPS = T::BSTRIP / 16;
        const int strip = clamp_strip(strip0 + s / UPS);
        boff[i] = ((int64_t)strip * nsteps) * T::BSTRIP + (s % UPS) * 16;
    }
    // scale unit of this thread (tid < SC_UNITS): strip and part
    const int sc_strip = clamp_strip(strip0 + (WNA16 ? (tid < 2 * NSTRIP ? tid / 2 : tid - 2 * NSTRIP) : tid / 4));

    // global -> registers (issued early, in flight during the MFMAs) ...
    v4u ra[NIA], rb[NIB], rs;
    auto gload = [&](int ks) {
        const char* ga = Abase + (int64_t)ks * AROW;
#pragma unroll
        for (int i = 0; i < NIA; ++i) ra[i] = *(const v4u*)(ga + aoff[i]);
        const char* gb = Wbase + (int64_t)ks * T::BSTRIP;
#pragma unroll
        for (int i = 0; i < NIB; ++i) rb[i] = __builtin_nontemporal_load((const v4u*)(gb + boff[i]));
        if constexpr (WNA16) {
            const int g = ks / p.gsteps;
            if (tid < 2 * NSTRIP) {
                rs = *(const v4u*)(Sbase + (((int64_t)sc_strip * p.ngroups + g) * 16 + (tid & 1) * 8) * 2);
            } else if (tid < 3 * NSTRIP) {
                rs = v4u{0x88888888u, 0x88888888u, 0u, 0u};
                if (p.Z) {
                    const uint32_t* zp = (const uint32_t*)p.Z + ((int64_t)sc_strip * p.ngroups + g) * 2;
                    rs[0] = zp[0];
                    rs[1] = zp[1];
                }
            }
        } else if constexpr (MX) {
            if (tid < SC_UNITS) rs = *(const v4u*)(Sbase + ((int64_t)sc_strip * nsteps + ks) * 64 + (tid & 3) * 16);
        }
    };
    // ... registers -> LDS stage (slot s of this lane: wave-major, 64 lanes per 1 KB)
    auto swrite = [&](int stage) {
        char* sA = smem + stage * STAGE;
        char* sB = sA + A_STAGE;
#pragma unroll
        for (int i = 0; i < NIA; ++i) *(v4u*)(sA + ((wave * NIA + i) * 64 + lane) * 16) = ra[i];
#pragma unroll
        for (int i = 0; i < NIB; ++i) *(v4u*)(sB + ((wave * NIB + i) * 64 + lane) * 16) = rb[i];
        if constexpr (SC_STAGE > 0) {
            char* sS = sB + B_STAGE;
            if constexpr (WNA16) {
                if (tid < 2 * NSTRIP) *(v4u*)(sS + tid * 16) = rs;
                else if (tid < 3 * NSTRIP) *(uint64_t*)(sS + SC_Z + (tid - 2 * NSTRIP) * 8) = ((uint64_t)rs[1] << 32) | rs[0];
            } else {
                if (tid < SC_UNITS) *(v4u*)(sS + tid * 16) = rs;
            }
        }
    };

    Acc acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = Acc{0, 0, 0, 0};

    gload(0);
    swrite(0);
    __syncthreads();

    for (int ks = 0; ks < nsteps; ++ks) {
        const int stage = ks & 1;
        if (ks + 1 < nsteps) gload(ks + 1);
        const char* sA = smem + stage * STAGE;
        const char* sB = sA + A_STAGE;
        const char* sS = sB + B_STAGE;

        // this wave's packed weight words: one 16-byte read per strip (per 64-K half for INT8)
        v4u bw[NT][T::BSTRIP / 1024];
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int h = 0; h < T::BSTRIP / 1024; ++h)
                bw[j][h] = *(const v4u*)(sB + (wn * NT + j) * T::BSTRIP + h * 1024 + lane * 16);

        if constexpr (F == Fmt::WNA16_F16) {
            uint32_t s2[NT], nb2[NT];
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const int sl = wn * NT + j;
                const uint32_t sc = ((const uint16_t*)sS)[sl * 16 + col];
                const uint32_t z = (((const uint32_t*)(sS + SC_Z))[sl * 2 + (col >> 3)] >> (4 * (col & 7))) & 15u;
                s2[j] = sc | (sc << 16);
                const uint32_t nbz = 0xE400u | z;
                nb2[j] = nbz | (nbz << 16);
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                Frag8 b[NT];
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    uint32_t w = bw[j][0][t];
                    if (!p.Z) w ^= 0x88888888u;
                    b[j] = deq4_f16_scaled(w, nb2[j], s2[j]);
                }
#pragma unroll
                for (int i = 0; i < MT; ++i) {
                    const int row = wm * (BM / 2) + i * 16 + col;
                    Frag8 a;
                    a.u = *(const v4u*)(sA + row * AROW + (((4 * quad + t) ^ swz(row, AUNITS)) * 16));
#pragma unroll
                    for (int j = 0; j < NT; ++j) acc[i][j] = mfma16<false>(a, b[j], acc[i][j]);
                }
            }
        } else if constexpr (F == Fmt::WNA16_BF16) {
            float sc[NT], zc[NT];
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const int sl = wn * NT + j;
                sc[j] = bits16_to_f32<true>(((const uint16_t*)sS)[sl * 16 + col]);
                const uint32_t z = (((const uint32_t*)(sS + SC_Z))[sl * 2 + (col >> 3)] >> (4 * (col & 7))) & 15u;
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
                    if (!p.Z) w ^= 0x88888888u;
                    b[j] = deq4_bf16_offset(w);
                }
#pragma unroll
                for (int i = 0; i < MT; ++i) {
                    const int row = wm * (BM / 2) + i * 16 + col;
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
        } else if constexpr (F == Fmt::W4A8_MX) {
            int bsc[NT];
#pragma unroll
            for (int j = 0; j < NT; ++j) bsc[j] = (int)((const uint8_t*)sS)[(wn * NT + j) * 64 + lane];
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                const int row = wm * (BM / 2) + i * 16 + col;
                const int sw = swz(row, AUNITS);
                const v4u lo = *(const v4u*)(sA + row * AROW + ((quad ^ sw) * 16));
                const v4u hi = *(const v4u*)(sA + row * AROW + (((4 + quad) ^ sw) * 16));
                const v8i a = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    const v8i b = v8i{(int)bw[j][0][0], (int)bw[j][0][1], (int)bw[j][0][2], (int)bw[j][0][3], 0, 0, 0, 0};
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[i][j], 0, 4, 0, 0x7F, 0, bsc[j]);
                }
            }
        } else if constexpr (F == Fmt::W8A8_I8) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i = 0; i < MT; ++i) {
                    const int row = wm * (BM / 2) + i * 16 + col;
                    const v4u a = *(const v4u*)(sA + row * AROW + (((4 * h + quad) ^ swz(row, AUNITS)) * 16));
#pragma unroll
                    for (int j = 0; j < NT; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(v4i, a), __builtin_bit_cast(v4i, bw[j][h]), acc[i][j], 0, 0, 0);
                }
        } else {  // MOE_MX
            float sf[NT];
#pragma unroll
            for (int j = 0; j < NT; ++j) sf[j] = e8m0_to_f32(((const uint8_t*)sS)[(wn * NT + j) * 64 + lane]);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                Frag8 b[NT];
#pragma unroll
                for (int j = 0; j < NT; ++j) b[j] = fp4_to_bf16(bw[j][0][t], sf[j]);
#pragma unroll
                for (int i = 0; i < MT; ++i) {
                    const int row = wm * (BM / 2) + i * 16 + col;
                    Frag8 a;
                    a.u = *(const v4u*)(sA + row * AROW + (((4 * quad + t) ^ swz(row, AUNITS)) * 16));
#pragma unroll
                    for (int j = 0; j < NT; ++j) acc[i][j] = mfma16<true>(a, b[j], acc[i][j]);
                }
            }
        }
        // stage s+1 was last read in step s-1 (before the previous barrier)
        if (ks + 1 < nsteps) swrite(stage ^ 1);
        __syncthreads();
    }

    // ---- epilogue: lane (col, quad) holds rows 4*quad + r of column col in each 16x16 tile ----
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int lrow = wm * (BM / 2) + i * 16 + quad * 4 + r;
            const int drow = rowinfo[BM + lrow];
            if (drow < 0) continue;
            float as = 1.f;
            if constexpr (F == Fmt::W4A8_MX || F == Fmt::W8A8_I8) as = p.a_scale[rowinfo[lrow]];
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const int n = (pid_n * NSTRIP + wn * NT + j) * 16 + col;
                if (n >= p.N) continue;
                const int64_t o = (int64_t)drow * p.N + n;
                if constexpr (F == Fmt::WNA16_F16) {
                    ((uint16_t*)p.D)[o] = f32_to_16<false>(acc[i][j][r]);
                } else if constexpr (F == Fmt::W8A8_I8) {
                    if (p.raw_i32) ((int*)p.D)[o] = acc[i][j][r];
                    else ((uint16_t*)p.D)[o] = f32_to_bf16_bits((float)acc[i][j][r] * as * ((const float*)Sbase)[n]);
                } else if constexpr (F == Fmt::W4A8_MX) {
                    ((uint16_t*)p.D)[o] = f32_to_bf16_bits(acc[i][j][r] * as);
                } else {
                    ((uint16_t*)p.D)[o] = f32_to_bf16_bits(acc[i][j][r]);
                }
            }
        }
}

}  // namespace hq
