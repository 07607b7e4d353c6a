// W4A16 kernels for gfx950: D[M,N] = A[M,K] x dequant(W), W symmetric INT4 or
// UINT4 with zero-points, one 16-bit scale per (group of G along K, column).
//
// Method: "Humming wird angekuendigt", section "WnA16" (dense W4A16 with
// fp16/bf16 activations) and section "Gemeinsam genutzte CUDA-Komponenten"
// (dequantisation and scaling fused into the GEMM's compute).  The design
// below is our own for CDNA4: 64-wide wavefronts, MFMA 16x16x32, packed
// weights laid out so that one 16-byte load per lane is one MFMA B fragment
// for four consecutive K steps.
//
// Small M (M <= 64): a GEMV-like schedule (see the skinny kernel below).  The
// group scale is applied to the fp32 accumulator once per 128-K chunk, so the
// dequantised operand (q - z, an integer in [-15, 15]) is exact in both bf16
// and fp16.  Large M: the LDS-tiled MFMA template in tile_gemm.hpp.
#include "hq_device.hpp"
#include "hq_internal.h"
#include "tile_gemm.hpp"

namespace hq {

// -------------------------------------------------------------------------
// 4-bit decode.  A packed word holds eight codes in pair order: nibble p is
// element {0,2,4,6,1,3,5,7}[p], so (w >> 4s) & 0x000F000F puts elements 2s
// and 2s+1 in the low and high 16-bit halves.
// -------------------------------------------------------------------------

// fp16: (0x6400 | u) is 1024 + u exactly; one packed add of -(1024 + z)
// gives u - z exactly.
__device__ __forceinline__ Frag8 deq4_f16(uint32_t w, uint32_t nbias2) {
    const uint32_t m = 0x000F000Fu, c = 0x64006400u;
    const v2h nb = __builtin_bit_cast(v2h, nbias2);
    Frag8 f;
    f.u[0] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, (w & m) | c) + nb);
    f.u[1] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, ((w >> 4) & m) | c) + nb);
    f.u[2] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, ((w >> 8) & m) | c) + nb);
    f.u[3] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, ((w >> 12) & m) | c) + nb);
    return f;
}

// bf16: (0x4300 | u) is 128 + u exactly.  The offset -(128 + z) is added by a
// second MFMA against a constant fragment, which keeps every operand exact.
__device__ __forceinline__ Frag8 deq4_bf16_biased(uint32_t w) {
    const uint32_t m = 0x000F000Fu, c = 0x43004300u;
    Frag8 f;
    f.u[0] = (w & m) | c;
    f.u[1] = ((w >> 4) & m) | c;
    f.u[2] = ((w >> 8) & m) | c;
    f.u[3] = ((w >> 12) & m) | c;
    return f;
}

// -------------------------------------------------------------------------
// small-M kernel
//
// Workgroup = 4 waves covering NS strips (16 columns each) and one K slice.
// Waves split the workgroup as WS strip-columns x WK K-parts; each wave owns
// SPW strips.  Every wave first issues all of its packed-weight loads into
// registers (the HBM stream), then the workgroup copies the A slice, the
// slice's group scales and zero-points into LDS with direct-to-LDS loads; one
// wait, one barrier, then decode + MFMA with A fragments read from LDS.  The
// K-parts reduce through LDS; K slices (split-K) write fp32 partial tiles to
// the workspace and a finalize kernel sums them in slice order.
// -------------------------------------------------------------------------

constexpr int kSkinnyLds = 150 * 1024;

__device__ __forceinline__ void lds_dma16(const void* g, char* lds_wave_base) {
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}
__device__ __forceinline__ void lds_dma4(const void* g, char* lds_wave_base) {
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_wave_base, 4, 0, 0);
}

struct SkinnyArgs {
    const uint16_t* A;
    const v4u* W;
    const uint16_t* S;
    const uint32_t* Z;   // packed zero-points as 32-bit words (two per strip-group)
    uint16_t* D;
    float* part;
    int M, K, N, Np, nc, ngroups, gchunks, splits;
    int NS, WS;          // strips per workgroup, wave strip-columns (WK = 4 / WS)
    int a_off, s_off, z_off, gslab_max;  // LDS layout (bytes / groups)
};

template <bool BF16, bool ZP, int MT, int SPW, int CPW>
__global__ __launch_bounds__(256) void wna16_skinny_kernel(SkinnyArgs p) {
    __shared__ __attribute__((aligned(1024))) char lds[kSkinnyLds];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, quad = lane >> 4;
    const int WS = p.WS, WK = 4 / WS;
    const int ws = wave % WS, wk = wave / WS;
    const int nstrips = p.Np / 16;
    const int strip_base = blockIdx.x * p.NS;
    const int split = blockIdx.y;
    // K slice of the workgroup, in 128-K chunks, and of this wave
    const int c0 = (int)((int64_t)split * p.nc / p.splits), c1 = (int)((int64_t)(split + 1) * p.nc / p.splits);
    const int cw0 = c0 + (c1 - c0) * wk / WK, cw1 = c0 + (c1 - c0) * (wk + 1) / WK;
    const int g0 = c0 / p.gchunks, gslab = (c1 - 1) / p.gchunks - g0 + 1;
    const int U = (c1 - c0) * 16;  // 16-byte units per A row in LDS

    // ---- 1. A slice, scales and zero-points -> LDS (direct loads, issued first) ----
    {
        const int slots = p.M * U;
        const char* Abase = (const char*)p.A + (size_t)c0 * 256;
        for (int ib = wave * 64; ib < slots; ib += 256) {
            const int s = ib + lane;
            if (s < slots) {
                const int row = s / U, pos = s % U;
                const int unit = pos ^ (row & 15);
                lds_dma16(Abase + (size_t)row * p.K * 2 + unit * 16, lds + p.a_off + ib * 16);
            }
        }
        const int sunits = p.NS * gslab * 2;  // 32 bytes of scales per (strip, group)
        for (int ib = wave * 64; ib < sunits; ib += 256) {
            const int s = ib + lane;
            if (s < sunits) {
                const int j = s / (gslab * 2), u = s % (gslab * 2);
                const int st = strip_base + j < nstrips ? strip_base + j : nstrips - 1;
                lds_dma16((const char*)p.S + ((size_t)st * p.ngroups + g0) * 32 + u * 16, lds + p.s_off + ib * 16);
            }
        }
        if constexpr (ZP) {
            const int zwords = p.NS * gslab * 2;  // two 32-bit words per (strip, group)
            for (int ib = wave * 64; ib < zwords; ib += 256) {
                const int s = ib + lane;
                if (s < zwords) {
                    const int j = s / (gslab * 2), u = s % (gslab * 2);
                    const int st = strip_base + j < nstrips ? strip_base + j : nstrips - 1;
                    lds_dma4(p.Z + ((size_t)st * p.ngroups + g0) * 2 + u, lds + p.z_off + ib * 4);
                }
            }
        }
    }

    // ---- 2. the wave's packed weights: CPW loads per strip, all in flight at once.
    //         Indices past the wave's range repeat its last chunk (never used); a wave
    //         with an empty range (more K-parts than chunks) re-reads the slice's first
    //         chunk, so every load stays inside the strip. ----
    const int wlast = cw1 > cw0 ? cw1 - 1 : c0;
    v4u w[SPW][CPW];
    int wstrip[SPW];
#pragma unroll
    for (int sp = 0; sp < SPW; ++sp) {
        wstrip[sp] = strip_base + ws * SPW + sp;
        const int st = wstrip[sp] < nstrips ? wstrip[sp] : nstrips - 1;
        const v4u* Wst = p.W + (size_t)st * p.nc * 64 + lane;
#pragma unroll
        for (int i = 0; i < CPW; ++i) w[sp][i] = ld_nt(Wst + (size_t)min(cw0 + i, wlast) * 64);
    }
    // wait for this wave's LDS copies (issued before the SPW*CPW weight loads), then for everyone's
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(SPW * CPW) : "memory");
    __syncthreads();

    // ---- 3. decode + MFMA, group scale on the fp32 accumulator ----
    v4f acc[SPW][MT];
#pragma unroll
    for (int sp = 0; sp < SPW; ++sp)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[sp][mt] = v4f{0.f, 0.f, 0.f, 0.f};
    const char* lA = lds + p.a_off;
    const uint16_t* lS = (const uint16_t*)(lds + p.s_off);
    const uint32_t* lZ = (const uint32_t*)(lds + p.z_off);
    Frag8 ones;
    ones.u = v4u{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};

    for (int cb = cw0; cb < cw1; cb += CPW) {
        if (cb != cw0) {  // K longer than one register batch: fetch the next batch
#pragma unroll
            for (int sp = 0; sp < SPW; ++sp) {
                const int st = wstrip[sp] < nstrips ? wstrip[sp] : nstrips - 1;
                const v4u* Wst = p.W + (size_t)st * p.nc * 64 + lane;
#pragma unroll
                for (int i = 0; i < CPW; ++i) w[sp][i] = ld_nt(Wst + (size_t)min(cb + i, cw1 - 1) * 64);
            }
        }
#pragma unroll
        for (int i = 0; i < CPW; ++i) {
            const int c = cb + i;
            if (c >= cw1) break;
            // A fragments of this chunk (rows >= M read row M-1; their outputs are dropped)
            Frag8 af[MT][4];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                int row = mt * 16 + col;
                row = row < p.M ? row : p.M - 1;
                const char* ar = lA + (size_t)row * U * 16;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int unit = (c - c0) * 16 + 4 * quad + t;
                    af[mt][t].u = *(const v4u*)(ar + ((unit ^ (row & 15)) * 16));
                }
            }
            const int g = c / p.gchunks - g0;
            v4f rs[MT];
            if constexpr (BF16) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    rs[mt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int t = 0; t < 4; ++t) rs[mt] = mfma16<true>(af[mt][t], ones, rs[mt]);
                }
            }
#pragma unroll
            for (int sp = 0; sp < SPW; ++sp) {
                const int j = ws * SPW + sp;
                const float sc = bits16_to_f32<BF16>(lS[(j * gslab + g) * 16 + col]);
                uint32_t z = 8;
                if constexpr (ZP) z = (lZ[(j * gslab + g) * 2 + (col >> 3)] >> (4 * (col & 7))) & 15u;
                v4f gacc[MT];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) gacc[mt] = v4f{0.f, 0.f, 0.f, 0.f};
                const uint32_t nbz = 0xE400u | z;  // fp16 bits of -(1024 + z)
                const uint32_t nbias2 = nbz | (nbz << 16);
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    uint32_t word = w[sp][i][t];
                    if constexpr (!ZP) word ^= 0x88888888u;  // two's complement -> offset binary
                    Frag8 b;
                    if constexpr (BF16) b = deq4_bf16_biased(word);
                    else b = deq4_f16(word, nbias2);
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) gacc[mt] = mfma16<BF16>(af[mt][t], b, gacc[mt]);
                }
                if constexpr (BF16) {
                    const float zc = (float)(128u + z);
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) acc[sp][mt] += sc * (gacc[mt] - zc * rs[mt]);
                } else {
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) acc[sp][mt] += sc * gacc[mt];
                }
            }
        }
    }

    // ---- 4. reduce the K-parts of the workgroup through LDS ----
    if (WK > 1) {
        __syncthreads();  // the A slice is no longer needed
        float* red = (float*)lds;
        if (wk > 0) {
#pragma unroll
            for (int sp = 0; sp < SPW; ++sp)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        red[((((wk - 1) * WS + ws) * SPW + sp) * MT * 4 + mt * 4 + r) * 64 + lane] = acc[sp][mt][r];
        }
        __syncthreads();
        if (wk == 0)
            for (int k2 = 1; k2 < WK; ++k2)
#pragma unroll
            for (int sp = 0; sp < SPW; ++sp)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                            acc[sp][mt][r] += red[((((k2 - 1) * WS + ws) * SPW + sp) * MT * 4 + mt * 4 + r) * 64 + lane];
    }
    // waves of K-part 0 own the results; the others stay alive for the barriers below
    const bool owner = wk == 0;

    // ---- 5. output: lane (col, quad) holds rows mt*16 + 4*quad + r of its strip's column col ----
    if (p.splits == 1) {
        if (!owner) return;
#pragma unroll
        for (int sp = 0; sp < SPW; ++sp) {
            const int n = wstrip[sp] * 16 + col;
            if (wstrip[sp] >= nstrips || n >= p.N) continue;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = mt * 16 + quad * 4 + r;
                    if (m < p.M) p.D[(size_t)m * p.N + n] = f32_to_16<BF16>(acc[sp][mt][r]);
                }
        }
        return;
    }
#pragma unroll
    for (int sp = 0; sp < SPW; ++sp) {
        if (!owner || wstrip[sp] >= nstrips) continue;
        const int n = wstrip[sp] * 16 + col;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = mt * 16 + quad * 4 + r;
                if (m < p.M) p.part[((size_t)split * p.M + m) * p.Np + n] = acc[sp][mt][r];
            }
    }
}

// Split-K finalize: D[m][n] = sum over slices s = 0..S-1 (in order) of part[s][m][n].
template <bool BF16>
__global__ __launch_bounds__(256) void splitk_finalize_kernel(const float* __restrict__ part, int S, int M, int N, int Np,
                                                              uint16_t* __restrict__ D) {
    const int64_t total = (int64_t)M * N;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
        const int m = (int)(e / N), n = (int)(e % N);
        const float* pp = part + (size_t)m * Np + n;
        float v = 0.f;
        for (int sl = 0; sl < S; ++sl) v += pp[(size_t)sl * M * Np];
        D[e] = f32_to_16<BF16>(v);
    }
}

// -------------------------------------------------------------------------
// host-side planning and launch
// -------------------------------------------------------------------------

namespace {

struct SkinnyPlan {
    int NS, WS, SPW, splits, MT, CPW;
    int a_off, s_off, z_off;
    int64_t groups_x;
};

SkinnyPlan plan_skinny(int64_t M, int64_t Np, int64_t K, int G) {
    const int64_t nstrips = Np / 16, nc = K / 128, gch = G / 128;
    SkinnyPlan p{};
    // strips per workgroup grow with M so the A slice is re-read ~nstrips/NS times
    p.NS = M <= 8 ? 1 : M <= 16 ? 2 : M <= 32 ? 4 : 8;
    while (p.NS > 1 && p.NS > nstrips) p.NS /= 2;
    p.SPW = p.NS <= 4 ? 1 : p.NS / 4;
    p.WS = p.NS / p.SPW;  // 1, 2 or 4 wave strip-columns
    const int WK = 4 / p.WS;
    p.groups_x = cdiv(nstrips, p.NS);
    // K slices: enough workgroups to cover the chip, A slice within the LDS budget
    int64_t S = cdiv(256, p.groups_x);
    auto lds_need = [&](int64_t s) {
        const int64_t cmax = cdiv(nc, s);
        const int64_t gmax = cmax / gch + 2;
        const int64_t a = ((M * cmax * 256 + 1023) / 1024) * 1024;
        const int64_t sc = ((p.NS * gmax * 32 + 1023) / 1024) * 1024;
        const int64_t z = ((p.NS * gmax * 8 + 1023) / 1024) * 1024;
        return a + sc + z;
    };
    while (S < nc / WK && lds_need(S) > kSkinnyLds) ++S;
    if (S > nc / WK) S = nc / WK > 0 ? nc / WK : 1;
    if (S < 1) S = 1;
    p.splits = (int)S;
    const int64_t cmax = cdiv(nc, S), gmax = cmax / gch + 2;
    p.a_off = 0;
    p.s_off = (int)(((M * cmax * 256 + 1023) / 1024) * 1024);
    p.z_off = p.s_off + (int)(((p.NS * gmax * 32 + 1023) / 1024) * 1024);
    p.MT = (int)cdiv(M < 1 ? 1 : M, 16);
    // weight loads per wave and strip: the smallest instantiated batch that covers the wave's chunks
    const int64_t per = cdiv(cmax, WK);
    if (p.SPW == 1) p.CPW = per <= 2 ? 2 : per <= 4 ? 4 : per <= 8 ? 8 : per <= 14 ? 14 : 16;
    else p.CPW = per <= 4 ? 4 : per <= 7 ? 7 : 8;
    return p;
}

template <bool BF16, bool ZP, int MT, int SPW, int CPW>
hipError_t launch_skinny_k(const SkinnyPlan& pl, const SkinnyArgs& a, hipStream_t st) {
    dim3 grid((unsigned)pl.groups_x, (unsigned)pl.splits), block(256);
    hipLaunchKernelGGL((wna16_skinny_kernel<BF16, ZP, MT, SPW, CPW>), grid, block, 0, st, a);
    return hipGetLastError();
}

template <bool BF16, bool ZP, int MT, int SPW>
hipError_t launch_skinny_mt(const SkinnyPlan& pl, const SkinnyArgs& a, hipStream_t st) {
    if constexpr (SPW == 1) {
        switch (pl.CPW) {
            case 2: return launch_skinny_k<BF16, ZP, MT, 1, 2>(pl, a, st);
            case 4: return launch_skinny_k<BF16, ZP, MT, 1, 4>(pl, a, st);
            case 8: return launch_skinny_k<BF16, ZP, MT, 1, 8>(pl, a, st);
            case 14: return launch_skinny_k<BF16, ZP, MT, 1, 14>(pl, a, st);
            default: return launch_skinny_k<BF16, ZP, MT, 1, 16>(pl, a, st);
        }
    } else {
        switch (pl.CPW) {
            case 4: return launch_skinny_k<BF16, ZP, MT, 2, 4>(pl, a, st);
            case 7: return launch_skinny_k<BF16, ZP, MT, 2, 7>(pl, a, st);
            default: return launch_skinny_k<BF16, ZP, MT, 2, 8>(pl, a, st);
        }
    }
}

template <bool BF16, bool ZP>
hipError_t launch_skinny(const DenseArgs& a) {
    SkinnyPlan pl = plan_skinny(a.M, a.Np, a.K, a.group_size);
    if (pl.z_off + ((pl.NS * (cdiv(a.K / 128, pl.splits) / (a.group_size / 128) + 2) * 8 + 1023) / 1024) * 1024 > kSkinnyLds)
        return hipErrorInvalidValue;  // shape beyond the LDS plan (validated on the host side)
    SkinnyArgs s{};
    s.A = (const uint16_t*)a.A;
    s.W = (const v4u*)a.w;
    s.S = (const uint16_t*)a.s;
    s.Z = (const uint32_t*)a.z;
    s.D = (uint16_t*)a.D;
    s.part = (float*)a.ws;
    s.M = (int)a.M;
    s.K = (int)a.K;
    s.N = (int)a.N;
    s.Np = (int)a.Np;
    s.nc = (int)(a.K / 128);
    s.ngroups = (int)(a.K / a.group_size);
    s.gchunks = a.group_size / 128;
    s.splits = pl.splits;
    s.NS = pl.NS;
    s.WS = pl.WS;
    s.a_off = pl.a_off;
    s.s_off = pl.s_off;
    s.z_off = pl.z_off;
    hipError_t e;
    if (pl.SPW == 2) {
        switch (pl.MT) {
            case 1: e = launch_skinny_mt<BF16, ZP, 1, 2>(pl, s, a.stream); break;
            case 2: e = launch_skinny_mt<BF16, ZP, 2, 2>(pl, s, a.stream); break;
            case 3: e = launch_skinny_mt<BF16, ZP, 3, 2>(pl, s, a.stream); break;
            default: e = launch_skinny_mt<BF16, ZP, 4, 2>(pl, s, a.stream); break;
        }
    } else {
        switch (pl.MT) {
            case 1: e = launch_skinny_mt<BF16, ZP, 1, 1>(pl, s, a.stream); break;
            case 2: e = launch_skinny_mt<BF16, ZP, 2, 1>(pl, s, a.stream); break;
            case 3: e = launch_skinny_mt<BF16, ZP, 3, 1>(pl, s, a.stream); break;
            default: e = launch_skinny_mt<BF16, ZP, 4, 1>(pl, s, a.stream); break;
        }
    }
    if (e != hipSuccess || pl.splits == 1) return e;
    int64_t blocks = cdiv(a.M * a.N, 256);
    if (blocks > 2048) blocks = 2048;
    hipLaunchKernelGGL((splitk_finalize_kernel<BF16>), dim3((unsigned)blocks), dim3(256), 0, a.stream, (const float*)s.part,
                       pl.splits, (int)a.M, (int)a.N, (int)a.Np, (uint16_t*)a.D);
    return hipGetLastError();
}

template <Fmt F>
hipError_t launch_tile(const DenseArgs& a) {
    TileArgs p{};
    p.A = a.A;
    p.W = a.w;
    p.S = a.s;
    p.Z = a.z;
    p.D = a.D;
    p.part = a.ws;
    p.M = (int)a.M;
    p.a_rows = (int)a.M;
    p.N = (int)a.N;
    p.K = (int)a.K;
    p.Np = (int)a.Np;
    p.ngroups = (int)(a.K / a.group_size);
    p.gsteps = a.group_size / 128;
    return launch_dense_plan<F>(plan_tile(a.M, a.Np, a.K, has_big_tile(F)), p, a.stream);
}

template <bool BF16, bool ZP>
hipError_t launch_all(const DenseArgs& a) {
    if (a.M <= 64) return launch_skinny<BF16, ZP>(a);
    if constexpr (BF16) return launch_tile<Fmt::WNA16_BF16>(a);
    return launch_tile<Fmt::WNA16_F16>(a);
}

}  // namespace

size_t wna16_workspace(int64_t M, int64_t N, int64_t K, int group_size, bool bf16) {
    const int64_t Np = pad16(N);
    if (M > 64) return tile_workspace(plan_tile(M, Np, K, has_big_tile(bf16 ? Fmt::WNA16_BF16 : Fmt::WNA16_F16)), M, Np);
    SkinnyPlan p = plan_skinny(M, Np, K, group_size);
    if (p.splits <= 1) return 0;
    return (size_t)p.splits * (size_t)M * (size_t)Np * sizeof(float);
}

hipError_t wna16_launch(const DenseArgs& a, bool bf16, bool zp) {
    if (bf16) return zp ? launch_all<true, true>(a) : launch_all<true, false>(a);
    return zp ? launch_all<false, true>(a) : launch_all<false, false>(a);
}

}  // namespace hq
