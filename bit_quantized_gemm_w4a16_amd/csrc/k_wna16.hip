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
// Small M (M <= 64): a GEMV-like schedule.  Each workgroup owns one 16-column
// strip; its waves split K; every wave issues all of its weight loads first
// (the data is streamed once from HBM), then decodes and multiplies.  The
// group scale is applied to the fp32 accumulator once per 128-K chunk, so the
// dequantised operand (q - z, an integer in [-15, 15]) is exact in both bf16
// and fp16.  Waves reduce through LDS; when K is split across workgroups the
// last workgroup to arrive sums the partial tiles in a fixed order.
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
// -------------------------------------------------------------------------

constexpr int kGemvMaxWaves = 8;

template <bool BF16, bool ZP, int MT, int KC>
__global__ __launch_bounds__(64 * kGemvMaxWaves) void wna16_gemv_kernel(
    const uint16_t* __restrict__ A, int M, int K, const v4u* __restrict__ W,
    const uint16_t* __restrict__ S, const uint64_t* __restrict__ Z, int nc, int ngroups,
    int gchunks, uint16_t* __restrict__ D, int N, int Np, float* __restrict__ part,
    unsigned* __restrict__ counters, int splits) {
    __shared__ float red[kGemvMaxWaves * MT * 256];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, WK = blockDim.x >> 6;
    const int strip = blockIdx.x, split = blockIdx.y;
    const int TW = WK * splits, gw = split * WK + wave;
    const int c_begin = (int)((int64_t)gw * nc / TW), c_end = (int)((int64_t)(gw + 1) * nc / TW);
    const int col = lane & 15, quad = lane >> 4;

    v4f acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = v4f{0.f, 0.f, 0.f, 0.f};

    const v4u* Wst = W + (size_t)strip * nc * 64 + lane;
    const uint16_t* Sst = S + (size_t)strip * ngroups * 16 + col;
    for (int cb = c_begin; cb < c_end; cb += KC) {
        v4u w[KC];
#pragma unroll
        for (int i = 0; i < KC; ++i)
            if (cb + i < c_end) w[i] = ld_nt(Wst + (size_t)(cb + i) * 64);
#pragma unroll
        for (int i = 0; i < KC; ++i) {
            const int c = cb + i;
            if (c >= c_end) break;
            const int g = c / gchunks;
            const float sc = bits16_to_f32<BF16>(Sst[(size_t)g * 16]);
            uint32_t z = 8;
            if constexpr (ZP) z = (uint32_t)(Z[(size_t)strip * ngroups + g] >> (4 * col)) & 15u;
            Frag8 af[MT][4];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int row = mt * 16 + col;
                const uint16_t* ap = A + (size_t)row * K + (size_t)c * 128 + quad * 32;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    if (row < M) af[mt][t].u = ld16(ap + 8 * t);
                    else af[mt][t].u = v4u{0u, 0u, 0u, 0u};
                }
            }
            v4f gacc[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) gacc[mt] = v4f{0.f, 0.f, 0.f, 0.f};
            Frag8 bc;
            uint32_t nbias2 = 0;
            if constexpr (BF16) {
                const uint32_t nb = 0xC300u | z;  // bf16 bits of -(128 + z)
                bc.u = v4u{nb | (nb << 16), nb | (nb << 16), nb | (nb << 16), nb | (nb << 16)};
            } else {
                const uint32_t nb = 0xE400u | z;  // fp16 bits of -(1024 + z)
                nbias2 = nb | (nb << 16);
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                uint32_t word = w[i][t];
                if constexpr (!ZP) word ^= 0x88888888u;  // two's complement -> offset binary
                Frag8 b;
                if constexpr (BF16) b = deq4_bf16_biased(word);
                else b = deq4_f16(word, nbias2);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    gacc[mt] = mfma16<BF16>(af[mt][t], b, gacc[mt]);
                    if constexpr (BF16) gacc[mt] = mfma16<BF16>(af[mt][t], bc, gacc[mt]);
                }
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[mt] += sc * gacc[mt];
        }
    }

    if (WK > 1) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[((wave * MT + mt) * 4 + r) * 64 + lane] = acc[mt][r];
        __syncthreads();
        if (wave != 0) return;
        for (int w2 = 1; w2 < WK; ++w2)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[mt][r] += red[((w2 * MT + mt) * 4 + r) * 64 + lane];
    }

    // lane (col, quad) holds rows mt*16 + 4*quad + r of column strip*16 + col
    const int n = strip * 16 + col;
    if (splits == 1) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = mt * 16 + quad * 4 + r;
                if (m < M && n < N) D[(size_t)m * N + n] = f32_to_16<BF16>(acc[mt][r]);
            }
        return;
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = mt * 16 + quad * 4 + r;
            if (m < M) part[((size_t)split * M + m) * Np + n] = acc[mt][r];
        }
    __threadfence();
    unsigned prev = 0;
    if (lane == 0) prev = atomicAdd(&counters[strip], 1u);
    prev = __shfl(prev, 0);
    if (prev != (unsigned)(splits - 1)) return;
    __threadfence();
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = mt * 16 + quad * 4 + r;
            if (m >= M) continue;
            float v = 0.f;
            for (int s = 0; s < splits; ++s) v += part[((size_t)s * M + m) * Np + n];
            if (n < N) D[(size_t)m * N + n] = f32_to_16<BF16>(v);
        }
    if (lane == 0) counters[strip] = 0u;
}

// -------------------------------------------------------------------------
// host-side planning and launch
// -------------------------------------------------------------------------

namespace {

struct GemvPlan {
    int WK, splits, KC, MT;
};

GemvPlan plan_gemv(int64_t M, int64_t Np, int64_t K) {
    const int64_t nstrips = Np / 16, nc = K / 128;
    int64_t target = 2048 / nstrips;  // waves per strip for ~8 waves per CU
    if (target < 1) target = 1;
    if (target > nc) target = nc;
    GemvPlan p;
    p.WK = (int)(target < kGemvMaxWaves ? target : kGemvMaxWaves);
    p.splits = (int)cdiv(target, p.WK);
    if (nstrips > kMaxCounters) p.splits = 1;
    const int64_t per = cdiv(nc, (int64_t)p.WK * p.splits);
    p.KC = per <= 1 ? 1 : per <= 2 ? 2 : per <= 4 ? 4 : 8;
    p.MT = (int)cdiv(M < 1 ? 1 : M, 16);
    return p;
}

template <bool BF16, bool ZP, int MT>
hipError_t launch_mt(const GemvPlan& p, dim3 grid, dim3 block, const DenseArgs& a, int64_t m0,
                     int64_t Mslab, float* part, unsigned* counters) {
    const uint16_t* A = (const uint16_t*)a.A + m0 * a.K;
    uint16_t* D = (uint16_t*)a.D + m0 * a.N;
    const int nc = (int)(a.K / 128), ngroups = (int)(a.K / a.group_size), gchunks = a.group_size / 128;
#define HQ_GEMV_ARGS                                                                                  \
    A, (int)Mslab, (int)a.K, (const v4u*)a.w, (const uint16_t*)a.s, (const uint64_t*)a.z, nc, ngroups, \
        gchunks, D, (int)a.N, (int)a.Np, part, counters, p.splits
    switch (p.KC) {
        case 1: hipLaunchKernelGGL((wna16_gemv_kernel<BF16, ZP, MT, 1>), grid, block, 0, a.stream, HQ_GEMV_ARGS); break;
        case 2: hipLaunchKernelGGL((wna16_gemv_kernel<BF16, ZP, MT, 2>), grid, block, 0, a.stream, HQ_GEMV_ARGS); break;
        case 4: hipLaunchKernelGGL((wna16_gemv_kernel<BF16, ZP, MT, 4>), grid, block, 0, a.stream, HQ_GEMV_ARGS); break;
        default: hipLaunchKernelGGL((wna16_gemv_kernel<BF16, ZP, MT, 8>), grid, block, 0, a.stream, HQ_GEMV_ARGS); break;
    }
#undef HQ_GEMV_ARGS
    return hipGetLastError();
}

template <bool BF16, bool ZP>
hipError_t launch_gemv(const DenseArgs& a, int64_t m0, int64_t Mslab) {
    GemvPlan p = plan_gemv(Mslab, a.Np, a.K);
    dim3 grid((unsigned)(a.Np / 16), (unsigned)p.splits), block(64 * p.WK);
    unsigned* counters = (unsigned*)a.ws;
    float* part = a.ws ? (float*)((char*)a.ws + kCounterBytes) : nullptr;
    switch (p.MT) {
        case 1: return launch_mt<BF16, ZP, 1>(p, grid, block, a, m0, Mslab, part, counters);
        case 2: return launch_mt<BF16, ZP, 2>(p, grid, block, a, m0, Mslab, part, counters);
        case 3: return launch_mt<BF16, ZP, 3>(p, grid, block, a, m0, Mslab, part, counters);
        default: return launch_mt<BF16, ZP, 4>(p, grid, block, a, m0, Mslab, part, counters);
    }
}

template <Fmt F, int BM>
hipError_t launch_tile(const DenseArgs& a) {
    TileArgs p{};
    p.A = a.A;
    p.W = a.w;
    p.S = a.s;
    p.Z = a.z;
    p.D = a.D;
    p.M = (int)a.M;
    p.N = (int)a.N;
    p.K = (int)a.K;
    p.Np = (int)a.Np;
    p.ngroups = (int)(a.K / a.group_size);
    p.gsteps = a.group_size / 128;
    p.tiles_m = (int)cdiv(a.M, BM);
    p.tiles_n = (int)cdiv(a.Np, 128);
    hipLaunchKernelGGL((tile_gemm_kernel<F, BM, 128>), dim3(p.tiles_m * p.tiles_n), dim3(256), 0, a.stream, p);
    return hipGetLastError();
}

template <bool BF16, bool ZP>
hipError_t launch_all(const DenseArgs& a) {
    if (a.M <= 64) return launch_gemv<BF16, ZP>(a, 0, a.M);
    if constexpr (BF16) return launch_tile<Fmt::WNA16_BF16, 128>(a);
    const int64_t tiles_n = cdiv(a.Np, 128);
    if (cdiv(a.M, 256) * tiles_n >= 256) return launch_tile<Fmt::WNA16_F16, 256>(a);
    return launch_tile<Fmt::WNA16_F16, 128>(a);
}

}  // namespace

size_t wna16_workspace(int64_t M, int64_t N, int64_t K, int group_size) {
    (void)group_size;
    const int64_t Np = pad16(N);
    if (M > 64) return 0;  // the tiled kernel needs no workspace
    GemvPlan p = plan_gemv(M, Np, K);
    if (p.splits <= 1) return 0;
    return kCounterBytes + (size_t)p.splits * (size_t)M * (size_t)Np * sizeof(float);
}

hipError_t wna16_launch(const DenseArgs& a, bool bf16, bool zp) {
    if (bf16) return zp ? launch_all<true, true>(a) : launch_all<true, false>(a);
    return zp ? launch_all<false, true>(a) : launch_all<false, false>(a);
}

}  // namespace hq
