// Small utility kernels: workspace zero-fill.
#include "hq_device.hpp"
#include "hq_internal.h"

namespace hq {

__global__ void fill_zero_kernel(v4u* p, size_t n16) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) p[i] = v4u{0u, 0u, 0u, 0u};
}

hipError_t fill_zero_launch(void* p, size_t bytes, hipStream_t stream) {
    const size_t n16 = bytes / 16;
    size_t blocks = (n16 + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (v4u*)p, n16);
    return hipGetLastError();
}

}  // namespace hq

namespace hq {

// Tokenwise E4M3 activation quantisation: one workgroup per row.
// s = max|x| / 448 (correctly rounded fp32 division, the HIP default; 1 for
// an all-zero row), q = E4M3(x / s)
// with round-to-nearest-even; |x / s| is clamped to 448 first, which equals
// saturating rounding since every quotient lies within rounding of +-448.
// Non-finite input: NaN elements take no part in the maximum (fmaxf returns
// the other operand) and encode as 0x7F, the E4M3 NaN; an infinite element
// makes s infinite, so finite elements of its row encode as +-0 and the
// infinite ones (Inf / Inf) as NaN.
__device__ __forceinline__ uint32_t e4m3_nan_fix(uint32_t codes, int byte, float v) {
    return v != v ? (codes & ~(0xFFu << (8 * byte))) | (0x7Fu << (8 * byte)) : codes;
}

__global__ __launch_bounds__(256) void quant_e4m3_kernel(const float* __restrict__ x, int K,
                                                         uint8_t* __restrict__ q, float* __restrict__ s) {
    __shared__ float red[256];
    const int64_t row = blockIdx.x;
    const float* xr = x + row * K;
    float amax = 0.f;
    for (int k = threadIdx.x; k < K; k += 256) amax = fmaxf(amax, fabsf(xr[k]));
    red[threadIdx.x] = amax;
    __syncthreads();
    for (int off = 128; off > 0; off >>= 1) {
        if (threadIdx.x < off) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + off]);
        __syncthreads();
    }
    amax = red[0];
    const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
    if (threadIdx.x == 0) s[row] = sc;
    uint8_t* qr = q + row * K;
    for (int k = 2 * threadIdx.x; k < K; k += 512) {
        const float va = xr[k] / sc, vb = k + 1 < K ? xr[k + 1] / sc : 0.f;
        const float a = fminf(fmaxf(va, -448.f), 448.f);
        const float b = fminf(fmaxf(vb, -448.f), 448.f);
        const uint32_t pk = e4m3_nan_fix(e4m3_nan_fix((uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false), 0, va), 1, vb);
        qr[k] = (uint8_t)(pk & 0xFF);
        if (k + 1 < K) qr[k + 1] = (uint8_t)((pk >> 8) & 0xFF);
    }
}

// The same quantisation for rows whose length K is a multiple of 4 and at
// most 1024 * NV: each thread holds NV groups of 4 consecutive elements in
// registers (16-byte loads, x read once), the row maximum is reduced across
// the wave by shuffles and across the 4 waves through LDS, and each group's
// four codes leave as one coalesced 32-bit store.  Same arithmetic as above,
// so both kernels give identical codes and scales.
template <int NV>
__global__ __launch_bounds__(256) void quant_e4m3_rows_kernel(const float4* __restrict__ x, int K4,
                                                              uint32_t* __restrict__ q, float* __restrict__ s) {
    __shared__ float red[4];
    const int64_t row = blockIdx.x;
    const float4* xr = x + row * K4;
    float4 v[NV];
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int i = j * 256 + (int)threadIdx.x;
        v[j] = i < K4 ? xr[i] : make_float4(0.f, 0.f, 0.f, 0.f);
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[j].x), fabsf(v[j].y)), fmaxf(fabsf(v[j].z), fabsf(v[j].w))));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
    if (threadIdx.x == 0) s[row] = sc;
    uint32_t* qr = q + row * K4;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int i = j * 256 + (int)threadIdx.x;
        if (i < K4) {
            const float va = v[j].x / sc, vb = v[j].y / sc, vc = v[j].z / sc, vd = v[j].w / sc;
            const float a = fminf(fmaxf(va, -448.f), 448.f);
            const float b = fminf(fmaxf(vb, -448.f), 448.f);
            const float c = fminf(fmaxf(vc, -448.f), 448.f);
            const float d = fminf(fmaxf(vd, -448.f), 448.f);
            int pk = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);  // bytes 0, 1
            pk = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, pk, true);      // bytes 2, 3
            uint32_t u = (uint32_t)pk;
            u = e4m3_nan_fix(u, 0, va);
            u = e4m3_nan_fix(u, 1, vb);
            u = e4m3_nan_fix(u, 2, vc);
            u = e4m3_nan_fix(u, 3, vd);
            qr[i] = u;
        }
    }
}

hipError_t quant_e4m3_launch(int64_t M, int64_t K, const float* x, uint8_t* q, float* s, hipStream_t st) {
    const dim3 grid((unsigned)M), blk(256);
    if (K % 4 == 0 && K <= 8192) {  // x and q are 16-byte aligned: 16-byte rows of x, 4-byte rows of q
        const int K4 = (int)(K / 4), nv = (K4 + 255) / 256;
        const float4* xv = (const float4*)x;
        uint32_t* qv = (uint32_t*)q;
        if (nv <= 1)
            hipLaunchKernelGGL(quant_e4m3_rows_kernel<1>, grid, blk, 0, st, xv, K4, qv, s);
        else if (nv <= 2)
            hipLaunchKernelGGL(quant_e4m3_rows_kernel<2>, grid, blk, 0, st, xv, K4, qv, s);
        else if (nv <= 4)
            hipLaunchKernelGGL(quant_e4m3_rows_kernel<4>, grid, blk, 0, st, xv, K4, qv, s);
        else
            hipLaunchKernelGGL(quant_e4m3_rows_kernel<8>, grid, blk, 0, st, xv, K4, qv, s);
    } else {
        hipLaunchKernelGGL(quant_e4m3_kernel, grid, blk, 0, st, x, (int)K, q, s);
    }
    return hipGetLastError();
}

}  // namespace hq

namespace hq {

// MX activation quantisation (OCP Microscaling Formats v1.0, section 6.3):
// per row and block of 32 along K the shared exponent is floor(log2(amax))
// minus the largest exponent of the element format (E4M3 8, E2M1 2), as an
// E8M0 byte clamped to 0..254 (0 for an all-zero block, 0xFF -- NaN -- for a
// block holding a NaN or an infinity, whose codes are then 0); each element
// x * 2^(127 - E) (an exact power-of-two scaling) is rounded to nearest even
// and saturated.  For normal amax, floor(log2(amax)) is its exponent field
// minus 127.  One thread per 8 consecutive elements, 4 threads per block.
//
// E2M1 rounding: |v| is compared with the midpoints of the grid
// 0, 0.5, 1, 1.5, 2, 3, 4, 6; a midpoint itself goes to the neighbour with
// the even mantissa bit, hence strict ">" at 0.25, 1.25, 2.5, 5 and ">=" at
// 0.75, 1.75, 3.5.  The sign is that of x (so -0 and tiny negatives give 8).
__device__ __forceinline__ uint32_t e2m1_code(float x, float v) {
    const float a = fabsf(v);
    const uint32_t mag = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) + (uint32_t)(a >= 1.75f) +
                         (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
    return mag | ((__float_as_uint(x) >> 28) & 8u);
}

template <bool FP4>
__global__ __launch_bounds__(256) void quant_mx_kernel(const float4* __restrict__ x, int64_t ngroups, int K8,
                                                       uint8_t* __restrict__ q, uint8_t* __restrict__ e) {
    constexpr int EMAX = FP4 ? 2 : 8;
    for (int64_t g0 = (int64_t)blockIdx.x * 256; g0 < ngroups; g0 += (int64_t)gridDim.x * 256) {
        const int64_t g = g0 + threadIdx.x;  // group of 8 elements; 4 consecutive groups form a block
        const bool live = g < ngroups;
        float v[8];
        if (live) {
            const float4 a = x[2 * g], b = x[2 * g + 1];
            v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = 0.f;
        }
        float amax = 0.f;
        uint32_t bad = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            bad |= (uint32_t)((__float_as_uint(v[i]) & 0x7F800000u) == 0x7F800000u);
            amax = fmaxf(amax, fabsf(v[i]));
        }
        // the 4 groups of a block are lanes 4j..4j+3 of the wave (ngroups is a multiple of 4)
        amax = fmaxf(amax, __shfl_xor(amax, 1));
        amax = fmaxf(amax, __shfl_xor(amax, 2));
        bad |= __shfl_xor(bad, 1);
        bad |= __shfl_xor(bad, 2);
        int E = 0;
        if (bad) {
            E = 255;
        } else if (amax > 0.f) {
            E = (int)((__float_as_uint(amax) >> 23) & 0xFFu) - EMAX;
            E = E < 0 ? 0 : E > 254 ? 254 : E;
        }
        if (!live) continue;
        const int sh = 127 - (E == 255 ? 127 : E);
        if constexpr (FP4) {
            uint32_t w = 0;
            if (E != 255) {
#pragma unroll
                for (int i = 0; i < 8; ++i) w |= e2m1_code(v[i], ldexpf(v[i], sh)) << (4 * i);
            }
            ((uint32_t*)q)[g] = w;
        } else {
            uint32_t lo = 0, hi = 0;
            if (E != 255) {
                float c[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) c[i] = fminf(fmaxf(ldexpf(v[i], sh), -448.f), 448.f);
                lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
                lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], (int)lo, true);
                hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c[4], c[5], 0, false);
                hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c[6], c[7], (int)hi, true);
            }
            ((uint2*)q)[g] = make_uint2(lo, hi);
        }
        if ((g & 3) == 0) e[g >> 2] = (uint8_t)E;
        (void)K8;
    }
}

hipError_t quant_mx_launch(bool fp4, int64_t M, int64_t K, const float* x, uint8_t* q, uint8_t* e, hipStream_t st) {
    const int64_t ngroups = M * (K / 8);
    int64_t blocks = (ngroups + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) return hipSuccess;
    if (fp4)
        hipLaunchKernelGGL(quant_mx_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, st, (const float4*)x, ngroups, (int)(K / 8), q, e);
    else
        hipLaunchKernelGGL(quant_mx_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, st, (const float4*)x, ngroups, (int)(K / 8), q, e);
    return hipGetLastError();
}

}  // namespace hq

namespace hq {

// SwiGLU between the MoE projections: out[r][i] = bf16(silu(g) * u) with
// g = in[r][i], u = in[r][I + i], computed in fp32 (exact bf16 -> fp32 inputs)
// and rounded once to nearest even.  silu(g) = g / (1 + e^-g), evaluated as
// g / (1 + t) for g >= 0 and g t / (1 + t) for g < 0 with t = e^-|g| <= 1: the
// plain form overflows e^-g for g below about -88.7 and returns 0 where the
// result is still a normal bf16.  One thread per 8 outputs (16-byte loads of
// gate and up, one 16-byte store); HBM-bound.
__global__ __launch_bounds__(256) void silu_mul_kernel(const v4u* __restrict__ in, int64_t rows, int I8,
                                                       v4u* __restrict__ out) {
    const int64_t total = rows * I8;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
        const int64_t r = i / I8, c = i - r * I8;
        const v4u g = in[r * 2 * I8 + c], u = in[r * 2 * I8 + I8 + c];
        v4u o;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float g0 = __uint_as_float(g[k] << 16), g1 = __uint_as_float(g[k] & 0xFFFF0000u);
            const float u0 = __uint_as_float(u[k] << 16), u1 = __uint_as_float(u[k] & 0xFFFF0000u);
            const float t0 = expf(-fabsf(g0)), t1 = expf(-fabsf(g1));
            const float y0 = (g0 >= 0.f ? g0 : g0 * t0) / (1.0f + t0) * u0;
            const float y1 = (g1 >= 0.f ? g1 : g1 * t1) / (1.0f + t1) * u1;
            o[k] = (uint32_t)f32_to_bf16_bits(y0) | ((uint32_t)f32_to_bf16_bits(y1) << 16);
        }
        out[i] = o;
    }
}

hipError_t silu_mul_launch(int64_t rows, int64_t I, const void* in, void* out, hipStream_t st) {
    const int64_t total = rows * (I / 8);
    int64_t blocks = (total + 255) / 256;
    if (blocks > 16384) blocks = 16384;
    if (blocks < 1) return hipSuccess;
    hipLaunchKernelGGL(silu_mul_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (const v4u*)in, rows, (int)(I / 8),
                       (v4u*)out);
    return hipGetLastError();
}

}  // namespace hq
