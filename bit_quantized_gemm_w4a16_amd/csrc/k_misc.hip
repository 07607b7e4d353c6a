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
        const float a = fminf(fmaxf(xr[k] / sc, -448.f), 448.f);
        const float b = k + 1 < K ? fminf(fmaxf(xr[k + 1] / sc, -448.f), 448.f) : 0.f;
        const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
        qr[k] = (uint8_t)(pk & 0xFF);
        if (k + 1 < K) qr[k + 1] = (uint8_t)((pk >> 8) & 0xFF);
    }
}

hipError_t quant_e4m3_launch(int64_t M, int64_t K, const float* x, uint8_t* q, float* s, hipStream_t st) {
    hipLaunchKernelGGL(quant_e4m3_kernel, dim3((unsigned)M), dim3(256), 0, st, x, (int)K, q, s);
    return hipGetLastError();
}

}  // namespace hq
