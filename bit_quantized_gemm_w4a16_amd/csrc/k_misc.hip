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
