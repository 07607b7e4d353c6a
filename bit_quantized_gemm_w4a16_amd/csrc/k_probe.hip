// Measurement probes: the attainable HBM read rate and dense MFMA rate of the
// device the library runs on, so kernel timings can be set against what the
// chip delivers as well as against its published peaks.  Neither is part of
// any GEMM; both run only when called.
#include "hq_device.hpp"
#include "hq_internal.h"

namespace hq {

// Read stream: every 16 bytes of src read once with 16-byte loads (grid-stride,
// consecutive lanes on consecutive addresses), folded into an XOR that is
// stored only if it equals a value no real fold is expected to produce, so the
// loads cannot be dropped and nothing is written in practice.
__global__ __launch_bounds__(256) void probe_stream_kernel(const v4u* __restrict__ src, size_t n16, uint32_t* sink) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    v4u acc = v4u{0u, 0u, 0u, 0u};
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {  // four loads in flight per lane
        const v4u a = __builtin_nontemporal_load(src + i), b = __builtin_nontemporal_load(src + i + stride);
        const v4u c = __builtin_nontemporal_load(src + i + 2 * stride), d = __builtin_nontemporal_load(src + i + 3 * stride);
        acc ^= a ^ b ^ c ^ d;
    }
    for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(src + i);
    const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    if (x == 0x9E3779B9u) sink[0] = x;
}

hipError_t probe_stream_launch(const void* src, size_t bytes, void* sink, int reps, hipStream_t st) {
    const size_t n16 = bytes / 16;
    for (int r = 0; r < reps; ++r) {
        hipLaunchKernelGGL(probe_stream_kernel, dim3(4096), dim3(256), 0, st, (const v4u*)src, n16, (uint32_t*)sink);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// MFMA rate: each wave runs `iters` rounds of 8 independent MFMAs of the
// type's dense 16x16 instruction on register operands (enough chains to cover
// the instruction's latency), then stores its accumulators to sink.
template <int DT>
__device__ __forceinline__ v4f probe_mfma(uint32_t u, v4f c) {
    if constexpr (DT == HQ_DT_FP16) {
        const v8h a = __builtin_bit_cast(v8h, v4u{u, u, u, u});
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, a, c, 0, 0, 0);
    } else if constexpr (DT == HQ_DT_BF16) {
        const v8bf a = __builtin_bit_cast(v8bf, v4u{u, u, u, u});
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, a, c, 0, 0, 0);
    } else if constexpr (DT == HQ_DT_FP8_E4M3) {
        const v8i a = v8i{(int)u, (int)u, (int)u, (int)u, (int)u, (int)u, (int)u, (int)u};
        return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, a, c, 0, 0, 0, 0x7F, 0, 0x7F);
    } else if constexpr (DT == HQ_DT_FP4_E2M1) {
        const v8i a = v8i{(int)u, (int)u, (int)u, (int)u, 0, 0, 0, 0};
        return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, a, c, 4, 4, 0, 0x7F, 0, 0x7F);
    } else {
        const v4i a = v4i{(int)u, (int)u, (int)u, (int)u};
        return __builtin_bit_cast(v4f, __builtin_amdgcn_mfma_i32_16x16x64_i8(a, a, __builtin_bit_cast(v4i, c), 0, 0, 0));
    }
}

template <int DT>
__global__ __launch_bounds__(256) void probe_mfma_kernel(int iters, uint32_t seed, float* __restrict__ sink) {
    const uint32_t u = 0x3C003C00u ^ ((seed + threadIdx.x) & 0x003F003Fu);  // finite fp16/bf16/fp8/fp4/int8 patterns
    v4f a0 = v4f{0.f, 0.f, 0.f, 0.f}, a1 = a0, a2 = a0, a3 = a0, a4 = a0, a5 = a0, a6 = a0, a7 = a0;
    for (int it = 0; it < iters; ++it) {
        a0 = probe_mfma<DT>(u, a0);
        a1 = probe_mfma<DT>(u, a1);
        a2 = probe_mfma<DT>(u, a2);
        a3 = probe_mfma<DT>(u, a3);
        a4 = probe_mfma<DT>(u, a4);
        a5 = probe_mfma<DT>(u, a5);
        a6 = probe_mfma<DT>(u, a6);
        a7 = probe_mfma<DT>(u, a7);
    }
    const v4f t = (a0 + a1) + (a2 + a3) + (a4 + a5) + (a6 + a7);  // int8: bit patterns, summed as floats
    sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = t[0] + t[1] + t[2] + t[3];
}

hipError_t probe_mfma_launch(int dtype, int64_t workgroups, int iters, void* sink, hipStream_t st) {
    const dim3 g((unsigned)workgroups), b(256);
    float* out = (float*)sink;
    switch (dtype) {
        case HQ_DT_FP16: hipLaunchKernelGGL(probe_mfma_kernel<HQ_DT_FP16>, g, b, 0, st, iters, 1u, out); break;
        case HQ_DT_BF16: hipLaunchKernelGGL(probe_mfma_kernel<HQ_DT_BF16>, g, b, 0, st, iters, 1u, out); break;
        case HQ_DT_FP8_E4M3: hipLaunchKernelGGL(probe_mfma_kernel<HQ_DT_FP8_E4M3>, g, b, 0, st, iters, 1u, out); break;
        case HQ_DT_FP4_E2M1: hipLaunchKernelGGL(probe_mfma_kernel<HQ_DT_FP4_E2M1>, g, b, 0, st, iters, 1u, out); break;
        case HQ_DT_INT8: hipLaunchKernelGGL(probe_mfma_kernel<HQ_DT_INT8>, g, b, 0, st, iters, 1u, out); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace hq
