// Internal interfaces between the C-ABI layer (hq_api.cpp) and the kernel
// translation units (*.hip).  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "../../include/hq.h"

namespace hq {

// Row/column counts padded to the packed layout.
inline int64_t pad16(int64_t n) { return (n + 15) / 16 * 16; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Workspace carve-up shared by every dense split-K launch:
//   [0, kCounterBytes)       uint32 arrival counters, one per output tile
//   [kCounterBytes, ...)     fp32 / int32 partial tiles
constexpr size_t kCounterBytes = 64 * 1024;
constexpr int kMaxCounters = (int)(kCounterBytes / 4);

struct DenseArgs {
    int64_t M, N, K, Np;
    int group_size;
    const void* A;
    const float* a_scale;
    const void* w;
    const void* s;
    const void* z;
    void* D;
    void* ws;
    size_t ws_bytes;
    hipStream_t stream;
};

// W4A16 (INT4 / UINT4+zp; bf16 / fp16 activations)
size_t wna16_workspace(int64_t M, int64_t N, int64_t K, int group_size);
hipError_t wna16_launch(const DenseArgs& a, bool bf16, bool zp);

// fill kernel used by hq_workspace_init
hipError_t fill_zero_launch(void* p, size_t bytes, hipStream_t stream);

}  // namespace hq
