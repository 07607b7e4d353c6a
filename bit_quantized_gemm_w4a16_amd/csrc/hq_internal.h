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

// Launch planning without launching: while a PlanRecorder is active on the
// calling thread, the dense launchers append the name, grid and split of each
// kernel they would enqueue to it and return hipSuccess without any HIP call
// (hq_gemm_plan).  The same code path chooses the kernels in both modes.
// The launchers also report the workspace bytes their launches read and write,
// so hq_workspace_bytes and the workspace check of hq_gemm follow the exact
// plan the call will run.
struct PlanRecorder {
    char* buf;     // launch names (may be null: only the workspace is wanted)
    size_t len, used;
    size_t ws;     // workspace bytes the planned launches need
    size_t base;   // offset added to the needs noted from here on (a region in front is taken)
};
PlanRecorder* plan_recorder();                     // the active recorder of this thread, or null
void plan_record(const char* fmt, ...);            // appends one launch (no-op without a recorder)
void plan_workspace(size_t bytes);                 // notes a workspace need (no-op without a recorder)
void plan_workspace_base(size_t base);             // the following needs start `base` bytes into the workspace

struct DenseArgs {
    int64_t M, N, K, Np;
    int group_size;
    const void* A;
    const float* a_scale;   // per-token fp32 scales (W4A8 tokenwise, W8A8)
    const uint8_t* a_e8;    // MX activation scales, E8M0 [M][K/32]
    const float* a_blk;     // blockwise fp8 activation scales, fp32 [M][K/128]
    const void* w;
    const void* s;
    const void* z;
    const float* s2;        // second-level weight scale (NVFP4), fp32 [1]
    void* D;
    void* ws;
    size_t ws_bytes;
    hipStream_t stream;
    // compute / tuning options from the descriptor
    bool invariant;       // batch-invariant mode: results per row independent of M
    int tune_path;        // 0: library's choice; else a TunePath override
    int tune_splits;      // K slices of the override (0: the planner's)
    int wbits = 4;        // W4A16 kinds: weight code width (1-3: the low-bit planes)
};

// W4A16 (INT4 / UINT4+zp; bf16 / fp16 activations)
hipError_t wna16_launch(const DenseArgs& a, bool bf16, bool zp);  // also the 1-3-bit widths (a.wbits)

// W4A8-MXFP4 and W8A8-INT8 (split-K workspace for mid M)
hipError_t w4a8_launch(const DenseArgs& a);
hipError_t w8a8_launch(const DenseArgs& a, bool raw_i32);
hipError_t mx_act_launch(const DenseArgs& a, bool fp4_act);  // MX activations x MXFP4 weights
hipError_t fp8_block_launch(const DenseArgs& a);              // FP8 W8A8 with blockwise scales
hipError_t w8a16_launch(const DenseArgs& a, bool bf16, bool fp8);  // bf16 / fp16 A x INT8 / E4M3 weights, per-channel scale
// 16-bit A (bf16, or fp16 when !bf16) x MXFP4 (0) / NVFP4 (1) / MXINT4 (2) / MXFP8 (3) / MXFP6 E2M3 (4) / E3M2 (5)
hipError_t fp4_a16_launch(const DenseArgs& a, int kind, bool bf16);
hipError_t fp4w_launch_bf16(const DenseArgs& a, int kind);  // kinds 0-2 (k_fp4w_bf16.hip)
hipError_t fp4w_launch_f16(const DenseArgs& a, int kind);
hipError_t mxfw_launch_bf16(const DenseArgs& a, int kind);  // kinds 3-5 (k_mxfw_bf16.hip)
hipError_t mxfw_launch_f16(const DenseArgs& a, int kind);

// MoE
struct MoeLayout {  // byte offsets into the MoE workspace
    size_t hist, lrank, offsets, sorted, tiles_tier[4], ntiles, bytes;
    int64_t max_tier[4];  // bounds of the per-tier m-tile lists (by expert row count)
};
MoeLayout moe_layout(int64_t T, int top_k, int E, bool indexed);
size_t moe_align_workspace(int64_t T, int top_k, int E);

struct MoeArgs {
    int64_t T, N, K, Np;
    int top_k, E;
    bool indexed;
    const void* A;
    const int* topk_ids;
    const int* expert_offsets;
    const void* w;
    const void* s;
    void* D;
    int64_t w_estride, s_estride;
    void* ws;
    hipStream_t stream;
};
hipError_t moe_gemm_launch(const MoeArgs& a);
struct MoeTiers;
hipError_t moe_align_launch(int64_t T, int top_k, int E, const int* ids, int* offsets, int* sorted, void* ws,
                            const MoeTiers* tiers, hipStream_t st);
hipError_t moe_gather_launch(const void* A, const int* sorted, int64_t P, int top_k, int64_t row_bytes, void* out,
                             hipStream_t st);

// activation quantisation (tokenwise E4M3)
hipError_t quant_e4m3_launch(int64_t M, int64_t K, const float* x, uint8_t* q, float* s, hipStream_t st);
hipError_t quant_mx_launch(bool fp4, int64_t M, int64_t K, const float* x, uint8_t* q, uint8_t* e, hipStream_t st);
hipError_t silu_mul_launch(int64_t rows, int64_t I, const void* in, void* out, hipStream_t st);

// measurement probes
hipError_t probe_stream_launch(const void* src, size_t bytes, void* sink, int reps, hipStream_t st);
hipError_t probe_mfma_launch(int dtype, int64_t workgroups, int iters, void* sink, hipStream_t st);

// fill kernel used by hq_workspace_init
hipError_t fill_zero_launch(void* p, size_t bytes, hipStream_t stream);

}  // namespace hq
