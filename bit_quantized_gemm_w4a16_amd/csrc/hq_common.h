// Host-only definitions shared by the C-ABI layer and the repack code.
// No HIP types: this header compiles with any C++17 compiler.
#pragma once

#include <cstddef>
#include <cstdint>

#include "../../include/hq.h"

namespace hq {

// The operation families the kernels implement (one per supported row of the
// descriptor table in include/hq.h).
enum class Kind {
    WNA16,        // bf16/fp16 A, INT4 or UINT4+zp W, 16-bit group scales
    W4A8_MX,      // fp8-e4m3 A (per-token fp32 scale), e2m1 W, E8M0 per 32 K
    W8A8,         // int8 A (per-token fp32 scale), int8 W, fp32 per-channel
    MOE_MX_BF16,  // MoE: bf16 A, e2m1 W, E8M0 per 32 K
    MXA_MX,       // MX activations (E4M3 or E2M1, E8M0 per 32 K) x e2m1 W, E8M0 per 32 K
    FP8_BLOCK,    // fp8-e4m3 A (fp32 per row and 128-K block) x fp8-e4m3 W (fp32 per 128 x 128 block)
    FP4_A16,      // bf16 A, e2m1 W with E8M0 per 32 K (MXFP4) or E4M3 per 16 K + fp32 per tensor (NVFP4);
                  // also INT4 W with E8M0 per 32 K (MXINT4), and E4M3 / E2M3 / E3M2 W with
                  // E8M0 per 32 K (MXFP8, MXFP6)
    W8A16,        // bf16/fp16 A, int8 or fp8-e4m3 W, fp32 per-channel
};

struct LayerInfo {
    Kind kind;
    int64_t N, K, Np, E, G;
    bool a_bf16;   // WNA16: activations (and scales, output) are bf16
    bool zp;       // WNA16: UINT4 codes with UINT4 zero-points
    bool out_i32;  // W8A8: raw int32 accumulators
    bool a_fp4;    // MXA_MX: E2M1 activations (else E4M3)
    bool nv;       // FP4_A16: NVFP4 (E4M3 per 16 K, per-tensor second-level scale), else MXFP4
    bool i4;       // FP4_A16: MXINT4 (two's-complement INT4 codes, E8M0 per 32 K) instead of e2m1
    bool w_fp8;    // W8A16: E4M3 weight codes instead of INT8
    int mxf;       // FP4_A16: MX float codes, 1 = E4M3 (MXFP8), 2 = E2M3, 3 = E3M2 (MXFP6); 0 = none
    int bits;      // WNA16: weight code width (4, or 1 / 2 / 3 for the low-bit widths)
    bool zp8;      // WNA16 at 5-8 bits: unsigned codes with UINT8 zero-points
    int e0m;       // WNA16 / W8A16: e0mN codes (n = 1, 2, 3 or 7; 0 = none), converted at repack to the
                   // two's-complement container of width n + 1
    bool invariant;        // HQ_FLAG_BATCH_INVARIANT
    int tune_path, tune_splits;  // HQ_TUNE override (0, 0: the library's choice)
};

// Validates a descriptor; fills `info` on success.  Sets the thread-local
// error message on failure.
hq_status describe(const hq_layer_desc* d, LayerInfo* info);

void packed_sizes(const LayerInfo& L, size_t* w, size_t* s, size_t* z, size_t* s2);
void repack_all(const LayerInfo& L, const void* w, const void* s, const void* z, const void* s2, void* w_out,
                void* s_out, void* z_out, void* s2_out);

hq_status set_error(hq_status st, const char* fmt, ...);

}  // namespace hq
