// MX float (MXFP8 E4M3, MXFP6 E2M3 / E3M2) weight-only launches with bf16 activations.
//
// FP4 weights with 16-bit activations (section "WnA16": FP4 among the weight
// formats; NVFP4 with its second-level scale, section "Eine einheitliche
// Quantisierungsdarstellung"): e2m1 codes converted to 16-bit operands of the
// activation type with the lane's E8M0 or E4M3 group scale (exact; with fp16
// inside fp16's range), MFMA of that type, the per-tensor scale on the output.
// The same for MXINT4 and for the MX float widths (section "WnA16": float
// weights of any width; OCP MX v1.0): E4M3 (MXFP8) and E2M3 / E3M2 (MXFP6)
// codes under E8M0 per 32 K, the FP6 ones converted 32 at a time by the packed
// FP6 convert (widened to E4M3 for the tiles).
#include "dense_launch.hpp"

namespace hq {

hipError_t mxfw_launch_bf16(const DenseArgs& a, int kind) {
    switch (kind) {
        case 3: return launch<Fmt::MXF8_BF16>(a, 0);
        case 4: return launch<Fmt::MXF6E2_BF16>(a, 0);
        case 5: return launch<Fmt::MXF6E3_BF16>(a, 0);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace hq
