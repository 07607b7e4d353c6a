// Dense W4A8-MXFP4, MX-activation, FP8-blockwise and W8A8-INT8 launches (the
// weight-only formats with 16-bit activations are in k_w8a16.hip, k_fp4w_*.hip
// and k_mxfw_*.hip).
//
// W4A8-MXFP4 ("Humming wird angekuendigt", section "W8A8 / W4A8 / W4A4"):
// fp8-e4m3 activations with a per-token fp32 scale times e2m1 weights with an
// E8M0 scale per 32 K.  The pages' NVIDIA design converts MXFP4 to FP8 in the
// kernel because those parts lack native MXFP4 MMA; gfx950 has a scaled MFMA
// that takes the e2m1 codes and the E8M0 exponents directly
// (v_mfma_scale_f32_16x16x128_f8f6f4), so the weights are never dequantised.
//
// MX activations (same section, W4A4 and W4A8 on microscaling formats; section
// "Auswahl von Aktivierungstypen" for MXFP8 activations): E4M3 or E2M1 codes
// with one E8M0 scale per 32 K per row, fed with the weights' E8M0 scales to
// the same scaled MFMA; no epilogue scale.
//
// FP8 W8A8 with blockwise scales (same section: the Hopper-era FP8 path with
// blockwise scaling; "Humming v0.1.0-0.1.4" for the per-K-block activation
// scale indexing): fp8 x fp8 on the scaled MFMA per 128-K block, the partial
// scaled by the row's block scale times the 128 x 128 weight block scale.
//
// W8A8-INT8 (same section, INT8 through integer MMA): int8 x int8 into exact
// int32 accumulators (v_mfma_i32_16x16x64_i8), then acc * s_a[m] * s_w[n] in
// fp32, or the raw int32 accumulators.
#include "dense_launch.hpp"

namespace hq {

hipError_t w4a8_launch(const DenseArgs& a) { return launch<Fmt::W4A8_MX>(a, 0); }

hipError_t w8a8_launch(const DenseArgs& a, bool raw_i32) { return launch<Fmt::W8A8_I8>(a, raw_i32 ? 1 : 0); }

hipError_t fp8_block_launch(const DenseArgs& a) { return launch<Fmt::W8A8_F8B>(a, 0); }

hipError_t mx_act_launch(const DenseArgs& a, bool fp4_act) {
    return fp4_act ? launch<Fmt::W4A4_MX>(a, 0) : launch<Fmt::W4A8_MXA>(a, 0);
}

}  // namespace hq
