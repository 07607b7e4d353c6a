// Dense W4A8-MXFP4 and W8A8-INT8 launches of the tiled MFMA template.
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
// FP4 weights with bf16 activations (section "WnA16": FP4 among the weight
// formats; NVFP4 with its second-level scale, section "Eine einheitliche
// Quantisierungsdarstellung"): e2m1 codes converted to bf16 with the lane's
// E8M0 or E4M3 group scale (exact), bf16 MFMA, the per-tensor scale on the output.
// The same for the MX float widths (section "WnA16": float weights of any
// width; OCP MX v1.0): E4M3 (MXFP8) and E2M3 / E3M2 (MXFP6) codes under E8M0
// per 32 K, the FP6 ones converted 32 at a time by the packed FP6 convert.
//
// FP8 W8A8 with blockwise scales (same section: the Hopper-era FP8 path with
// blockwise scaling; "Humming v0.1.0-0.1.4" for the per-K-block activation
// scale indexing): fp8 x fp8 on the scaled MFMA per 128-K block, the partial
// scaled by the row's block scale times the 128 x 128 weight block scale.
//
// W8A8-INT8 (same section, INT8 through integer MMA): int8 x int8 into exact
// int32 accumulators (v_mfma_i32_16x16x64_i8), then acc * s_a[m] * s_w[n] in
// fp32, or the raw int32 accumulators.
#include "hq_device.hpp"
#include "hq_internal.h"
#include "skinny.hpp"

namespace hq {

namespace {

template <Fmt F>
hipError_t launch(const DenseArgs& a, int raw_i32) {
    SkinnyArgs s{};
    s.A = a.A;
    s.a_scale = a.a_scale;
    s.a_e8 = a.a_e8;
    s.a_blk = a.a_blk;
    s.s2 = a.s2;
    s.W = a.w;
    s.S = a.s;
    s.D = a.D;
    s.part = a.ws;
    s.M = (int)a.M;
    s.K = (int)a.K;
    s.N = (int)a.N;
    s.Np = (int)a.Np;
    s.nc = (int)(a.K / 128);
    s.ngroups = 1;
    s.gchunks = 1;
    s.raw_i32 = raw_i32;
    TileArgs p{};
    p.A = a.A;
    p.a_scale = a.a_scale;
    p.a_e8 = a.a_e8;
    p.a_blk = a.a_blk;
    p.s2 = a.s2;
    p.W = a.w;
    p.S = a.s;
    p.D = a.D;
    p.part = a.ws;
    p.M = (int)a.M;
    p.a_rows = (int)a.M;
    p.N = (int)a.N;
    p.K = (int)a.K;
    p.Np = (int)a.Np;
    p.ngroups = 1;
    p.gsteps = 1;
    p.raw_i32 = raw_i32;
    return dense_dispatch<F>(a, s, p, 128);
}

}  // namespace

hipError_t w4a8_launch(const DenseArgs& a) { return launch<Fmt::W4A8_MX>(a, 0); }

hipError_t w8a8_launch(const DenseArgs& a, bool raw_i32) { return launch<Fmt::W8A8_I8>(a, raw_i32 ? 1 : 0); }

hipError_t fp8_block_launch(const DenseArgs& a) { return launch<Fmt::W8A8_F8B>(a, 0); }

hipError_t w8a16_launch(const DenseArgs& a, bool bf16, bool fp8) {
    if (fp8) return bf16 ? launch<Fmt::F8W_BF16>(a, 0) : launch<Fmt::F8W_F16>(a, 0);
    return bf16 ? launch<Fmt::W8A16_BF16>(a, 0) : launch<Fmt::W8A16_F16>(a, 0);
}

hipError_t fp4_a16_launch(const DenseArgs& a, int kind) {
    switch (kind) {
        case 1: return launch<Fmt::NVFP4_BF16>(a, 0);
        case 2: return launch<Fmt::MXINT4_BF16>(a, 0);
        case 3: return launch<Fmt::MXF8_BF16>(a, 0);
        case 4: return launch<Fmt::MXF6E2_BF16>(a, 0);
        case 5: return launch<Fmt::MXF6E3_BF16>(a, 0);
        default: return launch<Fmt::MXFP4_BF16>(a, 0);
    }
}

hipError_t mx_act_launch(const DenseArgs& a, bool fp4_act) {
    return fp4_act ? launch<Fmt::W4A4_MX>(a, 0) : launch<Fmt::W4A8_MXA>(a, 0);
}

}  // namespace hq
