// Dense W4A8-MXFP4 and W8A8-INT8 launches of the tiled MFMA template.
//
// W4A8-MXFP4 ("Humming wird angekuendigt", section "W8A8 / W4A8 / W4A4"):
// fp8-e4m3 activations with a per-token fp32 scale times e2m1 weights with an
// E8M0 scale per 32 K.  The pages' NVIDIA design converts MXFP4 to FP8 in the
// kernel because those parts lack native MXFP4 MMA; gfx950 has a scaled MFMA
// that takes the e2m1 codes and the E8M0 exponents directly
// (v_mfma_scale_f32_16x16x128_f8f6f4), so the weights are never dequantised.
//
// W8A8-INT8 (same section, INT8 through integer MMA): int8 x int8 into exact
// int32 accumulators (v_mfma_i32_16x16x64_i8), then acc * s_a[m] * s_w[n] in
// fp32, or the raw int32 accumulators.
#include "hq_device.hpp"
#include "hq_internal.h"
#include "tile_gemm.hpp"

namespace hq {

namespace {

template <Fmt F, int BM>
hipError_t launch(const DenseArgs& a, int raw_i32) {
    TileArgs p{};
    p.A = a.A;
    p.a_scale = a.a_scale;
    p.W = a.w;
    p.S = a.s;
    p.D = a.D;
    p.M = (int)a.M;
    p.N = (int)a.N;
    p.K = (int)a.K;
    p.Np = (int)a.Np;
    p.ngroups = 1;
    p.gsteps = 1;
    p.raw_i32 = raw_i32;
    p.tiles_m = (int)cdiv(a.M, BM);
    p.tiles_n = (int)cdiv(a.Np, 128);
    hipLaunchKernelGGL((tile_gemm_kernel<F, BM, 128>), dim3(p.tiles_m * p.tiles_n), dim3(256), 0, a.stream, p);
    return hipGetLastError();
}

template <Fmt F>
hipError_t launch_any(const DenseArgs& a, int raw_i32) {
    const int64_t tiles_n = cdiv(a.Np, 128);
    if (cdiv(a.M, 256) * tiles_n >= 256) return launch<F, 256>(a, raw_i32);
    return launch<F, 128>(a, raw_i32);
}

}  // namespace

hipError_t w4a8_launch(const DenseArgs& a) { return launch_any<Fmt::W4A8_MX>(a, 0); }

hipError_t w8a8_launch(const DenseArgs& a, bool raw_i32) { return launch_any<Fmt::W8A8_I8>(a, raw_i32 ? 1 : 0); }

}  // namespace hq
