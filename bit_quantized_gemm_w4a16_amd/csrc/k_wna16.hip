// W4A16 kernels for gfx950: D[M,N] = A[M,K] x dequant(W), W symmetric INT4 or
// UINT4 with zero-points, one 16-bit scale per (group of G along K, column).
//
// Method: "Humming wird angekuendigt", section "WnA16" (dense W4A16 with
// fp16/bf16 activations) and section "Gemeinsam genutzte CUDA-Komponenten"
// (dequantisation and scaling fused into the GEMM's compute).  The design
// below is our own for CDNA4: 64-wide wavefronts, MFMA 16x16x32, packed
// weights laid out so that one 16-byte load per lane is one MFMA B fragment
// for four consecutive K steps.
//
// Small M (M <= 64): the GEMV-like weight stream of skinny.hpp, where the
// group scale multiplies the fp32 partial of each 128-K chunk, so the
// dequantised operand (q - z, an integer in [-15, 15]) is exact in both bf16
// and fp16.  Large M: the LDS-tiled MFMA template in tile_gemm.hpp.
#include "hq_device.hpp"
#include "hq_internal.h"
#include "skinny.hpp"

namespace hq {

// -------------------------------------------------------------------------
// host-side planning and launch
// -------------------------------------------------------------------------

namespace {

template <Fmt F>
hipError_t launch_all(const DenseArgs& a) {
    SkinnyArgs s{};
    s.A = a.A;
    s.W = a.w;
    s.S = a.s;
    s.Z = a.z;
    s.D = a.D;
    s.part = a.ws;
    s.M = (int)a.M;
    s.K = (int)a.K;
    s.N = (int)a.N;
    s.Np = (int)a.Np;
    s.nc = (int)(a.K / 128);
    s.ngroups = (int)(a.K / a.group_size);
    s.gchunks = a.group_size / 128;
    s.wbits = a.wbits;
    TileArgs p{};
    p.A = a.A;
    p.W = a.w;
    p.S = a.s;
    p.Z = a.z;
    p.D = a.D;
    p.part = a.ws;
    p.M = (int)a.M;
    p.a_rows = (int)a.M;
    p.N = (int)a.N;
    p.K = (int)a.K;
    p.Np = (int)a.Np;
    p.ngroups = (int)(a.K / a.group_size);
    p.gsteps = a.group_size / 128;
    return dense_dispatch<F>(a, s, p, a.group_size);
}

}  // namespace

hipError_t wna16_launch(const DenseArgs& a, bool bf16, bool zp) {
    (void)zp;  // zero-points travel as a pointer (null for symmetric INT4)
    return bf16 ? launch_all<Fmt::WNA16_BF16>(a) : launch_all<Fmt::WNA16_F16>(a);
}

}  // namespace hq
