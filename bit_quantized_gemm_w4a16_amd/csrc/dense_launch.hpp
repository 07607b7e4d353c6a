// The dense launch of one format: the small-M weight stream or the tiled
// kernels (dense_dispatch), with the format's kernel arguments filled in from
// the validated call.  Included by the per-family translation units so that
// they compile in parallel.
#pragma once

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

}  // namespace hq
