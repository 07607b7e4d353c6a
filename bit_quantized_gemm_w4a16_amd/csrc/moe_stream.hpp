// MoE experts with few rows (W4A16-MXFP4, bf16 tokens): a weight stream in
// which every wave owns whole output strips.
//
// The pages give the shape of the problem, not the code: below a few rows per
// expert the MoE GEMM is a set of GEMVs bound by the weight traffic
// ("Humming wird angekuendigt", section "WnA16", the MoE Indexed and Grouped
// paths; the weight-streaming idea of section "Tuning und JIT-Kompilierung
// fuer jeden Workload").  The schedule below is our own for CDNA4.
//
// Workgroup = 4 waves sharing one m-tile (expert, at most a few rows), whose
// A rows sit in LDS for all of K.  Wave w of workgroup x takes the strips
// (16 output columns) 4x + w, 4x + w + 4 gridDim.x, ... of the tile and runs
// along K in NB batches of CB 128-K chunks per strip: the packed weights (16
// bytes per lane and chunk = one MFMA B fragment per K sub-step) and E8M0
// bytes (one per lane and chunk) of the next batch are in flight while the
// current one is decoded and fed to the MFMA, and the last batches of a strip
// already load the first two of the next, so a wave keeps loading from its
// first batch to its last with no reduction between waves and no barrier
// between strips.  blockIdx.y walks the m-tile list.
//
// The batch sequence of a strip is unrolled at compile time and every refill
// is unconditional, so each point of the loop has the same loads outstanding
// on every path: the explicit waits then hold for the compiler too, and it
// adds none of its own.  Loads that have nothing to fetch (chunks past K, the
// strip after a wave's last) use an offset past the buffer resource, which
// the range check answers with zeros without touching memory; chunks past K
// are not computed.
#pragma once

#include "skinny.hpp"

namespace hq {

struct MoeStreamArgs {
    const void* A;          // tokens [T][K] (Indexed) or expert-sorted rows [P][K] (Grouped), bf16
    const void* W;          // packed MXFP4 weights of expert 0 (experts w_estride bytes apart)
    const void* S;          // packed E8M0 scales of expert 0 (s_estride bytes apart)
    void* D;                // output [P][N] bf16, row = pair (Indexed) or sorted row (Grouped)
    int64_t w_estride, s_estride;
    int K, N, Np;
    int nc;                 // 128-K chunks in K
    int top_k;
    // blockIdx.y walks the m-tile list (expert, first sorted row, rows)
    const int* tile_info;
    const int* ntiles;
    const int* sorted;      // Indexed: sorted pair ids; Grouped: null
    // at most kRouteMaxP pairs: instead of tile_info / ntiles / sorted, every
    // workgroup derives the m-tile list itself from the top-k ids (Indexed)
    // or the expert offsets (Grouped), in tiles of at most route_cap rows
    const int* route_ids;
    const int* route_off;
    int route_P, route_E, route_cap;
};
constexpr int kRouteMaxP = 64;  // one pair (or sorted row) per lane of a wave

// The m-tile list of a MoE launch with at most kRouteMaxP pairs, built by
// every workgroup in LDS (one launch less than a routing pass of its own).
// Rows of the expert-sorted order carry their expert (or -1), their rank
// among the expert's rows and the expert's row count; a tile starts at every
// row whose rank is a multiple of route_cap and holds the next
// min(route_cap, count - rank) rows.  Indexed: pairs are sorted stably by
// expert (rank = equal ids before the pair), ids outside [0, E) are dropped.
// Grouped: row i belongs to the expert whose clamped offset range holds it.
// Returns the tile count (at most kRouteMaxP: every tile holds a row).  All
// threads of the workgroup call it.
__device__ __forceinline__ int moe_route_inline(const MoeStreamArgs& p, int* tile, int* srt, int* rexp, int* rrank,
                                                int* key, int* ntl) {
    const int tid = threadIdx.x, P = p.route_P, E = p.route_E, cap = p.route_cap;
    int id = -1;
    if (p.route_ids && tid < P) {
        const int v = p.route_ids[tid];
        id = v >= 0 && v < E ? v : -1;
    }
    if (tid < kRouteMaxP) {
        rexp[tid] = -1;
        key[tid] = id;  // the pair's expert, read back by every pair below
    }
    __syncthreads();
    if (p.route_ids) {
        if (id >= 0) {
            int pos = 0, rank = 0, cnt = 0;
            for (int j = 0; j < P; ++j) {
                const int v = key[j];
                pos += (v >= 0 && (v < id || (v == id && j < tid))) ? 1 : 0;
                rank += (v == id && j < tid) ? 1 : 0;
                cnt += v == id ? 1 : 0;
            }
            srt[pos] = tid;
            rexp[pos] = id;
            rrank[pos] = rank | (cnt << 8);  // rank and count (both at most kRouteMaxP)
        }
    } else {
        for (int e = tid; e < E; e += blockDim.x) {
            const int lo = min(max(p.route_off[e], 0), P), hi = min(max(p.route_off[e + 1], lo), P);
            for (int i = lo; i < hi; ++i) rexp[i] = e;  // overlapping ranges (malformed offsets): one owner wins
        }
    }
    __syncthreads();
    if (tid < kRouteMaxP) {  // wave 0: lane = row of the sorted order
        const int i = tid;
        const int e = i < P ? rexp[i] : -1;
        int rank = 0, cnt = 0;
        if (e >= 0) {
            if (p.route_ids) {
                rank = rrank[i] & 255;
                cnt = rrank[i] >> 8;
            } else {
                const int lo = min(max(p.route_off[e], 0), P), hi = min(max(p.route_off[e + 1], lo), P);
                rank = i - lo;
                cnt = hi - lo;
            }
        }
        const bool start = e >= 0 && rank % cap == 0;
        const unsigned long long bal = __ballot(start);
        const int t = __popcll(bal & ((1ull << i) - 1ull));
        if (start) {
            tile[3 * t] = e;
            tile[3 * t + 1] = i;
            tile[3 * t + 2] = min(cap, cnt - rank);
        }
        if (i == 0) *ntl = __popcll(bal);
    }
    __syncthreads();
    return *ntl;
}

template <int CB, int NB>
__global__ __launch_bounds__(256) void moe_stream_kernel(MoeStreamArgs p) {
    static_assert(NB % 2 == 0, "a strip ends on buffer 1, so the next starts on buffer 0");
    extern __shared__ __attribute__((aligned(1024))) char lds[];  // A rows of the tile: rows x K bf16 (swizzled)
    __shared__ int rowinfo[2 * 16];  // [0,16): A row of each local row; [16,32): D row or -1
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, quad = lane >> 4;
    const int nstrips = p.Np / 16, nc = p.nc;
    constexpr int UPC = 16;     // 16-byte A units per chunk and row (bf16)
    const int U = nc * UPC;     // A units per LDS row

    // ---- the m-tile list ----
    const int* tinfo = p.tile_info;
    const int* srt = p.sorted;
    int nt;
    if (p.route_ids || p.route_off) {
        __shared__ int rt_tile[3 * kRouteMaxP], rt_srt[kRouteMaxP], rt_exp[kRouteMaxP], rt_rank[kRouteMaxP],
            rt_tmp[kRouteMaxP], rt_n;
        nt = moe_route_inline(p, rt_tile, rt_srt, rt_exp, rt_rank, rt_tmp, &rt_n);
        tinfo = rt_tile;
        srt = p.route_ids ? rt_srt : nullptr;
    } else {
        nt = *p.ntiles;
    }

    // ---- this wave's strips ----
    const int gw = blockIdx.x * 4 + wave, wstride = gridDim.x * 4;
    const int nsw = gw < nstrips ? (nstrips - 1 - gw) / wstride + 1 : 0;  // strips of this wave per tile

    for (int t = blockIdx.y; t < nt; t += gridDim.y) {
        // the tile's fields are the same for the whole workgroup: scalar registers
        const int e = __builtin_amdgcn_readfirstlane(tinfo[3 * t]);
        const int first = __builtin_amdgcn_readfirstlane(tinfo[3 * t + 1]);
        const int rows = __builtin_amdgcn_readfirstlane(tinfo[3 * t + 2]);
        if (tid < 16) {
            const int rr = tid < rows ? tid : rows - 1;
            const int pos = first + rr;
            const int pair = srt ? srt[pos] : pos;
            rowinfo[tid] = srt ? pair / p.top_k : pos;
            rowinfo[16 + tid] = tid < rows ? pair : -1;
        }
        __syncthreads();  // no load is in flight yet, so this drains nothing
        const char* Wb = (const char*)p.W + (int64_t)e * p.w_estride;
        const uint8_t* Sb = (const uint8_t*)p.S + (int64_t)e * p.s_estride;

        // ---- 1. the tile's A rows -> LDS (direct loads, 64 units per wave instruction) ----
        {
            const int nblk = (U + 63) >> 6;
            int r = 0, blk = wave;
            while (r < rows && blk >= nblk) {
                blk -= nblk;
                ++r;
            }
            while (r < rows) {
                const int pos = blk * 64 + lane;
                const char* arow = (const char*)p.A + (size_t)rowinfo[r] * p.K * 2;
                if (pos < U) lds_dma16(arow + ((pos ^ skinny_swz<UPC>(r)) * 16), lds + (r * U + blk * 64) * 16);
                blk += 4;
                while (r < rows && blk >= nblk) {
                    blk -= nblk;
                    ++r;
                }
            }
        }

        // ---- 2. NB batches of CB chunks per strip, two in flight ----
        // Buffer loads: the expert's weights and E8M0 bytes as resources, the
        // lane's offset in a VGPR and the chunk's offset in an SGPR.
        const rsrc_t rW = make_rsrc(Wb, (uint32_t)p.w_estride), rS = make_rsrc(Sb, (uint32_t)p.s_estride);
        const uint32_t wl = (uint32_t)lane * 16u, sl = (uint32_t)lane;
        constexpr uint32_t kNone = 0x80000000u;  // past every resource: reads zeros
        v4u w[2][CB];
        uint32_t sc[2][CB];
        // batch b of strip j of this wave -> buffer B
        auto issue = [&](auto bufc, int j, int b) {
            constexpr int B = decltype(bufc)::value;
            const bool live = j < nsw;
            const uint32_t s0 = (uint32_t)(gw + j * wstride) * (uint32_t)nc;
#pragma unroll
            for (int c = 0; c < CB; ++c) {
                const int k = b * CB + c;
                const bool ok = live && k < nc;
                w[B][c] = buf16<true>(rW, wl, ok ? (s0 + (uint32_t)k) * 1024u : kNone);
                sc[B][c] = buf1(rS, sl, ok ? (s0 + (uint32_t)k) * 64u : kNone);
            }
        };
        using Z0 = std::integral_constant<int, 0>;
        using Z1 = std::integral_constant<int, 1>;
        issue(Z0{}, 0, 0);
        __builtin_amdgcn_sched_barrier(0);  // buffer 0's loads all before buffer 1's, as in the loop
        issue(Z1{}, 0, 1);
        __builtin_amdgcn_sched_barrier(0);
        // the A copies were issued before the batch loads: once only those are
        // outstanding, this wave's copies have landed
        wait_vmcnt<4 * CB>();
        lds_barrier();

        // This lane's A units of K sub-step tt (rows past the tile read its last
        // row).  A tile has at most 16 rows, so the swizzle only permutes the 16
        // units of a chunk: chunk k's unit is this base + k * 256, an immediate
        // offset once the batch sequence is unrolled.
        const int arow = min(col, rows - 1);
        const int asw = skinny_swz<UPC>(arow);
        const char* abase[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) abase[tt] = lds + (size_t)arow * U * 16 + ((4 * quad + tt) ^ asw) * 16;
        // batch b from buffer B into the two accumulators (chunks past K skipped)
        auto compute = [&](auto bufc, int b, v4f(&acc)[2]) {
            constexpr int B = decltype(bufc)::value;
#pragma unroll
            for (int c = 0; c < CB; ++c) {
                const int k = b * CB + c;
                if (k < nc) {
                    const float sf = e8m0_to_f32(sc[B][c]);
                    Frag8 a[4];
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt) a[tt].u = *(const v4u*)(abase[tt] + k * 256);
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt) {
                        const Frag8 bf = fp4_to_bf16(w[B][c][tt], sf);
                        acc[tt & 1] = mfma16<true>(a[tt], bf, acc[tt & 1]);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);  // one chunk at a time
            }
        };
        for (int j = 0; j < nsw; ++j) {
            v4f acc[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                wait_vmcnt<2 * CB>();  // batch b has landed; batch b + 1 may still fly
                __builtin_amdgcn_sched_barrier(0);
                if (b & 1) {
                    compute(Z1{}, b, acc);
                    if (b + 2 < NB) issue(Z1{}, j, b + 2);
                    else issue(Z1{}, j + 1, b + 2 - NB);
                } else {
                    compute(Z0{}, b, acc);
                    if (b + 2 < NB) issue(Z0{}, j, b + 2);
                    else issue(Z0{}, j + 1, b + 2 - NB);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            // the strip's rows: lane (col, quad) holds rows 4 quad + r of column col
            const v4f o = acc[0] + acc[1];
            const int n = (gw + j * wstride) * 16 + col;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = quad * 4 + r;
                const int drow = rowinfo[16 + m];
                if (drow >= 0 && n < p.N) ((uint16_t*)p.D)[(int64_t)drow * p.N + n] = f32_to_bf16_bits(o[r]);
            }
        }
        wait_vmcnt<0>();  // the two batches past the wave's last strip (zeros)
        __syncthreads();  // the next tile overwrites A and rowinfo
    }
}

// Launch over the m-tiles of `s` (tile list, or routing in the kernel):
// `gy` workgroup rows walk the tiles, and enough workgroup columns that the
// chip holds about four workgroups per CU, each wave taking at least one strip.
// The strip's batches come from the smallest instantiated CB x NB that covers
// K (K=7168: 7 x 8 exactly; K=2048: 8 x 2).
inline bool moe_stream_fits(int nc) { return nc <= 8 * 16; }

template <int CB, int NB>
hipError_t launch_moe_stream_k(const MoeStreamArgs& s, size_t lds, dim3 grid, hipStream_t st) {
    static const hipError_t attr = hipFuncSetAttribute((const void*)moe_stream_kernel<CB, NB>,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, kSkinnyLds);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((moe_stream_kernel<CB, NB>), grid, dim3(256), lds, st, s);
    return hipGetLastError();
}

inline hipError_t launch_moe_stream(const MoeStreamArgs& s, int rows_max, int64_t gy, hipStream_t st) {
    const int64_t lds = (int64_t)rows_max * s.nc * 256;  // A rows: rows x K bf16
    if (!moe_stream_fits(s.nc) || lds < 1 || lds > kSkinnyLds) return hipErrorInvalidValue;
    if (gy < 1) gy = 1;
    const int64_t nstrips = s.Np / 16;
    int64_t gx = cdiv(1024, gy);
    const int64_t gxmax = cdiv(nstrips, 4);
    if (gx > gxmax) gx = gxmax;
    if (gx < 1) gx = 1;
    const dim3 grid((unsigned)gx, (unsigned)gy);
    const int nc = s.nc;
    if (nc <= 8) return launch_moe_stream_k<4, 2>(s, (size_t)lds, grid, st);
    if (nc <= 16) return launch_moe_stream_k<8, 2>(s, (size_t)lds, grid, st);  // K = 2048 (down projection)
    if (nc <= 32) return launch_moe_stream_k<8, 4>(s, (size_t)lds, grid, st);
    if (nc <= 56) return launch_moe_stream_k<7, 8>(s, (size_t)lds, grid, st);
    if (nc <= 64) return launch_moe_stream_k<8, 8>(s, (size_t)lds, grid, st);
    return launch_moe_stream_k<8, 16>(s, (size_t)lds, grid, st);
}

}  // namespace hq
