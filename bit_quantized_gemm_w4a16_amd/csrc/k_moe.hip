// MoE: routing metadata, Grouped-path gather, and the expert GEMM launches.
//
// "Humming wird angekuendigt", section "WnA16": MoE runs on an Indexed path
// (token rows gathered per expert by index) and a Grouped path (tokens sorted
// by expert, contiguous per expert); the work per expert varies with the
// routing.  Both paths share one schedule over device-built lists of m-tiles
// (expert, first sorted row, row count), one list per tier of experts by row
// count: the weight-streaming kernel (moe_stream.hpp) for experts with a few
// rows, tiled MFMA kernels of growing height for the rest.  Experts with many
// tokens get many tiles, experts with none get none, and each grid is sized by
// the host from an upper bound so no host synchronisation is needed.
//
// Routing metadata is a stable counting sort of the flattened pairs
// p = t * top_k + j by expert id: per-chunk histograms and in-chunk ranks,
// a per-expert scan over chunks, one workgroup for the expert offsets and the
// m-tile lists, then the scatter (one workgroup does it all up to 1024 pairs;
// up to 64 pairs the streaming kernel's workgroups build their list in LDS).
#include "hq_device.hpp"
#include "hq_internal.h"
#include "moe_stream.hpp"

namespace hq {

constexpr int kMoeChunk = 256;  // pairs per histogram chunk
constexpr int kMoeBM = 128;     // rows per m-tile of the tiled expert GEMM
// Experts are served in four tiers by their row count: up to kMoeSmallRows
// rows on the weight-streaming kernel (one m-tile, its A rows in LDS for all
// of K), up to kMoeMidMax rows on the tiled kernel with kMoeMidBM-row tiles,
// up to kMoeBigMax on kMoeBM-row tiles and the rest on kMoeHugeBM-row tiles,
// so no expert pads its rows more than ~2x and the busiest ones get the most
// efficient tile.
constexpr int kMoeSmallRows = 4;
constexpr int kMoeAllSmallP = 64;  // at most this many pairs: every expert on the streaming path
constexpr int kMoeSmallGridY = 32;  // workgroup rows walking the tier-0 m-tiles
constexpr int kMoeMidBM = 32;
constexpr int kMoeMidMax = 64;
constexpr int kMoeBigMax = 256;  // up to this many rows: kMoeBM-row tiles; beyond: kMoeHugeBM
constexpr int kMoeHugeBM = 256;

// ---- 1. per-chunk histogram + rank of each pair among equal ids before it ----
// hist is expert-major: hist[e * C + c].
__global__ __launch_bounds__(256) void moe_hist_kernel(const int* __restrict__ ids, int P, int E, int C,
                                                       int* __restrict__ hist, int* __restrict__ lrank) {
    extern __shared__ int sh[];  // [E] histogram, then [kMoeChunk] ids
    int* h = sh;
    int* cid = sh + E;
    const int c = blockIdx.x, t = threadIdx.x, p = c * kMoeChunk + t;
    for (int e = t; e < E; e += 256) h[e] = 0;
    const int id = p < P ? ids[p] : -1;
    cid[t] = id;
    __syncthreads();
    if (id >= 0 && id < E) {
        int r = 0;
        for (int j = 0; j < t; ++j) r += cid[j] == id;
        lrank[p] = r;
        atomicAdd(&h[id], 1);
    }
    __syncthreads();
    for (int e = t; e < E; e += 256) hist[(int64_t)e * C + c] = h[e];
}

// ---- 2a. per expert (one wave): exclusive scan of its chunk counts, total ----
__global__ __launch_bounds__(64) void moe_colscan_kernel(int* __restrict__ hist, int C, int* __restrict__ counts) {
    const int e = blockIdx.x, l = threadIdx.x;
    int* row = hist + (int64_t)e * C;
    int carry = 0;
    for (int c0 = 0; c0 < C; c0 += 64) {
        const int v = c0 + l < C ? row[c0 + l] : 0;
        int incl = v;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int o = __shfl_up(incl, off, 64);
            if (l >= off) incl += o;
        }
        if (c0 + l < C) row[c0 + l] = carry + incl - v;
        carry += __shfl(incl, 63, 64);
    }
    if (l == 0) counts[e] = carry;
}

// Block-wide exclusive scans of N values per thread over 1024 threads: a
// shuffle scan inside each wave, then the 16 wave totals through LDS
// (tmp holds 16 * N ints); two barriers for all N values.
template <int N>
__device__ void block_excl_scan_1024(int (&v)[N], int* tmp) {
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    int incl[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
        incl[i] = v[i];
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int o = __shfl_up(incl[i], off, 64);
            if (lane >= off) incl[i] += o;
        }
        if (lane == 63) tmp[wave * N + i] = incl[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < N; ++i) {
        int before = 0;
        for (int w = 0; w < wave; ++w) before += tmp[w * N + i];
        v[i] = before + incl[i] - v[i];
    }
    __syncthreads();
}

// ---- 2b. expert offsets and the m-tile lists (one workgroup) ----
// Counts come from `counts` (Indexed) or from the caller's offsets (Grouped).
// Caller-given offsets are clamped to [0, P] so malformed input can never
// address rows outside A or D.  An expert with c rows goes to the first tier
// with c <= upto: the tier's list gets ceil(c / bm) m-tiles of at most bm rows
// (at most max_tiles entries per list).
struct TileList {
    int* tiles;   // per tile: expert, first sorted row, row count (null: no list)
    int* ntiles;  // number of valid tiles
    int max_tiles, bm, upto;
};
constexpr int kMoeTiers = 4;
struct MoeTiers {
    TileList t[kMoeTiers];
};

// Expert offsets and tier lists from per-expert counts (`counts`, global or
// LDS) or from caller-given offsets; one workgroup of 1024 threads.  The
// offsets also go to `off_lds` when it is not null.
__device__ void moe_offsets_and_tiers(const int* counts, const int* __restrict__ given_off, int E, int P,
                                      int* __restrict__ offsets, int* off_lds, const MoeTiers& tiers, int* tmp,
                                      int* carry) {
    const int t = threadIdx.x;
    if (t <= kMoeTiers) carry[t] = 0;
    __syncthreads();
    for (int e0 = 0; e0 < E; e0 += 4096) {  // 4 experts per thread per round
        int cnt[4], tier[4], ntl[4], sum = 0, tsum[kMoeTiers] = {};
        for (int k = 0; k < 4; ++k) {
            const int e = e0 + 4 * t + k;
            int c = 0;
            if (e < E) {
                if (counts) {
                    c = counts[e];
                } else {
                    const int lo = min(max(given_off[e], 0), P), hi = min(max(given_off[e + 1], lo), P);
                    c = hi - lo;
                }
            }
            cnt[k] = c;
            // first tier with c <= upto (static indices only: a dynamic index into
            // the kernel-argument struct would copy it to scratch memory)
            int q = kMoeTiers - 1, bm = tiers.t[kMoeTiers - 1].bm;
#pragma unroll
            for (int i = kMoeTiers - 2; i >= 0; --i)
                if (c <= tiers.t[i].upto) {
                    q = i;
                    bm = tiers.t[i].bm;
                }
            tier[k] = q;
            ntl[k] = (c + bm - 1) / bm;
            sum += c;
#pragma unroll
            for (int i = 0; i < kMoeTiers; ++i) tsum[i] += i == q ? ntl[k] : 0;
        }
        int sc[1 + kMoeTiers];
        sc[0] = sum;
#pragma unroll
        for (int i = 0; i < kMoeTiers; ++i) sc[1 + i] = tsum[i];
        block_excl_scan_1024(sc, tmp);
        int run = carry[0] + sc[0];
        int trun[kMoeTiers];
#pragma unroll
        for (int i = 0; i < kMoeTiers; ++i) trun[i] = carry[1 + i] + sc[1 + i];
        for (int k = 0; k < 4; ++k) {
            const int e = e0 + 4 * t + k;
            if (e < E) {
                const int start = counts ? run : min(max(given_off[e], 0), P);
                if (offsets) offsets[e] = start;
                if (off_lds) off_lds[e] = start;
#pragma unroll
                for (int i = 0; i < kMoeTiers; ++i) {
                    const TileList& L = tiers.t[i];
                    if (i != tier[k] || !L.tiles) continue;
                    for (int q = 0; q < ntl[k] && trun[i] + q < L.max_tiles; ++q) {
                        L.tiles[3 * (trun[i] + q)] = e;
                        L.tiles[3 * (trun[i] + q) + 1] = start + q * L.bm;
                        L.tiles[3 * (trun[i] + q) + 2] = min(L.bm, cnt[k] - q * L.bm);
                    }
                }
            }
            run += cnt[k];
#pragma unroll
            for (int i = 0; i < kMoeTiers; ++i) trun[i] += i == tier[k] ? ntl[k] : 0;
        }
        __syncthreads();
        if (t == 1023) {
            carry[0] = run;
#pragma unroll
            for (int i = 0; i < kMoeTiers; ++i) carry[1 + i] = trun[i];
        }
        __syncthreads();
    }
    if (t == 0) {
        if (offsets) offsets[E] = carry[0];
#pragma unroll
        for (int i = 0; i < kMoeTiers; ++i)
            if (tiers.t[i].ntiles) *tiers.t[i].ntiles = min(carry[1 + i], tiers.t[i].max_tiles);
    }
    __syncthreads();
}

__global__ __launch_bounds__(1024) void moe_offsets_kernel(const int* __restrict__ counts, const int* __restrict__ given_off,
                                                           int E, int P, int* __restrict__ offsets, MoeTiers tiers) {
    __shared__ int tmp[1024];
    __shared__ int carry[1 + kMoeTiers];
    moe_offsets_and_tiers(counts, given_off, E, P, offsets, nullptr, tiers, tmp, carry);
}

// ---- routing of at most 1024 pairs in one workgroup: counts, offsets, tier
// lists and the stable placement (rank = equal ids before the pair) ----
constexpr int kMoeSmallP = 1024;
__global__ __launch_bounds__(1024) void moe_route_small_kernel(const int* __restrict__ ids, int P, int E,
                                                               int* __restrict__ offsets, int* __restrict__ sorted,
                                                               MoeTiers tiers) {
    __shared__ int cnt[4096];
    __shared__ int off[4096];
    __shared__ int cid[kMoeSmallP];
    __shared__ int tmp[1024];
    __shared__ int carry[1 + kMoeTiers];
    const int t = threadIdx.x;
    for (int e = t; e < E; e += 1024) cnt[e] = 0;
    const int id = t < P ? ids[t] : -1;
    const bool ok = id >= 0 && id < E;
    cid[t] = ok ? id : -1;
    __syncthreads();
    if (ok) atomicAdd(&cnt[id], 1);
    __syncthreads();
    moe_offsets_and_tiers(cnt, nullptr, E, P, offsets, off, tiers, tmp, carry);
    if (ok) {
        int r = 0;
        for (int j = 0; j < t; ++j) r += cid[j] == id;
        sorted[off[id] + r] = t;
    }
}

// ---- 3. scatter: sorted[offset(id) + chunk base(id) + rank] = p ----
__global__ __launch_bounds__(256) void moe_place_kernel(const int* __restrict__ ids, int P, int E, int C,
                                                        const int* __restrict__ hist, const int* __restrict__ offsets,
                                                        const int* __restrict__ lrank, int* __restrict__ sorted) {
    const int c = blockIdx.x, p = c * kMoeChunk + threadIdx.x;
    if (p >= P) return;
    const int id = ids[p];
    if (id < 0 || id >= E) return;
    sorted[offsets[id] + hist[(int64_t)id * C + c] + lrank[p]] = p;
}

// ---- gather for the Grouped path: out[i] = A[sorted[i] / top_k] ----
__global__ __launch_bounds__(256) void moe_gather_kernel(const char* __restrict__ A, const int* __restrict__ sorted,
                                                         int P, int top_k, int row_bytes, char* __restrict__ out) {
    const int units = row_bytes / 16;
    const int64_t total = (int64_t)P * units;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
        const int r = (int)(i / units), u = (int)(i % units);
        const int src = min(max(sorted[r], 0), P - 1) / top_k;  // clamped: never outside A
        ((v4u*)(out + (int64_t)r * row_bytes))[u] = ((const v4u*)(A + (int64_t)src * row_bytes))[u];
    }
}

// -------------------------------------------------------------------------
// host side
// -------------------------------------------------------------------------

namespace {
size_t al16(size_t b) { return (b + 15) / 16 * 16; }
}  // namespace

// Upper bounds of the tier lists (the real lengths are known only on the device).
static int64_t moe_max_tiles(int tier, int64_t P, int E) {
    const int64_t ex = E < P ? E : P;  // experts that can hold a row
    if (tier == 0)                     // one m-tile of at most kMoeSmallRows rows per small expert
        return ex;
    if (tier == 1) {                   // at most kMoeMidMax / kMoeMidBM tiles per mid expert
        const int64_t a = cdiv(kMoeMidMax, kMoeMidBM) * ex, b = cdiv(P, kMoeMidBM) + ex;
        return a < b ? a : b;
    }
    if (tier == 2) {                   // experts with kMoeMidMax < rows <= kMoeBigMax
        const int64_t n = P / (kMoeMidMax + 1), ne = E < n ? E : n;
        const int64_t a = cdiv(kMoeBigMax, kMoeBM) * ne, b = cdiv(P, kMoeBM) + ne;
        return a < b ? a : b;
    }
    const int64_t n = P / (kMoeBigMax + 1);
    return cdiv(P, kMoeHugeBM) + (E < n ? E : n);
}

MoeLayout moe_layout(int64_t T, int top_k, int E, bool indexed) {
    MoeLayout L{};
    const int64_t P = T * top_k;
    size_t o = 0;
    L.hist = o;  // hist + lrank + counts (the align scratch)
    o += indexed ? moe_align_workspace(T, top_k, E) : 0;
    L.offsets = o;
    o += indexed ? al16((size_t)(E + 1) * 4) : 0;
    L.sorted = o;
    o += indexed ? al16((size_t)P * 4) : 0;
    for (int i = 0; i < 4; ++i) {
        L.max_tier[i] = moe_max_tiles(i, P, E);
        L.tiles_tier[i] = o;
        o += al16((size_t)(L.max_tier[i] > 0 ? L.max_tier[i] : 1) * 12);
    }
    L.ntiles = o;  // one count per tier
    o += 16;
    L.bytes = o;
    return L;
}

size_t moe_align_workspace(int64_t T, int top_k, int E) {
    const int64_t P = T * top_k, C = cdiv(P, kMoeChunk);
    return al16((size_t)(C * E) * 4) + al16((size_t)P * 4) + al16((size_t)E * 4);
}

hipError_t moe_align_launch(int64_t T, int top_k, int E, const int* ids, int* offsets, int* sorted, void* ws,
                            const MoeTiers* tiers, hipStream_t st) {
    const int P = (int)(T * top_k), C = (int)cdiv(P, kMoeChunk);
    MoeTiers none{};
    for (int i = 0; i < kMoeTiers; ++i) none.t[i] = TileList{nullptr, nullptr, 0, 1, 0};
    const MoeTiers& tl = tiers ? *tiers : none;
    if (P <= kMoeSmallP && E <= 4096) {  // one launch for the whole routing
        hipLaunchKernelGGL(moe_route_small_kernel, dim3(1), dim3(1024), 0, st, ids, P, E, offsets, sorted, tl);
        return hipGetLastError();
    }
    int* hist = (int*)ws;
    int* lrank = (int*)((char*)ws + al16((size_t)C * E * 4));
    int* counts = (int*)((char*)lrank + al16((size_t)P * 4));
    hipLaunchKernelGGL(moe_hist_kernel, dim3(C), dim3(256), (size_t)(E + kMoeChunk) * 4, st, ids, P, E, C, hist, lrank);
    hipLaunchKernelGGL(moe_colscan_kernel, dim3(E), dim3(64), 0, st, hist, C, counts);
    hipLaunchKernelGGL(moe_offsets_kernel, dim3(1), dim3(1024), 0, st, (const int*)counts, (const int*)nullptr, E, P,
                       offsets, tl);
    hipLaunchKernelGGL(moe_place_kernel, dim3(C), dim3(256), 0, st, ids, P, E, C, (const int*)hist,
                       (const int*)offsets, (const int*)lrank, sorted);
    return hipGetLastError();
}

hipError_t moe_gather_launch(const void* A, const int* sorted, int64_t P, int top_k, int64_t row_bytes, void* out,
                             hipStream_t st) {
    const int64_t units = P * (row_bytes / 16);
    int64_t blocks = cdiv(units, 256);
    if (blocks > 8192) blocks = 8192;
    if (blocks < 1) return hipSuccess;
    hipLaunchKernelGGL(moe_gather_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (const char*)A, sorted, (int)P,
                       top_k, (int)row_bytes, (char*)out);
    return hipGetLastError();
}

// Arguments of the MoE weight-streaming kernel.
static MoeStreamArgs moe_stream_args(const MoeArgs& a, int nc) {
    MoeStreamArgs s{};
    s.A = a.A;
    s.W = a.w;
    s.S = a.s;
    s.D = a.D;
    s.w_estride = a.w_estride;
    s.s_estride = a.s_estride;
    s.K = (int)a.K;
    s.N = (int)a.N;
    s.Np = (int)a.Np;
    s.nc = nc;
    s.top_k = a.top_k;
    return s;
}

// At most kMoeAllSmallP pairs: one launch of the weight-streaming kernel, whose
// workgroups each build the m-tile list from the ids or offsets (no routing
// pass; measured faster than a routing launch of its own at every such size).
// A token picks an expert at most once, so an expert has at most T rows: tiles
// of min(T, kMoeSmallRows) rows cover each expert in as few tiles as the
// streaming kernel's row limit allows, and below kMoeSmallRows tokens the A
// rows held in LDS shrink with T, which leaves room for more workgroups per
// CU.  (Tiles never exceed that many rows whatever the ids, so repeated ids
// only cost extra tiles.)
static_assert(kMoeAllSmallP <= kRouteMaxP, "the in-kernel routing handles one pair per lane");
static hipError_t moe_all_small_launch(const MoeArgs& a, int64_t P, int nc) {
    const int cap = (int)(a.T < kMoeSmallRows ? a.T : kMoeSmallRows);
    MoeStreamArgs s = moe_stream_args(a, nc);
    s.route_ids = a.indexed ? a.topk_ids : nullptr;
    s.route_off = a.indexed ? nullptr : a.expert_offsets;
    s.route_P = (int)P;
    s.route_E = a.E;
    s.route_cap = cap;
    // every tile holds a row, so at most P tiles
    return launch_moe_stream(s, cap, P < kMoeSmallGridY ? P : kMoeSmallGridY, a.stream);
}

// Experts with few rows (the common case below a few thousand tokens) run on
// the weight-streaming kernel in m-tiles of kMoeSmallRows rows: their
// weights are read once per m-tile without padding the tile to 128 rows.
// Experts with more rows run on the tiled MFMA kernel.
hipError_t moe_gemm_launch(const MoeArgs& a) {
    const int64_t P = a.T * a.top_k;
    // The weight-streaming path holds a tile's A rows for all of K in LDS; a
    // larger K sends its experts to the mid tier.
    const int nc = (int)(a.K / 128);
    const bool small_ok = moe_stream_fits(nc) && (int64_t)kMoeSmallRows * nc * 256 <= kSkinnyLds;
    // With few pairs in total no expert can fill a tile: every expert takes the
    // streaming path (several m-tiles if it must) and no tiled launch is made.
    const bool all_small = small_ok && P <= kMoeAllSmallP;
    if (all_small) return moe_all_small_launch(a, P, nc);
    MoeLayout L = moe_layout(a.T, a.top_k, a.E, a.indexed);
    char* ws = (char*)a.ws;
    int* ntiles = (int*)(ws + L.ntiles);
    int* tl[4];
    for (int i = 0; i < 4; ++i) tl[i] = (int*)(ws + L.tiles_tier[i]);
    MoeTiers tiers{};
    tiers.t[0] = TileList{tl[0], ntiles + 0, (int)L.max_tier[0], kMoeSmallRows, small_ok ? kMoeSmallRows : 0};
    tiers.t[1] = TileList{tl[1], ntiles + 1, (int)L.max_tier[1], kMoeMidBM, kMoeMidMax};
    tiers.t[2] = TileList{tl[2], ntiles + 2, (int)L.max_tier[2], kMoeBM, kMoeBigMax};
    tiers.t[3] = TileList{tl[3], ntiles + 3, (int)L.max_tier[3], kMoeHugeBM, 1 << 30};
    const int* sorted = nullptr;
    hipError_t e;
    if (a.indexed) {  // routing builds the tier lists from the counts
        int* offsets = (int*)(ws + L.offsets);
        int* srt = (int*)(ws + L.sorted);
        e = moe_align_launch(a.T, a.top_k, a.E, a.topk_ids, offsets, srt, ws + L.hist, &tiers, a.stream);
        if (e != hipSuccess) return e;
        sorted = srt;
    } else {  // Grouped: tier lists from the caller's offsets
        hipLaunchKernelGGL(moe_offsets_kernel, dim3(1), dim3(1024), 0, a.stream, (const int*)nullptr, a.expert_offsets,
                           a.E, (int)P, (int*)nullptr, tiers);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // tier 0 (at most kMoeSmallRows rows): weight-streaming kernel, persistent over its m-tiles
    if (small_ok) {
        MoeStreamArgs s = moe_stream_args(a, nc);
        s.tile_info = tl[0];
        s.ntiles = ntiles + 0;
        s.sorted = sorted;
        e = launch_moe_stream(s, kMoeSmallRows, L.max_tier[0] < kMoeSmallGridY ? L.max_tier[0] : kMoeSmallGridY,
                              a.stream);
        if (e != hipSuccess) return e;
    }
    // tiers 1 and 2: tiled MFMA kernel over m-tiles of kMoeMidBM / kMoeBM rows
    TileArgs p{};
    p.A = a.A;
    p.W = a.w;
    p.S = a.s;
    p.D = a.D;
    p.N = (int)a.N;
    p.K = (int)a.K;
    p.Np = (int)a.Np;
    p.M = (int)P;
    p.a_rows = (int)(a.indexed ? a.T : P);
    p.ngroups = 1;
    p.gsteps = 1;
    p.w_estride = a.w_estride;
    p.s_estride = a.s_estride;
    p.tiles_n = (int)cdiv(a.Np, 256);
    p.splits = 1;
    p.sorted = sorted;
    p.top_k = a.top_k;
    p.tiles_m = (int)L.max_tier[1];
    p.tile_info = tl[1];
    p.ntiles = ntiles + 1;
    if (p.tiles_m > 0) {
        hipLaunchKernelGGL((tile_gemm_kernel<Fmt::MOE_MX, kMoeMidBM, 256, 1, 8, 0>), dim3((unsigned)(p.tiles_m * p.tiles_n)),
                           dim3(512), 0, a.stream, p);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // experts with more than kMoeMidMax rows: 256-column tiles of 8 waves side by
    // side (each wave decodes its weight strips once; the 256-row tile keeps one
    // weight LDS stage and feeds each decoded fragment to 16 MFMAs)
    p.tiles_m = (int)L.max_tier[2];
    p.tile_info = tl[2];
    p.ntiles = ntiles + 2;
    if (p.tiles_m > 0) {
        hipLaunchKernelGGL((tile_gemm_kernel<Fmt::MOE_MX, kMoeBM, 256, 1, 8, 0>), dim3((unsigned)(p.tiles_m * p.tiles_n)),
                           dim3(512), 0, a.stream, p);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    p.tiles_m = (int)L.max_tier[3];
    p.tile_info = tl[3];
    p.ntiles = ntiles + 3;
    if (p.tiles_m > 0) {
        hipLaunchKernelGGL((tile_gemm_kernel<Fmt::MOE_MX, kMoeHugeBM, 256, 1, 8, 3>), dim3((unsigned)(p.tiles_m * p.tiles_n)),
                           dim3(512), 0, a.stream, p);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace hq
