// hq_repack: host-side transform from the logical export form to the packed
// layout every hq kernel reads.  Integer bit permutation only (exact).
//
// The pages describe this step as converting each export format into one
// standard representation and then validating, padding and repacking it into
// a layout suited to the target kernel ("Humming wird angekuendigt", sections
// "Eine einheitliche Quantisierungsdarstellung" and "Tuning und
// JIT-Kompilierung fuer jeden Workload").  The packed layout below is our own,
// chosen for CDNA4: a wavefront's 64 lanes read 1 KB contiguous with one
// 16-byte load each, and that 16-byte load is directly the MFMA operand
// fragment (see include/hq.h for the exact layout).
#include <cstdint>
#include <cstring>
#include <vector>

#include "hq_common.h"

namespace hq {

namespace {

// nibble position p of a packed INT4/UINT4 word holds element kPairOrder[p]
constexpr int kPairOrder[8] = {0, 2, 4, 6, 1, 3, 5, 7};

inline uint32_t logical_word(const uint32_t* w, int64_t N, int64_t j, int64_t n) {
    return w[j * N + n];
}

void repack_4bit(const LayerInfo& L, const uint32_t* w, uint8_t* out, bool pair_order) {
    const int64_t N = L.N, K = L.K, nst = L.Np / 16, nc = K / 128;
    for (int64_t e = 0; e < L.E; ++e) {
        const uint32_t* we = w + e * (K / 8) * N;
        uint32_t* oe = (uint32_t*)(out + (size_t)e * (size_t)(nst * nc * 1024));
        for (int64_t st = 0; st < nst; ++st)
            for (int64_t c = 0; c < nc; ++c)
                for (int lane = 0; lane < 64; ++lane) {
                    const int64_t n = st * 16 + (lane & 15);
                    for (int t = 0; t < 4; ++t) {
                        const int64_t j = (c * 128 + 32 * (lane >> 4) + 8 * t) / 8;
                        const uint32_t src = n < N ? logical_word(we, N, j, n) : 0u;
                        uint32_t dst = src;
                        if (pair_order) {
                            dst = 0;
                            for (int p = 0; p < 8; ++p) dst |= ((src >> (4 * kPairOrder[p])) & 15u) << (4 * p);
                        }
                        oe[((st * nc + c) * 64 + lane) * 4 + t] = dst;
                    }
                }
    }
}

// Low-bit codes (one per byte, [K][N]) into bit planes: a 2-bit plane
// [Np/16][K/128][64 lanes][2 words] (widths 2 and 3: the low two bits), then a
// 1-bit plane [Np/16][K/128][64 lanes][1 word] (width 1: the bit; width 3: bit
// 2).  Code j (0..7) of sub-step t (0..3) of the lane's 32 K (k = 128*chunk +
// 32*(lane >> 4) + 8*t + j) sits at bit 16*(j&1) + 8*(t&1) + 2*(j>>1) of 2-bit
// word t>>1 and at bit 16*(j&1) + 4*t + (j>>1) of the 1-bit word: the two codes
// of a pair (2s, 2s+1) share an offset in the two 16-bit halves, as the two
// 16-bit operands of the kernels' decode.  Codes keep their two's-complement
// bits; padding columns hold 0.
void repack_lowbit(const LayerInfo& L, const int8_t* w, uint8_t* out) {
    const int64_t N = L.N, K = L.K, nst = L.Np / 16, nc = K / 128;
    const int b = L.bits;
    const bool two = b >= 2, one = b != 2;
    uint32_t* p2 = (uint32_t*)out;
    uint32_t* p1 = (uint32_t*)(out + (two ? (size_t)(nst * nc * 512) : 0));
    for (int64_t st = 0; st < nst; ++st)
        for (int64_t c = 0; c < nc; ++c)
            for (int lane = 0; lane < 64; ++lane) {
                const int64_t n = st * 16 + (lane & 15), slot = (st * nc + c) * 64 + lane;
                uint32_t x[2] = {0u, 0u}, y = 0u;
                for (int t = 0; t < 4; ++t)
                    for (int j = 0; j < 8; ++j) {
                        const int64_t k = c * 128 + 32 * (lane >> 4) + 8 * t + j;
                        const uint32_t code = n < N ? (uint32_t)(uint8_t)w[k * N + n] : 0u;
                        x[t >> 1] |= (code & 3u) << (16 * (j & 1) + 8 * (t & 1) + 2 * (j >> 1));
                        y |= ((b == 1 ? code : code >> 2) & 1u) << (16 * (j & 1) + 4 * t + (j >> 1));
                    }
                if (two) {
                    p2[slot * 2] = x[0];
                    p2[slot * 2 + 1] = x[1];
                }
                if (one) p1[slot] = y;
            }
}

// FP6 codes (one per byte, [K][N], the low six bits) into two planes that
// together hold a lane's 32 codes of a chunk as one 192-bit group, code j
// (k = 128*chunk + 32*(lane >> 4) + j) at bits 6j..6j+5 (the element order of
// the packed FP6 convert): bits 0-127 in a 16-byte plane [Np/16][K/128][64
// lanes][16 B], bits 128-191 after it in an 8-byte plane [Np/16][K/128][64
// lanes][8 B].  Padding columns hold code 0.
void repack_fp6(const LayerInfo& L, const uint8_t* w, uint8_t* out) {
    const int64_t N = L.N, K = L.K, nst = L.Np / 16, nc = K / 128;
    uint32_t* pa = (uint32_t*)out;
    uint32_t* pb = (uint32_t*)(out + (size_t)(nst * nc * 1024));
    for (int64_t st = 0; st < nst; ++st)
        for (int64_t c = 0; c < nc; ++c)
            for (int lane = 0; lane < 64; ++lane) {
                const int64_t n = st * 16 + (lane & 15), slot = (st * nc + c) * 64 + lane;
                uint32_t x[6] = {0u, 0u, 0u, 0u, 0u, 0u};
                for (int j = 0; j < 32; ++j) {
                    const int64_t k = c * 128 + 32 * (lane >> 4) + j;
                    const uint64_t code = n < N ? (uint64_t)(w[k * N + n] & 63u) : 0u;
                    const int bit = 6 * j;
                    const uint64_t v = code << (bit & 31);
                    x[bit >> 5] |= (uint32_t)v;
                    if ((bit & 31) > 26) x[(bit >> 5) + 1] |= (uint32_t)(v >> 32);
                }
                for (int d = 0; d < 4; ++d) pa[slot * 4 + d] = x[d];
                pb[slot * 2] = x[4];
                pb[slot * 2 + 1] = x[5];
            }
}

// 5-8-bit codes (one per byte, [K][N]): the low nibble of every code in the
// 4-bit layout (pair order), then the high bits: width 5-7 as the low-bit planes
// of a (bits - 4)-bit code (2-bit plane, then 1-bit plane), width 8 as a second
// 4-bit word set.  Signed codes keep their two's-complement bits.
void repack_wide(const LayerInfo& L, const uint8_t* w, uint8_t* out) {
    const int64_t N = L.N, K = L.K, nst = L.Np / 16, nc = K / 128;
    const int e = L.bits - 4;
    std::vector<uint32_t> lo((size_t)(K / 8 * N), 0u), hi4(e == 4 ? (size_t)(K / 8 * N) : 0, 0u);
    std::vector<int8_t> hi((size_t)(e < 4 ? K * N : 0));
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n) {
            const uint32_t c = w[k * N + n];
            lo[(size_t)((k / 8) * N + n)] |= (c & 15u) << (4 * (k % 8));
            if (e == 4) hi4[(size_t)((k / 8) * N + n)] |= ((c >> 4) & 15u) << (4 * (k % 8));
            else hi[(size_t)(k * N + n)] = (int8_t)((c >> 4) & ((1u << e) - 1u));
        }
    repack_4bit(L, lo.data(), out, true);
    uint8_t* o2 = out + (size_t)(nst * nc * 1024);
    if (e == 4) {
        repack_4bit(L, hi4.data(), o2, true);
    } else {
        LayerInfo Lh = L;
        Lh.bits = e;
        repack_lowbit(Lh, hi.data(), o2);
    }
}

// UINT8 zero-points [K/G][N] -> [Np/16][K/G][16] bytes (padding columns 0)
void repack_zero8(const LayerInfo& L, const uint8_t* z, uint8_t* out) {
    const int64_t N = L.N, ng = L.K / L.G, nst = L.Np / 16;
    for (int64_t st = 0; st < nst; ++st)
        for (int64_t g = 0; g < ng; ++g)
            for (int i = 0; i < 16; ++i) {
                const int64_t n = st * 16 + i;
                out[(st * ng + g) * 16 + i] = n < N ? z[g * N + n] : 0;
            }
}

void repack_int8(const LayerInfo& L, const int8_t* w, int8_t* out) {
    const int64_t N = L.N, K = L.K, nst = L.Np / 16, nc = K / 64;
    for (int64_t e = 0; e < L.E; ++e) {
        const int8_t* we = w + e * K * N;
        int8_t* oe = out + (size_t)e * (size_t)(nst * nc * 1024);
        for (int64_t st = 0; st < nst; ++st)
            for (int64_t c = 0; c < nc; ++c)
                for (int lane = 0; lane < 64; ++lane) {
                    const int64_t n = st * 16 + (lane & 15);
                    for (int j = 0; j < 16; ++j) {
                        const int64_t k = c * 64 + 16 * (lane >> 4) + j;
                        oe[((st * nc + c) * 64 + lane) * 16 + j] = n < N ? we[k * N + n] : 0;
                    }
                }
    }
}

// INT8 weight-only: [E][Np/16][K/128][2 halves][64 lanes][16 B]; lane l holds column
// 16*strip + (l & 15) and, in half h, K = 128*chunk + 32*(l >> 4) + 16*h + j (a lane's
// 32 consecutive K of the chunk, the K order of the 16-bit activation fragments).
void repack_int8_k32(const LayerInfo& L, const int8_t* w, int8_t* out) {
    const int64_t N = L.N, K = L.K, nst = L.Np / 16, nc = K / 128;
    for (int64_t e = 0; e < L.E; ++e) {
        const int8_t* we = w + e * K * N;
        int8_t* oe = out + (size_t)e * (size_t)(nst * nc * 2048);
        for (int64_t st = 0; st < nst; ++st)
            for (int64_t c = 0; c < nc; ++c)
                for (int h = 0; h < 2; ++h)
                    for (int lane = 0; lane < 64; ++lane) {
                        const int64_t n = st * 16 + (lane & 15);
                        for (int j = 0; j < 16; ++j) {
                            const int64_t k = c * 128 + 32 * (lane >> 4) + 16 * h + j;
                            oe[(((st * nc + c) * 2 + h) * 64 + lane) * 16 + j] = n < N ? we[k * N + n] : 0;
                        }
                    }
    }
}

void repack_scale16(const LayerInfo& L, const uint16_t* s, uint16_t* out, uint16_t one) {
    const int64_t N = L.N, nst = L.Np / 16, ng = L.K / L.G;
    for (int64_t e = 0; e < L.E; ++e) {
        const uint16_t* se = s + e * ng * N;
        uint16_t* oe = out + e * nst * ng * 16;
        for (int64_t st = 0; st < nst; ++st)
            for (int64_t g = 0; g < ng; ++g)
                for (int i = 0; i < 16; ++i) {
                    const int64_t n = st * 16 + i;
                    oe[(st * ng + g) * 16 + i] = n < N ? se[g * N + n] : one;
                }
    }
}

void repack_zero4(const LayerInfo& L, const uint32_t* z, uint64_t* out) {
    const int64_t N = L.N, nst = L.Np / 16, ng = L.K / L.G, zw = (N + 7) / 8;
    for (int64_t e = 0; e < L.E; ++e) {
        const uint32_t* ze = z + e * ng * zw;
        uint64_t* oe = out + e * nst * ng;
        for (int64_t st = 0; st < nst; ++st)
            for (int64_t g = 0; g < ng; ++g) {
                uint64_t v = 0;
                for (int i = 0; i < 16; ++i) {
                    const int64_t n = st * 16 + i;
                    const uint64_t code = n < N ? (ze[g * zw + n / 8] >> (4 * (n % 8))) & 15u : 0u;
                    v |= code << (4 * i);
                }
                oe[st * ng + g] = v;
            }
    }
}

void repack_e8m0(const LayerInfo& L, const uint8_t* s, uint8_t* out) {
    const int64_t N = L.N, nst = L.Np / 16, nc = L.K / 128, nb = L.K / 32;
    for (int64_t e = 0; e < L.E; ++e) {
        const uint8_t* se = s + e * nb * N;
        uint8_t* oe = out + (size_t)e * (size_t)(nst * nc * 64);
        for (int64_t st = 0; st < nst; ++st)
            for (int64_t c = 0; c < nc; ++c)
                for (int lane = 0; lane < 64; ++lane) {
                    const int64_t n = st * 16 + (lane & 15);
                    oe[(st * nc + c) * 64 + lane] = n < N ? se[(4 * c + (lane >> 4)) * N + n] : (uint8_t)127;
                }
    }
}

// NVFP4 group scales (E4M3 per 16 K): [E][Np/16][K/128][64 lanes][2 bytes]; lane
// l holds column 16*strip + (l & 15), groups 8*chunk + 2*(l >> 4) + {0, 1}
// (the two 16-K halves of the lane's 32 K); padding columns hold 0x38 (1.0).
void repack_e4m3_g16(const LayerInfo& L, const uint8_t* s, uint8_t* out) {
    const int64_t N = L.N, nst = L.Np / 16, nc = L.K / 128, ng = L.K / 16;
    for (int64_t e = 0; e < L.E; ++e) {
        const uint8_t* se = s + e * ng * N;
        uint8_t* oe = out + (size_t)e * (size_t)(nst * nc * 128);
        for (int64_t st = 0; st < nst; ++st)
            for (int64_t c = 0; c < nc; ++c)
                for (int lane = 0; lane < 64; ++lane) {
                    const int64_t n = st * 16 + (lane & 15);
                    for (int h = 0; h < 2; ++h)
                        oe[((st * nc + c) * 64 + lane) * 2 + h] = n < N ? se[(8 * c + 2 * (lane >> 4) + h) * N + n] : (uint8_t)0x38;
                }
    }
}

void repack_chan32(const LayerInfo& L, const float* s, float* out) {
    for (int64_t e = 0; e < L.E; ++e)
        for (int64_t n = 0; n < L.Np; ++n) out[e * L.Np + n] = n < L.N ? s[e * L.N + n] : 1.0f;
}

}  // namespace

void packed_sizes(const LayerInfo& L, size_t* w, size_t* s, size_t* z, size_t* s2) {
    const size_t E = (size_t)L.E, nst = (size_t)(L.Np / 16);
    *w = *s = *z = *s2 = 0;
    switch (L.kind) {
        case Kind::WNA16:
            // 4-bit: 16 B per lane and chunk; low-bit: an 8-B plane (widths 2, 3)
            // and a 4-B plane (widths 1, 3)
            // (5-8 bits: the 4-bit word set plus the high-bit planes, or a second word set)
            *w = E * nst * (size_t)(L.K / 128) *
                 (L.bits == 4 ? 1024 : L.bits < 4 ? (L.bits >= 2 ? 512 : 0) + (L.bits != 2 ? 256 : 0)
                                : 1024 + (L.bits == 8 ? 1024 : (L.bits >= 6 ? 512 : 0) + (L.bits != 6 ? 256 : 0)));
            *s = E * nst * (size_t)(L.K / L.G) * 16 * 2;
            if (L.zp) *z = E * nst * (size_t)(L.K / L.G) * (L.zp8 ? 16 : 8);
            break;
        case Kind::W4A8_MX:
        case Kind::MXA_MX:
        case Kind::MOE_MX_BF16:
            *w = E * nst * (size_t)(L.K / 128) * 1024;
            *s = E * nst * (size_t)(L.K / 128) * 64;
            break;
        case Kind::W8A8:
            *w = E * nst * (size_t)(L.K / 64) * 1024;
            *s = E * (size_t)L.Np * 4;
            break;
        case Kind::W8A16:
            *w = E * nst * (size_t)(L.K / 128) * 2048;
            *s = E * (size_t)L.Np * 4;
            break;
        case Kind::FP4_A16:
            // MXFP8: the 8-bit weight-only layout; MXFP6: a 16-byte and an 8-byte plane
            *w = E * nst * (size_t)(L.K / 128) * (L.mxf == 1 ? 2048 : L.mxf ? 1536 : 1024);
            *s = E * nst * (size_t)(L.K / 128) * (L.nv ? 128 : 64);
            if (L.nv) *s2 = E * 4;
            break;
        case Kind::FP8_BLOCK:
            *w = E * nst * (size_t)(L.K / 64) * 1024;
            *s = E * (size_t)(L.K / 128) * (size_t)((L.N + 127) / 128) * 4;
            break;
    }
}

// e0mN code (sign bit n, magnitude in bits 0..n-1) -> its two's-complement value
static int8_t e0m_value(uint32_t c, int n) {
    const int m = (int)(c & ((1u << n) - 1u));
    return (int8_t)(((c >> n) & 1u) ? -m : m);
}

// e0mN codes -> the two's-complement container of width n + 1 in the logical
// input form of that container (4-bit words for e0m3, one byte per code else)
static std::vector<uint32_t> e0m_to_int(const LayerInfo& L, const void* w) {
    const int64_t KN = L.E * L.K * L.N;
    if (L.e0m == 3) {
        std::vector<uint32_t> q((size_t)(KN / 8));
        const uint32_t* src = (const uint32_t*)w;
        for (int64_t i = 0; i < KN / 8; ++i) {
            uint32_t o = 0;
            for (int j = 0; j < 8; ++j) o |= ((uint32_t)e0m_value((src[i] >> (4 * j)) & 15u, 3) & 15u) << (4 * j);
            q[(size_t)i] = o;
        }
        return q;
    }
    std::vector<uint32_t> q((size_t)((KN + 3) / 4));
    const uint8_t* src = (const uint8_t*)w;
    int8_t* dst = (int8_t*)q.data();
    for (int64_t i = 0; i < KN; ++i) dst[i] = e0m_value(src[i], L.e0m);
    return q;
}

void repack_all(const LayerInfo& L, const void* w, const void* s, const void* z, const void* s2, void* w_out,
                void* s_out, void* z_out, void* s2_out) {
    switch (L.kind) {
        case Kind::WNA16: {
            std::vector<uint32_t> conv;
            if (L.e0m) {
                conv = e0m_to_int(L, w);
                w = conv.data();
            }
            if (L.bits > 4) repack_wide(L, (const uint8_t*)w, (uint8_t*)w_out);
            else if (L.bits < 4) repack_lowbit(L, (const int8_t*)w, (uint8_t*)w_out);
            else repack_4bit(L, (const uint32_t*)w, (uint8_t*)w_out, true);
            repack_scale16(L, (const uint16_t*)s, (uint16_t*)s_out, L.a_bf16 ? 0x3F80 : 0x3C00);
            if (L.zp8) repack_zero8(L, (const uint8_t*)z, (uint8_t*)z_out);
            else if (L.zp) repack_zero4(L, (const uint32_t*)z, (uint64_t*)z_out);
            break;
        }
        case Kind::W4A8_MX:
        case Kind::MXA_MX:
        case Kind::MOE_MX_BF16:
            repack_4bit(L, (const uint32_t*)w, (uint8_t*)w_out, false);
            repack_e8m0(L, (const uint8_t*)s, (uint8_t*)s_out);
            break;
        case Kind::W8A8:
            repack_int8(L, (const int8_t*)w, (int8_t*)w_out);
            repack_chan32(L, (const float*)s, (float*)s_out);
            break;
        case Kind::W8A16: {
            std::vector<uint32_t> conv;
            if (L.e0m) {
                conv = e0m_to_int(L, w);
                w = conv.data();
            }
            repack_int8_k32(L, (const int8_t*)w, (int8_t*)w_out);
            repack_chan32(L, (const float*)s, (float*)s_out);
            break;
        }
        case Kind::FP4_A16:
            if (L.mxf == 1) repack_int8_k32(L, (const int8_t*)w, (int8_t*)w_out);
            else if (L.mxf) repack_fp6(L, (const uint8_t*)w, (uint8_t*)w_out);
            else repack_4bit(L, (const uint32_t*)w, (uint8_t*)w_out, false);
            if (L.nv) repack_e4m3_g16(L, (const uint8_t*)s, (uint8_t*)s_out);
            else repack_e8m0(L, (const uint8_t*)s, (uint8_t*)s_out);
            if (L.nv) std::memcpy(s2_out, s2, (size_t)L.E * 4);
            break;
        case Kind::FP8_BLOCK:
            // E4M3 codes take the INT8 byte layout (code 0 = +0 in the padding); the
            // 128 x 128 block scales keep their logical [K/128][ceil(N/128)] order
            repack_int8(L, (const int8_t*)w, (int8_t*)w_out);
            std::memcpy(s_out, s, (size_t)(L.K / 128) * (size_t)((L.N + 127) / 128) * 4 * (size_t)L.E);
            break;
    }
}

}  // namespace hq
