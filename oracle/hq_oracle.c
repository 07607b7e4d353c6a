/*
 * hq_oracle.c -- plain CPU oracle for the quantized GEMM  D = A x dequant(W).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library links, includes or calls
 * this file; only the test-suite, the smoke check and the benchmark's CPU
 * baseline leg load it.  It shares no code, header, table or helper with the
 * HIP path.
 *
 * What it computes (the plain definition the method reaches up to rounding
 * order): decode every quantized weight to its real value, decode every
 * activation to its real value, multiply-accumulate in fp64, apply the
 * per-token / per-channel epilogue scales last.  The pages ("Humming wird
 * angekuendigt", section "Eine einheitliche Quantisierungsdarstellung") give the
 * parameters -- weight format, scale granularity and dtype, zero-points --
 * and the readers' checklist ("Humming v0.1.0-0.1.4", section
 * "上手核对清单") compares outputs against an unquantized matmul; that
 * matmul is what is written here.
 *
 * Number formats come from the OCP Microscaling Formats (MX) specification
 * v1.0 (FP4 E2M1 and the E8M0 scale) and the OCP 8-bit floating point
 * specification (E4M3, the "FN" variant without infinities).
 *
 * Logical layouts (the "export" form):
 *   4-bit codes   uint32 [K/8][N]   code k=8j+i of column n in bits 4i..4i+3 of word [j][n]
 *   INT8 weights  int8   [K][N]
 *   group scales  [K/G][N]  (bf16 / fp16 raw bits)
 *   zero-points   uint32 [K/G][ceil(N/8)]  column n=8j+i in bits 4i..4i+3 of word [g][j]
 *   E8M0          uint8  [K/32][N]
 *   activations   [M][K] row-major
 *
 * Every GEMM entry computes only the output rows listed in rows[0..nrows)
 * (or all rows when rows == NULL) and writes them densely to out[nrows][N].
 * Loop order is k-outer so that each weight is decoded once per call; the
 * arithmetic per output is the textbook sum over k in increasing order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* scalar decoders                                                      */
/* ------------------------------------------------------------------ */

/* OCP MX v1.0, FP4 E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit;
 * exponent field 0 is subnormal with value 0.5*m. */
double hq_oracle_e2m1(unsigned code)
{
    unsigned s = (code >> 3) & 1u, e = (code >> 1) & 3u, m = code & 1u;
    double mag = (e == 0) ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
    return s ? -mag : mag;
}

/* OCP MX v1.0, E8M0 scale: 2^(e-127); 0xFF is NaN. */
double hq_oracle_e8m0(unsigned e)
{
    if ((e & 0xFFu) == 0xFFu) return NAN;
    return ldexp(1.0, (int)(e & 0xFFu) - 127);
}

/* OCP FP8 E4M3 (bias 7, no infinities, S.1111.111 is NaN). */
double hq_oracle_e4m3(unsigned code)
{
    unsigned s = (code >> 7) & 1u, e = (code >> 3) & 15u, m = code & 7u;
    double mag;
    if (e == 15u && m == 7u) return NAN;
    if (e == 0) mag = ldexp((double)m, -9);                 /* m/8 * 2^(1-7) */
    else        mag = ldexp(1.0 + (double)m / 8.0, (int)e - 7);
    return s ? -mag : mag;
}

/* OCP MX v1.0, FP6: E2M3 (e3m2 = 0: 1 sign, 2 exponent bits with bias 1, 3
 * mantissa bits) or E3M2 (e3m2 = 1: 3 exponent bits with bias 3, 2 mantissa
 * bits); exponent field 0 is subnormal, 2^(1-bias) * m / 2^mbits; no
 * infinities or NaN.  code: the 6 low bits. */
double hq_oracle_fp6(unsigned code, int e3m2)
{
    const int eb = e3m2 ? 3 : 2, mb = e3m2 ? 2 : 3, bias = e3m2 ? 3 : 1;
    unsigned s = (code >> 5) & 1u, e = (code >> mb) & ((1u << eb) - 1u), m = code & ((1u << mb) - 1u);
    double frac = (double)m / (double)(1u << mb);
    double mag = (e == 0) ? ldexp(frac, 1 - bias) : ldexp(1.0 + frac, (int)e - bias);
    return s ? -mag : mag;
}

/* Zero-exponent float e0mN ("Humming wird angekuendigt", section on the weight
 * and activation combinations: a float format without exponent bits whose
 * values are the symmetric integers of the same width): 1 sign bit (bit n)
 * and n mantissa bits read as an integer magnitude, so the code's value is
 * -m or +m (the sign with magnitude 0 is zero).  Returns 0 and sets *ok = 0 if
 * the code has a bit above bit n. */
double hq_oracle_e0m(unsigned code, int n, int* ok)
{
    *ok = (code >> (n + 1)) == 0u;
    if (!*ok) return 0.0;
    const unsigned m = code & ((1u << n) - 1u);
    return ((code >> n) & 1u) ? -(double)m : (double)m;
}

/* Round-to-nearest-even fp32 -> E4M3 with saturation to +-448 (satfinite). */
unsigned hq_oracle_e4m3_encode(float x)
{
    if (isnan(x)) return 0x7Fu;
    unsigned sign = signbit(x) ? 0x80u : 0u;
    double a = fabs((double)x);
    if (a > 448.0) return sign | 0x7Eu;
    if (a < ldexp(1.0, -6)) {                 /* subnormal range, step 2^-9 */
        double m = nearbyint(a * 512.0);      /* m == 8 lands on code 0x08 = 2^-6 */
        return sign | (unsigned)m;
    }
    int ex;
    double f = frexp(a, &ex);                 /* a = f * 2^ex, f in [0.5, 1) */
    int eu = ex - 1;                          /* a = (2f) * 2^eu, 2f in [1, 2) */
    double m = nearbyint((2.0 * f - 1.0) * 8.0);
    if (m == 8.0) { m = 0.0; eu += 1; }
    unsigned code = (unsigned)(((eu + 7) << 3) | (int)m);
    if (code > 0x7Eu) code = 0x7Eu;
    return sign | code;
}

double hq_oracle_bf16(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

double hq_oracle_fp16(uint16_t h)
{
    unsigned s = (h >> 15) & 1u, e = (h >> 10) & 31u, m = h & 1023u;
    double mag;
    if (e == 31u) mag = m ? NAN : INFINITY;
    else if (e == 0) mag = ldexp((double)m, -24);
    else mag = ldexp(1.0 + (double)m / 1024.0, (int)e - 15);
    return s ? -mag : mag;
}

static double act16(int is_bf16, uint16_t v) { return is_bf16 ? hq_oracle_bf16(v) : hq_oracle_fp16(v); }

static unsigned nib_along_k(const uint32_t* q, int64_t N, int64_t k, int64_t n)
{
    return (q[(k >> 3) * N + n] >> (4 * (k & 7))) & 15u;
}

static int64_t row_of(const int64_t* rows, int64_t r) { return rows ? rows[r] : r; }

/* ------------------------------------------------------------------ */
/* activation quantisation (tokenwise E4M3)                             */
/* ------------------------------------------------------------------ */

/* Per row m: s[m] = max_k |x| / 448 in fp32 (1 for an all-zero row), and
 * q[m][k] = E4M3_RNE_satfinite(x / s[m]) with the division in fp32. */
void hq_oracle_quant_act_e4m3(int64_t M, int64_t K, const float* x, uint8_t* q, float* s)
{
    for (int64_t m = 0; m < M; ++m) {
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float a = fabsf(x[m * K + k]);
            if (a > amax) amax = a;
        }
        float sc = (amax > 0.0f) ? amax / 448.0f : 1.0f;
        s[m] = sc;
        for (int64_t k = 0; k < K; ++k) {
            float v = x[m * K + k] / sc;
            q[m * K + k] = (uint8_t)hq_oracle_e4m3_encode(v);
        }
    }
}

/* Per row m and block b of B consecutive elements along K (K % B == 0):
 * s[m][b] = max |x| over the block / 448 in fp32 (1 for an all-zero block),
 * q = E4M3_RNE_satfinite(x / s) with the division in fp32.  B == K is the
 * tokenwise case above; B == 128 is the 1 x 128 activation blocks of FP8
 * W8A8 with blockwise scales. */
int hq_oracle_quant_act_e4m3_blocks(int64_t M, int64_t K, int64_t B, const float* x, uint8_t* q, float* s)
{
    if (B <= 0 || K % B) return 1;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t b = 0; b < K / B; ++b) {
            const float* xb = x + m * K + b * B;
            float amax = 0.0f;
            for (int64_t k = 0; k < B; ++k) {
                float a = fabsf(xb[k]);
                if (a > amax) amax = a;
            }
            float sc = (amax > 0.0f) ? amax / 448.0f : 1.0f;
            s[m * (K / B) + b] = sc;
            for (int64_t k = 0; k < B; ++k) q[m * K + b * B + k] = (uint8_t)hq_oracle_e4m3_encode(xb[k] / sc);
        }
    return 0;
}

/* ------------------------------------------------------------------ */
/* MX activation quantisation (OCP MX v1.0: one E8M0 scale per 32)      */
/* ------------------------------------------------------------------ */

/* Nearest E2M1 value to v, ties to the even mantissa bit, saturating at
 * +-6; the sign of v is kept (so -0.0 and tiny negatives give code 8). */
unsigned hq_oracle_e2m1_encode(double v)
{
    static const double grid[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    if (v != v) return 0u;
    unsigned sign = signbit(v) ? 8u : 0u;
    double a = fabs(v);
    if (a >= 6.0) return sign | 7u;          /* saturation (also avoids distances lost to rounding) */
    unsigned best = 0;
    for (unsigned c = 1; c < 8; ++c) {
        double dc = fabs(a - grid[c]), db = fabs(a - grid[best]);
        if (dc < db || (dc == db && (c & 1u) == 0u)) best = c;
    }
    return sign | best;
}

/* One block of 32 values x[0..31] -> E8M0 exponent and element codes
 * (elem 0: E4M3, codes one per byte; elem 1: E2M1, codes in code[0..31]).
 * OCP MX v1.0, section 6.3: the shared exponent is floor(log2(max|x|))
 * minus the largest exponent of the element format (E4M3: 8, since
 * 448 = 1.75 * 2^8; E2M1: 2, since 6 = 1.5 * 2^2), as an E8M0 value
 * clamped to 0..254 (0 for an all-zero block); each element is x / 2^(E-127)
 * rounded to nearest-even and saturated.  A block holding a NaN or an
 * infinity gets the NaN scale 0xFF and zero codes. */
static unsigned mx_block(const float* x, int elem, unsigned* code)
{
    double amax = 0.0;
    for (int i = 0; i < 32; ++i) {
        if (!isfinite(x[i])) {
            for (int j = 0; j < 32; ++j) code[j] = 0;
            return 0xFFu;
        }
        if (fabs((double)x[i]) > amax) amax = fabs((double)x[i]);
    }
    int E = 0;
    if (amax > 0.0) {
        int ex;
        frexp(amax, &ex);                           /* amax = f * 2^ex, f in [0.5, 1) */
        E = (ex - 1) - (elem ? 2 : 8) + 127;
        if (E < 0) E = 0;
        if (E > 254) E = 254;
    }
    for (int i = 0; i < 32; ++i) {
        double v = ldexp((double)x[i], 127 - E);   /* exact power-of-two scaling */
        code[i] = elem ? hq_oracle_e2m1_encode(v) : hq_oracle_e4m3_encode((float)v);
    }
    return (unsigned)E;
}

/* x fp32 [M][K] (K % 32 == 0) -> codes (E4M3: uint8 [M][K]; E2M1: uint8
 * [M][K/2], element k in the low nibble of byte k/2 when k is even) and
 * E8M0 scales uint8 [M][K/32]. */
int hq_oracle_quant_act_mx(int64_t M, int64_t K, int elem, const float* x, uint8_t* q, uint8_t* e)
{
    if (K % 32 || (elem != 0 && elem != 1)) return 1;
    unsigned code[32];
    for (int64_t m = 0; m < M; ++m)
        for (int64_t b = 0; b < K / 32; ++b) {
            e[m * (K / 32) + b] = (uint8_t)mx_block(x + m * K + b * 32, elem, code);
            for (int i = 0; i < 32; ++i) {
                int64_t k = b * 32 + i;
                if (elem == 0) q[m * K + k] = (uint8_t)code[i];
                else if ((k & 1) == 0) q[m * (K / 2) + k / 2] = (uint8_t)code[i];
                else q[m * (K / 2) + k / 2] |= (uint8_t)(code[i] << 4);
            }
        }
    return 0;
}

/* ------------------------------------------------------------------ */
/* dense GEMMs                                                          */
/* ------------------------------------------------------------------ */

/* W4A16: W[k][n] = (code - zero) * s[k/G][n]
 *   w_signed = 1: code is two's-complement INT4 (-8..7), zero = 0
 *   w_signed = 0: code is UINT4 (0..15), zero from z (or 0 when z == NULL)
 * A and s are bf16 (a_bf16 = 1) or fp16 (a_bf16 = 0) raw bits. */
int hq_oracle_gemm_wna16(int64_t M, int64_t N, int64_t K, int64_t G, int a_bf16,
                         const uint16_t* A, int w_signed, const uint32_t* q,
                         const uint16_t* s, const uint32_t* z,
                         const int64_t* rows, int64_t nrows, double* out)
{
    if (K % 8 || G <= 0 || K % G) return 1;
    int64_t R = rows ? nrows : M;
    int64_t zw = (N + 7) / 8;
    double* a = (double*)malloc(sizeof(double) * (size_t)(R * K + 1));
    if (!a) return 2;
    for (int64_t r = 0; r < R; ++r)
        for (int64_t k = 0; k < K; ++k) a[r * K + k] = act16(a_bf16, A[row_of(rows, r) * K + k]);
    memset(out, 0, sizeof(double) * (size_t)(R * N));
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            int64_t g = k / G;
            int code = (int)nib_along_k(q, N, k, n);
            int zero = 0;
            if (w_signed) code = code >= 8 ? code - 16 : code;
            else if (z) zero = (int)((z[g * zw + n / 8] >> (4 * (n % 8))) & 15u);
            double w = (double)(code - zero) * act16(a_bf16, s[g * N + n]);
            for (int64_t r = 0; r < R; ++r) out[r * N + n] += a[r * K + k] * w;
        }
    }
    free(a);
    return 0;
}

/* Low-bit WnA16 ("Humming wird angekuendigt", section WnA16: INT1, INT2 and INT3
 * weights among the widths; section "Eine einheitliche Quantisierungsdarstellung":
 * the width, zero-points and scale granularity are separate parameters).  One
 * code per byte, codes[k][n]: signed widths hold the two's-complement value
 * -2^(bits-1) .. 2^(bits-1)-1 (W = code * s), unsigned widths hold 0 .. 2^bits-1
 * with a 4-bit zero-point per group and column (W = (code - z) * s; z in the
 * UINT4 container of the W4A16 layer, [K/G][ceil(N/8)] words).  D = A x W in
 * fp64.  Returns 3 when a code lies outside its width. */
int hq_oracle_gemm_wnlow(int64_t M, int64_t N, int64_t K, int64_t G, int a_bf16, int bits, int w_signed,
                         const uint16_t* A, const int8_t* codes, const uint16_t* s, const uint32_t* z,
                         const int64_t* rows, int64_t nrows, double* out)
{
    if (bits < 1 || bits > 3 || G <= 0 || K % G) return 1;
    const int lo = w_signed ? -(1 << (bits - 1)) : 0, hi = w_signed ? (1 << (bits - 1)) - 1 : (1 << bits) - 1;
    for (int64_t i = 0; i < K * N; ++i) {
        const int c = w_signed ? (int)codes[i] : (int)(uint8_t)codes[i];
        if (c < lo || c > hi) return 3;
    }
    int64_t R = rows ? nrows : M;
    int64_t zw = (N + 7) / 8;
    double* a = (double*)malloc(sizeof(double) * (size_t)(R * K + 1));
    if (!a) return 2;
    for (int64_t r = 0; r < R; ++r)
        for (int64_t k = 0; k < K; ++k) a[r * K + k] = act16(a_bf16, A[row_of(rows, r) * K + k]);
    memset(out, 0, sizeof(double) * (size_t)(R * N));
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            const int64_t g = k / G;
            const int code = w_signed ? (int)codes[k * N + n] : (int)(uint8_t)codes[k * N + n];
            const int zero = (!w_signed && z) ? (int)((z[g * zw + n / 8] >> (4 * (n % 8))) & 15u) : 0;
            const double w = (double)(code - zero) * act16(a_bf16, s[g * N + n]);
            for (int64_t r = 0; r < R; ++r) out[r * N + n] += a[r * K + k] * w;
        }
    }
    free(a);
    return 0;
}

/* WnA16 at the widths above 4 bits ("Humming wird angekuendigt", section
 * WnA16: INT1-INT8 weights, symmetric or with dynamic zero-points): one code per
 * byte, codes[k][n] (int8 two's complement for signed widths, uint8 0 .. 2^bits-1
 * for unsigned ones), 16-bit group scales s[K/G][N]; unsigned widths take one
 * 8-bit zero-point per group and column, z8[K/G][N] (uint8):
 *   W = code * s (signed) or (code - z) * s (unsigned),  D = A x W in fp64.
 * Returns 3 when a code lies outside its width. */
int hq_oracle_gemm_wnwide(int64_t M, int64_t N, int64_t K, int64_t G, int a_bf16, int bits, int w_signed,
                          const uint16_t* A, const uint8_t* codes, const uint16_t* s, const uint8_t* z8,
                          const int64_t* rows, int64_t nrows, double* out)
{
    if (bits < 5 || bits > 8 || G <= 0 || K % G || (!w_signed && !z8)) return 1;
    const int lo = w_signed ? -(1 << (bits - 1)) : 0, hi = w_signed ? (1 << (bits - 1)) - 1 : (1 << bits) - 1;
    for (int64_t i = 0; i < K * N; ++i) {
        const int c = w_signed ? (int)(int8_t)codes[i] : (int)codes[i];
        if (c < lo || c > hi) return 3;
    }
    int64_t R = rows ? nrows : M;
    double* a = (double*)malloc(sizeof(double) * (size_t)(R * K + 1));
    if (!a) return 2;
    for (int64_t r = 0; r < R; ++r)
        for (int64_t k = 0; k < K; ++k) a[r * K + k] = act16(a_bf16, A[row_of(rows, r) * K + k]);
    memset(out, 0, sizeof(double) * (size_t)(R * N));
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            const int64_t g = k / G;
            const int c = w_signed ? (int)(int8_t)codes[k * N + n] : (int)codes[k * N + n];
            const int zero = w_signed ? 0 : (int)z8[g * N + n];
            const double w = (double)(c - zero) * act16(a_bf16, s[g * N + n]);
            for (int64_t r = 0; r < R; ++r) out[r * N + n] += a[r * K + k] * w;
        }
    free(a);
    return 0;
}

/* W4A8-MXFP4: W[k][n] = e2m1(code) * 2^(E[k/32][n]-127),
 * A_real[m][k] = e4m3(qa[m][k]) * s_a[m];  D = A_real x W. */
int hq_oracle_gemm_w4a8_mxfp4(int64_t M, int64_t N, int64_t K, const uint8_t* qa,
                              const float* s_a, const uint32_t* q, const uint8_t* e8,
                              const int64_t* rows, int64_t nrows, double* out)
{
    if (K % 32) return 1;
    int64_t R = rows ? nrows : M;
    double* a = (double*)malloc(sizeof(double) * (size_t)(R * K + 1));
    if (!a) return 2;
    for (int64_t r = 0; r < R; ++r)
        for (int64_t k = 0; k < K; ++k) a[r * K + k] = hq_oracle_e4m3(qa[row_of(rows, r) * K + k]);
    memset(out, 0, sizeof(double) * (size_t)(R * N));
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            double w = hq_oracle_e2m1(nib_along_k(q, N, k, n)) * hq_oracle_e8m0(e8[(k / 32) * N + n]);
            for (int64_t r = 0; r < R; ++r) out[r * N + n] += a[r * K + k] * w;
        }
        for (int64_t r = 0; r < R; ++r) out[r * N + n] *= (double)s_a[row_of(rows, r)];
    }
    free(a);
    return 0;
}

/* MX activations x MXFP4 weights (W4A4 with E2M1 activations, W4A8 with
 * MXFP8 E4M3 activations): A_real[m][k] = dec(qa code) * 2^(ea[m][k/32]-127),
 * W_real as in the W4A8-MXFP4 entry, D = A_real x W_real.
 * a_elem 0: qa is E4M3 uint8 [M][K]; a_elem 1: qa is E2M1 uint8 [M][K/2]
 * (element k in the low nibble of byte k/2 when k is even). */
int hq_oracle_gemm_mx_mxfp4(int64_t M, int64_t N, int64_t K, int a_elem, const uint8_t* qa,
                            const uint8_t* ea, const uint32_t* q, const uint8_t* e8,
                            const int64_t* rows, int64_t nrows, double* out)
{
    if (K % 32 || (a_elem != 0 && a_elem != 1)) return 1;
    int64_t R = rows ? nrows : M;
    double* a = (double*)malloc(sizeof(double) * (size_t)(R * K + 1));
    if (!a) return 2;
    for (int64_t r = 0; r < R; ++r) {
        int64_t m = row_of(rows, r);
        for (int64_t k = 0; k < K; ++k) {
            double v = a_elem ? hq_oracle_e2m1((qa[m * (K / 2) + k / 2] >> (4 * (k & 1))) & 15u)
                              : hq_oracle_e4m3(qa[m * K + k]);
            a[r * K + k] = v * hq_oracle_e8m0(ea[m * (K / 32) + k / 32]);
        }
    }
    memset(out, 0, sizeof(double) * (size_t)(R * N));
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            double w = hq_oracle_e2m1(nib_along_k(q, N, k, n)) * hq_oracle_e8m0(e8[(k / 32) * N + n]);
            for (int64_t r = 0; r < R; ++r) out[r * N + n] += a[r * K + k] * w;
        }
    free(a);
    return 0;
}

/* FP4 weights with 16-bit activations (WnA16, FP4): W_real[k][n] =
 * e2m1(q) * scale * s2, where scale_kind 0 (MXFP4) is an E8M0 byte per 32 K
 * (scales uint8 [K/32][N]) and scale_kind 1 (NVFP4) an E4M3 byte per 16 K
 * (scales uint8 [K/16][N]); s2 is the second-level fp32 scale per tensor
 * (NULL: 1).  A is bf16 (a_bf16 = 1) or fp16 raw bits [M][K]; D = A x W_real. */
int hq_oracle_gemm_fp4_a16(int64_t M, int64_t N, int64_t K, int a_bf16, const uint16_t* A, const uint32_t* q,
                           int scale_kind, const uint8_t* scales, const float* s2,
                           const int64_t* rows, int64_t nrows, double* out)
{
    const int64_t G = scale_kind ? 16 : 32;
    if (K % G || (scale_kind != 0 && scale_kind != 1)) return 1;
    int64_t R = rows ? nrows : M;
    double* a = (double*)malloc(sizeof(double) * (size_t)(R * K + 1));
    if (!a) return 2;
    for (int64_t r = 0; r < R; ++r)
        for (int64_t k = 0; k < K; ++k) a[r * K + k] = act16(a_bf16, A[row_of(rows, r) * K + k]);
    const double t2 = s2 ? (double)s2[0] : 1.0;
    memset(out, 0, sizeof(double) * (size_t)(R * N));
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            uint8_t sc = scales[(k / G) * N + n];
            double w = hq_oracle_e2m1(nib_along_k(q, N, k, n)) * (scale_kind ? hq_oracle_e4m3(sc) : hq_oracle_e8m0(sc)) * t2;
            for (int64_t r = 0; r < R; ++r) out[r * N + n] += a[r * K + k] * w;
        }
    free(a);
    return 0;
}

/* MXINT4 weights with 16-bit activations: two's-complement INT4 codes (-8..7)
 * with one E8M0 scale per 32 consecutive K of a column (the OCP MX integer
 * element type MXINT4 under the MX block scale):
 *   W_real[k][n] = int4(q[k][n]) * 2^(e8[k/32][n] - 127),  D = A x W_real (fp64).
 * q uint32 [K/8][N] (4-bit layout above), e8 uint8 [K/32][N]. */
int hq_oracle_gemm_mxint4_a16(int64_t M, int64_t N, int64_t K, int a_bf16, const uint16_t* A, const uint32_t* q,
                              const uint8_t* e8, const int64_t* rows, int64_t nrows, double* out)
{
    if (K % 32) return 1;
    int64_t R = rows ? nrows : M;
    double* a = (double*)malloc(sizeof(double) * (size_t)(R * K + 1));
    if (!a) return 2;
    for (int64_t r = 0; r < R; ++r)
        for (int64_t k = 0; k < K; ++k) a[r * K + k] = act16(a_bf16, A[row_of(rows, r) * K + k]);
    memset(out, 0, sizeof(double) * (size_t)(R * N));
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int code = (int)nib_along_k(q, N, k, n);
            code = code >= 8 ? code - 16 : code;
            double w = (double)code * hq_oracle_e8m0(e8[(k / 32) * N + n]);
            for (int64_t r = 0; r < R; ++r) out[r * N + n] += a[r * K + k] * w;
        }
    free(a);
    return 0;
}

/* FP8 W8A8 with blockwise scales: A_real[m][k] = e4m3(qa[m][k]) * sa[m][k/128],
 * W_real[k][n] = e4m3(w[k][n]) * sw[k/128][n/128], D = A_real x W_real.
 * qa uint8 [M][K], sa fp32 [M][K/128], w uint8 [K][N], sw fp32 [K/128][ceil(N/128)]. */
int hq_oracle_gemm_fp8_blockwise(int64_t M, int64_t N, int64_t K, const uint8_t* qa, const float* sa,
                                 const uint8_t* w, const float* sw, const int64_t* rows, int64_t nrows,
                                 double* out)
{
    if (K % 128) return 1;
    int64_t R = rows ? nrows : M, nbn = (N + 127) / 128;
    double* a = (double*)malloc(sizeof(double) * (size_t)(R * K + 1));
    if (!a) return 2;
    for (int64_t r = 0; r < R; ++r) {
        int64_t m = row_of(rows, r);
        for (int64_t k = 0; k < K; ++k) a[r * K + k] = hq_oracle_e4m3(qa[m * K + k]) * (double)sa[m * (K / 128) + k / 128];
    }
    memset(out, 0, sizeof(double) * (size_t)(R * N));
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            double wv = hq_oracle_e4m3(w[k * N + n]) * (double)sw[(k / 128) * nbn + n / 128];
            for (int64_t r = 0; r < R; ++r) out[r * N + n] += a[r * K + k] * wv;
        }
    free(a);
    return 0;
}

/* W8A8 INT8: acc[m][n] = sum_k a[m][k] * w[k][n] (exact, int64; returns 3 if
 * any |acc| exceeds int32), D = acc * s_a[m] * s_w[n]. */
int hq_oracle_gemm_w8a8(int64_t M, int64_t N, int64_t K, const int8_t* a, const float* s_a,
                        const int8_t* w, const float* s_w, const int64_t* rows, int64_t nrows,
                        int64_t* acc, double* out)
{
    int64_t R = rows ? nrows : M;
    int overflow = 0;
    memset(acc, 0, sizeof(int64_t) * (size_t)(R * N));
#pragma omp parallel for schedule(static) reduction(| : overflow)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            int64_t wv = w[k * N + n];
            for (int64_t r = 0; r < R; ++r) acc[r * N + n] += (int64_t)a[row_of(rows, r) * K + k] * wv;
        }
        for (int64_t r = 0; r < R; ++r) {
            int64_t v = acc[r * N + n];
            if (v > INT32_MAX || v < INT32_MIN) overflow = 1;
            out[r * N + n] = (double)v * (double)s_a[row_of(rows, r)] * (double)s_w[n];
        }
    }
    return overflow ? 3 : 0;
}

/* INT8 weight-only (W8A16): two's-complement INT8 weights with one fp32 scale per
 * output column and 16-bit activations:
 *   D[m][n] = (sum_k A[m][k] * w[k][n]) * s_w[n]   (fp64).
 * A uint16 [M][K] (bf16 or fp16 bits), w int8 [K][N], s_w fp32 [N]. */
int hq_oracle_gemm_w8a16(int64_t M, int64_t N, int64_t K, int a_bf16, const uint16_t* A, const int8_t* w,
                         const float* s_w, const int64_t* rows, int64_t nrows, double* out)
{
    int64_t R = rows ? nrows : M;
    double* a = (double*)malloc(sizeof(double) * (size_t)(R * K + 1));
    if (!a) return 2;
    for (int64_t r = 0; r < R; ++r)
        for (int64_t k = 0; k < K; ++k) a[r * K + k] = act16(a_bf16, A[row_of(rows, r) * K + k]);
    memset(out, 0, sizeof(double) * (size_t)(R * N));
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            double wv = (double)w[k * N + n];
            for (int64_t r = 0; r < R; ++r) out[r * N + n] += a[r * K + k] * wv;
        }
        for (int64_t r = 0; r < R; ++r) out[r * N + n] *= (double)s_w[n];
    }
    free(a);
    return 0;
}

/* FP8 weight-only: E4M3 weights with one fp32 scale per output column and 16-bit
 * activations:  D[m][n] = (sum_k A[m][k] * e4m3(w[k][n])) * s_w[n]   (fp64).
 * A uint16 [M][K] (bf16 or fp16 bits), w uint8 [K][N] (E4M3 codes), s_w fp32 [N]. */
int hq_oracle_gemm_fp8w_a16(int64_t M, int64_t N, int64_t K, int a_bf16, const uint16_t* A, const uint8_t* w,
                            const float* s_w, const int64_t* rows, int64_t nrows, double* out)
{
    int64_t R = rows ? nrows : M;
    double* a = (double*)malloc(sizeof(double) * (size_t)(R * K + 1));
    if (!a) return 2;
    for (int64_t r = 0; r < R; ++r)
        for (int64_t k = 0; k < K; ++k) a[r * K + k] = act16(a_bf16, A[row_of(rows, r) * K + k]);
    memset(out, 0, sizeof(double) * (size_t)(R * N));
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            double wv = hq_oracle_e4m3(w[k * N + n]);
            for (int64_t r = 0; r < R; ++r) out[r * N + n] += a[r * K + k] * wv;
        }
        for (int64_t r = 0; r < R; ++r) out[r * N + n] *= (double)s_w[n];
    }
    free(a);
    return 0;
}

/* MX-scaled float weights with 16-bit activations (the WnA16 float widths of
 * "Humming wird angekuendigt", section WnA16, under the OCP MX v1.0 block
 * scale): elem 0 = FP8 E4M3 (MXFP8), 1 = FP6 E2M3, 2 = FP6 E3M2 (MXFP6);
 *   W_real[k][n] = elem(codes[k][n]) * 2^(e8[k/32][n] - 127),  D = A x W_real (fp64).
 * codes uint8 [K][N] (FP6: the low 6 bits; returns 3 if a higher bit is set),
 * e8 uint8 [K/32][N], A uint16 [M][K] (bf16 or fp16 bits). */
int hq_oracle_gemm_mxf_a16(int64_t M, int64_t N, int64_t K, int a_bf16, const uint16_t* A, int elem,
                           const uint8_t* codes, const uint8_t* e8, const int64_t* rows, int64_t nrows, double* out)
{
    if (K % 32 || elem < 0 || elem > 2) return 1;
    if (elem)
        for (int64_t i = 0; i < K * N; ++i)
            if (codes[i] & 0xC0u) return 3;
    int64_t R = rows ? nrows : M;
    double* a = (double*)malloc(sizeof(double) * (size_t)(R * K + 1));
    if (!a) return 2;
    for (int64_t r = 0; r < R; ++r)
        for (int64_t k = 0; k < K; ++k) a[r * K + k] = act16(a_bf16, A[row_of(rows, r) * K + k]);
    memset(out, 0, sizeof(double) * (size_t)(R * N));
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            const unsigned c = codes[k * N + n];
            double w = elem == 0 ? hq_oracle_e4m3(c) : hq_oracle_fp6(c, elem == 2);
            w *= hq_oracle_e8m0(e8[(k / 32) * N + n]);
            for (int64_t r = 0; r < R; ++r) out[r * N + n] += a[r * K + k] * w;
        }
    free(a);
    return 0;
}

/* ------------------------------------------------------------------ */
/* MoE                                                                   */
/* ------------------------------------------------------------------ */

/* Routing metadata over the flattened pairs p = t*top_k + j:
 * counts[e] = #pairs routed to e, offsets = exclusive prefix sum (E+1),
 * perm = pairs stably sorted by expert (counting sort). Returns 1 on a bad id. */
int hq_oracle_moe_route(int64_t T, int64_t top_k, int64_t E, const int32_t* ids,
                        int64_t* counts, int64_t* offsets, int64_t* perm)
{
    int64_t P = T * top_k;
    for (int64_t e = 0; e < E; ++e) counts[e] = 0;
    for (int64_t p = 0; p < P; ++p) {
        if (ids[p] < 0 || ids[p] >= E) return 1;
        counts[ids[p]]++;
    }
    offsets[0] = 0;
    for (int64_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int64_t* cur = (int64_t*)malloc(sizeof(int64_t) * (size_t)(E + 1));
    if (!cur) return 2;
    for (int64_t e = 0; e < E; ++e) cur[e] = offsets[e];
    for (int64_t p = 0; p < P; ++p) perm[cur[ids[p]]++] = p;
    free(cur);
    return 0;
}

/* bf16 bits of x rounded to nearest, ties to even (overflow -> inf, NaN -> quiet
 * NaN).  Exact: |x| / q with q the bf16 quantum of x's binade (2^(E-7), or
 * 2^-133 below the normal range) is a power-of-two scaling, nearbyint rounds
 * it to an integer under the default round-to-nearest-even mode, and r * q is
 * representable in bf16, hence in float, whose top 16 bits are its encoding. */
static uint16_t bf16_rne(double x)
{
    if (x != x) return 0x7FC0;
    const uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);                       /* a = m * 2^e, m in [0.5, 1): binade exponent e - 1 */
    const int E = e - 1 < -126 ? -126 : e - 1;
    const int qexp = e - 1 < -126 ? -133 : E - 7;
    const double r = nearbyint(ldexp(a, -qexp));
    const double v = ldexp(r, qexp);
    if (v > 3.3895313892515355e38) return sign | 0x7F80;   /* beyond the largest bf16 */
    const float f = (float)v;
    uint32_t bits;
    memcpy(&bits, &f, 4);
    return sign | (uint16_t)(bits >> 16);
}

uint16_t hq_oracle_bf16_encode(double x) { return bf16_rne(x); }

/* The activation between the MoE gate-up and down projections ("Humming wird
 * angekuendigt", section "Leistung": the MoE figures add the gate-up and down
 * GEMMs; the pages name no activation, and the plain reading of a fused gate+up
 * output is SiLU(gate) * up with the gate in the first half of each row).
 * in [rows][2I] bf16 bits; out[r][i] = bf16_rne(silu(g) * u), g = in[r][i],
 * u = in[r][I + i], silu(g) = g / (1 + e^-g), all in double. */
void hq_oracle_silu_mul_bf16(int64_t rows, int64_t I, const uint16_t* in, uint16_t* out)
{
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t i = 0; i < I; ++i) {
            const double g = hq_oracle_bf16(in[r * 2 * I + i]), u = hq_oracle_bf16(in[r * 2 * I + I + i]);
            out[r * I + i] = bf16_rne(g / (1.0 + exp(-g)) * u);
        }
}

/* MoE W4A16-MXFP4 (bf16 tokens): for each requested pair p (t = p / top_k),
 * out[i][:] = A[t][:] x W_real[ids[p]] with W_real as in the W4A8-MXFP4 entry.
 * q is expert-stacked [E][K/8][N], e8 is [E][K/32][N]. Each expert's weights
 * are decoded once for all of its requested pairs. */
int hq_oracle_moe_mxfp4_bf16(int64_t T, int64_t top_k, int64_t E, int64_t N, int64_t K,
                             const uint16_t* A, const int32_t* ids, const uint32_t* q,
                             const uint8_t* e8, const int64_t* pairs, int64_t npairs, double* out)
{
    if (K % 32) return 1;
    for (int64_t i = 0; i < npairs; ++i)
        if (pairs[i] < 0 || pairs[i] >= T * top_k || ids[pairs[i]] < 0 || ids[pairs[i]] >= E) return 1;
    memset(out, 0, sizeof(double) * (size_t)(npairs * N));
    int64_t* sel = (int64_t*)malloc(sizeof(int64_t) * (size_t)(npairs + 1));
    double* a = (double*)malloc(sizeof(double) * (size_t)(npairs * K + 1));
    if (!sel || !a) { free(sel); free(a); return 2; }
    for (int64_t e = 0; e < E; ++e) {
        int64_t R = 0;
        for (int64_t i = 0; i < npairs; ++i)
            if (ids[pairs[i]] == e) sel[R++] = i;
        if (!R) continue;
        for (int64_t r = 0; r < R; ++r) {
            int64_t t = pairs[sel[r]] / top_k;
            for (int64_t k = 0; k < K; ++k) a[r * K + k] = hq_oracle_bf16(A[t * K + k]);
        }
        const uint32_t* qe = q + e * (K / 8) * N;
        const uint8_t* ee = e8 + e * (K / 32) * N;
#pragma omp parallel for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            for (int64_t k = 0; k < K; ++k) {
                double w = hq_oracle_e2m1(nib_along_k(qe, N, k, n)) * hq_oracle_e8m0(ee[(k / 32) * N + n]);
                for (int64_t r = 0; r < R; ++r) out[sel[r] * N + n] += a[r * K + k] * w;
            }
        }
    }
    free(sel);
    free(a);
    return 0;
}
