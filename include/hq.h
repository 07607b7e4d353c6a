/*
 * hq.h -- C ABI of the hq quantized-GEMM library for AMD Instinct MI355X (gfx950).
 *
 *   D[M,N] = A[M,K] x dequant(W[K,N])
 *
 * for weight-only W4A16 (symmetric INT4, or UINT4 with zero-points; group
 * scales along K), W4A8 with MXFP4 weights (e2m1 codes, E8M0 scale per 32 K)
 * and tokenwise FP8-e4m3 activations, W8A8 INT8 with a per-token x
 * per-channel epilogue, and the MoE Indexed / Grouped variants; further
 * W4A4 (MXFP4 x MXFP4) and MXFP8 x MXFP4 with the activations' own E8M0
 * scales, FP8 W8A8 with blockwise scales (1 x 128 activation blocks, 128 x 128
 * weight blocks), and 16-bit activations with FP4 weights (MXFP4, or NVFP4
 * with E4M3 scales per 16 K and a per-tensor second-level scale), MXINT4
 * weights, or INT8 / FP8-E4M3 weights with per-channel scales.  A layer
 * descriptor may ask for a batch-invariant reduction order or override the
 * kernel choice (tuning); two probes measure the device's attainable peaks.
 *
 * Sources.  The operation and its parameters follow the Humming pages:
 *  - "Humming wird angekuendigt", section "Eine einheitliche
 *    Quantisierungsdarstellung": weights, scales, zero-points and second-level
 *    scales are separate tensors; weight format, scale granularity and scale
 *    dtype are separate parameters; activations have their own format.
 *  - same page, section "Tuning und JIT-Kompilierung fuer jeden Workload":
 *    preprocessing validates, pads and repacks into a kernel layout; a layer
 *    description (shapes, dtypes, quantization parameters) plus a compute
 *    description (GEMM type, input-scale layout) configure the kernel; the
 *    kernel is chosen per input-size range at run time.
 *  - same page, sections "WnA16" and "W8A8 / W4A8 / W4A4": the dense
 *    W4A16, MoE Indexed / Grouped, W8A8 and W4A8-MXFP4 paths.
 *  - "Humming v0.1.0-0.1.4", section "v0.1.1": low launch CPU overhead and a
 *    stable launcher ABI.
 * Number formats: OCP Microscaling Formats v1.0 (E2M1, E8M0) and OCP 8-bit
 * floating point (E4M3, no infinities).
 *
 * Conventions (all entry points):
 *  - Every function returns hq_status.  HQ_OK = 0.  Arguments are validated
 *    before any HIP call; on an error nothing is launched and the stream is
 *    not touched.  hq_last_error() returns a thread-local message for the
 *    last failing call on this thread.
 *  - The caller owns every buffer.  The library never allocates device
 *    memory, never synchronises, and keeps no pointer after returning.
 *  - Device entry points enqueue work asynchronously on `stream` (a
 *    hipStream_t passed as void*; NULL is the default stream).  Device-side
 *    faults surface at the caller's next synchronisation.
 *  - Device pointers must be 16-byte aligned (HQ_ERR_ALIGNMENT otherwise).
 *  - A workspace is needed only where hq_workspace_bytes() says so (split-K
 *    partial tiles, MoE routing metadata, and at larger M the weights of the
 *    1-3-bit, 5-8-bit and MXFP6 formats rewritten in the layout the tiled
 *    kernels read: 4-bit words, one byte per code, or MXFP8 codes).  Every kernel writes what it later
 *    reads within the same call, so its contents need no initialisation and
 *    are meaningless between calls.  Two calls that share a workspace must not
 *    run concurrently.
 *  - Thread safety: the library holds no mutable global state besides
 *    per-device caches filled once (kernel attributes, the device address of
 *    hq_gemm_noalloc's scratch array).
 */
#ifndef HQ_H
#define HQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HQ_ABI_VERSION 1

typedef void* hq_stream_t; /* a hipStream_t */

typedef enum hq_status {
    HQ_OK = 0,
    HQ_ERR_INVALID_ARG = 1,  /* null pointer, negative size, bad enum           */
    HQ_ERR_UNSUPPORTED = 2,  /* dtype combination or shape the kernels lack     */
    HQ_ERR_ALIGNMENT = 3,    /* a device pointer is not 16-byte aligned         */
    HQ_ERR_WORKSPACE = 4,    /* workspace missing or smaller than required      */
    HQ_ERR_ABI = 5,          /* descriptor abi_version != HQ_ABI_VERSION        */
    HQ_ERR_HIP = 6           /* a HIP call failed; message has the HIP error    */
} hq_status;

typedef enum hq_dtype {
    HQ_DT_NONE = 0,
    HQ_DT_BF16 = 1,
    HQ_DT_FP16 = 2,
    HQ_DT_FP32 = 3,
    HQ_DT_FP8_E4M3 = 4,  /* OCP E4M3 ("fn": no inf, S.1111.111 = NaN) */
    HQ_DT_INT8 = 5,
    HQ_DT_INT4 = 6,      /* two's-complement nibble, -8..7             */
    HQ_DT_UINT4 = 7,     /* 0..15; with zero-points: value = q - z     */
    HQ_DT_FP4_E2M1 = 8,  /* OCP MX E2M1                                */
    HQ_DT_E8M0 = 9,      /* OCP MX shared scale, 2^(e-127)             */
    HQ_DT_INT32 = 10,
    /* low-bit weight codes (WnA16): signed widths are two's complement,
       unsigned ones take 4-bit zero-points; one code per byte on input */
    HQ_DT_INT1 = 11,     /* -1..0                                      */
    HQ_DT_UINT1 = 12,    /* 0..1                                       */
    HQ_DT_INT2 = 13,     /* -2..1                                      */
    HQ_DT_UINT2 = 14,    /* 0..3                                       */
    HQ_DT_INT3 = 15,     /* -4..3                                      */
    HQ_DT_UINT3 = 16,    /* 0..7                                       */
    /* OCP MX v1.0 FP6 element types (MXFP6 weights); one code per byte on input */
    HQ_DT_FP6_E2M3 = 17, /* 2 exponent bits (bias 1), 3 mantissa bits  */
    HQ_DT_FP6_E3M2 = 18, /* 3 exponent bits (bias 3), 2 mantissa bits  */
    /* zero-exponent floats e0mN: sign bit n, integer magnitude in bits 0..n-1,
       values -(2^n - 1) .. 2^n - 1 (the symmetric integers of width n + 1) */
    HQ_DT_E0M1 = 19,     /* -1..1, one code per byte                   */
    HQ_DT_E0M2 = 20,     /* -3..3, one code per byte                   */
    HQ_DT_E0M3 = 21,     /* -7..7, 4-bit codes in the INT4 word layout */
    HQ_DT_E0M7 = 22,     /* -127..127, one code per byte               */
    /* wider WnA16 codes, one per byte (INT8 = HQ_DT_INT8 with 16-bit group
       scales); unsigned widths take UINT8 zero-points */
    HQ_DT_INT5 = 23,     /* -16..15                                    */
    HQ_DT_UINT5 = 24,    /* 0..31                                      */
    HQ_DT_INT6 = 25,     /* -32..31                                    */
    HQ_DT_UINT6 = 26,    /* 0..63                                      */
    HQ_DT_INT7 = 27,     /* -64..63                                    */
    HQ_DT_UINT7 = 28,    /* 0..127                                     */
    HQ_DT_UINT8 = 29,    /* 0..255; also the 8-bit zero-point dtype    */
    HQ_DT_E0M4 = 30,     /* -15..15, one code per byte                 */
    HQ_DT_E0M5 = 31,     /* -31..31, one code per byte                 */
    HQ_DT_E0M6 = 32      /* -63..63, one code per byte                 */
} hq_dtype;

typedef enum hq_scale_gran {
    HQ_GRAN_NONE = 0,
    HQ_GRAN_PER_GROUP_K = 1, /* one scale per (group of group_size along K, column) */
    HQ_GRAN_PER_CHANNEL = 2, /* one scale per output column                         */
    HQ_GRAN_BLOCK_128x128 = 3 /* one scale per 128 x 128 block: [K/128][ceil(N/128)] */
} hq_scale_gran;

typedef enum hq_ascale {
    HQ_ASCALE_NONE = 0,
    HQ_ASCALE_PER_TOKEN_F32 = 1, /* fp32 a_scale[M], applied in the epilogue              */
    HQ_ASCALE_MX_E8M0 = 2,       /* OCP MX: uint8 E8M0 a_scale[M][K/32], 2^(e-127) per 32 K */
    HQ_ASCALE_PER_BLOCK128_F32 = 3 /* fp32 a_scale[M][K/128], one per row and 128-K block   */
} hq_ascale;

typedef enum hq_scale2 {
    HQ_S2_NONE = 0,
    HQ_S2_PER_TENSOR_F32 = 1 /* one fp32 multiplier of the whole weight tensor (per expert) */
} hq_scale2;

typedef enum hq_moe_mode {
    HQ_MOE_INDEXED = 1, /* A is [T,K] token rows; rows are gathered by topk_ids      */
    HQ_MOE_GROUPED = 2  /* A is [T*top_k,K] already sorted by expert (offsets given) */
} hq_moe_mode;

/*
 * Layer descriptor: shapes, dtypes and quantization parameters of one linear
 * layer (dense when num_experts == 0, else expert-stacked).  Plain data,
 * copied by value inside every call.
 *
 * Supported combinations:
 *   a_dtype   w_dtype    w_scale (gran, group)         zp      a_scale   out
 *   BF16|FP16 INT4       same as a_dtype, PER_GROUP_K  NONE    NONE      a_dtype
 *   BF16|FP16 UINT4      same as a_dtype, PER_GROUP_K  UINT4   NONE      a_dtype
 *   BF16|FP16 INT1|INT2|INT3  same as a_dtype, PER_GROUP_K  NONE  NONE  a_dtype (low-bit WnA16)
 *   BF16|FP16 UINT1|UINT2|UINT3  same, PER_GROUP_K     UINT4   NONE      a_dtype (low-bit WnA16)
 *   BF16|FP16 INT5|INT6|INT7|INT8  same as a_dtype, PER_GROUP_K  NONE  NONE  a_dtype (5-8-bit WnA16)
 *   BF16|FP16 UINT5|UINT6|UINT7|UINT8  same, PER_GROUP_K  UINT8  NONE     a_dtype (5-8-bit WnA16)
 *   BF16|FP16 E0M1|E0M2|E0M3  same as a_dtype, PER_GROUP_K  NONE  NONE  a_dtype (e0mN: the INT2/3/4 kernels)
 *   BF16|FP16 E0M4|E0M5|E0M6  same as a_dtype, PER_GROUP_K  NONE  NONE  a_dtype (e0mN: the INT5/6/7 kernels)
 *   BF16|FP16 E0M7       FP32, PER_CHANNEL             NONE    NONE      a_dtype (e0m7: the INT8 kernels)
 *   BF16|FP16 FP8_E4M3   E8M0, PER_GROUP_K, group 32   NONE    NONE      a_dtype (MXFP8 weight-only)
 *   BF16|FP16 FP6_E2M3|FP6_E3M2  E8M0, PER_GROUP_K, 32  NONE   NONE      a_dtype (MXFP6 weight-only)
 * (With fp16 activations the E8M0- and E4M3-scaled weights become fp16
 * operands: exact while code x scale stays inside fp16's range, about
 * 2^-24 .. 65504; outside it they round to subnormals or saturate.)
 *   FP8_E4M3  FP4_E2M1   E8M0, PER_GROUP_K, group 32   NONE    PER_TOKEN BF16
 *   INT8      INT8       FP32, PER_CHANNEL             NONE    PER_TOKEN BF16|INT32
 *   FP8_E4M3  FP4_E2M1   E8M0, PER_GROUP_K, group 32   NONE    MX_E8M0   BF16   (MXFP8 x MXFP4)
 *   FP4_E2M1  FP4_E2M1   E8M0, PER_GROUP_K, group 32   NONE    MX_E8M0   BF16   (W4A4 MXFP4)
 *   FP8_E4M3  FP8_E4M3   FP32, BLOCK_128x128           NONE    PER_BLOCK128 BF16 (FP8 blockwise)
 *   BF16|FP16 FP4_E2M1   E8M0, PER_GROUP_K, group 32   NONE    NONE      a_dtype (FP4 WnA16, MXFP4)
 *   BF16|FP16 FP4_E2M1   FP8_E4M3, PER_GROUP_K, grp 16 NONE    NONE      a_dtype (NVFP4; scale2
 *                                                                               PER_TENSOR_F32)
 *   BF16      FP4_E2M1   E8M0, PER_GROUP_K, group 32   NONE    NONE      BF16   (MoE)
 *   BF16|FP16 INT4       E8M0, PER_GROUP_K, group 32   NONE    NONE      a_dtype (MXINT4)
 *   BF16|FP16 INT8       FP32, PER_CHANNEL             NONE    NONE      a_dtype (INT8 weight-only)
 *   BF16|FP16 FP8_E4M3   FP32, PER_CHANNEL             NONE    NONE      a_dtype (FP8 weight-only)
 * FP4_E2M1 activations are packed two per byte along K, element k in the low
 * nibble of byte k/2 when k is even (rows of K/2 bytes).
 * Group sizes for 16-bit scales: a multiple of 128 that divides K.
 * K: a multiple of 128 (every format), at most 2^24.  N: 1 .. 2^21 (a row
 * tile of the output is addressed through one 32-bit buffer range).
 * out_dtype INT32 returns the raw INT8 x INT8 accumulators (bit-exact).
 */
typedef struct hq_layer_desc {
    int32_t abi_version;    /* HQ_ABI_VERSION                                  */
    int32_t num_experts;    /* 0 = dense layer                                 */
    int64_t N;              /* output features                                 */
    int64_t K;              /* input features                                  */
    int32_t a_dtype;        /* hq_dtype of A                                   */
    int32_t a_scale;        /* hq_ascale                                       */
    int32_t w_dtype;        /* hq_dtype of the weight codes                    */
    int32_t w_scale_dtype;  /* hq_dtype of the weight scales                   */
    int32_t w_scale_gran;   /* hq_scale_gran                                   */
    int32_t group_size;     /* K elements per scale (PER_GROUP_K)              */
    int32_t zp_dtype;       /* HQ_DT_NONE or HQ_DT_UINT4                       */
    int32_t scale2;         /* hq_scale2                                       */
    int32_t out_dtype;      /* hq_dtype of D                                   */
    int32_t flags;          /* HQ_FLAG_* compute options (0: none)             */
    int32_t tune;           /* 0: the library's kernel choice; HQ_TUNE(...)    */
    int32_t reserved;       /* must be zero                                    */
} hq_layer_desc;

/*
 * Compute options ("Humming wird angekuendigt", section "Tuning und
 * JIT-Kompilierung fuer jeden Workload": the compute description carries
 * options such as batch invariance).
 *   HQ_FLAG_BATCH_INVARIANT  dense layers: every output row is computed in an
 *       order that does not depend on M or on the other rows (tiled kernels
 *       without a K split at every M), so a row gives bit-identical results
 *       whatever batch it is part of.  Slower at small M.
 */
#define HQ_FLAG_BATCH_INVARIANT 1

/*
 * Tuning override of the kernel choice for dense layers (same section: the
 * tuning description selects tile shape and pipeline; an autotuner times the
 * candidates on the device, "Humming wird angekuendigt", section "Zukuenftige
 * Plaene").  tune = HQ_TUNE(path, splits); splits = K slices (0: the
 * planner's choice for the stream path, 1 for tiles).  Paths:
 *   HQ_TUNE_STREAM  the small-M weight stream (M <= 64), A slice in LDS
 *   HQ_TUNE_T128    128 x 128 tiles          HQ_TUNE_T256  the 256-row tile
 *   HQ_TUNE_W128    128 x 256 tiles          HQ_TUNE_W256  256 x 256 tiles
 *   HQ_TUNE_STREAM8 the small-M weight stream on eight waves that load their
 *                   A fragments directly, one 16-column strip per workgroup
 *                   and no K split (16-bit activations, M <= 16, K / 128
 *                   between 8 and 64; splits 0 or 1)
 * A path the layer's format lacks, or a split the slice cannot take, returns
 * HQ_ERR_UNSUPPORTED at the call.  hq_gemm_plan and hq_workspace_bytes follow
 * the override.
 */
#define HQ_TUNE_STREAM 1
#define HQ_TUNE_T128 2
#define HQ_TUNE_T256 3
#define HQ_TUNE_W128 4
#define HQ_TUNE_W256 5
#define HQ_TUNE_STREAM8 6
#define HQ_TUNE(path, splits) ((int32_t)(path) | ((int32_t)(splits) << 8))

/* ---------------------------------------------------------------------- */
/* general                                                                 */
/* ---------------------------------------------------------------------- */

int32_t hq_abi_version(void);
const char* hq_status_str(hq_status s);
/* Message for the last failing call on the calling thread ("" if none). */
const char* hq_last_error(void);
/* Checks a descriptor against the supported combinations above. Host only. */
hq_status hq_desc_validate(const hq_layer_desc* desc);

/* ---------------------------------------------------------------------- */
/* repack (host only): logical export form -> hq standard packed layout     */
/* ---------------------------------------------------------------------- */

/*
 * Byte sizes of the four packed tensors (weights, scales, zero-points,
 * second-level scales), covering all experts.  Unused tensors report 0.
 */
hq_status hq_repacked_bytes(const hq_layer_desc* desc, size_t* w_bytes, size_t* s_bytes,
                            size_t* z_bytes, size_t* s2_bytes);

/*
 * Host-memory transform of one layer (all experts) from the logical export
 * form into the packed layout the kernels read.  Pure, deterministic,
 * thread-safe; integer bit permutation only (exact).  Outputs are allocated
 * by the caller with hq_repacked_bytes(); unused tensors are NULL.
 *
 * Logical inputs (per expert, experts stacked along a leading axis):
 *   w  4-bit codes: uint32 [K/8][N]; code k = 8j+i of column n in bits
 *      4i..4i+3 of word [j][n]            INT8 / FP8_E4M3: one byte [K][N]
 *      1-3-bit codes (WnA16 "Humming wird angekuendigt", section WnA16): one
 *      int8 per code [K][N], the two's-complement value for INT1..INT3,
 *      0 .. 2^b-1 for UINT1..UINT3; a code outside its width is
 *      HQ_ERR_INVALID_ARG.  Unsigned widths take UINT4 zero-points (below).
 *      5-8-bit codes (WnA16, same section): one byte per code [K][N], int8
 *      two's complement for INT5..INT8, uint8 0 .. 2^b-1 for UINT5..UINT8; a
 *      code outside its width is HQ_ERR_INVALID_ARG.  Unsigned widths take
 *      UINT8 zero-points (below).
 *      e0mN ("Humming wird angekuendigt": the zero-exponent float whose values
 *      are the symmetric integers of its width): e0m3 in the 4-bit word layout
 *      above, e0m1 / e0m2 / e0m4..e0m7 one code per byte [K][N]; bit n is the sign,
 *      bits 0..n-1 the magnitude.  The repack stores each code as the two's-
 *      complement code of width n + 1 (INT2 .. INT8) and the kernels of
 *      that width run it; a code with a bit above bit n is HQ_ERR_INVALID_ARG.
 *      MXFP8 / MXFP6: E4M3 / E2M3 / E3M2 codes, one per byte [K][N] (FP6 in the
 *      low six bits, a higher bit is HQ_ERR_INVALID_ARG); E8M0 [K/32][N].
 *   scale  [K/group][N] in w_scale_dtype (16-bit raw bits, uint8 for E8M0);
 *          PER_CHANNEL fp32: [N]; BLOCK_128x128 fp32: [K/128][ceil(N/128)]
 *   zp     UINT4: uint32 [K/group][ceil(N/8)]; column n = 8j+i in bits
 *          4i..4i+3 of word [g][j]
 *          UINT8 (5-8-bit widths): uint8 [K/group][N], each inside the codes'
 *          width (else HQ_ERR_INVALID_ARG)
 *   scale2 PER_TENSOR_F32: fp32 [E] (one per expert); otherwise NULL
 *
 * Packed outputs (N padded to Np = ceil(N/16)*16; padding decodes to 0 with
 * unit scale).  A "strip" is 16 consecutive columns; a lane is one of the 64
 * lanes of a wavefront reading 16 bytes:
 *   w  4-bit: [E][Np/16][K/128][64 lanes][16 B]; lane l holds column
 *      16*strip + (l & 15), k = 128*chunk + 32*(l >> 4) + j, j = 0..31,
 *      bytes 4t..4t+3 holding j = 8t..8t+7.  Inside a word FP4 codes are in
 *      natural order (j in nibble j%8); INT4/UINT4 codes are in pair order
 *      (nibble p holds j%8 = {0,2,4,6,1,3,5,7}[p]) so that one shift+mask
 *      yields two consecutive codes in the two 16-bit halves.
 *      1-3-bit (WnA16): the codes' low two bits and their third (b = 3) or
 *      only (b = 1) bit in separate planes.  Per slot = (strip * K/128 +
 *      chunk) * 64 + lane, code j = 0..7 of sub-step t = 0..3 is the code at
 *      k = 128*chunk + 32*(l >> 4) + 8*t + j of column 16*strip + (l & 15):
 *        2-bit plane (b = 2, 3), first: uint32 [slots][2]; bits
 *          16*(j&1) + 8*(t&1) + 2*(j>>1) .. +1 of word t>>1 hold its low two bits;
 *        1-bit plane (b = 1, 3), after it: uint32 [slots]; bit
 *          16*(j&1) + 4*t + (j>>1) holds its bit 0 (b = 1) or bit 2 (b = 3).
 *      Codes 2s and 2s+1 thus share an offset in the two 16-bit halves.
 *      5-8-bit (WnA16): the codes' low four bits as a 4-bit word set in the
 *        INT4/UINT4 layout above (pair order), then their high b - 4 bits:
 *        for b = 8 a second 4-bit word set of the same layout; for b = 5..7
 *        the planes above holding the (b - 4)-bit high code (a 2-bit plane for
 *        b = 6, 7, then a 1-bit plane for b = 5, 7, whose bit is bit 4 for
 *        b = 5 and bit 6 for b = 7 of the code).
 *      MXFP6: a lane's 32 codes of a chunk as one 192-bit group, code j at
 *        bits 6j..6j+5; bits 0-127 of every slot in a 16-byte plane
 *        [Np/16][K/128][64 lanes][16 B], bits 128-191 after it in an 8-byte
 *        plane [Np/16][K/128][64 lanes][8 B].  MXFP8: the INT8 weight-only
 *        layout below; both with the E8M0 layout below.
 *      INT8 and FP8_E4M3 with 8-bit activations (W8A8, FP8 blockwise):
 *      [Np/16][K/64][64 lanes][16 B]; lane l holds column 16*strip + (l & 15),
 *      k = 64*chunk + 16*(l >> 4) + j, j = 0..15.
 *      INT8 and FP8_E4M3 with 16-bit activations (weight-only):
 *      [Np/16][K/128][2 halves][64 lanes][16 B]; lane l holds column
 *      16*strip + (l & 15), k = 128*chunk + 32*(l >> 4) + 16*h + j, j = 0..15.
 *   scale  16-bit group scales: [E][Np/16][K/group][16];
 *          E8M0: [E][Np/16][K/128][64 lanes] bytes; lane l holds the
 *          exponent of column 16*strip + (l & 15), K-block 4*chunk + (l >> 4)
 *          (padding columns hold 127);
 *          E4M3 per 16 K (NVFP4): [E][Np/16][K/128][64 lanes][2] bytes; lane l
 *          holds column 16*strip + (l & 15), groups 8*chunk + 2*(l >> 4) + h
 *          (padding columns hold 0x38 = 1.0);
 *          PER_CHANNEL fp32: [Np]; BLOCK_128x128 fp32: unchanged [K/128][ceil(N/128)]
 *   zp     [E][Np/16][K/group] uint64, column 16*strip + i in bits 4i..4i+3
 *          UINT8: [Np/16][K/group][16] bytes, byte i for column 16*strip + i
 *          (padding columns 0)
 *   scale2 fp32 [E], copied
 */
hq_status hq_repack(const hq_layer_desc* desc, const void* w, const void* scale, const void* zp,
                    const void* scale2, void* w_out, void* s_out, void* z_out, void* s2_out);

/* ---------------------------------------------------------------------- */
/* workspace                                                               */
/* ---------------------------------------------------------------------- */

/*
 * Workspace bytes for a call with M rows (dense) or T tokens and top_k
 * (MoE; top_k is ignored for dense layers).  0 means none is needed.
 */
hq_status hq_workspace_bytes(const hq_layer_desc* desc, int64_t M_or_T, int32_t top_k, size_t* bytes);

/* Zero-fills a workspace on `stream` with a fill kernel (graph-capturable).
 * Never required by the GEMMs (they initialise what they read); kept for
 * callers that want deterministic workspace contents. */
hq_status hq_workspace_init(void* workspace, size_t bytes, hq_stream_t stream);

/* ---------------------------------------------------------------------- */
/* GEMMs (device)                                                          */
/* ---------------------------------------------------------------------- */

/*
 * Dense D[M,N] = A[M,K] x dequant(W).
 *   A        device, [M][K] row-major, a_dtype (E2M1: [M][K/2] bytes)
 *   a_scale  device; PER_TOKEN_F32: fp32 [M]; MX_E8M0: uint8 [M][K/32]
 *            (E8M0 of row m, K block b); PER_BLOCK128_F32: fp32 [M][K/128];
 *            NONE: NULL
 *   w, s, z, s2  device, packed by hq_repack (unused ones NULL; s2 4-byte aligned)
 *   D        device, [M][N] row-major, out_dtype
 * Floating outputs: fp32 accumulation, rounded once (RNE) to out_dtype.
 * M == 0 returns HQ_OK without launching.
 */
hq_status hq_gemm(const hq_layer_desc* desc, int64_t M, const void* A, const void* a_scale,
                  const void* w, const void* s, const void* z, const void* s2, void* D,
                  void* workspace, size_t ws_bytes, hq_stream_t stream);

/*
 * hq_gemm without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, kernels and results as hq_gemm;
 * where that call's plan needs split-K partial tiles, they go to a scratch
 * array of HQ_NOALLOC_SCRATCH_BYTES compiled into the library, one per GPU,
 * held until the process ends.  Calls whose plan needs more scratch return
 * HQ_ERR_WORKSPACE (hq_workspace_bytes() tells the need in advance).  Nothing
 * is allocated: no hipMalloc/hipFree, no allocating library call.  The first
 * call on a GPU looks up the array's device address once (hipGetSymbolAddress,
 * with that GPU made current for the lookup).  Every call on one GPU shares
 * its array, so calls that overlap in time on one GPU (other streams, other
 * threads) race and must be serialised by the caller; the kernels write every
 * scratch byte they read within the call, so nothing needs clearing.
 */
#define HQ_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
hq_status hq_gemm_noalloc(const hq_layer_desc* desc, int64_t M, const void* A, const void* a_scale,
                          const void* w, const void* s, const void* z, const void* s2, void* D, hq_stream_t stream);

/*
 * Host only, no HIP call: the kernel launches hq_gemm would enqueue for this
 * dense descriptor and M, written to buf (NUL-terminated, truncated to len)
 * as ';'-separated "kernel<template arguments> grid=... splits=..." items.
 * The same code path picks the kernels in hq_gemm ("Humming wird
 * angekuendigt", section "Tuning und JIT-Kompilierung fuer jeden Workload":
 * one prepared configuration per range of input sizes, chosen at run time).
 * M == 0 writes "" (no launch).
 */
hq_status hq_gemm_plan(const hq_layer_desc* desc, int64_t M, char* buf, size_t len);

/*
 * MoE GEMM over top_k experts per token (expert-stacked packed weights).
 *   INDEXED: A [T][K]; topk_ids device int32 [T][top_k] (distinct per token,
 *            0 <= id < num_experts); D [T*top_k][N], row t*top_k + j is
 *            A[t] x W[topk_ids[t][j]].  expert_offsets must be NULL.
 *   GROUPED: A [T*top_k][K] already sorted by expert; expert_offsets device
 *            int32 [num_experts+1] (nondecreasing, offsets[0] = 0,
 *            offsets[E] = T*top_k); D [T*top_k][N] in the same row order.
 *            topk_ids must be NULL.
 * Routing weights are not applied.  T == 0 returns HQ_OK.
 */
hq_status hq_moe_gemm(const hq_layer_desc* desc, int32_t mode, int64_t T, int32_t top_k,
                      const void* A, const float* a_scale, const int32_t* topk_ids,
                      const int32_t* expert_offsets, const void* w, const void* s, const void* z,
                      const void* s2, void* D, void* workspace, size_t ws_bytes, hq_stream_t stream);

/* ---------------------------------------------------------------------- */
/* input preparation (device)                                              */
/* ---------------------------------------------------------------------- */

/*
 * Tokenwise activation quantisation ("Humming wird angekuendigt", section
 * "End-to-End-Inferenzleistung": tokenwise FP8 activations for W4A8).
 * For each row m of x (fp32 [M][K]): s[m] = max_k |x| / 448 in fp32 (1 for an
 * all-zero row); q[m][k] = E4M3(x / s[m]), fp32 division, round to nearest
 * even, saturating at +-448.  out_dtype must be HQ_DT_FP8_E4M3.
 */
hq_status hq_quantize_act(int32_t out_dtype, int64_t M, int64_t K, const float* x, void* q, float* s,
                          hq_stream_t stream);

/*
 * Activation quantisation to E4M3 with one fp32 scale per row and block of
 * `block` consecutive elements along K ("Humming wird angekuendigt", section
 * "W8A8 / W4A8 / W4A4": FP8 W8A8 with blockwise scaling; block 128 gives the
 * 1 x 128 activation blocks of that path, block K the tokenwise case of
 * hq_quantize_act).  Per block: s = max |x| / 448 in fp32 (1 for an all-zero
 * block), q = E4M3(x / s) with fp32 division, round to nearest even,
 * saturating at +-448; NaN and infinity as in hq_quantize_act.
 *   x fp32 [M][K], q [M][K], s fp32 [M][K/block]; K a multiple of block,
 *   block a multiple of 4 unless it equals K; pointers 16-byte aligned.
 */
hq_status hq_quantize_act_blocks(int32_t out_dtype, int64_t M, int64_t K, int64_t block, const float* x, void* q,
                                 float* s, hq_stream_t stream);

/*
 * MX activation quantisation ("Humming wird angekuendigt", sections
 * "W8A8 / W4A8 / W4A4" and "Auswahl von Aktivierungstypen": W4A4 on MXFP4
 * and MXFP8 activations), OCP Microscaling Formats v1.0, section 6.3:
 * for each row m of x (fp32 [M][K], K a multiple of 32) and block b of 32 along K:
 *   e[m][b] = clamp(floor(log2(max|x|)) - emax, ...) as E8M0 (emax: E4M3 8,
 *             E2M1 2), i.e. the exponent field of max|x| minus emax, clamped
 *             to 0..254; 0 for an all-zero block; 0xFF (NaN) for a block
 *             holding a NaN or an infinity (its codes are then 0)
 *   q = x * 2^(127 - e) rounded to nearest even, saturated (E4M3 +-448,
 *       E2M1 +-6); E4M3 codes one per byte [M][K]; E2M1 codes two per byte
 *       [M][K/2], element k in the low nibble of byte k/2 when k is even.
 * out_dtype HQ_DT_FP8_E4M3 or HQ_DT_FP4_E2M1; pointers 16-byte aligned.
 */
hq_status hq_quantize_act_mx(int32_t out_dtype, int64_t M, int64_t K, const float* x, void* q, void* e,
                             hq_stream_t stream);

/*
 * SwiGLU between the MoE gate-up and down projections ("Humming wird
 * angekuendigt", section "Leistung": the MoE figures add the gate-up and down
 * GEMMs; the activation between them is the plain SiLU(gate) * up of a fused
 * gate+up output, gate in the first half of each row).
 *   gate_up  device bf16 [rows][2I]: row r = gate[r][0..I) | up[r][0..I)
 *   out      device bf16 [rows][I]: bf16(silu(gate) * up), fp32 arithmetic with
 *            silu(g) = g / (1 + e^-g) (evaluated without overflow for large
 *            negative g), rounded once to nearest even
 * dtype must be HQ_DT_BF16; I a multiple of 8; pointers 16-byte aligned; the
 * two buffers must not overlap.  rows == 0 returns HQ_OK.  The output feeds the
 * down projection as hq_moe_gemm INDEXED with T = rows, top_k = 1 and the
 * flattened top-k ids (each row its own token), or GROUPED on sorted rows.
 */
hq_status hq_silu_mul(int32_t dtype, int64_t rows, int64_t I, const void* gate_up, void* out, hq_stream_t stream);

/*
 * MoE routing metadata ("Humming wird angekuendigt", section "WnA16": the
 * Grouped path runs on expert-sorted tokens).  From topk_ids [T][top_k]:
 *   expert_offsets [E+1]: exclusive prefix sum of per-expert pair counts
 *   sorted_pairs   [T*top_k]: pair ids p = t*top_k + j stably sorted by expert
 * workspace: hq_workspace_bytes of a MoE descriptor with the same T, top_k.
 */
hq_status hq_moe_align(int64_t T, int32_t top_k, int32_t num_experts, const int32_t* topk_ids,
                       int32_t* expert_offsets, int32_t* sorted_pairs, void* workspace,
                       size_t ws_bytes, hq_stream_t stream);

/*
 * Builds the Grouped activation matrix: A_sorted[i] = A[sorted_pairs[i] / top_k]
 * for i < T*top_k; rows of K elements of `dtype` (BF16, FP16, FP8_E4M3, INT8).
 */
hq_status hq_moe_gather(int32_t dtype, int64_t T, int32_t top_k, int64_t K, const void* A,
                        const int32_t* sorted_pairs, void* A_sorted, hq_stream_t stream);

/*
 * Measurement probes (not part of the GEMM path): what the device delivers, for
 * setting kernel timings against measured as well as published peaks.
 *
 * hq_probe_stream: reads the `bytes` of device buffer src once per repetition
 * (16-byte non-temporal loads, grid-stride, 4096 workgroups of 256 threads),
 * `reps` times back to back on `stream`; nothing is written in practice (sink,
 * 16 device bytes, is stored to only if the XOR of all loaded words takes one
 * fixed value).  bytes a positive multiple of 16, src and sink 16-byte aligned,
 * reps 1..1000.
 *
 * hq_probe_mfma: `workgroups` workgroups of 4 waves; each wave runs `iters`
 * rounds of 8 independent MFMAs of the dense 16x16 instruction of `dtype` on
 * register operands: HQ_DT_FP16 / HQ_DT_BF16 16x16x32 (16384 flops each),
 * HQ_DT_FP8_E4M3 and HQ_DT_FP4_E2M1 16x16x128 (65536), HQ_DT_INT8 16x16x64
 * (32768 ops); flops per call = workgroups * 4 * iters * 8 * that.  sink: device
 * fp32 [workgroups * 256], written (one sum per thread).  workgroups 1..65536,
 * iters 1..1000000.
 */
hq_status hq_probe_stream(const void* src, size_t bytes, void* sink, int32_t reps, hq_stream_t stream);
hq_status hq_probe_mfma(int32_t dtype, int64_t workgroups, int32_t iters, void* sink, hq_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* HQ_H */
