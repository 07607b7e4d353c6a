// hq_api.cpp -- the extern "C" boundary of libhq: descriptor validation,
// sizing, repack, workspace queries and per-call dispatch to the kernels.
//
// Dispatch follows the pages' scheme of configurations prepared per range of
// input sizes and selected at run time ("Humming wird angekuendigt", section
// "Tuning und JIT-Kompilierung fuer jeden Workload"), with kernels compiled
// ahead of time.  The host path does O(1) checks and no allocation, in the
// spirit of the launch-overhead work in "Humming v0.1.0-0.1.4", section
// "v0.1.1".
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "hq_common.h"
#include "hq_internal.h"

namespace hq {

namespace {
thread_local char g_err[512] = {0};

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
}  // namespace

hq_status set_error(hq_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

namespace {
thread_local PlanRecorder* g_plan = nullptr;
}

PlanRecorder* plan_recorder() { return g_plan; }

void plan_workspace(size_t bytes) {
    if (g_plan && g_plan->base + bytes > g_plan->ws) g_plan->ws = g_plan->base + bytes;
}

void plan_workspace_base(size_t base) {
    if (g_plan) g_plan->base = base;
}

void plan_record(const char* fmt, ...) {
    PlanRecorder* r = g_plan;
    if (!r || !r->buf || r->used + 1 >= r->len) return;
    if (r->used) r->buf[r->used++] = ';';
    va_list ap;
    va_start(ap, fmt);
    const int n = vsnprintf(r->buf + r->used, r->len - r->used, fmt, ap);
    va_end(ap);
    if (n > 0) r->used += (size_t)n < r->len - r->used ? (size_t)n : r->len - r->used - 1;
}

static hq_status ok() {
    g_err[0] = 0;
    return HQ_OK;
}

// mantissa width n of the zero-exponent float dtypes e0mN (0 for the others)
static int e0m_width(int w) {
    switch (w) {
        case HQ_DT_E0M1: return 1;
        case HQ_DT_E0M2: return 2;
        case HQ_DT_E0M3: return 3;
        case HQ_DT_E0M4: return 4;
        case HQ_DT_E0M5: return 5;
        case HQ_DT_E0M6: return 6;
        case HQ_DT_E0M7: return 7;
        default: return 0;
    }
}

// code width and signedness of the 5-8-bit WnA16 dtypes (0 for the others; INT8
// is one of them only with 16-bit group scales)
static int wide_width(int w, int scale_dtype, bool* is_signed) {
    *is_signed = w == HQ_DT_INT5 || w == HQ_DT_INT6 || w == HQ_DT_INT7 || w == HQ_DT_INT8 || w == HQ_DT_E0M4 ||
                 w == HQ_DT_E0M5 || w == HQ_DT_E0M6;
    switch (w) {
        case HQ_DT_E0M4: return 5;  // e0m4..e0m6: sign and magnitude, converted at repack
        case HQ_DT_E0M5: return 6;  // to the two's-complement codes of width n + 1
        case HQ_DT_E0M6: return 7;
        case HQ_DT_INT5: case HQ_DT_UINT5: return 5;
        case HQ_DT_INT6: case HQ_DT_UINT6: return 6;
        case HQ_DT_INT7: case HQ_DT_UINT7: return 7;
        case HQ_DT_UINT8: return 8;
        case HQ_DT_INT8: return scale_dtype == HQ_DT_BF16 || scale_dtype == HQ_DT_FP16 ? 8 : 0;
        default: return 0;
    }
}

// code width of the low-bit weight dtypes (0 for the others)
int lowbit_width(int w) {
    switch (w) {
        case HQ_DT_INT1: case HQ_DT_UINT1: return 1;
        case HQ_DT_INT2: case HQ_DT_UINT2: return 2;
        case HQ_DT_INT3: case HQ_DT_UINT3: return 3;
        default: return 0;
    }
}

hq_status describe(const hq_layer_desc* d, LayerInfo* L) {
    if (!d) return set_error(HQ_ERR_INVALID_ARG, "descriptor is NULL");
    if (d->abi_version != HQ_ABI_VERSION)
        return set_error(HQ_ERR_ABI, "descriptor abi_version %d, library %d", d->abi_version, HQ_ABI_VERSION);
    if (d->reserved) return set_error(HQ_ERR_INVALID_ARG, "reserved fields must be zero");
    if (d->flags & ~HQ_FLAG_BATCH_INVARIANT) return set_error(HQ_ERR_INVALID_ARG, "unknown flags 0x%x", d->flags);
    const int tune_path = d->tune & 0xFF, tune_splits = (d->tune >> 8) & 0xFFFF;
    if (tune_path > HQ_TUNE_STREAM8 || (d->tune >> 24) || (tune_path == 0 && tune_splits))
        return set_error(HQ_ERR_INVALID_ARG, "bad tune value 0x%x", d->tune);
    if ((d->flags || d->tune) && d->num_experts)
        return set_error(HQ_ERR_UNSUPPORTED, "batch invariance and tuning overrides apply to dense layers");
    // N <= 2^21: the tile epilogues address a tile's rows of the output (or of a
    // partial tile) through one 32-bit buffer range (256 rows x N x 4 bytes)
    if (d->N < 1 || d->K < 1 || d->N > (1LL << 21) || d->K > (1LL << 24))
        return set_error(HQ_ERR_INVALID_ARG, "N=%lld K=%lld out of range (N in [1, 2^21], K in [1, 2^24])", (long long)d->N,
                         (long long)d->K);
    if (d->num_experts < 0 || d->num_experts > 4096)
        return set_error(HQ_ERR_INVALID_ARG, "num_experts=%d out of range [0, 4096]", d->num_experts);
    if (d->scale2 != HQ_S2_NONE && d->scale2 != HQ_S2_PER_TENSOR_F32)
        return set_error(HQ_ERR_INVALID_ARG, "bad scale2 kind %d", d->scale2);
    LayerInfo I{};
    I.bits = 4;
    I.invariant = (d->flags & HQ_FLAG_BATCH_INVARIANT) != 0;
    I.tune_path = tune_path;
    I.tune_splits = tune_splits;
    I.N = d->N;
    I.K = d->K;
    I.Np = pad16(d->N);
    I.E = d->num_experts ? d->num_experts : 1;
    I.G = d->group_size;
    const int a = d->a_dtype, w = d->w_dtype;
    bool wide_signed = false;
    if (w == HQ_DT_INT4 && (a == HQ_DT_BF16 || a == HQ_DT_FP16) && d->w_scale_dtype == HQ_DT_E8M0) {
        // MXINT4: two's-complement INT4 codes with one E8M0 scale per 32 K (the
        // FP4 weight-only path with an integer decode)
        I.kind = Kind::FP4_A16;
        I.i4 = true;
        I.a_bf16 = a == HQ_DT_BF16;
        if (d->num_experts) return set_error(HQ_ERR_UNSUPPORTED, "MXINT4 is dense-only");
        if (d->w_scale_gran != HQ_GRAN_PER_GROUP_K || d->group_size != 32)
            return set_error(HQ_ERR_UNSUPPORTED, "MXINT4 needs E8M0 scales per 32 K elements");
        if (d->a_scale != HQ_ASCALE_NONE) return set_error(HQ_ERR_UNSUPPORTED, "16-bit A x MXINT4 takes no activation scale");
        if (d->K % 128) return set_error(HQ_ERR_UNSUPPORTED, "MXINT4 needs K %% 128 == 0 (K=%lld)", (long long)d->K);
        if (d->zp_dtype != HQ_DT_NONE) return set_error(HQ_ERR_UNSUPPORTED, "MXINT4 takes no zero-points");
        if (d->out_dtype != a) return set_error(HQ_ERR_UNSUPPORTED, "MXINT4 weight-only outputs the activation dtype");
        I.G = 32;
    } else if ((a == HQ_DT_BF16 || a == HQ_DT_FP16) && wide_width(w, d->w_scale_dtype, &wide_signed)) {
        // WnA16 at 5-8 bits: the low nibble in the 4-bit layout, the high bits in
        // planes; 16-bit group scales, UINT8 zero-points for unsigned codes
        I.kind = Kind::WNA16;
        I.a_bf16 = a == HQ_DT_BF16;
        I.bits = wide_width(w, d->w_scale_dtype, &wide_signed);
        I.e0m = e0m_width(w);
        I.zp = I.zp8 = !wide_signed;
        if (d->num_experts) return set_error(HQ_ERR_UNSUPPORTED, "WnA16 at 5-8 bits is dense-only");
        if (d->w_scale_dtype != a) return set_error(HQ_ERR_UNSUPPORTED, "WnA16 scale dtype must equal the activation dtype");
        if (d->w_scale_gran != HQ_GRAN_PER_GROUP_K) return set_error(HQ_ERR_UNSUPPORTED, "WnA16 needs per-group scales");
        if (d->group_size < 128 || d->group_size % 128 || d->K % d->group_size)
            return set_error(HQ_ERR_UNSUPPORTED, "WnA16 group_size=%d must be a multiple of 128 dividing K=%lld",
                             d->group_size, (long long)d->K);
        if (d->zp_dtype != (I.zp8 ? HQ_DT_UINT8 : HQ_DT_NONE))
            return set_error(HQ_ERR_UNSUPPORTED, "zero-points: unsigned 5-8-bit codes need UINT8 zero-points, signed codes none");
        if (d->a_scale != HQ_ASCALE_NONE) return set_error(HQ_ERR_UNSUPPORTED, "WnA16 takes no activation scale");
        if (d->out_dtype != a) return set_error(HQ_ERR_UNSUPPORTED, "WnA16 output dtype must equal the activation dtype");
    } else if ((a == HQ_DT_BF16 || a == HQ_DT_FP16) &&
               (w == HQ_DT_INT4 || w == HQ_DT_UINT4 || lowbit_width(w) || (e0m_width(w) && e0m_width(w) <= 3))) {
        // W4A16, the low-bit widths on the same kernels (1-3-bit codes widened
        // to 4-bit ones in registers), and e0m1..e0m3 (sign and magnitude,
        // converted at repack to the two's-complement codes of width n + 1)
        I.kind = Kind::WNA16;
        I.a_bf16 = a == HQ_DT_BF16;
        I.e0m = e0m_width(w);
        I.bits = I.e0m ? I.e0m + 1 : lowbit_width(w) ? lowbit_width(w) : 4;
        I.zp = w == HQ_DT_UINT4 || w == HQ_DT_UINT1 || w == HQ_DT_UINT2 || w == HQ_DT_UINT3;
        if (d->num_experts) return set_error(HQ_ERR_UNSUPPORTED, "W4A16 INT4/UINT4 is dense-only");
        if (d->w_scale_dtype != a) return set_error(HQ_ERR_UNSUPPORTED, "W4A16 scale dtype must equal the activation dtype");
        if (d->w_scale_gran != HQ_GRAN_PER_GROUP_K) return set_error(HQ_ERR_UNSUPPORTED, "W4A16 needs per-group scales");
        if (d->group_size < 128 || d->group_size % 128 || d->K % d->group_size)
            return set_error(HQ_ERR_UNSUPPORTED, "W4A16 group_size=%d must be a multiple of 128 dividing K=%lld",
                             d->group_size, (long long)d->K);
        if (d->zp_dtype != (I.zp ? HQ_DT_UINT4 : HQ_DT_NONE))
            return set_error(HQ_ERR_UNSUPPORTED, "zero-points: unsigned codes need UINT4 zero-points, signed codes none");
        if (d->a_scale != HQ_ASCALE_NONE) return set_error(HQ_ERR_UNSUPPORTED, "W4A16 takes no activation scale");
        if (d->out_dtype != a) return set_error(HQ_ERR_UNSUPPORTED, "W4A16 output dtype must equal the activation dtype");
    } else if (w == HQ_DT_FP4_E2M1 && (a == HQ_DT_FP8_E4M3 || a == HQ_DT_FP4_E2M1) && d->a_scale == HQ_ASCALE_MX_E8M0) {
        I.kind = Kind::MXA_MX;
        I.a_fp4 = a == HQ_DT_FP4_E2M1;
        if (d->num_experts) return set_error(HQ_ERR_UNSUPPORTED, "MX activations are built for dense layers");
        if (d->w_scale_dtype != HQ_DT_E8M0 || d->w_scale_gran != HQ_GRAN_PER_GROUP_K || d->group_size != 32)
            return set_error(HQ_ERR_UNSUPPORTED, "MXFP4 needs E8M0 scales per 32 K elements");
        if (d->K % 128) return set_error(HQ_ERR_UNSUPPORTED, "MXFP4 needs K %% 128 == 0 (K=%lld)", (long long)d->K);
        if (d->zp_dtype != HQ_DT_NONE) return set_error(HQ_ERR_UNSUPPORTED, "MXFP4 takes no zero-points");
        if (d->out_dtype != HQ_DT_BF16) return set_error(HQ_ERR_UNSUPPORTED, "MXFP4 paths output bf16");
        I.G = 32;
    } else if (w == HQ_DT_FP4_E2M1 && (a == HQ_DT_BF16 || a == HQ_DT_FP16) && !d->num_experts) {
        I.kind = Kind::FP4_A16;
        I.a_bf16 = a == HQ_DT_BF16;
        I.nv = d->w_scale_dtype == HQ_DT_FP8_E4M3;
        if (d->a_scale != HQ_ASCALE_NONE) return set_error(HQ_ERR_UNSUPPORTED, "bf16 x FP4 takes no activation scale");
        if (I.nv) {
            if (d->w_scale_gran != HQ_GRAN_PER_GROUP_K || d->group_size != 16)
                return set_error(HQ_ERR_UNSUPPORTED, "NVFP4 needs E4M3 scales per 16 K elements");
            if (d->scale2 != HQ_S2_PER_TENSOR_F32)
                return set_error(HQ_ERR_UNSUPPORTED, "NVFP4 needs a per-tensor fp32 second-level scale");
        } else if (d->w_scale_dtype != HQ_DT_E8M0 || d->w_scale_gran != HQ_GRAN_PER_GROUP_K || d->group_size != 32) {
            return set_error(HQ_ERR_UNSUPPORTED, "FP4 weights need E8M0 scales per 32 K (MXFP4) or E4M3 per 16 K (NVFP4)");
        }
        if (d->K % 128) return set_error(HQ_ERR_UNSUPPORTED, "FP4 weights need K %% 128 == 0 (K=%lld)", (long long)d->K);
        if (d->zp_dtype != HQ_DT_NONE) return set_error(HQ_ERR_UNSUPPORTED, "FP4 weights take no zero-points");
        if (d->out_dtype != a) return set_error(HQ_ERR_UNSUPPORTED, "FP4 weight-only outputs the activation dtype");
        I.G = I.nv ? 16 : 32;
    } else if (w == HQ_DT_FP4_E2M1 && (a == HQ_DT_FP8_E4M3 || a == HQ_DT_BF16)) {
        const bool moe = d->num_experts > 0;
        if (a == HQ_DT_FP8_E4M3) {
            if (moe) return set_error(HQ_ERR_UNSUPPORTED, "W4A8-MXFP4 MoE is not built");
            I.kind = Kind::W4A8_MX;
            if (d->a_scale != HQ_ASCALE_PER_TOKEN_F32) return set_error(HQ_ERR_UNSUPPORTED, "W4A8 needs per-token fp32 activation scales");
        } else {
            if (!moe) return set_error(HQ_ERR_UNSUPPORTED, "bf16 x MXFP4 is built for MoE layers only");
            I.kind = Kind::MOE_MX_BF16;
            if (d->a_scale != HQ_ASCALE_NONE) return set_error(HQ_ERR_UNSUPPORTED, "bf16 MoE takes no activation scale");
        }
        if (d->w_scale_dtype != HQ_DT_E8M0 || d->w_scale_gran != HQ_GRAN_PER_GROUP_K || d->group_size != 32)
            return set_error(HQ_ERR_UNSUPPORTED, "MXFP4 needs E8M0 scales per 32 K elements");
        if (d->K % 128) return set_error(HQ_ERR_UNSUPPORTED, "MXFP4 needs K %% 128 == 0 (K=%lld)", (long long)d->K);
        if (d->zp_dtype != HQ_DT_NONE) return set_error(HQ_ERR_UNSUPPORTED, "MXFP4 takes no zero-points");
        if (d->out_dtype != HQ_DT_BF16) return set_error(HQ_ERR_UNSUPPORTED, "MXFP4 paths output bf16");
        I.G = 32;
    } else if (a == HQ_DT_FP8_E4M3 && w == HQ_DT_FP8_E4M3) {
        I.kind = Kind::FP8_BLOCK;
        if (d->num_experts) return set_error(HQ_ERR_UNSUPPORTED, "blockwise FP8 is built for dense layers");
        if (d->a_scale != HQ_ASCALE_PER_BLOCK128_F32)
            return set_error(HQ_ERR_UNSUPPORTED, "FP8 W8A8 needs fp32 activation scales per 128-K block");
        if (d->w_scale_dtype != HQ_DT_FP32 || d->w_scale_gran != HQ_GRAN_BLOCK_128x128)
            return set_error(HQ_ERR_UNSUPPORTED, "FP8 W8A8 needs fp32 weight scales per 128 x 128 block");
        if (d->zp_dtype != HQ_DT_NONE) return set_error(HQ_ERR_UNSUPPORTED, "FP8 W8A8 takes no zero-points");
        if (d->K % 128) return set_error(HQ_ERR_UNSUPPORTED, "FP8 W8A8 needs K %% 128 == 0 (K=%lld)", (long long)d->K);
        if (d->out_dtype != HQ_DT_BF16) return set_error(HQ_ERR_UNSUPPORTED, "FP8 W8A8 outputs bf16");
        I.G = 128;
    } else if (a == HQ_DT_INT8 && w == HQ_DT_INT8) {
        I.kind = Kind::W8A8;
        if (d->num_experts) return set_error(HQ_ERR_UNSUPPORTED, "W8A8 is dense-only");
        if (d->a_scale != HQ_ASCALE_PER_TOKEN_F32) return set_error(HQ_ERR_UNSUPPORTED, "W8A8 needs per-token fp32 activation scales");
        if (d->w_scale_dtype != HQ_DT_FP32 || d->w_scale_gran != HQ_GRAN_PER_CHANNEL)
            return set_error(HQ_ERR_UNSUPPORTED, "W8A8 needs fp32 per-channel weight scales");
        if (d->zp_dtype != HQ_DT_NONE) return set_error(HQ_ERR_UNSUPPORTED, "W8A8 takes no zero-points");
        if (d->K % 128) return set_error(HQ_ERR_UNSUPPORTED, "W8A8 needs K %% 128 == 0 (K=%lld)", (long long)d->K);
        if (d->out_dtype != HQ_DT_BF16 && d->out_dtype != HQ_DT_INT32)
            return set_error(HQ_ERR_UNSUPPORTED, "W8A8 outputs bf16 or raw int32");
        I.out_i32 = d->out_dtype == HQ_DT_INT32;
        I.G = d->K;
    } else if ((a == HQ_DT_BF16 || a == HQ_DT_FP16) &&
               (w == HQ_DT_FP6_E2M3 || w == HQ_DT_FP6_E3M2 || (w == HQ_DT_FP8_E4M3 && d->w_scale_dtype == HQ_DT_E8M0))) {
        // MX float weights: E4M3 (MXFP8) or E2M3 / E3M2 (MXFP6) codes with one
        // E8M0 scale per 32 K, converted to bf16 operands with the scale (exact)
        I.kind = Kind::FP4_A16;
        I.mxf = w == HQ_DT_FP8_E4M3 ? 1 : w == HQ_DT_FP6_E2M3 ? 2 : 3;
        I.a_bf16 = a == HQ_DT_BF16;
        if (d->num_experts) return set_error(HQ_ERR_UNSUPPORTED, "MX float weights are dense-only");
        if (d->w_scale_dtype != HQ_DT_E8M0 || d->w_scale_gran != HQ_GRAN_PER_GROUP_K || d->group_size != 32)
            return set_error(HQ_ERR_UNSUPPORTED, "MXFP8 / MXFP6 weights need E8M0 scales per 32 K elements");
        if (d->a_scale != HQ_ASCALE_NONE) return set_error(HQ_ERR_UNSUPPORTED, "MX float weight-only takes no activation scale");
        if (d->K % 128) return set_error(HQ_ERR_UNSUPPORTED, "MX float weights need K %% 128 == 0 (K=%lld)", (long long)d->K);
        if (d->zp_dtype != HQ_DT_NONE) return set_error(HQ_ERR_UNSUPPORTED, "MX float weights take no zero-points");
        if (d->out_dtype != a) return set_error(HQ_ERR_UNSUPPORTED, "MX float weight-only outputs the activation dtype");
        I.G = 32;
    } else if ((a == HQ_DT_BF16 || a == HQ_DT_FP16) && (w == HQ_DT_INT8 || w == HQ_DT_FP8_E4M3 || w == HQ_DT_E0M7)) {
        // (e0m7: sign and magnitude, converted at repack to INT8 -127..127)
        I.kind = Kind::W8A16;
        I.e0m = e0m_width(w);
        I.a_bf16 = a == HQ_DT_BF16;
        I.w_fp8 = w == HQ_DT_FP8_E4M3;
        if (d->num_experts) return set_error(HQ_ERR_UNSUPPORTED, "INT8 weight-only is dense-only");
        if (d->a_scale != HQ_ASCALE_NONE) return set_error(HQ_ERR_UNSUPPORTED, "INT8 weight-only takes no activation scale");
        if (d->w_scale_dtype != HQ_DT_FP32 || d->w_scale_gran != HQ_GRAN_PER_CHANNEL)
            return set_error(HQ_ERR_UNSUPPORTED, "INT8 weight-only needs fp32 per-channel weight scales");
        if (d->zp_dtype != HQ_DT_NONE) return set_error(HQ_ERR_UNSUPPORTED, "INT8 weight-only takes no zero-points");
        if (d->K % 128) return set_error(HQ_ERR_UNSUPPORTED, "INT8 weight-only needs K %% 128 == 0 (K=%lld)", (long long)d->K);
        if (d->out_dtype != a)
            return set_error(HQ_ERR_UNSUPPORTED, "INT8 weight-only output dtype must equal the activation dtype");
        I.G = d->K;
    } else {
        return set_error(HQ_ERR_UNSUPPORTED, "unsupported activation/weight dtype pair (%d, %d)", a, w);
    }
    if (d->scale2 != HQ_S2_NONE && !(I.kind == Kind::FP4_A16 && I.nv))
        return set_error(HQ_ERR_UNSUPPORTED, "second-level scales are built for NVFP4 weights only");
    {
        // the kernels address one expert's packed tensors with 32-bit buffer offsets
        LayerInfo one = I;
        one.E = 1;
        size_t wb, sb, zb, s2b;
        packed_sizes(one, &wb, &sb, &zb, &s2b);
        if (wb >= ((size_t)1 << 32) || sb >= ((size_t)1 << 32))
            return set_error(HQ_ERR_UNSUPPORTED, "one expert's packed weights or scales reach 4 GiB (N=%lld K=%lld)",
                             (long long)d->N, (long long)d->K);
    }
    *L = I;
    return HQ_OK;
}

static hq_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    if (e == hipErrorNotSupported)
        return set_error(HQ_ERR_UNSUPPORTED, "%s: the tuning override does not apply to this layer and M", what);
    return set_error(HQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

hipError_t fp4_a16_launch(const DenseArgs& a, int kind, bool bf16) {
    if (kind >= 3) return bf16 ? mxfw_launch_bf16(a, kind) : mxfw_launch_f16(a, kind);
    return bf16 ? fp4w_launch_bf16(a, kind) : fp4w_launch_f16(a, kind);
}

static hq_status dense_launch(const LayerInfo& L, const DenseArgs& a) {
    switch (L.kind) {
        case Kind::WNA16: return hip_status(wna16_launch(a, L.a_bf16, L.zp), "hq_gemm(W4A16)");
        case Kind::W4A8_MX: return hip_status(w4a8_launch(a), "hq_gemm(W4A8-MXFP4)");
        case Kind::W8A8: return hip_status(w8a8_launch(a, L.out_i32), "hq_gemm(W8A8)");
        case Kind::W8A16:
            return hip_status(w8a16_launch(a, L.a_bf16, L.w_fp8), L.w_fp8 ? "hq_gemm(FP8-weight-only)" : "hq_gemm(W8A16)");
        case Kind::MXA_MX: return hip_status(mx_act_launch(a, L.a_fp4), L.a_fp4 ? "hq_gemm(W4A4-MXFP4)" : "hq_gemm(W4A8-MXFP8xMXFP4)");
        case Kind::FP8_BLOCK: return hip_status(fp8_block_launch(a), "hq_gemm(FP8-blockwise)");
        case Kind::FP4_A16:
            return hip_status(fp4_a16_launch(a, L.nv ? 1 : L.i4 ? 2 : L.mxf ? 2 + L.mxf : 0, L.a_bf16),
                              L.nv ? "hq_gemm(NVFP4-A16)" : L.i4 ? "hq_gemm(MXINT4-A16)"
                              : L.mxf == 1 ? "hq_gemm(MXFP8-A16)" : L.mxf ? "hq_gemm(MXFP6-A16)" : "hq_gemm(MXFP4-A16)");
        default: return set_error(HQ_ERR_UNSUPPORTED, "this layer kind runs through hq_moe_gemm");
    }
}

// Runs the dense dispatch in planning mode (no HIP call): fills buf (if any)
// with the launches and returns the workspace they need in *ws.
static hq_status dense_plan(const LayerInfo& L, int64_t M, char* buf, size_t len, size_t* ws) {
    PlanRecorder rec{buf, len, 0, 0, 0};
    if (buf) buf[0] = 0;
    if (M == 0) {
        *ws = 0;
        return HQ_OK;
    }
    g_plan = &rec;
    DenseArgs a{};  // shapes only: the planning run touches no pointer
    a.M = M;
    a.N = L.N;
    a.K = L.K;
    a.Np = L.Np;
    a.group_size = (int)L.G;
    a.invariant = L.invariant;
    a.tune_path = L.tune_path;
    a.tune_splits = L.tune_splits;
    a.wbits = L.bits;
    const hq_status st = dense_launch(L, a);
    g_plan = nullptr;
    if (buf) buf[rec.used < len ? rec.used : len - 1] = 0;
    *ws = rec.ws;
    return st;
}

static size_t dense_workspace(const LayerInfo& L, int64_t M) {
    size_t ws = 0;
    return dense_plan(L, M, nullptr, 0, &ws) == HQ_OK ? ws : 0;
}

// ---- scratch memory of the no-allocation entry point ----
// One array in every device's copy of the code object, used by
// hq_gemm_noalloc in place of a caller's workspace.  In host code the array's
// name is only a stand-in: its device address is looked up once per device
// (with that device current) and kept in scratch_dev[].
static __device__ __align__(256) char scratch[HQ_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> scratch_dev[kMaxDevices];
std::mutex scratch_mu;
}  // namespace

// Device address of `scratch` on the device that runs `stream`.
static hq_status scratch_for_stream(hipStream_t stream, void** out) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return set_error(HQ_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    int dev = cur;
    if (stream) {
        hipDevice_t d = 0;
        e = hipStreamGetDevice(stream, &d);
        if (e != hipSuccess) return set_error(HQ_ERR_HIP, "hipStreamGetDevice: %s", hipGetErrorString(e));
        dev = (int)d;
    }
    if (dev < 0 || dev >= kMaxDevices) return set_error(HQ_ERR_UNSUPPORTED, "device %d beyond the scratch table", dev);
    void* p = scratch_dev[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lk(scratch_mu);
        p = scratch_dev[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess)
                return set_error(HQ_ERR_HIP, "hipSetDevice(%d): %s", dev, hipGetErrorString(e));
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (dev != cur) {
                const hipError_t e2 = hipSetDevice(cur);
                if (e == hipSuccess) e = e2;
            }
            if (e != hipSuccess || !p)
                return set_error(HQ_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
            scratch_dev[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return HQ_OK;
}

}  // namespace hq

using namespace hq;

extern "C" {

int32_t hq_abi_version(void) { return HQ_ABI_VERSION; }

const char* hq_status_str(hq_status s) {
    switch (s) {
        case HQ_OK: return "HQ_OK";
        case HQ_ERR_INVALID_ARG: return "HQ_ERR_INVALID_ARG";
        case HQ_ERR_UNSUPPORTED: return "HQ_ERR_UNSUPPORTED";
        case HQ_ERR_ALIGNMENT: return "HQ_ERR_ALIGNMENT";
        case HQ_ERR_WORKSPACE: return "HQ_ERR_WORKSPACE";
        case HQ_ERR_ABI: return "HQ_ERR_ABI";
        case HQ_ERR_HIP: return "HQ_ERR_HIP";
    }
    return "HQ_ERR_UNKNOWN";
}

const char* hq_last_error(void) { return g_err; }

hq_status hq_desc_validate(const hq_layer_desc* desc) {
    LayerInfo L;
    hq_status st = describe(desc, &L);
    return st == HQ_OK ? ok() : st;
}

hq_status hq_repacked_bytes(const hq_layer_desc* desc, size_t* w, size_t* s, size_t* z, size_t* s2) {
    LayerInfo L;
    hq_status st = describe(desc, &L);
    if (st != HQ_OK) return st;
    if (!w || !s || !z || !s2) return set_error(HQ_ERR_INVALID_ARG, "size outputs must be non-NULL");
    packed_sizes(L, w, s, z, s2);
    return ok();
}

hq_status hq_repack(const hq_layer_desc* desc, const void* w, const void* scale, const void* zp,
                    const void* scale2, void* w_out, void* s_out, void* z_out, void* s2_out) {
    LayerInfo L;
    hq_status st = describe(desc, &L);
    if (st != HQ_OK) return st;
    if (!w || !scale || !w_out || !s_out) return set_error(HQ_ERR_INVALID_ARG, "weights and scales are required");
    const bool need_z = L.kind == Kind::WNA16 && L.zp;
    if (need_z && (!zp || !z_out)) return set_error(HQ_ERR_INVALID_ARG, "zero-points are required for UINT4 weights");
    if (!need_z && (zp || z_out)) return set_error(HQ_ERR_INVALID_ARG, "zero-point buffers must be NULL for this format");
    const bool need_s2 = desc->scale2 != HQ_S2_NONE;
    if (need_s2 && (!scale2 || !s2_out)) return set_error(HQ_ERR_INVALID_ARG, "second-level scale buffers are required");
    if (!need_s2 && (scale2 || s2_out)) return set_error(HQ_ERR_INVALID_ARG, "second-level scale buffers must be NULL");
    if (L.kind == Kind::FP4_A16 && L.mxf >= 2) {
        // FP6 codes, one per byte: the low six bits
        const uint8_t* c = (const uint8_t*)w;
        for (int64_t i = 0; i < L.K * L.N; ++i)
            if (c[i] & 0xC0u)
                return set_error(HQ_ERR_INVALID_ARG, "FP6 code 0x%02x at k=%lld n=%lld has bits above bit 5", c[i],
                                 (long long)(i / L.N), (long long)(i % L.N));
    }
    if (L.e0m && L.e0m != 3 && L.e0m != 7) {
        // e0m1 / e0m2 / e0m4..e0m6 codes, one per byte: the sign bit n and n magnitude bits
        const uint8_t* c = (const uint8_t*)w;
        for (int64_t i = 0; i < L.K * L.N; ++i)
            if (c[i] >> (L.e0m + 1))
                return set_error(HQ_ERR_INVALID_ARG, "e0m%d code 0x%02x at k=%lld n=%lld has bits above bit %d", L.e0m,
                                 c[i], (long long)(i / L.N), (long long)(i % L.N), L.e0m);
    } else if (L.kind == Kind::WNA16 && L.bits > 4 && L.bits < 8) {
        // 5-7-bit codes, one per byte: each must lie inside its width
        const int lo = L.zp8 ? 0 : -(1 << (L.bits - 1)), hi = L.zp8 ? (1 << L.bits) - 1 : (1 << (L.bits - 1)) - 1;
        const int8_t* c = (const int8_t*)w;
        for (int64_t i = 0; i < L.K * L.N; ++i) {
            const int v = L.zp8 ? (int)(uint8_t)c[i] : (int)c[i];
            if (v < lo || v > hi)
                return set_error(HQ_ERR_INVALID_ARG, "code %d at k=%lld n=%lld outside the %d-bit width", v,
                                 (long long)(i / L.N), (long long)(i % L.N), L.bits);
        }
        if (L.zp8) {
            // UINT8 zero-points [K/G][N]: inside the codes' width too
            const uint8_t* z = (const uint8_t*)zp;
            if (!z) return set_error(HQ_ERR_INVALID_ARG, "zero-points required");
            for (int64_t i = 0; i < (L.K / L.G) * L.N; ++i)
                if (z[i] >> L.bits)
                    return set_error(HQ_ERR_INVALID_ARG, "zero-point %d at group %lld n=%lld outside the %d-bit width",
                                     (int)z[i], (long long)(i / L.N), (long long)(i % L.N), L.bits);
        }
    } else if (L.kind == Kind::WNA16 && L.bits < 4) {
        // low-bit codes, one per byte: each must lie inside its width
        const int lo = L.zp ? 0 : -(1 << (L.bits - 1)), hi = L.zp ? (1 << L.bits) - 1 : (1 << (L.bits - 1)) - 1;
        const int8_t* c = (const int8_t*)w;
        for (int64_t i = 0; i < L.K * L.N; ++i) {
            const int v = L.zp ? (int)(uint8_t)c[i] : (int)c[i];
            if (v < lo || v > hi)
                return set_error(HQ_ERR_INVALID_ARG, "code %d at k=%lld n=%lld outside the %d-bit width", v,
                                 (long long)(i / L.N), (long long)(i % L.N), L.bits);
        }
    }
    repack_all(L, w, scale, zp, scale2, w_out, s_out, z_out, s2_out);
    return ok();
}

hq_status hq_workspace_bytes(const hq_layer_desc* desc, int64_t M_or_T, int32_t top_k, size_t* bytes) {
    LayerInfo L;
    hq_status st = describe(desc, &L);
    if (st != HQ_OK) return st;
    if (!bytes) return set_error(HQ_ERR_INVALID_ARG, "bytes is NULL");
    if (M_or_T < 0 || M_or_T > (1LL << 30)) return set_error(HQ_ERR_INVALID_ARG, "M/T out of range");
    if (desc->num_experts) {
        if (top_k < 1 || top_k > desc->num_experts) return set_error(HQ_ERR_INVALID_ARG, "top_k out of range");
        *bytes = moe_layout(M_or_T, top_k, desc->num_experts, true).bytes;  // Indexed needs the most
    } else {
        *bytes = dense_workspace(L, M_or_T);
    }
    return ok();
}

hq_status hq_workspace_init(void* workspace, size_t bytes, hq_stream_t stream) {
    if (!bytes) return ok();
    if (!workspace) return set_error(HQ_ERR_INVALID_ARG, "workspace is NULL");
    if (!aligned16(workspace) || bytes % 16) return set_error(HQ_ERR_ALIGNMENT, "workspace must be 16-byte aligned and sized");
    return hip_status(fill_zero_launch(workspace, bytes, (hipStream_t)stream), "hq_workspace_init");
}

hq_status hq_gemm(const hq_layer_desc* desc, int64_t M, const void* A, const void* a_scale,
                  const void* w, const void* s, const void* z, const void* s2, void* D,
                  void* workspace, size_t ws_bytes, hq_stream_t stream) {
    LayerInfo L;
    hq_status st = describe(desc, &L);
    if (st != HQ_OK) return st;
    if (desc->num_experts) return set_error(HQ_ERR_INVALID_ARG, "hq_gemm takes a dense descriptor (num_experts == 0)");
    if (M < 0 || M > (1LL << 30)) return set_error(HQ_ERR_INVALID_ARG, "M=%lld out of range", (long long)M);
    if (M == 0) return ok();
    if (!A || !w || !s || !D) return set_error(HQ_ERR_INVALID_ARG, "A, w, s and D are required");
    const bool need_z = L.kind == Kind::WNA16 && L.zp;
    if (need_z != (z != nullptr)) return set_error(HQ_ERR_INVALID_ARG, need_z ? "zero-points required" : "z must be NULL");
    const bool need_as = desc->a_scale != HQ_ASCALE_NONE;
    if (need_as != (a_scale != nullptr)) return set_error(HQ_ERR_INVALID_ARG, need_as ? "a_scale required" : "a_scale must be NULL");
    const bool need_s2 = desc->scale2 != HQ_S2_NONE;
    if (need_s2 != (s2 != nullptr)) return set_error(HQ_ERR_INVALID_ARG, need_s2 ? "s2 required" : "s2 must be NULL");
    if (s2 && ((uintptr_t)s2 & 3u)) return set_error(HQ_ERR_ALIGNMENT, "s2 must be 4-byte aligned");
    if (!aligned16(A) || !aligned16(w) || !aligned16(s) || !aligned16(D) || (z && !aligned16(z)) ||
        (a_scale && !aligned16(a_scale)))
        return set_error(HQ_ERR_ALIGNMENT, "device pointers must be 16-byte aligned");
    const int64_t ab = desc->a_dtype == HQ_DT_BF16 || desc->a_dtype == HQ_DT_FP16 ? 2 : 1;  // fp4: bounded by 1
    if (M * L.K * ab >= (int64_t)1 << 32 || M * L.N >= (int64_t)1 << 31)
        return set_error(HQ_ERR_UNSUPPORTED, "M*K activation bytes must stay below 4 GiB and M*N below 2^31");
    const size_t need = dense_workspace(L, M);
    if (need) {
        if (!workspace || ws_bytes < need)
            return set_error(HQ_ERR_WORKSPACE, "workspace of %zu bytes required, %zu given", need, workspace ? ws_bytes : (size_t)0);
        if (!aligned16(workspace)) return set_error(HQ_ERR_ALIGNMENT, "workspace must be 16-byte aligned");
    }
    const bool mx = desc->a_scale == HQ_ASCALE_MX_E8M0, blk = desc->a_scale == HQ_ASCALE_PER_BLOCK128_F32;
    DenseArgs a{M, L.N, L.K, L.Np, (int)L.G, A, mx || blk ? nullptr : (const float*)a_scale,
                mx ? (const uint8_t*)a_scale : nullptr, blk ? (const float*)a_scale : nullptr,
                w, s, z, (const float*)s2, D, workspace, ws_bytes, (hipStream_t)stream,
                L.invariant, L.tune_path, L.tune_splits, L.bits};
    return dense_launch(L, a);
}

hq_status hq_gemm_noalloc(const hq_layer_desc* desc, int64_t M, const void* A, const void* a_scale,
                          const void* w, const void* s, const void* z, const void* s2, void* D, hq_stream_t stream) {
    LayerInfo L;
    hq_status st = describe(desc, &L);
    if (st != HQ_OK) return st;
    if (desc->num_experts) return set_error(HQ_ERR_INVALID_ARG, "hq_gemm_noalloc takes a dense descriptor (num_experts == 0)");
    if (M < 0 || M > (1LL << 30)) return set_error(HQ_ERR_INVALID_ARG, "M=%lld out of range", (long long)M);
    if (M == 0) return ok();
    const size_t need = dense_workspace(L, M);
    if (need > HQ_NOALLOC_SCRATCH_BYTES)
        return set_error(HQ_ERR_WORKSPACE, "this call needs %zu bytes of scratch; hq_gemm_noalloc holds %zu (use hq_gemm "
                         "with a workspace)", need, (size_t)HQ_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    if (need) {
        st = scratch_for_stream((hipStream_t)stream, &ws);
        if (st != HQ_OK) return st;
    }
    return hq_gemm(desc, M, A, a_scale, w, s, z, s2, D, ws, need ? (size_t)HQ_NOALLOC_SCRATCH_BYTES : 0, stream);
}

hq_status hq_gemm_plan(const hq_layer_desc* desc, int64_t M, char* buf, size_t len) {
    LayerInfo L;
    hq_status st = describe(desc, &L);
    if (st != HQ_OK) return st;
    if (desc->num_experts) return set_error(HQ_ERR_INVALID_ARG, "hq_gemm_plan takes a dense descriptor (num_experts == 0)");
    if (M < 0 || M > (1LL << 30)) return set_error(HQ_ERR_INVALID_ARG, "M=%lld out of range", (long long)M);
    if (!buf || len < 2) return set_error(HQ_ERR_INVALID_ARG, "buf must hold at least 2 bytes");
    size_t ws = 0;
    st = dense_plan(L, M, buf, len, &ws);
    return st == HQ_OK ? ok() : st;
}

hq_status hq_moe_gemm(const hq_layer_desc* desc, int32_t mode, int64_t T, int32_t top_k, const void* A,
                      const float* a_scale, const int32_t* topk_ids, const int32_t* expert_offsets,
                      const void* w, const void* s, const void* z, const void* s2, void* D,
                      void* workspace, size_t ws_bytes, hq_stream_t stream) {
    LayerInfo L;
    hq_status st = describe(desc, &L);
    if (st != HQ_OK) return st;
    if (!desc->num_experts || L.kind != Kind::MOE_MX_BF16)
        return set_error(HQ_ERR_INVALID_ARG, "hq_moe_gemm takes a MoE descriptor (num_experts > 0)");
    if (mode != HQ_MOE_INDEXED && mode != HQ_MOE_GROUPED) return set_error(HQ_ERR_INVALID_ARG, "bad MoE mode %d", mode);
    if (T < 0 || T > (1LL << 24)) return set_error(HQ_ERR_INVALID_ARG, "T=%lld out of range", (long long)T);
    if (top_k < 1 || top_k > desc->num_experts) return set_error(HQ_ERR_INVALID_ARG, "top_k=%d out of range", top_k);
    if (T == 0) return ok();
    const bool indexed = mode == HQ_MOE_INDEXED;
    if (!A || !w || !s || !D) return set_error(HQ_ERR_INVALID_ARG, "A, w, s and D are required");
    if (a_scale || z || s2) return set_error(HQ_ERR_INVALID_ARG, "a_scale, z and s2 must be NULL for this format");
    if (indexed && (!topk_ids || expert_offsets))
        return set_error(HQ_ERR_INVALID_ARG, "INDEXED takes topk_ids and no expert_offsets");
    if (!indexed && (topk_ids || !expert_offsets))
        return set_error(HQ_ERR_INVALID_ARG, "GROUPED takes expert_offsets and no topk_ids");
    const int64_t P = T * top_k;
    const int64_t arows = indexed ? T : P;
    if (arows * L.K * 2 >= (int64_t)1 << 32 || P * L.N >= (int64_t)1 << 31)
        return set_error(HQ_ERR_UNSUPPORTED, "activation bytes must stay below 4 GiB and rows*N below 2^31");
    if (!aligned16(A) || !aligned16(w) || !aligned16(s) || !aligned16(D) || (topk_ids && !aligned16(topk_ids)) ||
        (expert_offsets && !aligned16(expert_offsets)))
        return set_error(HQ_ERR_ALIGNMENT, "device pointers must be 16-byte aligned");
    const MoeLayout lay = moe_layout(T, top_k, desc->num_experts, indexed);
    if (!workspace || ws_bytes < lay.bytes)
        return set_error(HQ_ERR_WORKSPACE, "workspace of %zu bytes required, %zu given", lay.bytes,
                         workspace ? ws_bytes : (size_t)0);
    if (!aligned16(workspace)) return set_error(HQ_ERR_ALIGNMENT, "workspace must be 16-byte aligned");
    size_t wb, sb, zb, s2b;
    LayerInfo one = L;
    one.E = 1;
    packed_sizes(one, &wb, &sb, &zb, &s2b);
    MoeArgs a{};
    a.T = T;
    a.N = L.N;
    a.K = L.K;
    a.Np = L.Np;
    a.top_k = top_k;
    a.E = desc->num_experts;
    a.indexed = indexed;
    a.A = A;
    a.topk_ids = topk_ids;
    a.expert_offsets = expert_offsets;
    a.w = w;
    a.s = s;
    a.D = D;
    a.w_estride = (int64_t)wb;
    a.s_estride = (int64_t)sb;
    a.ws = workspace;
    a.stream = (hipStream_t)stream;
    return hip_status(moe_gemm_launch(a), indexed ? "hq_moe_gemm(INDEXED)" : "hq_moe_gemm(GROUPED)");
}

hq_status hq_quantize_act(int32_t out_dtype, int64_t M, int64_t K, const float* x, void* q, float* s,
                          hq_stream_t stream) {
    if (out_dtype != HQ_DT_FP8_E4M3) return set_error(HQ_ERR_UNSUPPORTED, "only FP8_E4M3 activation codes are built");
    if (M < 0 || K < 1 || M > (1LL << 30) || K > (1LL << 24)) return set_error(HQ_ERR_INVALID_ARG, "M/K out of range");
    if (M == 0) return ok();
    if (!x || !q || !s) return set_error(HQ_ERR_INVALID_ARG, "x, q and s are required");
    if (!aligned16(x) || !aligned16(q) || !aligned16(s)) return set_error(HQ_ERR_ALIGNMENT, "pointers must be 16-byte aligned");
    return hip_status(quant_e4m3_launch(M, K, x, (uint8_t*)q, s, (hipStream_t)stream), "hq_quantize_act");
}

hq_status hq_quantize_act_mx(int32_t out_dtype, int64_t M, int64_t K, const float* x, void* q, void* e,
                             hq_stream_t stream) {
    if (out_dtype != HQ_DT_FP8_E4M3 && out_dtype != HQ_DT_FP4_E2M1)
        return set_error(HQ_ERR_UNSUPPORTED, "MX activation codes are FP8_E4M3 or FP4_E2M1");
    if (M < 0 || K < 32 || M > (1LL << 30) || K > (1LL << 24) || K % 32)
        return set_error(HQ_ERR_INVALID_ARG, "M/K out of range (K a multiple of 32)");
    if (M * K >= (1LL << 34)) return set_error(HQ_ERR_UNSUPPORTED, "M*K too large");
    if (M == 0) return ok();
    if (!x || !q || !e) return set_error(HQ_ERR_INVALID_ARG, "x, q and e are required");
    if (!aligned16(x) || !aligned16(q) || !aligned16(e)) return set_error(HQ_ERR_ALIGNMENT, "pointers must be 16-byte aligned");
    return hip_status(quant_mx_launch(out_dtype == HQ_DT_FP4_E2M1, M, K, x, (uint8_t*)q, (uint8_t*)e, (hipStream_t)stream),
                      "hq_quantize_act_mx");
}

hq_status hq_quantize_act_blocks(int32_t out_dtype, int64_t M, int64_t K, int64_t block, const float* x, void* q,
                                 float* s, hq_stream_t stream) {
    if (out_dtype != HQ_DT_FP8_E4M3) return set_error(HQ_ERR_UNSUPPORTED, "only FP8_E4M3 activation codes are built");
    if (M < 0 || K < 1 || block < 1 || M > (1LL << 30) || K > (1LL << 24) || K % block)
        return set_error(HQ_ERR_INVALID_ARG, "M/K/block out of range (K a multiple of block)");
    if (M * (K / block) >= (1LL << 31)) return set_error(HQ_ERR_UNSUPPORTED, "too many blocks");
    if (M == 0) return ok();
    if (!x || !q || !s) return set_error(HQ_ERR_INVALID_ARG, "x, q and s are required");
    if (!aligned16(x) || !aligned16(q) || !aligned16(s)) return set_error(HQ_ERR_ALIGNMENT, "pointers must be 16-byte aligned");
    if ((block * 4) % 16 && K != block) return set_error(HQ_ERR_UNSUPPORTED, "block must be a multiple of 4 (or K)");
    // every block is its own row of a tokenwise problem: rows of `block` consecutive elements
    return hip_status(quant_e4m3_launch(M * (K / block), block, x, (uint8_t*)q, s, (hipStream_t)stream),
                      "hq_quantize_act_blocks");
}

hq_status hq_silu_mul(int32_t dtype, int64_t rows, int64_t I, const void* gate_up, void* out, hq_stream_t stream) {
    if (dtype != HQ_DT_BF16) return set_error(HQ_ERR_UNSUPPORTED, "only BF16 rows are built");
    if (rows < 0 || rows > (1LL << 30) || I < 8 || I > (1LL << 24) || I % 8)
        return set_error(HQ_ERR_INVALID_ARG, "rows/I out of range (I a multiple of 8)");
    if (rows == 0) return ok();
    if (!gate_up || !out) return set_error(HQ_ERR_INVALID_ARG, "gate_up and out are required");
    if (!aligned16(gate_up) || !aligned16(out)) return set_error(HQ_ERR_ALIGNMENT, "pointers must be 16-byte aligned");
    return hip_status(silu_mul_launch(rows, I, gate_up, out, (hipStream_t)stream), "hq_silu_mul");
}

hq_status hq_probe_stream(const void* src, size_t bytes, void* sink, int32_t reps, hq_stream_t stream) {
    if (bytes == 0 || bytes % 16 || reps < 1 || reps > 1000)
        return set_error(HQ_ERR_INVALID_ARG, "bytes must be a positive multiple of 16 and reps 1..1000");
    if (!src || !sink) return set_error(HQ_ERR_INVALID_ARG, "src and sink are required");
    if (!aligned16(src) || !aligned16(sink)) return set_error(HQ_ERR_ALIGNMENT, "pointers must be 16-byte aligned");
    return hip_status(probe_stream_launch(src, bytes, sink, reps, (hipStream_t)stream), "hq_probe_stream");
}

hq_status hq_probe_mfma(int32_t dtype, int64_t workgroups, int32_t iters, void* sink, hq_stream_t stream) {
    if (dtype != HQ_DT_FP16 && dtype != HQ_DT_BF16 && dtype != HQ_DT_FP8_E4M3 && dtype != HQ_DT_FP4_E2M1 &&
        dtype != HQ_DT_INT8)
        return set_error(HQ_ERR_UNSUPPORTED, "dtype %d has no MFMA probe", dtype);
    if (workgroups < 1 || workgroups > 65536 || iters < 1 || iters > 1000000)
        return set_error(HQ_ERR_INVALID_ARG, "workgroups 1..65536 and iters 1..1000000");
    if (!sink) return set_error(HQ_ERR_INVALID_ARG, "sink is required");
    if (!aligned16(sink)) return set_error(HQ_ERR_ALIGNMENT, "sink must be 16-byte aligned");
    return hip_status(probe_mfma_launch(dtype, workgroups, iters, sink, (hipStream_t)stream), "hq_probe_mfma");
}

hq_status hq_moe_align(int64_t T, int32_t top_k, int32_t num_experts, const int32_t* topk_ids,
                       int32_t* expert_offsets, int32_t* sorted_pairs, void* workspace, size_t ws_bytes,
                       hq_stream_t stream) {
    if (num_experts < 1 || num_experts > 4096) return set_error(HQ_ERR_INVALID_ARG, "num_experts out of range");
    if (top_k < 1 || top_k > num_experts) return set_error(HQ_ERR_INVALID_ARG, "top_k out of range");
    if (T < 0 || T > (1LL << 24)) return set_error(HQ_ERR_INVALID_ARG, "T out of range");
    if (T * top_k >= (1LL << 31)) return set_error(HQ_ERR_UNSUPPORTED, "T*top_k must stay below 2^31");
    if (T == 0) return ok();
    if (!topk_ids || !expert_offsets || !sorted_pairs) return set_error(HQ_ERR_INVALID_ARG, "pointers are required");
    if (!aligned16(topk_ids) || !aligned16(expert_offsets) || !aligned16(sorted_pairs))
        return set_error(HQ_ERR_ALIGNMENT, "pointers must be 16-byte aligned");
    const size_t need = moe_align_workspace(T, top_k, num_experts);
    if (!workspace || ws_bytes < need)
        return set_error(HQ_ERR_WORKSPACE, "workspace of %zu bytes required", need);
    if (!aligned16(workspace)) return set_error(HQ_ERR_ALIGNMENT, "workspace must be 16-byte aligned");
    return hip_status(moe_align_launch(T, top_k, num_experts, topk_ids, expert_offsets, sorted_pairs, workspace,
                                       nullptr, (hipStream_t)stream),
                      "hq_moe_align");
}

hq_status hq_moe_gather(int32_t dtype, int64_t T, int32_t top_k, int64_t K, const void* A,
                        const int32_t* sorted_pairs, void* A_sorted, hq_stream_t stream) {
    int64_t eb = 0;
    switch (dtype) {
        case HQ_DT_BF16:
        case HQ_DT_FP16: eb = 2; break;
        case HQ_DT_FP8_E4M3:
        case HQ_DT_INT8: eb = 1; break;
        default: return set_error(HQ_ERR_UNSUPPORTED, "gather dtype must be BF16, FP16, FP8_E4M3 or INT8");
    }
    if (T < 0 || top_k < 1 || K < 1 || T > (1LL << 24) || K > (1LL << 24) || top_k > 4096)
        return set_error(HQ_ERR_INVALID_ARG, "sizes out of range");
    if (T * top_k >= (1LL << 31)) return set_error(HQ_ERR_UNSUPPORTED, "T*top_k must stay below 2^31");
    if (T == 0) return ok();
    if ((K * eb) % 16) return set_error(HQ_ERR_UNSUPPORTED, "row bytes must be a multiple of 16");
    if (!A || !sorted_pairs || !A_sorted) return set_error(HQ_ERR_INVALID_ARG, "pointers are required");
    if (!aligned16(A) || !aligned16(sorted_pairs) || !aligned16(A_sorted))
        return set_error(HQ_ERR_ALIGNMENT, "pointers must be 16-byte aligned");
    return hip_status(moe_gather_launch(A, sorted_pairs, T * top_k, top_k, K * eb, A_sorted, (hipStream_t)stream),
                      "hq_moe_gather");
}

}  // extern "C"
