// INT8 and FP8-E4M3 weight-only launches with 16-bit activations ("Humming
// wird angekuendigt", section "WnA16": INT8 and FP8 among the weight widths):
// exact 16-bit operands from the codes, the fp32 per-channel scale in the
// epilogue.  (e0m7 weights arrive here as INT8 codes.)
#include "dense_launch.hpp"

namespace hq {

hipError_t w8a16_launch(const DenseArgs& a, bool bf16, bool fp8) {
    if (fp8) return bf16 ? launch<Fmt::F8W_BF16>(a, 0) : launch<Fmt::F8W_F16>(a, 0);
    return bf16 ? launch<Fmt::W8A16_BF16>(a, 0) : launch<Fmt::W8A16_F16>(a, 0);
}

}  // namespace hq
