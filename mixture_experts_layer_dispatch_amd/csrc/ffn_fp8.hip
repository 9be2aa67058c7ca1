// FP8 e4m3 x MXFP4 grouped GEMMs (S8-S9 in the FP8 x FP4 mode).
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

hipError_t launch_fp8_ffn(const Shape &s, const FfnPlan &p, const uint8_t *w1, const uint8_t *w1s,
                          const uint8_t *w2, const uint8_t *w2s, const uint8_t *xq, const float *xs,
                          const int32_t *offsets, const int32_t *row_to_slot, uint8_t *h, float *hs, void *y_perm,
                          const int32_t *ts1, const int32_t *ts2, hipStream_t st) {
    return hipErrorNotSupported;
}

}  // namespace moe
