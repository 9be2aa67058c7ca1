// Combine kernel (S10) and its launcher; the work item lives in combine_dev.hpp.
#include "combine_dev.hpp"
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

template <bool F32>
__global__ __launch_bounds__(256) void combine_kernel(const void *__restrict__ yp, const int32_t *__restrict__ s2r,
                                                     const float *__restrict__ gate, void *__restrict__ y, int T,
                                                     int k, int d, int S) {
    combine_lane<F32, false>(yp, s2r, gate, y, T, k, d, S, (long)blockIdx.x * blockDim.x + threadIdx.x);
}

hipError_t launch_combine(const Shape &s, const void *y_perm, const int32_t *slot_to_row, const float *gate,
                          void *y, hipStream_t st) {
    if (s.T == 0) return hipSuccess;
    const int V = s.mode == MODE_F32 ? 4 : 8;
    const long threads = (long)s.T * (s.d / V);
    dim3 grid((unsigned)((threads + 255) / 256));
    if (s.mode == MODE_F32)
        MOE_LAUNCH("combine", combine_kernel<true>, grid, dim3(256), 0, st, y_perm, slot_to_row, gate, y, s.T, s.k,
                   s.d, s.S);
    else
        MOE_LAUNCH("combine", combine_kernel<false>, grid, dim3(256), 0, st, y_perm, slot_to_row, gate, y, s.T, s.k,
                   s.d, s.S);
    return hipGetLastError();
}

}  // namespace moe
