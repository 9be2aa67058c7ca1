// Dispatch kernels (S5-S7) and their launchers; the work items live in dispatch_dev.hpp.
#include "common.hpp"
#include "dispatch_dev.hpp"
#include "kernels.hpp"

namespace moe {

int dispatch_blocks(int T) { return (T + kDispTok - 1) / kDispTok; }

__global__ __launch_bounds__(256) void dispatch_count_kernel(const int32_t *__restrict__ idx, int T, int k, int E,
                                                            int32_t *__restrict__ blockcounts, int32_t *err) {
    extern __shared__ unsigned long long masks[];  // [4][E]
    count_block<false>(idx, T, k, E, blockIdx.x, masks, blockcounts, err);
}

__global__ __launch_bounds__(256) void dispatch_scan_kernel(int32_t *__restrict__ blockcounts, int nblk, int T,
                                                           int E, int S, int32_t *__restrict__ counts,
                                                           int32_t *__restrict__ offsets) {
    __shared__ int32_t sh[1024 + 256];
    dispatch_scan_block<false>(blockcounts, nblk, T, E, S, counts, offsets, sh);
}

__global__ __launch_bounds__(256) void dispatch_scatter_kernel(const int32_t *__restrict__ idx, int T, int k, int E,
                                                              const int32_t *__restrict__ bases,
                                                              int32_t *__restrict__ slot_to_row,
                                                              int32_t *__restrict__ row_to_slot) {
    extern __shared__ unsigned long long masks[];  // [4][E]
    scatter_block<false>(idx, T, k, E, blockIdx.x, bases, slot_to_row, row_to_slot, masks);
}

hipError_t launch_dispatch(const Shape &s, const int32_t *idx, int32_t *blockcounts, int32_t *counts,
                           int32_t *offsets, int32_t *slot_to_row, int32_t *row_to_slot, int32_t *err,
                           hipStream_t st) {
    if (s.T == 0) return hipSuccess;
    const int nblk = dispatch_blocks(s.T);
    const size_t lds = (size_t)4 * s.E * sizeof(unsigned long long);
    MOE_LAUNCH("dispatch_count", dispatch_count_kernel, dim3(nblk), dim3(256), lds, st, idx, s.T, s.k, s.E,
               blockcounts, err);
    MOE_LAUNCH("dispatch_scan", dispatch_scan_kernel, dim3(1), dim3(256), 0, st, blockcounts, nblk, s.T, s.E, s.S,
               counts, offsets);
    MOE_LAUNCH("dispatch_scatter", dispatch_scatter_kernel, dim3(nblk), dim3(256), lds, st, idx, s.T, s.k, s.E,
               (const int32_t *)blockcounts, slot_to_row, row_to_slot);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void quant_x_kernel(const uint16_t *__restrict__ x, long nblocks,
                                                     uint8_t *__restrict__ xq, float *__restrict__ xs) {
    quant_x_lane<false>(x, nblocks, xq, xs, (long)blockIdx.x * blockDim.x + threadIdx.x);
}

hipError_t launch_quant_x(const Shape &s, const uint16_t *x, uint8_t *xq, float *xs, hipStream_t st) {
    const long nblocks = (long)s.T * s.d / 128;
    if (nblocks == 0) return hipSuccess;
    const long threads = nblocks * 16;
    MOE_LAUNCH("quant_x", quant_x_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, x, nblocks, xq,
               xs);
    return hipGetLastError();
}

}  // namespace moe
