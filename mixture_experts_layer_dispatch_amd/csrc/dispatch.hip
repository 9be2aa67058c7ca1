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

// One dispatch block (T <= 256 tokens): workgroup 0 runs histogram, scan and scatter in
// one pass through LDS, the others quantise x to e4m3 (an independent job; none when xq
// is null).
__global__ __launch_bounds__(256) void dispatch_one_kernel(const int32_t *__restrict__ idx, int T, int k, int E,
                                                          int S, int32_t *__restrict__ blockcounts,
                                                          int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
                                                          int32_t *__restrict__ slot_to_row,
                                                          int32_t *__restrict__ row_to_slot, int32_t *err,
                                                          const uint16_t *__restrict__ x, long nq,
                                                          uint8_t *__restrict__ xq, float *__restrict__ xs) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    if (blockIdx.x > 0) {
        for (long gid = (long)(blockIdx.x - 1) * blockDim.x + threadIdx.x; gid < nq * 16;
             gid += (long)(gridDim.x - 1) * blockDim.x)
            quant_x_lane<false>(x, nq, xq, xs, gid);
        return;
    }
    dispatch_single_block<false>(idx, T, k, E, S, counts, offsets, slot_to_row, row_to_slot, err, lds);
}

// Histogram of one dispatch block per workgroup; workgroups past nblk quantise x.
__global__ __launch_bounds__(256) void dispatch_count_quant_kernel(const int32_t *__restrict__ idx, int T, int k,
                                                                  int E, int nblk, int32_t *__restrict__ blockcounts,
                                                                  int32_t *err, const uint16_t *__restrict__ x,
                                                                  long nq, uint8_t *__restrict__ xq,
                                                                  float *__restrict__ xs) {
    extern __shared__ unsigned long long masks[];  // [4][E]
    if ((int)blockIdx.x >= nblk) {
        const long nqg = gridDim.x - nblk;
        for (long gid = (long)(blockIdx.x - nblk) * blockDim.x + threadIdx.x; gid < nq * 16; gid += nqg * blockDim.x)
            quant_x_lane<false>(x, nq, xq, xs, gid);
        return;
    }
    count_block<false>(idx, T, k, E, blockIdx.x, masks, blockcounts, err);
}

// x, xq, xs: the activations and their e4m3 codes and block scales, quantised alongside
// (FP8 mode), or null.
hipError_t launch_dispatch(const Shape &s, const int32_t *idx, int32_t *blockcounts, int32_t *counts,
                           int32_t *offsets, int32_t *slot_to_row, int32_t *row_to_slot, int32_t *err,
                           const uint16_t *x, uint8_t *xq, float *xs, hipStream_t st) {
    if (s.T == 0) return hipSuccess;
    const int nblk = dispatch_blocks(s.T);
    const size_t lds = (size_t)4 * s.E * sizeof(unsigned long long);
    const long nq = xq ? (long)s.T * s.d / 128 : 0;
    // quantisation workgroups: 16 lanes per 128-wide block, up to 4 blocks' worth per lane
    const long qwg = nq ? (nq * 16 + 1023) / 1024 : 0;
    if (nblk == 1) {
        const size_t l1 = lds + (size_t)(s.E + 256) * 4;
        MOE_LAUNCH("dispatch", dispatch_one_kernel, dim3((unsigned)(1 + qwg)), dim3(256), l1, st, idx, s.T, s.k, s.E,
                   s.S, blockcounts, counts, offsets, slot_to_row, row_to_slot, err, x, nq, xq, xs);
        return hipGetLastError();
    }
    MOE_LAUNCH("dispatch_count", dispatch_count_quant_kernel, dim3((unsigned)(nblk + qwg)), dim3(256), lds, st, idx,
               s.T, s.k, s.E, nblk, blockcounts, err, x, nq, xq, xs);
    MOE_LAUNCH("dispatch_scan", dispatch_scan_kernel, dim3(1), dim3(256), 0, st, blockcounts, nblk, s.T, s.E, s.S,
               counts, offsets);
    MOE_LAUNCH("dispatch_scatter", dispatch_scatter_kernel, dim3(nblk), dim3(256), lds, st, idx, s.T, s.k, s.E,
               (const int32_t *)blockcounts, slot_to_row, row_to_slot);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void dispatch_scan_cap_kernel(int32_t *__restrict__ blockcounts, int nblk, int T,
                                                               int E, int S, int cap, int32_t *__restrict__ counts,
                                                               int32_t *__restrict__ dropped,
                                                               int32_t *__restrict__ offsets,
                                                               int32_t *__restrict__ dbase) {
    __shared__ int32_t sh[2048 + 256];
    dispatch_scan_cap_block(blockcounts, nblk, T, E, S, cap, counts, dropped, offsets, dbase, sh);
}

__global__ __launch_bounds__(256) void dispatch_scatter_cap_kernel(const int32_t *__restrict__ idx, int T, int k,
                                                                  int E, int cap, const int32_t *__restrict__ ranks,
                                                                  const int32_t *__restrict__ offsets,
                                                                  const int32_t *__restrict__ dbase,
                                                                  int32_t *__restrict__ slot_to_row,
                                                                  int32_t *__restrict__ row_to_slot) {
    extern __shared__ unsigned long long masks[];  // [4][E]
    scatter_cap_block(idx, T, k, E, blockIdx.x, cap, ranks, offsets, dbase, slot_to_row, row_to_slot, masks);
}

// The capacity variant: histogram (with the FP8 activations alongside), scan, scatter.
hipError_t launch_dispatch_capacity(const Shape &s, const int32_t *idx, int cap, int32_t *blockcounts,
                                    int32_t *counts, int32_t *dropped, int32_t *offsets, int32_t *dbase,
                                    int32_t *slot_to_row, int32_t *row_to_slot, int32_t *err, const uint16_t *x,
                                    uint8_t *xq, float *xs, hipStream_t st) {
    if (s.T == 0) return hipSuccess;
    const int nblk = dispatch_blocks(s.T);
    const size_t lds = (size_t)4 * s.E * sizeof(unsigned long long);
    const long nq = xq ? (long)s.T * s.d / 128 : 0;
    const long qwg = nq ? (nq * 16 + 1023) / 1024 : 0;
    MOE_LAUNCH("dispatch_count", dispatch_count_quant_kernel, dim3((unsigned)(nblk + qwg)), dim3(256), lds, st, idx,
               s.T, s.k, s.E, nblk, blockcounts, err, x, nq, xq, xs);
    MOE_LAUNCH("dispatch_scan", dispatch_scan_cap_kernel, dim3(1), dim3(256), 0, st, blockcounts, nblk, s.T, s.E, s.S,
               cap, counts, dropped, offsets, dbase);
    MOE_LAUNCH("dispatch_scatter", dispatch_scatter_cap_kernel, dim3(nblk), dim3(256), lds, st, idx, s.T, s.k, s.E,
               cap, (const int32_t *)blockcounts, (const int32_t *)offsets, (const int32_t *)dbase, slot_to_row,
               row_to_slot);
    return hipGetLastError();
}

// Aux-loss-free balancing (MoE lesson, "The load-balancing problem", the DeepSeek-V3
// scheme): bias[e] -= gamma for an expert above the mean load of the E routed experts,
// += gamma below it, unchanged on it (counts[e] * E against the total, in integers).
// One workgroup.
__global__ __launch_bounds__(256) void bias_update_kernel(const int32_t *__restrict__ counts, int E,
                                                         float *__restrict__ bias, float gamma) {
    __shared__ long long part[256];
    long long s = 0;
    for (int e = threadIdx.x; e < E; e += blockDim.x) s += counts[e];
    part[threadIdx.x] = s;
    __syncthreads();
    for (int w = 128; w >= 1; w >>= 1) {
        if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
        __syncthreads();
    }
    const long long total = part[0];
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        const long long scaled = (long long)counts[e] * E;
        if (scaled > total) bias[e] = bias[e] - gamma;
        else if (scaled < total) bias[e] = bias[e] + gamma;
    }
}

hipError_t launch_bias_update(const int32_t *counts, int E, float *bias, float gamma, hipStream_t st) {
    MOE_LAUNCH("bias_update", bias_update_kernel, dim3(1), dim3(256), 0, st, counts, E, bias, gamma);
    return hipGetLastError();
}

// Stand-alone FP8 quantiser: rows of fp32 or bf16 values, 1024 lanes per workgroup (64
// blocks of 128), a grid-stride loop beyond 2^20 workgroups.
template <bool F32>
__global__ __launch_bounds__(256) void quant_e4m3_kernel(const void *__restrict__ in, long nblocks,
                                                        uint8_t *__restrict__ q, float *__restrict__ qs) {
    const long lanes = nblocks * 16;
    for (long gid = (long)blockIdx.x * blockDim.x + threadIdx.x; gid - threadIdx.x < lanes;
         gid += (long)gridDim.x * blockDim.x) {
        if constexpr (F32) quant_f32_lane((const float *)in, nblocks, q, qs, gid);
        else quant_x_lane<false>((const uint16_t *)in, nblocks, q, qs, gid);
    }
}

hipError_t launch_quant_e4m3(const void *in, bool f32, long nblocks, uint8_t *q, float *qs, hipStream_t st) {
    if (nblocks == 0) return hipSuccess;
    const long wg = (nblocks * 16 + 255) / 256;
    const dim3 grid((unsigned)(wg < (1L << 20) ? wg : (1L << 20)));
    if (f32) MOE_LAUNCH("quant_e4m3", quant_e4m3_kernel<true>, grid, dim3(256), 0, st, in, nblocks, q, qs);
    else MOE_LAUNCH("quant_e4m3", quant_e4m3_kernel<false>, grid, dim3(256), 0, st, in, nblocks, q, qs);
    return hipGetLastError();
}

}  // namespace moe
