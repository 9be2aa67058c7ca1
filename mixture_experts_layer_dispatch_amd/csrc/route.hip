// Router kernels (S1-S4) and their launcher; the work items live in route_dev.hpp.
#include "common.hpp"
#include "kernels.hpp"
#include "route_dev.hpp"

namespace moe {

template <bool F32, int CH>
__global__ __launch_bounds__(256) void route_valu_kernel(const void *__restrict__ x, const void *__restrict__ wr,
                                                        const float *__restrict__ bias, int T, int d, int E, int k,
                                                        int gating, int32_t *idx, float *gate, float *logits,
                                                        float *keys, int32_t *err) {
    extern __shared__ float lds_logits[];  // [4][E]
    route_valu_block<F32, CH, false>(x, wr, bias, T, d, E, k, gating, blockIdx.x, lds_logits, idx, gate, logits, keys,
                              err);
}

__global__ __launch_bounds__(256) void route_mfma_kernel(const uint16_t *__restrict__ x,
                                                        const uint16_t *__restrict__ wr,
                                                        const float *__restrict__ bias, int T, int d, int E, int k,
                                                        int gating, int32_t *idx, float *gate, float *logits,
                                                        float *keys, int32_t *err) {
    extern __shared__ float lds_logits[];  // [32][E]
    route_mfma_block<false>(x, wr, bias, T, d, E, k, gating, blockIdx.x, lds_logits, idx, gate, logits, keys, err);
}

// one wave per (expert tile, K slice, token tile)
__global__ __launch_bounds__(64) void route_splitk_kernel(const uint16_t *__restrict__ x,
                                                         const uint16_t *__restrict__ wr, int T, int d, int E,
                                                         int nks, float *__restrict__ part) {
    route_splitk_wave<false>(x, wr, T, d, E, nks, blockIdx.x, part);
}

// one workgroup per token
__global__ __launch_bounds__(256) void route_select_kernel(const float *__restrict__ part, int nks, int T, int E,
                                                          int k, int gating, const float *__restrict__ bias,
                                                          int32_t *idx, float *gate, float *logits, float *keys,
                                                          int32_t *err) {
    extern __shared__ float lg[];  // [E]
    route_sum_select<false>(part, nks, T, E, k, gating, bias, blockIdx.x, lg, idx, gate, logits, keys, err);
}

// Router work layout: bf16 activations with E a multiple of 32 use the split-K kernel at
// every T -- one wave per (32 tokens, 32 experts, K slice), with as many K slices (whole
// multiples of 64) as keep the waves near 2048, so that even a few tokens spread W_r over
// the whole chip.  fp32 or other E: the one-pass VALU kernel.
int route_splitk_slices(const Shape &s) {
    if (s.mode == MODE_F32 || s.E % 32 != 0 || s.T == 0) return 0;
    const long tiles = (long)(s.E / 32) * ((s.T + 31) / 32);
    int best = 1;
    for (int q = 1; q <= 64; ++q)
        if (s.d % (64 * q) == 0 && tiles * q <= 2048) best = q;
    return best;
}

long route_splitk_waves(const Shape &s, int nks) { return (long)(s.E / 32) * nks * ((s.T + 31) / 32); }

hipError_t launch_route(const Shape &s, const void *x, const void *wr, const float *bias, int32_t *idx,
                        float *gate, float *logits, float *keys, int32_t *err, float *part, hipStream_t st) {
    if (s.T == 0) return hipSuccess;
    const int nks = part ? route_splitk_slices(s) : 0;
    if (nks > 0) {
        dim3 grid((unsigned)(route_splitk_waves(s, nks)));
        MOE_LAUNCH("route", route_splitk_kernel, grid, dim3(64), 0, st, (const uint16_t *)x, (const uint16_t *)wr,
                   s.T, s.d, s.E, nks, part);
        MOE_LAUNCH("route_select", route_select_kernel, dim3(s.T), dim3(256), (size_t)s.E * sizeof(float),
                   st, (const float *)part, nks, s.T, s.E, s.k, s.gating, bias, idx, gate, logits, keys, err);
        return hipGetLastError();
    }
    if (s.mode != MODE_F32 && s.E % 32 == 0) {
        dim3 grid((s.T + kRouteTok - 1) / kRouteTok);
        size_t lds = (size_t)kRouteTok * s.E * sizeof(float);
        if (lds > 65536) {
            hipError_t e = hipFuncSetAttribute((const void *)route_mfma_kernel,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return e;
        }
        MOE_LAUNCH("route", route_mfma_kernel, grid, dim3(256), lds, st, (const uint16_t *)x, (const uint16_t *)wr,
                           bias, s.T, s.d, s.E, s.k, s.gating, idx, gate, logits, keys, err);
    } else {
        dim3 grid((s.T + 3) / 4);
        size_t lds = (size_t)4 * s.E * sizeof(float);
        bool f32 = s.mode == MODE_F32;
        if (s.E <= 8) {
            if (f32)
                MOE_LAUNCH("route", (route_valu_kernel<true, 8>), grid, dim3(256), lds, st, x, wr, bias, s.T, s.d,
                                   s.E, s.k, s.gating, idx, gate, logits, keys, err);
            else
                MOE_LAUNCH("route", (route_valu_kernel<false, 8>), grid, dim3(256), lds, st, x, wr, bias, s.T, s.d,
                                   s.E, s.k, s.gating, idx, gate, logits, keys, err);
        } else {
            if (f32)
                MOE_LAUNCH("route", (route_valu_kernel<true, 32>), grid, dim3(256), lds, st, x, wr, bias, s.T, s.d,
                                   s.E, s.k, s.gating, idx, gate, logits, keys, err);
            else
                MOE_LAUNCH("route", (route_valu_kernel<false, 32>), grid, dim3(256), lds, st, x, wr, bias, s.T,
                                   s.d, s.E, s.k, s.gating, idx, gate, logits, keys, err);
        }
    }
    return hipGetLastError();
}

}  // namespace moe
