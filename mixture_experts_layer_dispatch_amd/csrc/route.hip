// Router kernels (S1-S4) and their launcher; the work items live in route_dev.hpp.
#include "common.hpp"
#include "gemm_bf16_dev.hpp"
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

// Many tokens and E a multiple of 256: the router is a plain GEMM logits = x W_r^T, run on
// the 8-wave 256 x 256 bf16 tile (W_r and x rows staged through LDS) and split along K into
// nks slices so that the tiles fill the chip.  Tile b: slice b / per, then the 256-token
// tile fastest and the 256-expert tile; the slice's fp32 partial logits go to part[ks][t][e].
__global__ __launch_bounds__(512) void route_tile_kernel(const uint16_t *__restrict__ x, const uint16_t *__restrict__ wr,
                                                        int T, int d, int E, int nks, float *__restrict__ part) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int mtn = (T + 255) / 256, per = mtn * (E / 256);
    const int b = pick_tile(blockIdx.x, per * nks);
    if (b < 0) return;
    const int ks = b / per, rem = b % per;
    TileInfo ti;
    ti.g = 0;
    ti.mt = rem % mtn;
    ti.nt = rem / mtn;
    ti.row0 = ti.mt * 256;
    ti.nrows = min(256, T - ti.row0);
    GemmArgs a = {x, nullptr, wr, (uint16_t *)(part + (long)ks * T * E), nullptr, nullptr, T, 1, d, E, E, 1, 0};
    const int kchunk = d / nks;
    bf16_tile8_rows<false, false, true>(a, ti, d, ks * kchunk, kchunk / 32, lds);
}

// one workgroup per token
__global__ __launch_bounds__(256) void route_select_kernel(const float *__restrict__ part, int nks, int T, int E,
                                                          int k, int gating, const float *__restrict__ bias,
                                                          int32_t *idx, float *gate, float *logits, float *keys,
                                                          int32_t *err) {
    extern __shared__ float lg[];  // [2][E]: logits, then the bias
    route_sum_select<false>(part, nks, T, E, k, gating, bias, blockIdx.x, lg, idx, gate, logits, keys, err);
}

// one wave per token (few K slices): tokens 4 b .. 4 b + 3
__global__ __launch_bounds__(256) void route_select_wave_kernel(const float *__restrict__ part, int nks, int T, int E,
                                                               int k, int gating, const float *__restrict__ bias,
                                                               int32_t *idx, float *gate, float *logits, float *keys,
                                                               int32_t *err) {
    extern __shared__ float lgw[];  // [4][E]
    const int wave = threadIdx.x >> 6;
    const long t = (long)blockIdx.x * 4 + wave;
    if (t < T)
        route_sum_select_wave<false>(part, nks, T, E, k, gating, bias, t, lgw + wave * E, idx, gate, logits, keys, err);
}

// Selection after the split-K router: a wave per token when the slices are few (at most 16,
// E at most 256: all of a lane's loads in flight at once), else a workgroup per token.
static hipError_t launch_route_select(const Shape &s, int nks, const float *part, const float *bias, int32_t *idx,
                                      float *gate, float *logits, float *keys, int32_t *err, hipStream_t st) {
    if (route_select_by_wave(s.E, nks))
        MOE_LAUNCH("route_select", route_select_wave_kernel, dim3((unsigned)((s.T + 3) / 4)), dim3(256),
                   (size_t)4 * s.E * sizeof(float), st, part, nks, s.T, s.E, s.k, s.gating, bias, idx, gate, logits,
                   keys, err);
    else
        MOE_LAUNCH("route_select", route_select_kernel, dim3(s.T), dim3(256), (size_t)2 * s.E * sizeof(float), st, part,
                   nks, s.T, s.E, s.k, s.gating, bias, idx, gate, logits, keys, err);
    return hipGetLastError();
}

// Router work layout: bf16 activations with E a multiple of 256 and many tokens use the
// tiled GEMM above; otherwise, with E a multiple of 32, the split-K kernel at every T -- one wave per (32 tokens, 32 experts, K slice), with as many K slices (whole
// multiples of 64) as keep the waves near 2048, so that even a few tokens spread W_r over
// the whole chip.  fp32 or other E: the one-pass VALU kernel.
// K slices of the router.  With many tokens and E a multiple of 256 (bf16) the unfused
// path runs the tiled GEMM: the fewest slices (multiples of 64 wide, at least 512) that give
// 256 tiles.  Otherwise as many slices (multiples of 64 wide) as keep the split-K waves
// near 2048.  The persistent layer kernel's split-K waves use the same slices, and one MFMA
// chain over the same K slice gives the same partial sums in either kernel, so both entry
// points produce identical logits.
static bool route_tile_eligible(const Shape &s) {
    return s.mode != MODE_F32 && s.E % 256 == 0 && s.T >= 2048 && s.d % 64 == 0;
}

int route_splitk_slices(const Shape &s) {
    if (s.mode == MODE_F32 || s.E % 32 != 0 || s.T == 0) return 0;
    int best = 1;
    if (route_tile_eligible(s)) {
        const long tiles = (long)((s.T + 255) / 256) * (s.E / 256);
        for (int q = 1; q <= 64; ++q) {
            if (s.d % (64 * q) != 0 || s.d / q < 512) continue;
            best = q;
            if (tiles * q >= 256) break;
        }
        return best;
    }
    const long tiles = (long)(s.E / 32) * ((s.T + 31) / 32);
    for (int q = 1; q <= 64; ++q)
        if (s.d % (64 * q) == 0 && tiles * q <= 2048) best = q;
    return best;
}

int route_tile_slices(const Shape &s) { return route_tile_eligible(s) ? route_splitk_slices(s) : 0; }

long route_splitk_waves(const Shape &s, int nks) { return (long)(s.E / 32) * nks * ((s.T + 31) / 32); }

hipError_t launch_route(const Shape &s, const void *x, const void *wr, const float *bias, int32_t *idx,
                        float *gate, float *logits, float *keys, int32_t *err, float *part, hipStream_t st) {
    if (s.T == 0) return hipSuccess;
    const int tks = part ? route_tile_slices(s) : 0;
    if (tks > 0) {
        static bool attr = false;
        if (!attr) {
            hipError_t e = hipFuncSetAttribute((const void *)route_tile_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)bf16_tile8_lds());
            if (e != hipSuccess) return e;
            attr = true;
        }
        const long tiles = (long)((s.T + 255) / 256) * (s.E / 256) * tks;
        MOE_LAUNCH("route", route_tile_kernel, dim3((unsigned)((tiles + 7) / 8 * 8)), dim3(512), bf16_tile8_lds(), st,
                   (const uint16_t *)x, (const uint16_t *)wr, s.T, s.d, s.E, tks, part);
        return launch_route_select(s, tks, part, bias, idx, gate, logits, keys, err, st);
    }
    const int nks = part ? route_splitk_slices(s) : 0;
    if (nks > 0) {
        dim3 grid((unsigned)(route_splitk_waves(s, nks)));
        MOE_LAUNCH("route", route_splitk_kernel, grid, dim3(64), 0, st, (const uint16_t *)x, (const uint16_t *)wr,
                   s.T, s.d, s.E, nks, part);
        return launch_route_select(s, nks, part, bias, idx, gate, logits, keys, err, st);
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
