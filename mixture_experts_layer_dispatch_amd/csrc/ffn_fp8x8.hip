// FP8 e4m3 x e4m3 FFN kernels (S8-S9 in the FP8 x FP8 expert mode) and their launcher; the
// work items live in gemm_fp8x8_dev.hpp.
#include "common.hpp"
#include "gemm_fp8x8_dev.hpp"
#include "kernels.hpp"

namespace moe {

template <bool SWIGLU, bool GATHER, int BN>
__global__ __launch_bounds__(256) void gemm_fp8x8_kernel(Fp8Args a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tile = pick_tile(blockIdx.x, a.tile_start[a.G]);
    if (tile >= 0) fp8x8_tile<SWIGLU, GATHER, BN>(a, tile, lds);
}

template <bool SWIGLU, bool GATHER, int BN>
static hipError_t launch_fp8x8(const char *name, dim3 grid, const Fp8Args &a, hipStream_t st) {
    constexpr size_t lds = fp8x8_tile_lds<BN>();
    static bool attr = false;
    if (!attr) {
        hipError_t e = hipFuncSetAttribute((const void *)gemm_fp8x8_kernel<SWIGLU, GATHER, BN>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr = true;
    }
    MOE_LAUNCH(name, (gemm_fp8x8_kernel<SWIGLU, GATHER, BN>), grid, dim3(256), lds, st, a);
    return hipGetLastError();
}

// linear1 + SwiGLU (128 x 256 tiles: 128 gate + 128 up columns), then linear2 (128 x p.bn2),
// over the tile plans ts1, ts2 of the dispatched groups.
hipError_t launch_fp8x8_ffn(const Shape &s, const FfnPlan &p, const uint8_t *w1, const float *w1s, const uint8_t *w2,
                            const float *w2s, const uint8_t *xq, const float *xs, const int32_t *offsets,
                            const int32_t *row_to_slot, uint8_t *h, float *hs, void *y_perm, const int32_t *ts1,
                            const int32_t *ts2, hipStream_t st) {
    const long rows = s.rows();
    const int G = s.G();
    auto grid_for = [&](int bm, int ntn) {
        const long ub = ((rows + bm - 1) / bm + (G < rows ? G : rows)) * (long)ntn;
        return dim3((unsigned)((ub + 7) / 8 * 8));
    };
    const Fp8Args a1 = {xq, xs, row_to_slot, w1, (const uint8_t *)w1s, h, hs, offsets, ts1, s.T, s.k, s.d, 2 * s.F,
                        s.F, G, s.F};
    const Fp8Args a2 = {h, hs, nullptr, w2, (const uint8_t *)w2s, y_perm, nullptr, offsets, ts2, s.T, s.k, s.F, s.d,
                        s.d, G, s.F};
    hipError_t e = launch_fp8x8<true, true, 256>("linear1", grid_for(p.bm1, p.ntn1), a1, st);
    if (e != hipSuccess) return e;
    if (p.bn2 == 256) return launch_fp8x8<false, false, 256>("linear2", grid_for(p.bm2, p.ntn2), a2, st);
    return launch_fp8x8<false, false, 128>("linear2", grid_for(p.bm2, p.ntn2), a2, st);
}

}  // namespace moe
