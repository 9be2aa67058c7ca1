// Expert FFN kernels (S8-S9) and their launchers, bf16 and fp32; the work items live in
// gemm_bf16_dev.hpp, the FP8 x FP4 ones in ffn_fp8.hip.
#include "common.hpp"
#include "dispatch_dev.hpp"
#include "gemm_bf16_dev.hpp"
#include "kernels.hpp"

namespace moe {

__global__ __launch_bounds__(256) void tile_plan_kernel(const int32_t *__restrict__ offsets, int G, int bm1,
                                                       int ntn1, int bm2, int ntn2, int32_t *__restrict__ ts1,
                                                       int32_t *__restrict__ ts2) {
    __shared__ int32_t sh[2 * 1032 + 256];
    tile_plan_block<false>(offsets, G, bm1, ntn1, bm2, ntn2, ts1, ts2, sh);
}

template <int BM, int BN, bool SWIGLU, bool GATHER>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tile = pick_tile(blockIdx.x, a.tile_start[a.G]);
    if (tile >= 0) bf16_tile<BM, BN, SWIGLU, GATHER>(a, tile, lds);
}

// xcd_cus: CUs per XCD (one workgroup per CU), for the tail split
template <bool SWIGLU, bool GATHER>
__global__ __launch_bounds__(512) void gemm_bf16_kernel8(GemmArgs a, int xcd_cus) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    int half;
    const int tile = pick_tile_split(blockIdx.x, a.tile_start[a.G], xcd_cus, half);
    if (tile >= 0) bf16_tile8<SWIGLU, GATHER>(a, tile, lds, half);
}

__global__ __launch_bounds__(256) void ffn1_f32_kernel(const float *__restrict__ x, const int32_t *__restrict__ r2s,
                                                      const float *__restrict__ w1, const int32_t *__restrict__ offsets,
                                                      int G, int T, int k, int d, int F, long rows,
                                                      float *__restrict__ h) {
    ffn1_f32_lane(x, r2s, w1, offsets, G, T, k, d, F, rows, h, (long)blockIdx.x * blockDim.x + threadIdx.x);
}

__global__ __launch_bounds__(256) void ffn2_f32_kernel(const float *__restrict__ h, const float *__restrict__ w2,
                                                      const int32_t *__restrict__ offsets, int G, int d, int F,
                                                      long rows, float *__restrict__ y) {
    ffn2_f32_lane(h, w2, offsets, G, d, F, rows, y, (long)blockIdx.x * blockDim.x + threadIdx.x);
}

// ---- launch ------------------------------------------------------------------------

FfnPlan ffn_plan(const Shape &s) {
    FfnPlan p;
    const long rows = s.rows();
    const double per_group = (double)rows / s.G();
    // weight streaming below 20 rows per group, the tiled kernels (each weight tile streamed
    // through LDS for 256 rows) from there on.  DeepSeek-V3 FP8 x FP4 layer on MI355X, weight
    // streaming against tiled: 1.1 rows per group 0.93 / 1.11 ms, 2.2 1.29 / 1.43, 3.4
    // 1.43 / 1.66, 9 1.58 / 1.80, 13.4 1.65 / 1.82, 17.9 1.71 / 1.77
    p.decode = s.mode == MODE_FP8 && per_group < 20.0 && rows * (s.d > 2 * s.F ? s.d : 2 * s.F) < (1L << 31);
    if (p.decode) {
        // One 64-lane wave per (group, 32-row tile, 32 output columns, K slice).  linear1's
        // K slices are whole 256-wide chunks, the fewest that keep a slice within 1024: the
        // unfused kernel stages a slice of each activation row in LDS, and 4-wave groups
        // of these waves then stream every weight tile with four blocks in flight.  If d is
        // no multiple of 256, one slice.
        const int chunks = s.d % 256 == 0 ? s.d / 256 : 1;
        p.ks = 1;
        if (s.d % 256 == 0)
            for (int q = 1; q <= chunks; ++q)
                if (chunks % q == 0 && s.d / q <= 1024) { p.ks = q; break; }
        p.bm1 = p.bm2 = 32;
        p.bn1 = p.bn2 = 32;
        p.ntn1 = (2 * s.F / 32) * p.ks;
        p.ntn2 = s.d / 32;
        return p;
    }
    p.ks = 1;
    if (s.mode == MODE_FP8X8) {  // the 4-wave FP8 x FP8 tiles: 128 x 256 (linear1), 128 x 256
        p.bm1 = p.bm2 = 128;     // (linear2; 128 x 128 when d is no multiple of 256)
        p.bn1 = 256;
        p.bn2 = s.d % 256 == 0 ? 256 : 128;
        p.ntn1 = s.F / 128;
        p.ntn2 = s.d / p.bn2;
        return p;
    }
    p.bm1 = p.bm2 = per_group >= 160 ? 256 : 128;
    p.bn1 = 256;
    p.bn2 = s.d % 256 == 0 ? 256 : 128;
    p.ntn1 = s.F / (p.bn1 / 2);
    p.ntn2 = s.d / p.bn2;
    return p;
}

size_t ffn_partial_bytes(const Shape &s) {
    const FfnPlan p = ffn_plan(s);
    return p.decode ? (size_t)p.ks * s.rows() * 2 * s.F * sizeof(float) : 0;
}

template <int BM, int BN, bool SWIGLU, bool GATHER>
static hipError_t launch_gemm(const char *name, dim3 grid, const GemmArgs &a, hipStream_t st) {
    constexpr size_t lds = bf16_tile_lds<BM, BN>();
    static bool attr = false;
    if (!attr) {
        hipError_t e = hipFuncSetAttribute((const void *)gemm_bf16_kernel<BM, BN, SWIGLU, GATHER>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr = true;
    }
    MOE_LAUNCH(name, (gemm_bf16_kernel<BM, BN, SWIGLU, GATHER>), grid, dim3(256), lds, st, a);
    return hipGetLastError();
}

// CUs per XCD of the current device (eight XCDs)
int xcd_cus() {
    static int cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (!cached[dev]) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cached[dev] = cus / 8 > 0 ? cus / 8 : 1;
    }
    return cached[dev];
}

// 256 x 256 tiles: the 8-wave kernel.  ub: an upper bound of the tile count; the grid adds
// the blocks of the tail split.
template <bool SWIGLU, bool GATHER>
static hipError_t launch_gemm8(const char *name, long ub, const GemmArgs &a, hipStream_t st) {
    constexpr size_t lds = bf16_tile8_lds();
    static bool attr = false;
    if (!attr) {
        hipError_t e = hipFuncSetAttribute((const void *)gemm_bf16_kernel8<SWIGLU, GATHER>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr = true;
    }
    const int C = xcd_cus();
    if (C <= 0) return hipErrorInvalidDevice;
    const dim3 grid((unsigned)(8 * ((ub + 7) / 8 + C / 2)));
    MOE_LAUNCH(name, (gemm_bf16_kernel8<SWIGLU, GATHER>), grid, dim3(512), lds, st, a, C);
    return hipGetLastError();
}

hipError_t launch_fp8_ffn(const Shape &s, const FfnPlan &p, const uint8_t *w1, const uint8_t *w1s,
                          const uint8_t *w2, const uint8_t *w2s, const uint8_t *xq, const float *xs,
                          const int32_t *offsets, const int32_t *row_to_slot, uint8_t *h, float *hs, void *y_perm,
                          const int32_t *ts1, const int32_t *ts2, float *upart, hipStream_t st);

hipError_t launch_fp8x8_ffn(const Shape &s, const FfnPlan &p, const uint8_t *w1, const float *w1s, const uint8_t *w2,
                            const float *w2s, const uint8_t *xq, const float *xs, const int32_t *offsets,
                            const int32_t *row_to_slot, uint8_t *h, float *hs, void *y_perm, const int32_t *ts1,
                            const int32_t *ts2, hipStream_t st);

hipError_t launch_ffn(const Shape &s, const FfnPlan &p, const void *w1, const void *w1s, const void *w2,
                      const void *w2s, const void *x, const uint8_t *xq, const float *xs, const int32_t *offsets,
                      const int32_t *row_to_slot, void *h, float *hs, void *y_perm, int32_t *tile_start,
                      float *upart, hipStream_t st) {
    if (s.T == 0) return hipSuccess;
    const long rows = s.rows();
    const int G = s.G();
    if (s.mode == MODE_F32) {
        long n1 = rows * s.F, n2 = rows * s.d;
        MOE_LAUNCH("linear1", ffn1_f32_kernel, dim3((unsigned)((n1 + 255) / 256)), dim3(256), 0, st, (const float *)x,
                           row_to_slot, (const float *)w1, offsets, G, s.T, s.k, s.d, s.F, rows, (float *)h);
        MOE_LAUNCH("linear2", ffn2_f32_kernel, dim3((unsigned)((n2 + 255) / 256)), dim3(256), 0, st, (const float *)h,
                           (const float *)w2, offsets, G, s.d, s.F, rows, (float *)y_perm);
        return hipGetLastError();
    }
    int32_t *ts1 = tile_start, *ts2 = tile_start + (G + 1);
    const int ntn1 = p.ntn1, ntn2 = p.ntn2;
    if (!(s.mode == MODE_FP8 && fp8_gemv_ok(s, p)))
        MOE_LAUNCH("tile_plan", tile_plan_kernel, dim3(1), dim3(256), 0, st, offsets, G, p.bm1, ntn1, p.bm2, ntn2, ts1,
                   ts2);
    if (s.mode == MODE_FP8X8)
        return launch_fp8x8_ffn(s, p, (const uint8_t *)w1, (const float *)w1s, (const uint8_t *)w2, (const float *)w2s,
                                xq, xs, offsets, row_to_slot, (uint8_t *)h, hs, y_perm, ts1, ts2, st);
    if (s.mode == MODE_FP8)
        return launch_fp8_ffn(s, p, (const uint8_t *)w1, (const uint8_t *)w1s, (const uint8_t *)w2,
                              (const uint8_t *)w2s, xq, xs, offsets, row_to_slot, (uint8_t *)h, hs, y_perm, ts1, ts2,
                              upart, st);
    auto grid_for = [&](int bm, int ntn) {
        const long ub = ((rows + bm - 1) / bm + (G < rows ? G : rows)) * (long)ntn;
        return dim3((unsigned)((ub + 7) / 8 * 8));
    };
    GemmArgs a1 = {(const uint16_t *)x, row_to_slot, (const uint16_t *)w1, (uint16_t *)h, offsets, ts1,
                   s.T, s.k, s.d, 2 * s.F, s.F, G, s.F};
    GemmArgs a2 = {(const uint16_t *)h, nullptr, (const uint16_t *)w2, (uint16_t *)y_perm, offsets, ts2,
                   s.T, s.k, s.F, s.d, s.d, G, s.F};
    hipError_t e;
    auto ub_for = [&](int bm, int ntn) { return ((rows + bm - 1) / bm + (G < rows ? G : rows)) * (long)ntn; };
    if (p.bm1 == 256) e = launch_gemm8<true, true>("linear1", ub_for(p.bm1, ntn1), a1, st);
    else e = launch_gemm<128, 256, true, true>("linear1", grid_for(p.bm1, ntn1), a1, st);
    if (e != hipSuccess) return e;
    if (p.bm2 == 256 && p.bn2 == 256) e = launch_gemm8<false, false>("linear2", ub_for(p.bm2, ntn2), a2, st);
    else if (p.bn2 == 256) e = launch_gemm<128, 256, false, false>("linear2", grid_for(p.bm2, ntn2), a2, st);
    else if (p.bm2 == 256) e = launch_gemm<256, 128, false, false>("linear2", grid_for(p.bm2, ntn2), a2, st);
    else e = launch_gemm<128, 128, false, false>("linear2", grid_for(p.bm2, ntn2), a2, st);
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

}  // namespace moe
