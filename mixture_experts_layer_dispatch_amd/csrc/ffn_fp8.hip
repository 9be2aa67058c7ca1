// FP8 e4m3 x MXFP4 FFN kernels (S8-S9, S12) and their launchers; the work items live in
// gemm_fp8_dev.hpp.
#include "common.hpp"
#include "dispatch_dev.hpp"
#include "gemm_fp8_dev.hpp"
#include "kernels.hpp"

namespace moe {

template <int BM, int BN, int WM, bool SWIGLU, bool GATHER>
__global__ __launch_bounds__(256) void gemm_fp8_kernel(Fp8Args a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tile = pick_tile(blockIdx.x, a.tile_start[a.G]);
    if (tile >= 0) fp8_tile<BM, BN, WM, SWIGLU, GATHER>(a, tile, lds);
}

template <int BM, int BN, int WM, bool SWIGLU, bool GATHER>
static hipError_t launch_fp8(const char *name, dim3 grid, const Fp8Args &a, hipStream_t st) {
    constexpr size_t lds = fp8_tile_lds<BM, BN>();
    static bool attr = false;
    if (!attr) {
        hipError_t e = hipFuncSetAttribute((const void *)gemm_fp8_kernel<BM, BN, WM, SWIGLU, GATHER>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr = true;
    }
    MOE_LAUNCH(name, (gemm_fp8_kernel<BM, BN, WM, SWIGLU, GATHER>), grid, dim3(256), lds, st, a);
    return hipGetLastError();
}

// xcd_cus: CUs per XCD (one workgroup per CU), for the tail split
template <bool SWIGLU>
__global__ __launch_bounds__(512) void gemm_fp8_kernel8(Fp8Args a, int xcd_cus) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    int half;
    const int tile = pick_tile_split(blockIdx.x, a.tile_start[a.G], xcd_cus, half);
    if (tile >= 0) fp8_tile8<SWIGLU ? 1 : 2, SWIGLU ? 8 : 4, SWIGLU, SWIGLU>(a, tile, lds, half);
}

// 256 x 256 tiles: the 8-wave kernel (linear1 gathers its rows, linear2 does not).  ub: an
// upper bound of the tile count; the grid adds the blocks of the tail split.
template <bool SWIGLU>
static hipError_t launch_fp8_8(const char *name, long ub, const Fp8Args &a, hipStream_t st) {
    constexpr size_t lds = fp8_tile8_lds();
    static bool attr = false;
    if (!attr) {
        hipError_t e = hipFuncSetAttribute((const void *)gemm_fp8_kernel8<SWIGLU>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr = true;
    }
    const int C = xcd_cus();
    if (C <= 0) return hipErrorInvalidDevice;
    const dim3 grid((unsigned)(8 * ((ub + 7) / 8 + C / 2)));
    MOE_LAUNCH(name, gemm_fp8_kernel8<SWIGLU>, grid, dim3(512), lds, st, a, C);
    return hipGetLastError();
}

constexpr long kDecodeMaxWaves = 1L << 20;  // grid cap; the kernels stride over any excess tiles

// The grid is an upper bound of the tile count (non-empty groups only), so a tail round of
// a few waves after a full one never happens; excess waves exit at once.
template <bool LIN1>
__global__ __launch_bounds__(64) void fp8_decode_kernel(DecArgs a) {
    const int total = a.tile_start[a.G];
    for (int tile = blockIdx.x; tile < total; tile += gridDim.x) fp8_decode_tile<LIN1, false, true>(a, tile, a.tile_start, a.offsets);
}

// Weight ring depth (a divisor of the slice's blocks).  Measured on MI355X at decode shapes
// (9 groups, T = 1): eight blocks in flight per wave instead of four did not stream faster
// (linear2, 9 x 7168 x 2048: 19.4-22.9 us against 17.5-19.2 us), so four.
constexpr int gemv_ring(int, int) { return 4; }

// workgroup tiles: ts[G] / 4 of them
// ntn: 32-column tiles per row tile and group (the K slices included).  The tile plan --
// the prefix over groups of ceil(rows / 32) * ntn -- is built in LDS from the offsets.
template <bool LIN1, int QC, int NB>
__global__ __launch_bounds__(256) void fp8_gemv_kernel(DecArgs a, int rmax, int ntn) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    int32_t *plan = (int32_t *)lds;  // tile starts, then group offsets
    for (int i = threadIdx.x; i <= a.G; i += blockDim.x) plan[a.G + 1 + i] = a.offsets[i];
    __syncthreads();
    for (int g = threadIdx.x; g < a.G; g += blockDim.x)
        plan[g] = (plan[a.G + 2 + g] - plan[a.G + 1 + g] + 31) / 32 * ntn;
    __syncthreads();
    const int tot = block_exclusive_scan(plan, a.G, plan + 2 * (a.G + 1));
    if (threadIdx.x == 0) plan[a.G] = tot;
    __syncthreads();
    const int total = plan[a.G] / (4 * QC);
    for (int wt = blockIdx.x; wt < total; wt += gridDim.x) {
        fp8_gemv_tile<LIN1, QC, NB, gemv_ring(QC, NB)>(a, wt, rmax, plan, lds);
        __syncthreads();  // the next tile restages the LDS rows
    }
}

__global__ __launch_bounds__(256) void fp8_decode_swiglu_kernel(const float *__restrict__ part, long rows, int F,
                                                               int ks, uint8_t *__restrict__ hq,
                                                               float *__restrict__ hs) {
    const long wid = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (wid < rows * (F / 128)) decode_swiglu_wave<false>(part, rows, F, ks, hq, hs, wid);
}

// The workgroup decode kernels apply: K slices of whole 1024-wide blocks (at most 2048),
// column tiles in fours, and the staged rows (at most min(32, T) per tile) and the plan
// within 64 KB of LDS.  They build their own tile plan.
bool fp8_gemv_ok(const Shape &s, const FfnPlan &p) {
    if (!p.decode) return false;
    const int rmax = s.T < 32 ? s.T : 32, G = s.G();
    const int kc1 = s.d / p.ks, kc2 = s.F;
    return kc1 % 1024 == 0 && kc2 % 1024 == 0 && kc1 <= 2048 && kc2 <= 2048 && p.ntn1 % 4 == 0 &&
           p.ntn2 % 4 == 0 && fp8_gemv_lds_total(G, rmax, kc1) <= 65536 && fp8_gemv_lds_total(G, rmax, kc2) <= 65536;
}

template <bool LIN1, int QC, int NB>
static hipError_t launch_gemv(const char *name, dim3 grid, size_t lds, hipStream_t st, const DecArgs &a, int rmax,
                              int ntn) {
    static bool attr = false;
    if (!attr) {
        hipError_t e = hipFuncSetAttribute((const void *)fp8_gemv_kernel<LIN1, QC, NB>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 65536);
        if (e != hipSuccess) return e;
        attr = true;
    }
    MOE_LAUNCH(name, (fp8_gemv_kernel<LIN1, QC, NB>), grid, dim3(256), lds, st, a, rmax, ntn);
    return hipGetLastError();
}

// qc column quads per workgroup tile (1, 2 or 4); nb 256-wide blocks per K slice (4 or 8)
template <bool LIN1>
static hipError_t launch_gemv_any(int qc, int nb, const char *name, dim3 grid, size_t lds, hipStream_t st,
                                  const DecArgs &a, int rmax, int ntn) {
    if (nb == 4) {
        if (qc == 4) return launch_gemv<LIN1, 4, 4>(name, grid, lds, st, a, rmax, ntn);
        if (qc == 2) return launch_gemv<LIN1, 2, 4>(name, grid, lds, st, a, rmax, ntn);
        return launch_gemv<LIN1, 1, 4>(name, grid, lds, st, a, rmax, ntn);
    }
    if (qc == 4) return launch_gemv<LIN1, 4, 8>(name, grid, lds, st, a, rmax, ntn);
    if (qc == 2) return launch_gemv<LIN1, 2, 8>(name, grid, lds, st, a, rmax, ntn);
    return launch_gemv<LIN1, 1, 8>(name, grid, lds, st, a, rmax, ntn);
}

static hipError_t launch_fp8_decode(const Shape &s, const FfnPlan &p, const uint8_t *w1, const uint8_t *w1s,
                                    const uint8_t *w2, const uint8_t *w2s, const uint8_t *xq, const float *xs,
                                    const int32_t *offsets, const int32_t *row_to_slot, uint8_t *h, float *hs,
                                    void *y_perm, const int32_t *ts1, const int32_t *ts2, float *upart,
                                    hipStream_t st) {
    const long rows = s.rows();
    const int G = s.G();
    // one wave per tile: the row tiles number at most ceil(rows / 32) + (non-empty groups)
    auto grid_for = [&](int ntn) {
        const long ub = ((rows + 31) / 32 + (G < rows ? G : rows)) * (long)ntn;
        return dim3((unsigned)(ub < kDecodeMaxWaves ? ub : kDecodeMaxWaves));
    };
    DecArgs a1 = {xq, xs, row_to_slot, offsets, ts1, w1, w1s, upart, nullptr, rows, s.T, s.k, s.d, 2 * s.F, G, p.ks};
    DecArgs a2 = {h, hs, nullptr, offsets, ts2, w2, w2s, nullptr, (uint16_t *)y_perm, rows, s.T, s.k, s.F, s.d, G, 1};
    const int rmax = s.T < 32 ? s.T : 32;
    const int kc1 = s.d / p.ks, kc2 = s.F;
    const size_t l1 = fp8_gemv_lds_total(G, rmax, kc1), l2 = fp8_gemv_lds_total(G, rmax, kc2);
    const bool wg = fp8_gemv_ok(s, p);
    const long waves = rows * (s.F / 128);
    if (wg) {
        // column quads per workgroup tile: longer weight streams per wave, while keeping about
        // two workgroup tiles per CU (measured, 9 experts x 4096 x 7168: 42.6 us with one
        // quad, 36 with two, 32.5 with four); every group's quad count (ntn / 4) is a
        // multiple of the choice
        auto qc_for = [&](int ntn) {
            const long quads = (long)(grid_for(ntn).x) / 4;
            int qc = quads >= 1536 ? 4 : quads >= 768 ? 2 : 1;
            while ((ntn / 4) % qc) qc /= 2;
            return qc;
        };
        auto launch = [&](bool lin1, int ntn, const DecArgs &args, size_t lds) {
            const int qc = qc_for(ntn), nb = (lin1 ? kc1 : kc2) / 256;
            const unsigned tiles = (unsigned)((grid_for(ntn).x / 4 + qc - 1) / qc), cap = 256 * 4;
            const dim3 grid(tiles < cap ? tiles : cap);
            return lin1 ? launch_gemv_any<true>(qc, nb, "linear1", grid, lds, st, args, rmax, ntn)
                        : launch_gemv_any<false>(qc, nb, "linear2", grid, lds, st, args, rmax, ntn);
        };
        hipError_t e = launch(true, p.ntn1, a1, l1);
        if (e != hipSuccess) return e;
        MOE_LAUNCH("swiglu_quant", fp8_decode_swiglu_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, st,
                   (const float *)upart, rows, s.F, p.ks, h, hs);
        return launch(false, p.ntn2, a2, l2);
    }
    MOE_LAUNCH("linear1", fp8_decode_kernel<true>, grid_for(p.ntn1), dim3(64), 0, st, a1);
    MOE_LAUNCH("swiglu_quant", fp8_decode_swiglu_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, st,
               (const float *)upart, rows, s.F, p.ks, h, hs);
    MOE_LAUNCH("linear2", fp8_decode_kernel<false>, grid_for(p.ntn2), dim3(64), 0, st, a2);
    return hipGetLastError();
}

hipError_t launch_fp8_ffn(const Shape &s, const FfnPlan &p, const uint8_t *w1, const uint8_t *w1s,
                          const uint8_t *w2, const uint8_t *w2s, const uint8_t *xq, const float *xs,
                          const int32_t *offsets, const int32_t *row_to_slot, uint8_t *h, float *hs, void *y_perm,
                          const int32_t *ts1, const int32_t *ts2, float *upart, hipStream_t st) {
    if (p.decode)
        return launch_fp8_decode(s, p, w1, w1s, w2, w2s, xq, xs, offsets, row_to_slot, h, hs, y_perm, ts1, ts2,
                                 upart, st);
    const long rows = s.rows();
    const int G = s.G();
    const int ntn1 = p.ntn1, ntn2 = p.ntn2;
    auto grid_for = [&](int bm, int ntn) {
        const long ub = ((rows + bm - 1) / bm + (G < rows ? G : rows)) * (long)ntn;
        return dim3((unsigned)((ub + 7) / 8 * 8));
    };
    Fp8Args a1 = {xq, xs, row_to_slot, w1, w1s, h, hs, offsets, ts1, s.T, s.k, s.d, 2 * s.F, s.F, G, s.F};
    Fp8Args a2 = {h, hs, nullptr, w2, w2s, y_perm, nullptr, offsets, ts2, s.T, s.k, s.F, s.d, s.d, G, s.F};
    hipError_t e;
    // the 8-wave tiles address their A operand with 32-bit byte offsets
    const bool a1_small = (long)s.T * s.d < (1L << 32), a2_small = rows * (long)s.F < (1L << 32);
    auto ub_for = [&](int bm, int ntn) { return ((rows + bm - 1) / bm + (G < rows ? G : rows)) * (long)ntn; };
    if (p.bm1 == 256 && a1_small) e = launch_fp8_8<true>("linear1", ub_for(p.bm1, ntn1), a1, st);
    else if (p.bm1 == 256) e = launch_fp8<256, 256, 4, true, true>("linear1", grid_for(p.bm1, ntn1), a1, st);
    else e = launch_fp8<128, 256, 4, true, true>("linear1", grid_for(p.bm1, ntn1), a1, st);
    if (e != hipSuccess) return e;
    if (p.bm2 == 256 && p.bn2 == 256 && a2_small) e = launch_fp8_8<false>("linear2", ub_for(p.bm2, ntn2), a2, st);
    else if (p.bm2 == 256 && p.bn2 == 256) e = launch_fp8<256, 256, 2, false, false>("linear2", grid_for(p.bm2, ntn2), a2, st);
    else if (p.bn2 == 256) e = launch_fp8<128, 256, 2, false, false>("linear2", grid_for(p.bm2, ntn2), a2, st);
    else if (p.bm2 == 256) e = launch_fp8<256, 128, 2, false, false>("linear2", grid_for(p.bm2, ntn2), a2, st);
    else e = launch_fp8<128, 128, 2, false, false>("linear2", grid_for(p.bm2, ntn2), a2, st);
    return e;
}

}  // namespace moe
