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
template <bool SWIGLU, bool GATHER>
__global__ __launch_bounds__(512) void gemm_fp8_kernel8(Fp8Args a, int xcd_cus) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    int half;
    const int tile = pick_tile_split(blockIdx.x, a.tile_start[a.G], xcd_cus, half);
    if (tile >= 0) fp8_tile8<1, 8, SWIGLU, GATHER>(a, tile, lds, half);
}

// 256 x 256 tiles: the 8-wave kernel (the layer's linear1 gathers its rows, linear2 does
// not; rows that arrive grouped -- an expert-parallel receive buffer -- need no gather).
// ub: an upper bound of the tile count; the grid adds the blocks of the tail split.
template <bool SWIGLU, bool GATHER = SWIGLU>
static hipError_t launch_fp8_8(const char *name, long ub, const Fp8Args &a, hipStream_t st) {
    constexpr size_t lds = fp8_tile8_lds();
    static bool attr = false;
    if (!attr) {
        hipError_t e = hipFuncSetAttribute((const void *)gemm_fp8_kernel8<SWIGLU, GATHER>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr = true;
    }
    const int C = xcd_cus();
    if (C <= 0) return hipErrorInvalidDevice;
    const dim3 grid((unsigned)(8 * ((ub + 7) / 8 + C / 2)));
    MOE_LAUNCH(name, (gemm_fp8_kernel8<SWIGLU, GATHER>), grid, dim3(512), lds, st, a, C);
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

// workgroup tiles: ts[G] / 4 of them
// ntn: 32-column tiles per row tile and group (the K slices included).  The tile plan --
// the prefix over groups of ceil(rows / 32) * ntn -- is built in LDS from the offsets; then
// each workgroup streams its tiles (blockIdx.x, + gridDim.x, ...).  D: weight blocks in
// flight per wave -- 4 at two workgroups per CU (eight blocks instead of four streamed no
// faster there, measured on MI355X), 8 when the two activation buffers take more than half
// the LDS and one workgroup (a wave per SIMD) keeps the CU's loads in flight alone.
template <bool LIN1, int QC, int NB, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 4 ? 2 : 1))) void fp8_gemv_kernel(
    DecArgs a, int rmax, int ntn) {
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
    fp8_gemv_run<LIN1, QC, NB, D>(a, rmax, plan, lds, plan[a.G] / (4 * QC));
}

__global__ __launch_bounds__(256) void fp8_decode_swiglu_kernel(const float *__restrict__ part, long rows, int F,
                                                               int ks, uint8_t *__restrict__ hq,
                                                               float *__restrict__ hs) {
    const long wid = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (wid < rows * (F / 128)) decode_swiglu_wave<false>(part, rows, F, ks, hq, hs, wid);
}

// The workgroup decode kernels apply: K slices of whole 1024-wide blocks (at most 2048),
// column tiles in fours, and the plan, two sets of row_to_slot entries and two buffers of
// staged rows (at most min(32, T) per tile) within the 160 KB of LDS a workgroup can hold.
// Up to half of it (2 x 32 rows of a 1024-wide slice take 71 KB) two workgroups share a CU.
// They build their own tile plan.
constexpr size_t kGemvLdsMax = 160 * 1024, kGemvLdsTwo = 80 * 1024;

bool fp8_gemv_ok(const Shape &s, const FfnPlan &p) {
    if (!p.decode) return false;
    const int rmax = s.T < 32 ? s.T : 32, G = s.G();
    const int kc1 = s.d / p.ks, kc2 = s.F;
    return kc1 % 1024 == 0 && kc2 % 1024 == 0 && kc1 <= 2048 && kc2 <= 2048 && p.ntn1 % 4 == 0 &&
           p.ntn2 % 4 == 0 && fp8_gemv_lds_total(G, rmax, kc1) <= kGemvLdsMax &&
           fp8_gemv_lds_total(G, rmax, kc2) <= kGemvLdsMax;
}

template <bool LIN1, int QC, int NB, int D>
static hipError_t launch_gemv(const char *name, dim3 grid, size_t lds, hipStream_t st, const DecArgs &a, int rmax,
                              int ntn) {
    static bool attr = false;
    if (!attr) {
        hipError_t e = hipFuncSetAttribute((const void *)fp8_gemv_kernel<LIN1, QC, NB, D>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)kGemvLdsMax);
        if (e != hipSuccess) return e;
        attr = true;
    }
    MOE_LAUNCH(name, (fp8_gemv_kernel<LIN1, QC, NB, D>), grid, dim3(256), lds, st, a, rmax, ntn);
    return hipGetLastError();
}

// qc column quads per workgroup tile (1, 2 or 4); nb 256-wide blocks per K slice (4 or 8);
// two: two workgroups per CU (the ring of 4), else one (the ring of 8; 2048-wide slices only)
template <bool LIN1>
static hipError_t launch_gemv_any(int qc, int nb, bool two, const char *name, dim3 grid, size_t lds, hipStream_t st,
                                  const DecArgs &a, int rmax, int ntn) {
    if (nb == 4) {
        if (qc == 4) return launch_gemv<LIN1, 4, 4, 4>(name, grid, lds, st, a, rmax, ntn);
        if (qc == 2) return launch_gemv<LIN1, 2, 4, 4>(name, grid, lds, st, a, rmax, ntn);
        return launch_gemv<LIN1, 1, 4, 4>(name, grid, lds, st, a, rmax, ntn);
    }
    if (two) {
        if (qc == 4) return launch_gemv<LIN1, 4, 8, 4>(name, grid, lds, st, a, rmax, ntn);
        if (qc == 2) return launch_gemv<LIN1, 2, 8, 4>(name, grid, lds, st, a, rmax, ntn);
        return launch_gemv<LIN1, 1, 8, 4>(name, grid, lds, st, a, rmax, ntn);
    }
    if (qc == 4) return launch_gemv<LIN1, 4, 8, 8>(name, grid, lds, st, a, rmax, ntn);
    if (qc == 2) return launch_gemv<LIN1, 2, 8, 8>(name, grid, lds, st, a, rmax, ntn);
    return launch_gemv<LIN1, 1, 8, 8>(name, grid, lds, st, a, rmax, ntn);
}

int fp8_gemv_qc(const Shape &s, int ntn) {
    const long rows = s.rows();
    const int G = s.G();
    // the one-wave-per-tile grid bound of launch_fp8_decode, in quads of four waves
    long ub = ((rows + 31) / 32 + (G < rows ? G : rows)) * (long)ntn;
    if (ub > kDecodeMaxWaves) ub = kDecodeMaxWaves;
    const long quads = ub / 4;
    int qc = quads >= 1536 ? 4 : quads >= 768 ? 2 : 1;
    while ((ntn / 4) % qc) qc /= 2;
    return qc;
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
        auto qc_for = [&](int ntn) { return fp8_gemv_qc(s, ntn); };
        // one workgroup per resident slot (two or one per CU), each streaming its tiles
        const int cus = 8 * xcd_cus();
        if (cus <= 0) return hipErrorInvalidDevice;
        auto launch = [&](bool lin1, int ntn, const DecArgs &args, size_t lds) {
            const int qc = qc_for(ntn), nb = (lin1 ? kc1 : kc2) / 256;
            const bool two = nb == 4 || lds <= kGemvLdsTwo;
            const unsigned tiles = (unsigned)((grid_for(ntn).x / 4 + qc - 1) / qc), cap = (two ? 2 : 1) * cus;
            const dim3 grid(tiles < cap ? tiles : cap);
            return lin1 ? launch_gemv_any<true>(qc, nb, two, "linear1", grid, lds, st, args, rmax, ntn)
                        : launch_gemv_any<false>(qc, nb, two, "linear2", grid, lds, st, args, rmax, ntn);
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

// ---- grouped FP8 x FP4 FFN over rows that arrive grouped, and the dense GEMM ----------

// offsets and tile plans of an expert-parallel rank's receive buffer: rows of local expert
// e from source rank s are the block (e, s) of recv_counts [E, nsrc], expert-major.  The
// cumulative offsets are clamped at the buffer's capacity (an overflow is a device error),
// so no tile reaches past the buffer.  One workgroup.
__global__ __launch_bounds__(256) void ep_plan_kernel(const int32_t *__restrict__ recv_counts, int E, int nsrc,
                                                     long cap, int bm1, int ntn1, int bm2, int ntn2,
                                                     int32_t *__restrict__ offsets, int32_t *__restrict__ ts1,
                                                     int32_t *__restrict__ ts2, int32_t *err) {
    __shared__ int32_t sh[2 * 1032 + 256];
    if (threadIdx.x == 0) {
        long run = 0;
        bool over = false;
        for (int e = 0; e < E; ++e) {
            offsets[e] = (int32_t)run;
            long n = 0;
            for (int q = 0; q < nsrc; ++q) {
                const int c = recv_counts[(long)e * nsrc + q];
                n += c > 0 ? c : 0;
                over |= c < 0;
            }
            run += n;
            if (run > cap) {
                run = cap;
                over = true;
            }
        }
        offsets[E] = (int32_t)run;
        if (over) set_error(err, DEVERR_OVERFLOW);
    }
    __syncthreads();
    tile_plan_block<false>(offsets, E, bm1, ntn1, bm2, ntn2, ts1, ts2, sh);
}

// the plan of one group of n rows (the dense GEMM, the shared expert of a shard)
__global__ void one_group_plan_kernel(int32_t *__restrict__ plan, int n, int ntiles1, int ntiles2) {
    if (threadIdx.x == 0) {
        plan[0] = 0;
        plan[1] = n;
        plan[2] = 0;
        plan[3] = ntiles1;
        plan[4] = 0;
        plan[5] = ntiles2;
    }
}

// linear2-shaped GEMM over ungathered rows: y [*, N] bf16 = A [*, K] . B^T by tiles of the
// plan (offsets, ts) over G groups, rows at most `rows`, N tiles of bn
static hipError_t launch_fp8_plain(const char *name, const Fp8Args &a, long rows, int bm, int bn, hipStream_t st) {
    const int G = a.G, ntn = a.Ntot / bn;
    const long ub = ((rows + bm - 1) / bm + (G < rows ? G : rows)) * (long)ntn;
    const bool small = rows * (long)a.K < (1L << 32);
    if (bm == 256 && bn == 256 && small) return launch_fp8_8<false>(name, ub, a, st);
    const dim3 grid((unsigned)((ub + 7) / 8 * 8));
    if (bm == 256 && bn == 256) return launch_fp8<256, 256, 2, false, false>(name, grid, a, st);
    if (bn == 256) return launch_fp8<128, 256, 2, false, false>(name, grid, a, st);
    if (bm == 256) return launch_fp8<256, 128, 2, false, false>(name, grid, a, st);
    return launch_fp8<128, 128, 2, false, false>(name, grid, a, st);
}

// linear1 + SwiGLU over ungathered rows (h codes and scales out)
static hipError_t launch_fp8_swiglu_plain(const char *name, const Fp8Args &a, long rows, int bm, hipStream_t st) {
    const int G = a.G, ntn = a.F / 128;
    const long ub = ((rows + bm - 1) / bm + (G < rows ? G : rows)) * (long)ntn;
    const bool small = rows * (long)a.K < (1L << 32);
    if (bm == 256 && small) return launch_fp8_8<true, false>(name, ub, a, st);
    const dim3 grid((unsigned)((ub + 7) / 8 * 8));
    if (bm == 256) return launch_fp8<256, 256, 4, true, false>(name, grid, a, st);
    return launch_fp8<128, 256, 4, true, false>(name, grid, a, st);
}

hipError_t launch_gemm_fp8_dense(long M, int N, int K, const uint8_t *a, const float *as, const uint8_t *b,
                                 const uint8_t *bs, void *c, int32_t *plan, hipStream_t st) {
    if (M == 0) return hipSuccess;
    const int bm = M >= 160 ? 256 : 128, bn = N % 256 == 0 ? 256 : 128;
    const long tiles = (M + bm - 1) / bm * (long)(N / bn);
    MOE_LAUNCH("gemm_plan", one_group_plan_kernel, dim3(1), dim3(64), 0, st, plan, (int)M, (int)tiles, (int)tiles);
    const Fp8Args g = {a, as, nullptr, b, bs, c, nullptr, plan, plan + 2, 0, 1, K, N, N, 1, 0};
    return launch_fp8_plain("gemm_fp8_mxfp4", g, M, bm, bn, st);
}

// One expert-parallel rank: the E local experts over the receive buffer (rows grouped by
// local expert, then by source rank), then the shared expert over the rank's own T tokens.
// ws: plan ints (offsets [E + 1], ts1, ts2 [E + 1] each, then 6 for the shared group), h and
// its scales for cap + S * T rows.
hipError_t launch_ep_ffn(const Shape &s, int nsrc, const int32_t *recv_counts, long cap, const uint8_t *rq,
                         const float *rs, const uint8_t *w1, const uint8_t *w1s, const uint8_t *w2,
                         const uint8_t *w2s, void *y_recv, const uint8_t *xq, const float *xs, void *y_shared,
                         int32_t *plan, uint8_t *h, float *hs, int32_t *err, hipStream_t st) {
    const int E = s.E, d = s.d, F = s.F;
    const int bm = cap >= 160L * E ? 256 : 128, bn2 = d % 256 == 0 ? 256 : 128;
    const int ntn1 = F / 128, ntn2 = d / bn2;
    int32_t *offs = plan, *ts1 = plan + (E + 1), *ts2 = plan + 2 * (E + 1), *p1 = plan + 3 * (E + 1);
    hipError_t e = hipSuccess;
    if (cap > 0) {
        MOE_LAUNCH("ep_plan", ep_plan_kernel, dim3(1), dim3(256), 0, st, recv_counts, E, nsrc, cap, bm, ntn1, bm,
                   ntn2, offs, ts1, ts2, err);
        const Fp8Args a1 = {rq, rs, nullptr, w1, w1s, h, hs, offs, ts1, 0, 1, d, 2 * F, F, E, F};
        const Fp8Args a2 = {h, hs, nullptr, w2, w2s, y_recv, nullptr, offs, ts2, 0, 1, F, d, d, E, F};
        e = launch_fp8_swiglu_plain("linear1", a1, cap, bm, st);
        if (e == hipSuccess) e = launch_fp8_plain("linear2", a2, cap, bm, bn2, st);
        if (e != hipSuccess) return e;
    }
    if (s.S && s.T > 0) {
        const long T = s.T;
        const int bms = T >= 160 ? 256 : 128;
        const long t1 = (T + bms - 1) / bms * (long)ntn1, t2 = (T + bms - 1) / bms * (long)ntn2;
        MOE_LAUNCH("ep_plan", one_group_plan_kernel, dim3(1), dim3(64), 0, st, p1, (int)T, (int)t1, (int)t2);
        const size_t g1 = (size_t)E * 2 * F, g2 = (size_t)E * d;  // rows of W1, W2 before the shared expert
        uint8_t *hsh = h + (size_t)cap * F;
        float *hssh = hs + (size_t)cap * (F / 128);
        const Fp8Args a1 = {xq, xs, nullptr, w1 + g1 * (d / 2), w1s + g1 * (d / 32), hsh, hssh, p1, p1 + 2, 0, 1,
                            d, 2 * F, F, 1, F};
        const Fp8Args a2 = {hsh, hssh, nullptr, w2 + g2 * (F / 2), w2s + g2 * (F / 32), y_shared, nullptr, p1,
                            p1 + 4, 0, 1, F, d, d, 1, F};
        e = launch_fp8_swiglu_plain("linear1_shared", a1, T, bms, st);
        if (e == hipSuccess) e = launch_fp8_plain("linear2_shared", a2, T, bms, bn2, st);
    }
    return e;
}

}  // namespace moe
