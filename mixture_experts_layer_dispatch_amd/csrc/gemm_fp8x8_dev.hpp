// FP8 e4m3 x e4m3 grouped GEMM work items (S8-S9 in the FP8 x FP8 expert mode).
//
// Mega MoE blog (donniechu.com, spec table: DeepGEMM's FP8 GEMM next to the FP8 x FP4
// mega kernel): the expert weights in FP8 as well.  Weights take the activations' format,
// e4m3 codes with one power-of-two fp32 scale per 1x128 block along K, so both scales are
// e8m0 exponents the scaled MFMA applies in hardware (v_mfma_scale_f32_32x32x64_f8f6f4,
// A and B both fp8): no per-block promotion of the fp32 accumulators.
//
// Tiles: 128 rows x BN columns, 4 waves as 2 x 2, each 64 rows x BN/2 columns (32x32
// MFMA blocks).  B rows are 128 bytes per 128-wide K stage, like A's, so one stage of a
// 128 x 256 tile is 48 KB and three stages (two in flight, moved by LDS DMA) fit the CU's
// 160 KB.  linear1 (SWIGLU, BN = 256): the tile's first 128 B rows are gate rows f0 ..
// f0 + 127, the last 128 the matching up rows; wave column wn holds gate and up columns
// wn * 64 .. wn * 64 + 63, so h = silu(gate) * up stays in the wave, and the row maximum
// of the 128-column quantisation block of h is completed across the two column waves
// through LDS.  The k order of every output element is fixed (stage by stage, k64 halves
// in order), so results are deterministic.
#pragma once

#include "common.hpp"
#include "gemm_fp8_dev.hpp"

namespace moe {

template <int BN>
constexpr size_t fp8x8_tile_lds() {
    return 3 * ((size_t)128 * 128 + (size_t)BN * 128 + 128 * 4 + (size_t)BN * 4 + 256);
}

// One tile per call; same caller contract as fp8_tile.  Fp8Args: B [G, Ntot, K] e4m3 codes,
// Bs [G, Ntot, K/128] fp32 scales (passed as bytes).
template <bool SWIGLU, bool GATHER, int BN>
__device__ __forceinline__ void fp8x8_tile(const Fp8Args &a, int tile, uint8_t *lds) {
    constexpr int BM = 128, NS = 3, PD = 2;
    constexpr int TM = 2, TN = BN / 64;
    constexpr int PA = BM / 32, PB = BN / 32;      // 1 KB DMA instructions per wave and stage
    constexpr int NSC = (BM + BN) / 64;             // 64-row chunks of scale dwords
    constexpr int PS = (NSC + 3) / 4;               // scale instructions per wave and stage
    constexpr int PER = PA + PB + PS;
    constexpr int OFF_B = BM * 128, OFF_SA = OFF_B + BN * 128, OFF_SB = OFF_SA + BM * 4;
    constexpr int OFF_SPARE = OFF_SB + BN * 4, STAGE = OFF_SPARE + 256;
    static_assert(BN == 128 || BN == 256, "tile width");
    static_assert(!SWIGLU || BN == 256, "SwiGLU tiles hold 128 gate + 128 up columns");
    int g, row0, nrows, nt;
    {
        int lo = 0, hi = a.G - 1;
        while (lo < hi) {
            int mid = (lo + hi + 1) >> 1;
            if (a.tile_start[mid] <= tile) lo = mid; else hi = mid - 1;
        }
        g = lo;
        const int rb = a.offsets[g], cnt = a.offsets[g + 1] - rb;
        const int mtiles = (cnt + BM - 1) / BM, local = tile - a.tile_start[g];
        const int mt = local % mtiles;
        nt = local / mtiles;
        row0 = rb + mt * BM;
        nrows = min(BM, cnt - mt * BM);
    }
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1, khalf = lane >> 5;
    const int KB = a.K / 128;
    const int f0 = nt * (BN / 2), n0 = nt * BN;
    auto wrow_of = [&](int r) -> long { return SWIGLU ? (r < BN / 2 ? f0 + r : a.F + f0 + r - BN / 2) : n0 + r; };
    auto arow_src = [&](int r) -> long {
        const long grow = row0 + (r < nrows ? r : 0);
        return GATHER ? row_token(grow, a.row_to_slot, a.T, a.k) : grow;
    };

    // ---- DMA sources: instruction q of a wave fills 8 rows x 128 bytes (lane L: row L / 8,
    // physical chunk L % 8 = logical chunk ^ the row's swizzle key)
    const uint8_t *pa[PA], *pb[PB];
#pragma unroll
    for (int q = 0; q < PA; ++q) {
        const int r = 8 * (wave * PA + q) + (lane >> 3);
        pa[q] = a.A + arow_src(r) * a.K + (((lane & 7) ^ ((r >> 1) & 7)) << 4);
    }
#pragma unroll
    for (int q = 0; q < PB; ++q) {
        const int r = 8 * (wave * PB + q) + (lane >> 3);
        pb[q] = a.B + ((long)g * a.Ntot + wrow_of(r)) * a.K + (((lane & 7) ^ ((r >> 1) & 7)) << 4);
    }
    // scale chunk c = wave + 4 s: A rows 64 c + lane for c < BM / 64, then B rows, then (to keep
    // every wave's instruction count equal for the counted waits) a spare re-load of A row 0
    const uint8_t *psc[PS];
    int sdst[PS];
#pragma unroll
    for (int q = 0; q < PS; ++q) {
        const int c = wave + 4 * q;
        if (c < BM / 64) {
            psc[q] = (const uint8_t *)(a.As + arow_src(64 * c + lane) * KB);
            sdst[q] = OFF_SA + 64 * c * 4;
        } else if (c < NSC) {
            const int r = 64 * (c - BM / 64) + lane;
            psc[q] = (const uint8_t *)((const float *)a.Bs + ((long)g * a.Ntot + wrow_of(r)) * KB);
            sdst[q] = OFF_SB + 64 * (c - BM / 64) * 4;
        } else {
            psc[q] = (const uint8_t *)(a.As + arow_src(0) * KB);
            sdst[q] = OFF_SPARE;
        }
    }

    // ---- fragments: A of rows arow[i], B of tile rows brow[j]; for k64 half h, lane half kh
    // holds K {16 kh .. 16 kh + 15} and {32 + 16 kh .. 32 + 16 kh + 15} of the step (the fp8
    // operand layout of the scaled MFMA, for A and B alike): chunks 4 h + kh and 4 h + 2 + kh
    int arow[TM], brow[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) arow[i] = wm * 64 + i * 32 + (lane & 31);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        if (SWIGLU) brow[j] = (j < TN / 2 ? wn * 64 + j * 32 : BN / 2 + wn * 64 + (j - TN / 2) * 32) + (lane & 31);
        else brow[j] = wn * (BN / 2) + j * 32 + (lane & 31);
    }
    int aoff[2][TM][2], boff[2][TN][2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
#pragma unroll
            for (int i = 0; i < TM; ++i) aoff[h][i][c] = sw128(arow[i], h * 4 + 2 * c + khalf);
#pragma unroll
            for (int j = 0; j < TN; ++j) boff[h][j][c] = OFF_B + sw128(brow[j], h * 4 + 2 * c + khalf);
        }
    }

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = (f32x16){};

    // One wave per SIMD, so the wave interleaves its own work: the k64 half h = 0 of stage kt
    // is multiplied while the DMAs of stage kt + 2 and the half h = 1 fragments are issued
    // between its MFMAs; after the one barrier per stage (stage kt + 1 published, every wave
    // done with stage kt), half h = 1 is multiplied while stage kt + 1's h = 0 fragments are
    // read.  Every accumulator still takes its MFMAs stage by stage, h = 0 before h = 1, with
    // the same operands and scales, so the results are those of the plain pipeline.
#define X8_DMA(q, stg, kt_)                                                                          \
    do {                                                                                             \
        uint8_t *s_ = lds + (stg) * STAGE;                                                           \
        const int kt2_ = (kt_);                                                                      \
        if ((q) < PA) lds_dma16(pa[(q) < PA ? (q) : 0] + kt2_ * 128, s_ + (wave * PA + (q)) * 1024); \
        else if ((q) < PA + PB)                                                                      \
            lds_dma16(pb[(q) >= PA && (q) < PA + PB ? (q) - PA : 0] + kt2_ * 128,                    \
                      s_ + OFF_B + (wave * PB + (q) - PA) * 1024);                                   \
        else {                                                                                       \
            const int p_ = (q) - PA - PB < PS ? (q) - PA - PB : 0;                                   \
            lds_dma4(psc[p_] + kt2_ * 4, s_ + sdst[p_]);                                             \
        }                                                                                            \
    } while (0)
#define X8_FRAG(FA, FB, u, stg, h)                                                                   \
    do {                                                                                             \
        const uint8_t *s_ = lds + (stg) * STAGE;                                                     \
        if ((u) < 2 * TM) {                                                                          \
            const int i_ = ((u) >> 1) < TM ? ((u) >> 1) : 0, c_ = (u) & 1;                          \
            FA[i_][c_] = *(const i32x4 *)(s_ + aoff[h][i_][c_]);                                     \
        } else {                                                                                     \
            const int j_ = (((u) - 2 * TM) >> 1) < TN ? (((u) - 2 * TM) >> 1) : 0, c_ = (u) & 1;     \
            FB[j_][c_] = *(const i32x4 *)(s_ + boff[h][j_][c_]);                                     \
        }                                                                                            \
    } while (0)
#define X8_SCALES(SA, SB, stg)                                                                       \
    do {                                                                                             \
        const uint8_t *s_ = lds + (stg) * STAGE;                                                     \
        _Pragma("unroll") for (int i = 0; i < TM; ++i)                                               \
            SA[i] = (int)((*(const uint32_t *)(s_ + OFF_SA + arow[i] * 4) >> 23) & 0xFF);            \
        _Pragma("unroll") for (int j = 0; j < TN; ++j)                                               \
            SB[j] = (int)((*(const uint32_t *)(s_ + OFF_SB + brow[j] * 4) >> 23) & 0xFF);            \
    } while (0)
#define X8_MFMA(FA, FB, m)                                                                           \
    do {                                                                                             \
        const int i_ = (m) / TN, j_ = (m) % TN;                                                      \
        const i32x8 av_ = {FA[i_][0][0], FA[i_][0][1], FA[i_][0][2], FA[i_][0][3],                   \
                           FA[i_][1][0], FA[i_][1][1], FA[i_][1][2], FA[i_][1][3]};                  \
        const i32x8 bv_ = {FB[j_][0][0], FB[j_][0][1], FB[j_][0][2], FB[j_][0][3],                   \
                           FB[j_][1][0], FB[j_][1][1], FB[j_][1][2], FB[j_][1][3]};                  \
        acc[i_][j_] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av_, bv_, acc[i_][j_], 0, 0, 0, \
                                                                      sa0[i_], 0, sb0[j_]);          \
    } while (0)
#define X8_BARRIER()                           \
    do {                                       \
        asm volatile("" ::: "memory");         \
        __builtin_amdgcn_s_barrier();          \
        asm volatile("" ::: "memory");         \
    } while (0)

    constexpr int NR = 2 * TM + 2 * TN;  // fragment reads per k64 half
    constexpr int NG = TM * TN;          // issue groups per k64 half (one MFMA each)
    i32x4 fa0[TM][2], fb0[TN][2], fa1[TM][2], fb1[TN][2];
    int sa0[TM], sb0[TN];

#pragma unroll
    for (int s0 = 0; s0 < PD; ++s0)
#pragma unroll
        for (int q = 0; q < PER; ++q) X8_DMA(q, s0, s0 < KB ? s0 : KB - 1);
    wait_vmcnt<(PD - 1) * PER>();  // this wave's loads of stage 0 have landed
    X8_BARRIER();                  // ... and every wave's
#pragma unroll
    for (int u = 0; u < NR; ++u) X8_FRAG(fa0, fb0, u, 0, 0);
    X8_SCALES(sa0, sb0, 0);

    for (int kt = 0; kt < KB; ++kt) {
        const int cur = kt % NS, nxt = (kt + 1) % NS, pre = (kt + PD) % NS;
        const int kpre = kt + PD < KB ? kt + PD : KB - 1;  // the tail re-loads the last stage
        wait_lgkmcnt0();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
#pragma unroll
            for (int q = gi * PER / NG; q < (gi + 1) * PER / NG; ++q) X8_DMA(q, pre, kpre);
#pragma unroll
            for (int u = gi * NR / NG; u < (gi + 1) * NR / NG; ++u) X8_FRAG(fa1, fb1, u, cur, 1);
            X8_MFMA(fa0, fb0, gi);
            __builtin_amdgcn_sched_barrier(0);
        }
        wait_lgkmcnt0();
        wait_vmcnt<(PD - 1) * PER>();  // stage kt + 1 landed (this wave's loads)
        X8_BARRIER();                  // every wave's; and every wave is done with stage kt
        __builtin_amdgcn_sched_barrier(0);
        int sa1[TM], sb1[TN];
        X8_SCALES(sa1, sb1, nxt);
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
#pragma unroll
            for (int u = gi * NR / NG; u < (gi + 1) * NR / NG; ++u) X8_FRAG(fa0, fb0, u, nxt, 0);
            X8_MFMA(fa1, fb1, gi);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < TM; ++i) sa0[i] = sa1[i];
#pragma unroll
        for (int j = 0; j < TN; ++j) sb0[j] = sb1[j];
    }
    wait_vmcnt<0>();
#undef X8_DMA
#undef X8_FRAG
#undef X8_SCALES
#undef X8_MFMA
#undef X8_BARRIER

    // ---- epilogue ------------------------------------------------------------------------
    if constexpr (SWIGLU) {
        uint8_t *hq = (uint8_t *)a.C;
        float *xmax = (float *)lds;  // [2][BM]: each column wave's row maxima
        __syncthreads();             // every wave is done reading the stages
        constexpr int TNh = TN / 2;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = wm * 64 + i * 32 + 8 * (r >> 2) + 4 * khalf + (r & 3);
                float am = 0.0f;
#pragma unroll
                for (int j = 0; j < TNh; ++j) am = fmaxf(am, fabsf(swiglu(acc[i][j][r], acc[i][j + TNh][r])));
                am = half_wave_max(am);  // the row's 64 columns of this wave
                if ((lane & 31) == 0) xmax[wn * BM + row] = am;
            }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = wm * 64 + i * 32 + 8 * (r >> 2) + 4 * khalf + (r & 3);
                if (row >= nrows) continue;
                const float amax = fmaxf(xmax[row], xmax[BM + row]);  // the 128-column block
                const int e = e4m3_block_exponent(amax);
                const float inv = ldexpf(1.0f, -e);
                const long grow = row0 + row;
#pragma unroll
                for (int j = 0; j < TNh; ++j) {
                    const float hv = swiglu(acc[i][j][r], acc[i][j + TNh][r]);
                    hq[grow * a.F + f0 + wn * 64 + j * 32 + (lane & 31)] = (uint8_t)(cvt_e4m3x2(hv * inv, 0.0f) & 0xFFu);
                }
                if (wn == 0 && (lane & 31) == 0) a.Cs[grow * (a.F / 128) + f0 / 128] = ldexpf(1.0f, e);
            }
    } else {
        uint16_t *y = (uint16_t *)a.C;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = wm * 64 + i * 32 + 8 * (r >> 2) + 4 * khalf + (r & 3);
                if (row >= nrows) continue;
                const long grow = row0 + row;
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    y[grow * a.ldc + n0 + wn * (BN / 2) + j * 32 + (lane & 31)] = f32_to_bf16(acc[i][j][r]);
            }
    }
}

}  // namespace moe
