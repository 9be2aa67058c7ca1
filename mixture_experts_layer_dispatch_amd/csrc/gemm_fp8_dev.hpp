// FP8 e4m3 x MXFP4 grouped GEMM work items (S8-S9 in the FP8 x FP4 mode, S12).
//
// Mega MoE blog (donniechu.com, spec table) and Mega MoE wiki ("One-line definition"):
// both expert linears run as FP8 x FP4.  Activations are e4m3 with one power-of-two
// fp32 scale per 1x128 block along K; weights are MXFP4 (e2m1 pairs per byte, one
// e8m0 scale per 32 along K).  Because the activation scales are powers of two they
// are exactly e8m0 values, so v_mfma_scale_f32_32x32x64_f8f6f4 applies both scales in
// hardware (A: fp8 e4m3, B: fp4 e2m1) and the fp32 accumulators need no per-block
// promotion step.
//
// Tiling follows the bf16 kernel: BM x BN tiles over ragged expert groups, K advancing
// 128 per stage, stages moved by LDS DMA three buffers deep (two stages in flight), a
// mid-stage barrier, register double-buffered fragments and an issue order pinned to
// small {DMA, LDS read, MFMA} groups.  Per stage the DMA moves, for each tile row, 128
// bytes of A codes, 64 bytes of B codes, the row's fp32 A scale and the 4 e8m0 B scale
// bytes of this K range.
//
// linear1 (SWIGLU): waves are stacked along M (4 x 1), so one wave holds all 128 gate
// columns and the matching 128 up columns of its rows; the epilogue forms
// h = silu(gate) * up, takes the row's amax over those 128 columns (one quantisation
// block of h), and writes e4m3 codes plus the power-of-two scale.
#pragma once

#include "common.hpp"

namespace moe {

struct Fp8Args {
    const uint8_t *A;            // codes: linear1 xq [T, K] (gathered by row); linear2 hq [rows, K]
    const float *As;             // scales [*, K/128]
    const int32_t *row_to_slot;  // linear1 only
    const uint8_t *B;            // MXFP4 codes [G, Ntot, K/2]
    const uint8_t *Bs;           // e8m0 [G, Ntot, K/32]
    void *C;                     // linear1: hq codes [rows, F]; linear2: y_perm bf16 [rows, ldc]
    float *Cs;                   // linear1: h scales [rows, F/128]
    const int32_t *offsets, *tile_start;
    int T, k, K, Ntot, ldc, G, F;
};

// 16-byte-chunk swizzles of 128-byte (A codes) and 64-byte (B codes) LDS rows.
__device__ __forceinline__ int sw128(int row, int c) { return swz_off<64>(row, c); }
__device__ __forceinline__ int sw64(int row, int c) { return swz_off<32>(row, c); }

template <int BM, int BN>
constexpr size_t fp8_tile_lds() { return 3 * ((size_t)BM * 128 + BN * 64 + BM * 4 + BN * 4 + 256); }

// One tile per call; lds holds fp8_tile_lds<BM, BN>() bytes.  Every wave has waited for
// its own DMAs when it returns, but other waves may still read fragments: callers that
// reuse lds must pass a workgroup barrier first.
template <int BM, int BN, int WM, bool SWIGLU, bool GATHER>
__device__ __forceinline__ void fp8_tile(const Fp8Args &a, int tile, uint8_t *lds) {
    constexpr int WN = 4 / WM;
    constexpr int TM = BM / WM / 32, TN = BN / WN / 32;
    constexpr int PD = 2, NS = PD + 1;
    // DMA instructions per wave per stage: A codes (8 rows x 128 B each), B codes (16 rows
    // x 64 B each), one dword each for the A and B scales (64 rows per instruction)
    constexpr int PA = BM / 32, PB = BN / 64;
    static_assert(BM % 64 == 0 && BN % 64 == 0 && BM <= 256 && BN <= 256, "tile shape");
    constexpr int OFF_B = BM * 128, OFF_SA = OFF_B + BN * 64, OFF_SB = OFF_SA + BM * 4;
    constexpr int OFF_SPARE = OFF_SB + BN * 4;  // 256 B sink for the scale DMAs of idle waves
    constexpr int STAGE = OFF_SPARE + 256;
    static_assert(!SWIGLU || WN == 1, "the SwiGLU epilogue needs whole 128-column blocks per wave");
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
    const int wm = WN == 1 ? wave : wave >> 1, wn = WN == 1 ? 0 : wave & 1;
    const int KB = a.K / 128;  // stages

    // ---- DMA sources ------------------------------------------------------------------
    // A codes: instruction q (of this wave's PA) fills rows 8 (wave PA + q) + 0..7;
    // lane L owns row L/8, physical chunk L%8.
    const uint8_t *pa[PA];
#pragma unroll
    for (int q = 0; q < PA; ++q) {
        int r = 8 * (wave * PA + q) + (lane >> 3);
        long grow = row0 + (r < nrows ? r : 0);
        long src = GATHER ? row_token(grow, a.row_to_slot, a.T, a.k) : grow;
        pa[q] = a.A + src * a.K + (((lane & 7) ^ ((r >> 1) & 7)) << 4);
    }
    // A scales: wave w < ISA * 4 covers rows 64 w' .. (one dword per lane)
    const float *psa = nullptr;
    {
        int r = 64 * wave + lane;
        if (r < BM) {
            long grow = row0 + (r < nrows ? r : 0);
            long src = GATHER ? row_token(grow, a.row_to_slot, a.T, a.k) : grow;
            psa = a.As + src * KB;
        }
    }
    // B codes: instruction q fills rows 16 (wave PB + q) + 0..15; lane L owns row L/4, chunk L%4
    const int f0 = nt * (BN / 2), n0 = nt * BN;
    auto wrow_of = [&](int r) -> long {
        return SWIGLU ? (r < BN / 2 ? f0 + r : a.F + f0 + r - BN / 2) : n0 + r;
    };
    const uint8_t *pb[PB];
#pragma unroll
    for (int q = 0; q < PB; ++q) {
        int r = 16 * (wave * PB + q) + (lane >> 2);
        pb[q] = a.B + ((long)g * a.Ntot + wrow_of(r)) * (a.K / 2) + (((lane & 3) ^ ((r >> 2) & 3)) << 4);
    }
    const uint8_t *psb = nullptr;
    {
        int r = 64 * wave + lane;
        if (r < BN) psb = a.Bs + ((long)g * a.Ntot + wrow_of(r)) * (a.K / 32);
    }
    // Every wave issues exactly PER DMA instructions per stage, so the counted vmcnt waits
    // hold for all of them: a wave with no scale rows of its own re-loads row 0's scale
    // into the spare slot.
    const bool has_sa = 64 * wave < BM, has_sb = 64 * wave < BN;
    constexpr int PER = PA + PB + 2;
    if (!has_sa) psa = a.As + (GATHER ? row_token(row0, a.row_to_slot, a.T, a.k) : (long)row0) * KB;
    if (!has_sb) psb = a.Bs + ((long)g * a.Ntot + wrow_of(0)) * (a.K / 32);
    const int sa_dst = has_sa ? OFF_SA + wave * 256 : OFF_SPARE;
    const int sb_dst = has_sb ? OFF_SB + wave * 256 : OFF_SPARE;

    // ---- fragment offsets -------------------------------------------------------------
    const int khalf = lane >> 5;
    int aoff[2][TM][2], boff[2][TN], arow[TM], brow[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) arow[i] = wm * (BM / WM) + i * 32 + (lane & 31);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        int base;
        if (SWIGLU) base = j < TN / 2 ? j * 32 : BN / 2 + (j - TN / 2) * 32;
        else base = wn * (BN / WN) + j * 32;
        brow[j] = base + (lane & 31);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            // For the fp8 A operand of v_mfma_scale_f32_32x32x64_f8f6f4, lane half kh holds
            // K {16 kh .. 16 kh + 15} and {32 + 16 kh .. 32 + 16 kh + 15} of the 64-wide step
            // (while the fp4 B operand holds 32 consecutive K, its e8m0 block): chunks
            // 4 h + kh and 4 h + 2 + kh of the 128-byte row.  Verified against a CPU model
            // of the instruction, scales included.
            aoff[h][i][0] = sw128(arow[i], h * 4 + khalf);
            aoff[h][i][1] = sw128(arow[i], h * 4 + 2 + khalf);
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) boff[h][j] = OFF_B + sw64(brow[j], h * 2 + khalf);
    }

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = (f32x16){};

#define FP8_DMA(q, stg, kt_)                                                                        \
    do {                                                                                            \
        uint8_t *s_ = lds + (stg) * STAGE;                                                          \
        const int kt2_ = (kt_);                                                                     \
        if ((q) < PA) lds_dma16(pa[(q) < PA ? (q) : 0] + kt2_ * 128, s_ + (wave * PA + (q)) * 1024);    \
        else if ((q) < PA + PB)                                                                     \
            lds_dma16(pb[(q) >= PA && (q) < PA + PB ? (q) - PA : 0] + kt2_ * 64,                        \
                  s_ + OFF_B + (wave * PB + (q) - PA) * 1024);                                      \
        else if ((q) == PA + PB)                                                                    \
            lds_dma4(psa + kt2_, s_ + sa_dst);                                                          \
        else                                                                                        \
            lds_dma4(psb + kt2_ * 4, s_ + sb_dst);                                                      \
    } while (0)

    // fragments: A (two 16-byte reads), B (one read), for k64 step h of a stage
    i32x4 fa0[TM][2], fb0[TN], fa1[TM][2], fb1[TN];
    int sa0[TM], sb0[TN];  // e8m0 of the stage (A per row; B dword of 4 blocks per column)
#define FP8_FRAG(FA, FB, u, stg, h)                                                                 \
    do {                                                                                            \
        const uint8_t *s_ = lds + (stg) * STAGE;                                                    \
        if ((u) < 2 * TM) {                                                                         \
            const int i_ = (u) >> 1, c_ = (u) & 1;                                                  \
            FA[i_ < TM ? i_ : 0][c_] = *(const i32x4 *)(s_ + aoff[h][i_ < TM ? i_ : 0][c_]);        \
        } else {                                                                                    \
            const int j_ = (u) - 2 * TM;                                                            \
            FB[j_ < TN ? j_ : 0] = *(const i32x4 *)(s_ + boff[h][j_ < TN ? j_ : 0]);                \
        }                                                                                           \
    } while (0)
#define FP8_SCALES(SA, SB, stg)                                                                     \
    do {                                                                                            \
        const uint8_t *s_ = lds + (stg) * STAGE;                                                    \
        _Pragma("unroll") for (int i = 0; i < TM; ++i)                                              \
            SA[i] = (int)((*(const uint32_t *)(s_ + OFF_SA + arow[i] * 4) >> 23) & 0xFF);           \
        _Pragma("unroll") for (int j = 0; j < TN; ++j)                                              \
            SB[j] = *(const int *)(s_ + OFF_SB + brow[j] * 4);                                      \
    } while (0)
#define FP8_MFMA(FA, FB, m, h)                                                                      \
    do {                                                                                            \
        const int i_ = (m) / TN, j_ = (m) % TN;                                                     \
        i32x8 av_ = {FA[i_][0][0], FA[i_][0][1], FA[i_][0][2], FA[i_][0][3],                        \
                     FA[i_][1][0], FA[i_][1][1], FA[i_][1][2], FA[i_][1][3]};                       \
        i32x8 bv_ = {FB[j_][0], FB[j_][1], FB[j_][2], FB[j_][3], 0, 0, 0, 0};                       \
        const int sb_ = (sb0[j_] >> (8 * ((h) * 2 + khalf))) & 0xFF;                                \
        acc[i_][j_] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av_, bv_, acc[i_][j_], 0, 4, 0, \
                                                                      sa0[i_], 0, sb_);             \
    } while (0)
#define FP8_BARRIER()                          \
    do {                                       \
        asm volatile("" ::: "memory");         \
        __builtin_amdgcn_s_barrier();          \
        asm volatile("" ::: "memory");         \
    } while (0)

    constexpr int NR = 2 * TM + TN;  // fragment reads per k64 step
    constexpr int NM = TM * TN;      // MFMAs per k64 step
    constexpr int NG = NM;           // issue groups per k64 step (one MFMA each)

    // prologue
#pragma unroll
    for (int s0 = 0; s0 < PD; ++s0)
#pragma unroll
        for (int q = 0; q < PER; ++q) FP8_DMA(q, s0, s0 < KB ? s0 : KB - 1);
    wait_vmcnt<(PD - 1) * PER>();
    FP8_BARRIER();
#pragma unroll
    for (int u = 0; u < NR; ++u) FP8_FRAG(fa0, fb0, u, 0, 0);
    FP8_SCALES(sa0, sb0, 0);

    for (int kt = 0; kt < KB; ++kt) {
        const int cur = kt % NS, nxt = (kt + 1) % NS, pre = (kt + PD) % NS;
        const int kpre = kt + PD < KB ? kt + PD : KB - 1;
        wait_lgkmcnt0();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
#pragma unroll
            for (int q = gi * PER / NG; q < (gi + 1) * PER / NG; ++q) FP8_DMA(q, pre, kpre);
#pragma unroll
            for (int u = gi * NR / NG; u < (gi + 1) * NR / NG; ++u) FP8_FRAG(fa1, fb1, u, cur, 1);
            FP8_MFMA(fa0, fb0, gi, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        wait_lgkmcnt0();
        wait_vmcnt<(PD - 1) * PER>();
        FP8_BARRIER();
        __builtin_amdgcn_sched_barrier(0);
        int sa1[TM], sb1[TN];
        FP8_SCALES(sa1, sb1, nxt);
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
#pragma unroll
            for (int u = gi * NR / NG; u < (gi + 1) * NR / NG; ++u) FP8_FRAG(fa0, fb0, u, nxt, 0);
            FP8_MFMA(fa1, fb1, gi, 1);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < TM; ++i) sa0[i] = sa1[i];
#pragma unroll
        for (int j = 0; j < TN; ++j) sb0[j] = sb1[j];
    }
    wait_vmcnt<0>();
#undef FP8_DMA
#undef FP8_FRAG
#undef FP8_SCALES
#undef FP8_MFMA
#undef FP8_BARRIER

    // ---- epilogue -----------------------------------------------------------------------
    if (SWIGLU) {
        uint8_t *hq = (uint8_t *)a.C;
        constexpr int TNh = TN / 2;  // 4 column tiles of 32 = the 128-column block
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = wm * (BM / WM) + i * 32 + 8 * (r >> 2) + 4 * khalf + (r & 3);
                float hv[TNh];
                float amax = 0.0f;
#pragma unroll
                for (int j = 0; j < TNh; ++j) {
                    float gv = acc[i][j][r], uv = acc[i][j + TNh][r];
                    hv[j] = swiglu(gv, uv);
                    amax = fmaxf(amax, fabsf(hv[j]));
                }
                // the 32 lanes of this half-wave hold the 128 columns of the row
                amax = half_wave_max(amax);
                if (row < nrows) {
                    const int e = e4m3_block_exponent(amax);
                    const float inv = ldexpf(1.0f, -e);
                    const long grow = row0 + row;
#pragma unroll
                    for (int j = 0; j < TNh; ++j) {
                        uint32_t c = cvt_e4m3x2(hv[j] * inv, 0.0f) & 0xFFu;
                        hq[grow * a.F + f0 + j * 32 + (lane & 31)] = (uint8_t)c;
                    }
                    if ((lane & 31) == 0) a.Cs[grow * (a.F / 128) + f0 / 128] = ldexpf(1.0f, e);
                }
            }
        }
    } else {
        uint16_t *y = (uint16_t *)a.C;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = wm * (BM / WM) + i * 32 + 8 * (r >> 2) + 4 * khalf + (r & 3);
                if (row >= nrows) continue;
                const long grow = row0 + row;
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    int col = n0 + wn * (BN / WN) + j * 32 + (lane & 31);
                    y[grow * a.ldc + col] = f32_to_bf16(acc[i][j][r]);
                }
            }
        }
    }
}

// ---- 8 waves on a 256 x 256 tile ------------------------------------------------------
//
// Two waves per SIMD (512 threads), so one wave's MFMAs cover the other's LDS and barrier
// waits.  linear1: each wave owns 32 rows x (128 gate + 128 up) columns, which keeps the
// SwiGLU and h-quantisation epilogue inside the wave; linear2 the same 32 rows x 256 columns.
// K advances 128 per stage (two k64 MFMA steps); NS = 3 stages of 50 KB (A codes 256 x 128,
// B codes 256 x 64, A scales, B scale dwords).  Each pass multiplies k64 step 0 of stage kt
// while reading step 1's fragments, passes the one barrier (stage kt + 1 published, every
// wave done with stage kt), then multiplies step 1 while reading step 0 of stage kt + 1.
// Loads are split as in the bf16 8-wave tile: stage s's B codes and scale dword go out in
// the first half of pass s - NS + 1, its A codes in the second half of pass s - NS, both
// into the buffer freed by the barrier of pass s - NS, interleaved one by one with MFMAs.
// With one 32-row block per wave each B fragment feeds one MFMA per k64 step and
// is refilled right after it, which keeps the wave within 256 VGPRs without spilling.  A
// wave whose rows all lie past a group's last, partial tile skips its fragment reads and
// MFMAs (it still loads its share and keeps the barriers), and the row groups are laid out
// so that the first 128 rows take one wave per SIMD.  The k accumulation order is that of
// fp8_tile, so results are identical bit for bit.
//
// A codes are addressed by 32-bit byte offsets: callers keep A below 4 GiB.  One tile per
// call; lds holds fp8_tile8_lds() bytes; same caller contract as fp8_tile.
constexpr size_t fp8_tile8_lds() { return 3 * (size_t)(256 * 128 + 256 * 64 + 256 * 4 + 256 * 4); }

// TM x TN blocks of 32x32 per wave; linear1 (SWIGLU): TM = 1, TN = 8 (32 rows, 128 gate + 128 up
// columns); linear2 runs TM = 1, TN = 8 as well (32 rows x 256 columns: same DeepSeek-V3 linear2
// at T = 8192 in 1.39 against 1.56 ms with TM = 2, TN = 4, the same bits); TM = 2, TN = 4 (64
// rows x 128 columns, double-buffered fragments) stays available.  half: -1 the whole tile, 0 / 1
// its rows 0..127 / 128..255 (an empty half returns at once); the first 128 rows are one
// wave per SIMD's, and every output element takes the same k order either way.
template <int TM, int TN, bool SWIGLU, bool GATHER>
__device__ __forceinline__ void fp8_tile8(const Fp8Args &a, int tile, uint8_t *lds, int half = -1) {
    constexpr int BM = 256, BN = 256, NS = 3;
    constexpr int WMW = BM / (32 * TM), WNW = 8 / WMW;
    static_assert(WNW * TN * 32 == BN, "wave grid");
    static_assert(!SWIGLU || (TM == 1 && TN == 8), "SwiGLU needs 128 gate + 128 up columns per wave");
    constexpr int PA = 4, PB = 2;                       // A / B code DMA instructions per wave and stage
    constexpr int PER = PA + PB + 1;                    // + one scale instruction
    constexpr int OFF_B = BM * 128, OFF_SA = OFF_B + BN * 64, OFF_SB = OFF_SA + BM * 4;
    constexpr int STAGE = OFF_SB + BN * 4;

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
        int mt;
        grouped_tile<kTileGroup>(local, mtiles, (a.tile_start[g + 1] - a.tile_start[g]) / mtiles, mt, nt);
        row0 = rb + mt * BM;
        nrows = min(BM, cnt - mt * BM);
        if (half >= 0) {
            row0 += 128 * half;
            nrows = half ? nrows - 128 : min(nrows, 128);
        }
    }
    if (nrows <= 0) return;
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    // linear2: waves 0-3 (one per SIMD) cover rows 0-127, so a short tile keeps every SIMD busy
    const int wm = TM == 1 ? wave : (wave & 1) + 2 * (wave >> 2), wn = TM == 1 ? 0 : (wave >> 1) & 1;
    static_assert(TM == 1 || (WMW == 4 && WNW == 2), "wave grid");
    const int KB = a.K / 128;

    uint32_t pa_off[PA];  // A is at most 4 GiB: byte offsets from the uniform base
#pragma unroll
    for (int q = 0; q < PA; ++q) {
        const int r = 8 * (wave * PA + q) + (lane >> 3);
        const long grow = row0 + (r < nrows ? r : 0);
        const long src = GATHER ? row_token(grow, a.row_to_slot, a.T, a.k) : grow;
        pa_off[q] = (uint32_t)(src * a.K + (((lane & 7) ^ ((r >> 1) & 7)) << 4));
    }
#define pa_at(q, kt) (a.A + pa_off[q] + (uint32_t)(kt) * 128u)
    const int f0 = nt * (BN / 2), n0 = nt * BN;
    auto wrow_of = [&](int r) -> long { return SWIGLU ? (r < BN / 2 ? f0 + r : a.F + f0 + r - BN / 2) : n0 + r; };
    const uint8_t *pb[PB];
#pragma unroll
    for (int q = 0; q < PB; ++q) {
        const int r = 16 * (wave * PB + q) + (lane >> 2);
        pb[q] = a.B + ((long)g * a.Ntot + wrow_of(r)) * (a.K / 2) + (((lane & 3) ^ ((r >> 2) & 3)) << 4);
    }
    // scales: waves 0-3 load the A scales of rows 64 w + lane, waves 4-7 the B scale dwords
    const uint8_t *psc;
    int sc_dst, sc_step;
    if (wave < 4) {
        const int r = 64 * wave + lane;
        const long grow = row0 + (r < nrows ? r : 0);
        const long src = GATHER ? row_token(grow, a.row_to_slot, a.T, a.k) : grow;
        psc = (const uint8_t *)(a.As + src * KB);
        sc_dst = OFF_SA + wave * 256;
        sc_step = 4;
    } else {
        const int r = 64 * (wave - 4) + lane;
        psc = a.Bs + ((long)g * a.Ntot + wrow_of(r)) * (a.K / 32);
        sc_dst = OFF_SB + (wave - 4) * 256;
        sc_step = 4;
    }

    const int khalf = lane >> 5;
    int aoff[2][TM][2], boff[2][TN], arow[TM], brow[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) arow[i] = wm * (32 * TM) + i * 32 + (lane & 31);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int base = SWIGLU ? (j < TN / 2 ? j * 32 : BN / 2 + (j - TN / 2) * 32) : wn * (32 * TN) + j * 32;
        brow[j] = base + (lane & 31);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            aoff[h][i][0] = sw128(arow[i], h * 4 + khalf);
            aoff[h][i][1] = sw128(arow[i], h * 4 + 2 + khalf);
        }
        // the swizzle key of row 32 j + l does not depend on j: block j sits 2048 bytes further
#pragma unroll
        for (int j = 0; j < TN; ++j) boff[h][j] = OFF_B + sw64(brow[0], h * 2 + khalf) + (brow[j] - brow[0]) * 64;
    }

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = (f32x16){};

#define F8_BARRIER()                           \
    do {                                       \
        asm volatile("" ::: "memory");         \
        __builtin_amdgcn_s_barrier();          \
        asm volatile("" ::: "memory");         \
    } while (0)
    // part 1 of stage s: B codes and the scale dword; part 2: A codes
#define F8_DMA1(s)                                                                                  \
    do {                                                                                            \
        const int s_ = (s);                                                                         \
        uint8_t *st_ = lds + (s_ % NS) * STAGE;                                                     \
        const int kt_ = s_ < KB ? s_ : KB - 1;                                                      \
        _Pragma("unroll") for (int q = 0; q < PB; ++q)                                              \
            lds_dma16(pb[q] + kt_ * 64, st_ + OFF_B + (wave * PB + q) * 1024);                      \
        lds_dma4(psc + kt_ * sc_step, st_ + sc_dst);                                                \
    } while (0)
#define F8_DMA2(s)                                                                                  \
    do {                                                                                            \
        const int s_ = (s);                                                                         \
        uint8_t *st_ = lds + (s_ % NS) * STAGE;                                                     \
        const int kt_ = s_ < KB ? s_ : KB - 1;                                                      \
        _Pragma("unroll") for (int q = 0; q < PA; ++q)                                              \
            lds_dma16(pa_at(q, kt_), st_ + (wave * PA + q) * 1024);                             \
    } while (0)
#define F8_READ(FA, FB, s, h)                                                                       \
    do {                                                                                            \
        const uint8_t *st_ = lds + ((s) % NS) * STAGE;                                              \
        _Pragma("unroll") for (int i = 0; i < TM; ++i) {                                            \
            FA[i][0] = *(const i32x4 *)(st_ + aoff[h][i][0]);                                       \
            FA[i][1] = *(const i32x4 *)(st_ + aoff[h][i][1]);                                       \
        }                                                                                           \
        _Pragma("unroll") for (int j = 0; j < TN; ++j) FB[j] = *(const i32x4 *)(st_ + boff[h][j]); \
    } while (0)
#define F8_SCALES(SA, SB, s)                                                                        \
    do {                                                                                            \
        const uint8_t *st_ = lds + ((s) % NS) * STAGE;                                              \
        _Pragma("unroll") for (int i = 0; i < TM; ++i)                                              \
            SA[i] = (int)((*(const uint32_t *)(st_ + OFF_SA + arow[i] * 4) >> 23) & 0xFF);          \
        _Pragma("unroll") for (int j = 0; j < TN; ++j) SB[j] = *(const int *)(st_ + OFF_SB + brow[j] * 4); \
    } while (0)
#define F8_MMA(FA, FB, SA, SB, h)                                                                   \
    do {                                                                                            \
        _Pragma("unroll") for (int i = 0; i < TM; ++i)                                              \
            _Pragma("unroll") for (int j = 0; j < TN; ++j) {                                        \
                i32x8 av_ = {FA[i][0][0], FA[i][0][1], FA[i][0][2], FA[i][0][3],                    \
                             FA[i][1][0], FA[i][1][1], FA[i][1][2], FA[i][1][3]};                   \
                i32x8 bv_ = {FB[j][0], FB[j][1], FB[j][2], FB[j][3], 0, 0, 0, 0};                   \
                const int sb_ = (SB[j] >> (8 * ((h) * 2 + khalf))) & 0xFF;                          \
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av_, bv_, acc[i][j], 0, 4, 0, \
                                                                            SA[i], 0, sb_);         \
            }                                                                                       \
    } while (0)
#define F8_INTERLEAVE(NR, ND)                                                                       \
    do {                                                                                            \
        _Pragma("unroll") for (int m_ = 0; m_ < TM * TN; ++m_) {                                    \
            if (m_ < (ND)) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);                       \
            __builtin_amdgcn_sched_group_barrier(0x100, ((NR) + TM * TN - 1) / (TM * TN), 0);       \
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                      \
        }                                                                                           \
        __builtin_amdgcn_sched_barrier(0);                                                          \
    } while (0)

    if constexpr (TM == 1) {
        // one 32-row block per wave: each B fragment feeds one MFMA per k64 step, so it is
        // refilled right after that MFMA (register rotation); only the A fragment is doubled
        i32x4 fa0[2], fa1[2], fb[TN];
        int sa0, sb0[TN];
#define F8_RA(FA, s, h)                                                                             \
        do {                                                                                        \
            const uint8_t *st_ = lds + ((s) % NS) * STAGE;                                          \
            FA[0] = *(const i32x4 *)(st_ + aoff[h][0][0]);                                          \
            FA[1] = *(const i32x4 *)(st_ + aoff[h][0][1]);                                          \
        } while (0)
#define F8_RB(j, s, h) fb[j] = *(const i32x4 *)(lds + ((s) % NS) * STAGE + boff[h][j])
#define F8_M1(FA, j, h)                                                                             \
        do {                                                                                        \
            i32x8 av_ = {FA[0][0], FA[0][1], FA[0][2], FA[0][3], FA[1][0], FA[1][1], FA[1][2], FA[1][3]}; \
            i32x8 bv_ = {fb[j][0], fb[j][1], fb[j][2], fb[j][3], 0, 0, 0, 0};                       \
            const int sb_ = (sb0[j] >> (8 * ((h) * 2 + khalf))) & 0xFF;                             \
            acc[0][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av_, bv_, acc[0][j], 0, 4, 0, sa0, 0, sb_); \
        } while (0)
#define F8_SC(s)                                                                                    \
        do {                                                                                        \
            const uint8_t *st_ = lds + ((s) % NS) * STAGE;                                          \
            sa0 = (int)((*(const uint32_t *)(st_ + OFF_SA + arow[0] * 4) >> 23) & 0xFF);            \
            _Pragma("unroll") for (int j = 0; j < TN; ++j)                                          \
                sb0[j] = *(const int *)(st_ + OFF_SB + brow[0] * 4 + (j < TN / 2 ? j : BN / 2 / 32 + j - TN / 2) * 128); \
        } while (0)
        // single DMA instructions: part 1 (q < PB: B codes, q == PB: scales), part 2 (A codes)
#define F8_D1(s, q)                                                                                 \
        do {                                                                                        \
            const int s_ = (s);                                                                     \
            uint8_t *st_ = lds + (s_ % NS) * STAGE;                                                 \
            const int kt_ = s_ < KB ? s_ : KB - 1;                                                  \
            if ((q) < PB) lds_dma16(pb[(q) < PB ? (q) : 0] + kt_ * 64, st_ + OFF_B + (wave * PB + (q)) * 1024); \
            else lds_dma4(psc + kt_ * sc_step, st_ + sc_dst);                                       \
        } while (0)
#define F8_D2(s, q)                                                                                 \
        do {                                                                                        \
            const int s_ = (s);                                                                     \
            uint8_t *st_ = lds + (s_ % NS) * STAGE;                                                 \
            const int kt_ = s_ < KB ? s_ : KB - 1;                                                  \
            lds_dma16(pa_at(q, kt_), st_ + (wave * PA + (q)) * 1024);                           \
        } while (0)
#pragma unroll
        for (int s0 = 0; s0 < NS - 1; ++s0) {
            F8_DMA2(s0);
            F8_DMA1(s0);
        }
        F8_DMA2(NS - 1);
        wait_vmcnt<(NS - 2) * PER + PA>();
        F8_BARRIER();
        F8_RA(fa0, 0, 0);
#pragma unroll
        for (int j = 0; j < TN; ++j) F8_RB(j, 0, 0);
        F8_SC(0);
        wait_lgkmcnt0();
        // a wave whose 32 rows lie past the tile's rows only loads and keeps the barriers
#define F8_LOOP1(ACT)                                                                               \
        for (int kt = 0; kt < KB; ++kt) {                                                           \
            const int nx = kt + 1 < KB ? kt + 1 : kt;                                               \
            if (ACT) F8_RA(fa1, kt, 1);                                                             \
            __builtin_amdgcn_sched_barrier(0);                                                      \
            _Pragma("unroll") for (int j = 0; j < TN; ++j) {                                        \
                if (ACT) {                                                                          \
                    F8_M1(fa0, j, 0);                                                               \
                    F8_RB(j, kt, 1);                                                                \
                }                                                                                   \
                if ((j & 1) && j / 2 < PB + 1) F8_D1(kt + NS - 1, j / 2);                           \
                __builtin_amdgcn_sched_barrier(0);                                                  \
            }                                                                                       \
            wait_vmcnt<(NS - 2) * PER>();                                                           \
            wait_lgkmcnt0();                                                                        \
            F8_BARRIER();                                                                           \
            __builtin_amdgcn_sched_barrier(0);                                                      \
            if (ACT) F8_RA(fa0, nx, 0);                                                             \
            __builtin_amdgcn_sched_barrier(0);                                                      \
            _Pragma("unroll") for (int j = 0; j < TN; ++j) {                                        \
                if (ACT) {                                                                          \
                    F8_M1(fa1, j, 1);                                                               \
                    F8_RB(j, nx, 0);                                                                \
                }                                                                                   \
                if (!(j & 1)) F8_D2(kt + NS, j / 2);                                                \
                __builtin_amdgcn_sched_barrier(0);                                                  \
            }                                                                                       \
            if (ACT) F8_SC(nx); /* after every MFMA of stage kt has taken its scales */             \
            wait_lgkmcnt0();                                                                        \
        }
        if (wave * 32 < nrows) {
            F8_LOOP1(true)
        } else {
            F8_LOOP1(false)
        }
#undef F8_LOOP1
#undef F8_RA
#undef F8_RB
#undef F8_M1
#undef F8_SC
#undef F8_D1
#undef F8_D2
    } else {
    i32x4 fa0[TM][2], fb0[TN], fa1[TM][2], fb1[TN];
        int sa0[TM], sb0[TN];
        // prologue: stages 0 .. NS-2 whole and part 2 of stage NS-1; stage 0 published
    #pragma unroll
        for (int s0 = 0; s0 < NS - 1; ++s0) {
            F8_DMA2(s0);
            F8_DMA1(s0);
        }
        F8_DMA2(NS - 1);
        wait_vmcnt<(NS - 2) * PER + PA>();
        F8_BARRIER();
        F8_READ(fa0, fb0, 0, 0);
        F8_SCALES(sa0, sb0, 0);
        wait_lgkmcnt0();
        // a wave whose rows lie past the tile's rows only loads and keeps the barriers
#define F8_LOOP2(ACT)                                                                               \
        for (int kt = 0; kt < KB; ++kt) {                                                           \
            const int nx = kt + 1 < KB ? kt + 1 : kt;                                               \
            if (ACT) F8_READ(fa1, fb1, kt, 1);                                                      \
            F8_DMA1(kt + NS - 1);                                                                   \
            if (ACT) {                                                                              \
                F8_MMA(fa0, fb0, sa0, sb0, 0);                                                      \
                F8_INTERLEAVE(2 * TM + TN, PB + 1);                                                 \
            }                                                                                       \
            wait_vmcnt<(NS - 2) * PER>();                                                           \
            wait_lgkmcnt0();                                                                        \
            F8_BARRIER();                                                                           \
            __builtin_amdgcn_sched_barrier(0);                                                      \
            F8_DMA2(kt + NS);                                                                       \
            if (ACT) {                                                                              \
                F8_READ(fa0, fb0, nx, 0);                                                           \
                F8_MMA(fa1, fb1, sa0, sb0, 1);                                                      \
                F8_INTERLEAVE(2 * TM + TN, PA);                                                     \
                F8_SCALES(sa0, sb0, nx); /* after every MFMA of stage kt has taken its scales */    \
            }                                                                                       \
            wait_lgkmcnt0();                                                                        \
        }
        if (wm * 32 * TM < nrows) {
            F8_LOOP2(true)
        } else {
            F8_LOOP2(false)
        }
#undef F8_LOOP2
    }
    wait_vmcnt<0>();
#undef pa_at
#undef F8_BARRIER
#undef F8_DMA1
#undef F8_DMA2
#undef F8_READ
#undef F8_SCALES
#undef F8_MMA
#undef F8_INTERLEAVE

    if (SWIGLU) {
        uint8_t *hq = (uint8_t *)a.C;
        constexpr int TNh = TN / 2;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = wm * (32 * TM) + i * 32 + 8 * (r >> 2) + 4 * khalf + (r & 3);
                float hv[TNh];
                float amax = 0.0f;
#pragma unroll
                for (int j = 0; j < TNh; ++j) {
                    const float gv = acc[i][j][r], uv = acc[i][j + TNh][r];
                    hv[j] = swiglu(gv, uv);
                    amax = fmaxf(amax, fabsf(hv[j]));
                }
                amax = half_wave_max(amax);
                if (row < nrows) {
                    const int e = e4m3_block_exponent(amax);
                    const float inv = ldexpf(1.0f, -e);
                    const long grow = row0 + row;
#pragma unroll
                    for (int j = 0; j < TNh; ++j) {
                        const uint32_t c = cvt_e4m3x2(hv[j] * inv, 0.0f) & 0xFFu;
                        hq[grow * a.F + f0 + j * 32 + (lane & 31)] = (uint8_t)c;
                    }
                    if ((lane & 31) == 0) a.Cs[grow * (a.F / 128) + f0 / 128] = ldexpf(1.0f, e);
                }
            }
        }
    } else {
        uint16_t *y = (uint16_t *)a.C;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = wm * (32 * TM) + i * 32 + 8 * (r >> 2) + 4 * khalf + (r & 3);
                if (row >= nrows) continue;
                const long grow = row0 + row;
#pragma unroll
                for (int j = 0; j < TN; ++j) y[grow * a.ldc + n0 + wn * (32 * TN) + j * 32 + (lane & 31)] = f32_to_bf16(acc[i][j][r]);
            }
        }
    }
}

// ---- decode path: few rows per group ----------------------------------------------------
//
// With a handful of rows per expert the layer is weight streaming (HBM bound).  Each
// 64-lane wave owns one (group, 32-row tile, 32 output columns, K slice) and streams its
// 32 weight rows straight from HBM into the MFMA operands (no LDS), so thousands of
// independent waves keep enough loads in flight.  linear1 writes fp32 partial sums per K
// slice; a second pass adds the slices in order, applies SwiGLU and requantises h to e4m3
// per 128 columns; linear2 then streams W2 the same way and writes bf16 rows.

struct DecArgs {
    const uint8_t *A;            // linear1: xq [T, K] gathered by row; linear2: hq [rows, K]
    const float *As;             // [*, K/128]
    const int32_t *row_to_slot;  // linear1 only
    const int32_t *offsets, *tile_start;
    const uint8_t *B, *Bs;       // MXFP4 codes [G, N, K/2], e8m0 [G, N, K/32]
    float *part;                 // linear1: partials [ks][rows][N]
    uint16_t *Y;                 // linear2: y_perm [rows, N]
    long rows;
    int T, k, K, N, G, ks;
};

// One (group, 32-row tile, 32 output columns, K slice) tile; ts / offs may live in LDS.
// K advances 256 per iteration (four MFMAs): the four steps' B scales arrive in two dword
// loads and their A scales in two floats.
//
// COH (the persistent kernel): the outputs -- linear1 partial sums, linear2 rows -- are
// stored device-coherently, and linear2's A scales are loaded so (an h-scale line can
// hold rows of two row tiles, finished by different waves).  Every other input is read
// through the caches: each of its lines has a single writer, which finished before any
// reader was let in, so no cache can hold an older copy.
// PF: the next block's loads are issued before this block's MFMAs (two blocks in flight
// per wave, about 220 VGPRs); without PF one block at a time, for register-capped callers.
template <bool LIN1, bool COH, bool PF = false>
__device__ __forceinline__ void fp8_decode_tile(const DecArgs &a, int tile, const int32_t *ts, const int32_t *offs) {
    int lo = 0, hi = a.G - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (ts[mid] <= tile) lo = mid; else hi = mid - 1;
    }
    const int g = lo;
    const int rb = offs[g], cnt = offs[g + 1] - rb;
    const int mtiles = (cnt + 31) / 32, local = tile - ts[g];
    const int mt = local % mtiles, rest = local / mtiles;
    const int nt = LIN1 ? rest / a.ks : rest, ksl = LIN1 ? rest % a.ks : 0;
    const int row0 = rb + mt * 32, nrows = min(32, cnt - mt * 32);

    const int lane = lane_id(), kh = lane >> 5;
    const int r = lane & 31;
    const long grow = row0 + (r < nrows ? r : 0);
    const long src = LIN1 ? row_token(grow, a.row_to_slot, a.T, a.k) : grow;
    const int KB = a.K / 128;
    const size_t arow = (size_t)src * a.K;  // byte offset of the A row
    const float *psa = a.As + src * KB;
    const long n = (long)nt * 32 + r;
    const uint8_t *pb = a.B + ((long)g * a.N + n) * (a.K / 2);
    const uint8_t *psb = a.Bs + ((long)g * a.N + n) * (a.K / 32);
    const int kc = a.K / a.ks, kbeg = ksl * kc, kend = kbeg + kc;

    f32x16 acc = (f32x16){};
    int k0 = kbeg;
    // 256 of K per block (four MFMAs)
    struct Blk {
        i32x4 alo[4], ahi[4], bq[4];
        uint32_t sb01, sb23;
        float sa01, sa23;
    };
    auto load = [&](Blk &b, int kb) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int kk = kb + 64 * u;
            // fp8 A operand: K {16 kh..+15} and {32 + 16 kh..+15} of the 64-wide step
            b.alo[u] = *(const i32x4 *)(a.A + arow + kk + 16 * kh);
            b.ahi[u] = *(const i32x4 *)(a.A + arow + kk + 32 + 16 * kh);
            // fp4 B operand: 32 consecutive K from 32 kh, one e8m0 block
            b.bq[u] = *(const i32x4 *)(pb + (kk + 32 * kh) / 2);
        }
        b.sb01 = *(const uint32_t *)(psb + kb / 32);
        b.sb23 = *(const uint32_t *)(psb + kb / 32 + 4);
        b.sa01 = ldc<COH && !LIN1>(psa + kb / 128);
        b.sa23 = ldc<COH && !LIN1>(psa + kb / 128 + 1);
    };
    auto mma = [&](const Blk &b) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            i32x8 av = {b.alo[u][0], b.alo[u][1], b.alo[u][2], b.alo[u][3],
                        b.ahi[u][0], b.ahi[u][1], b.ahi[u][2], b.ahi[u][3]};
            i32x8 bv = {b.bq[u][0], b.bq[u][1], b.bq[u][2], b.bq[u][3], 0, 0, 0, 0};
            const uint32_t sbw = u < 2 ? b.sb01 : b.sb23;
            const int sb = (int)((sbw >> (8 * (2 * (u & 1) + kh))) & 0xFF);
            const int sa = (int)((__float_as_uint(u < 2 ? b.sa01 : b.sa23) >> 23) & 0xFF);
            acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 0, 4, 0, sa, 0, sb);
        }
    };
    const int nblk = (kend - kbeg) / 256;
    if (!PF) {
        for (int i = 0; i < nblk; ++i, k0 += 256) {
            Blk b0;
            load(b0, k0);
            mma(b0);
        }
    } else if (nblk > 0) {
        Blk b0, b1;
        load(b0, k0);
        int i = 0;
        for (; i + 2 <= nblk; i += 2) {
            if (i + 1 < nblk) load(b1, k0 + 256);
            mma(b0);
            if (i + 2 < nblk) load(b0, k0 + 512);
            mma(b1);
            k0 += 512;
        }
        if (i < nblk) {  // odd count: b0 holds the last block
            mma(b0);
            k0 += 256;
        }
    }
    for (; k0 < kend; k0 += 64) {
        const i32x4 lo4 = *(const i32x4 *)(a.A + arow + k0 + 16 * kh);
        const i32x4 hi4 = *(const i32x4 *)(a.A + arow + k0 + 32 + 16 * kh);
        const i32x4 b4 = *(const i32x4 *)(pb + (k0 + 32 * kh) / 2);
        const int sb = psb[(k0 + 32 * kh) / 32];
        const int sa = (int)((__float_as_uint(ldc<COH && !LIN1>(psa + k0 / 128)) >> 23) & 0xFF);
        i32x8 av = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
        i32x8 bv = {b4[0], b4[1], b4[2], b4[3], 0, 0, 0, 0};
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 0, 4, 0, sa, 0, sb);
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int row = 8 * (q >> 2) + 4 * kh + (q & 3);
        if (row >= nrows) continue;
        const long orow = row0 + row;
        if (LIN1) stc<COH>(a.part + ((long)ksl * a.rows + orow) * a.N + n, acc[q]);
        else stc16<COH>(a.Y, (size_t)(orow * a.N + n), f32_to_bf16(acc[q]));
    }
}

// Workgroup form of the decode tile (unfused path): four waves share one (group, 32-row
// tile, K slice) and take four neighbouring 32-column tiles, so workgroup tile w covers
// wave tiles whose order matches fp8_decode_tile's (row tile fastest, then K slice, then
// column tile) -- every group has a multiple of 4 column tiles, so the group's first
// workgroup tile is ts[g] / 4.  The MFMA operands and their order per K slice are those of
// fp8_decode_tile: results are identical bit for bit.  K / ks is a multiple of 1024 and at
// most 2048.
//
// Each workgroup runs a sequence of tiles (blockIdx.x, + gridDim.x, ...) as one stream:
// the weights are the only global loads of the K loop, D blocks of 256 K ahead through a
// register ring that runs on into the next tile's first blocks, and a tile's activation
// rows (at most rmax: a group never holds more rows than there are tokens) and their
// scales are copied into one of two LDS buffers by DMA while the previous tile streams.
// So a tile starts with its activations in LDS and its first weights in flight, instead of
// paying a chain of dependent round trips (the row's token, then its activations, then
// the weights) before its stream starts.  linear1 gathers its rows: the row_to_slot
// entries of a tile are copied into LDS one tile earlier still.  Every wait on that data
// rests on loads completing in order: a buffer's DMAs are issued before the weight loads
// of the tile before it, so the wait for that tile's last weight block covers them, and
// the barrier between tiles publishes every wave's copies.
//
// LDS: the tile plan (2 (G + 1) ints), then at the next 16-byte boundary two sets of 64
// row_to_slot entries, then two activation buffers, each rmax rows of K / ks + 16 bytes
// followed by their e8m0-carrying fp32 scales (rounded up to a whole 64-lane copy).
__host__ __device__ constexpr size_t fp8_gemv_off_src(int G) { return ((size_t)8 * (G + 1) + 15) / 16 * 16; }
__host__ __device__ constexpr size_t fp8_gemv_off_buf(int G) { return fp8_gemv_off_src(G) + 2 * 64 * 4; }
__host__ __device__ constexpr size_t fp8_gemv_scales(int rmax, int kc) {
    return ((size_t)rmax * (kc / 128) + 63) / 64 * 64;
}
__host__ __device__ constexpr size_t fp8_gemv_buf(int rmax, int kc) {
    return (size_t)rmax * (kc + 16) + fp8_gemv_scales(rmax, kc) * 4;
}
__host__ __device__ constexpr size_t fp8_gemv_lds(int G, int rmax, int kc) {
    return fp8_gemv_off_buf(G) + 2 * fp8_gemv_buf(rmax, kc);
}
// the tile plan is built in the same LDS before anything is staged (scan scratch included)
__host__ __device__ constexpr size_t fp8_gemv_lds_total(int G, int rmax, int kc) {
    const size_t a = fp8_gemv_lds(G, rmax, kc), b = (size_t)2 * (G + 1) * 4 + 256 * 4;
    return a > b ? a : b;
}

struct GemvTile {
    int g, row0, nrows, ksl, qc;
};

// Workgroup tile wt of the plan (tile starts, then group offsets); wave-uniform.
template <int QC>
__device__ __forceinline__ GemvTile gemv_tile(const int32_t *plan, int G, int ks, int rmax, int wt) {
    const int32_t *ts = plan, *offs = plan + G + 1;
    int lo = 0, hi = G - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (ts[mid] / (4 * QC) <= wt) lo = mid; else hi = mid - 1;
    }
    GemvTile t;
    t.g = __builtin_amdgcn_readfirstlane(lo);
    const int rb = __builtin_amdgcn_readfirstlane(offs[t.g]);
    const int cnt = __builtin_amdgcn_readfirstlane(offs[t.g + 1]) - rb;
    const int mtiles = (cnt + 31) / 32, local = wt - __builtin_amdgcn_readfirstlane(ts[t.g]) / (4 * QC);
    const int mt = local % mtiles, rest = local / mtiles;
    t.ksl = rest % ks;
    t.qc = rest / ks;
    t.row0 = rb + mt * 32;
    const int n = min(32, cnt - mt * 32);
    t.nrows = n < rmax ? n : rmax;  // rmax >= nrows whenever the routing is valid
    return t;
}

// The LDS copies of the weight stream, written as instructions the compiler does not see.
// It treats a pending global_load_lds as a FLAT access that may touch LDS and then answers
// every vmcnt wait it needs -- also the ones for the register loads of the weight ring --
// with vmcnt(0) until one has retired it; at a loop head this holds on every trip.  Hidden
// from it, the copies only make its own waits stricter than needed (loads complete in
// order), never too weak, and the caller waits for them itself.  M0 holds the LDS address;
// the LDS DMA reads M0 one wait state after the SALU write.  No output registers.  (m0 is
// reserved: nothing keeps a value in it across these -- every other LDS copy sets it right
// before its instruction.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ int lds_u32(const void *lds_block) {
    return __builtin_amdgcn_readfirstlane((int)(uintptr_t)(const __attribute__((address_space(3))) void *)lds_block);
}
__device__ __forceinline__ void lds_dma16_hidden(const void *g, uint8_t *lds_block) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds_u32(lds_block))
                 : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4_hidden(const void *g, uint8_t *lds_block) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds_u32(lds_block))
                 : "memory", "m0");
}
// the same copy at device scope (sc1): past the XCD's L2, for data other XCDs wrote
// coherently during the same launch
__device__ __forceinline__ void lds_dma4_hidden_sc1(const void *g, uint8_t *lds_block) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off sc1" ::"v"(g), "s"(lds_u32(lds_block))
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// The workgroup barrier of the weight stream: s_barrier with compiler fences only.  The
// memory-model barrier would wait for every outstanding load -- the LDS copies count as
// LDS writes -- and so drain the weight ring at each tile; here every wave waits for its
// own copies itself before the barrier (no LDS is written otherwise).
__device__ __forceinline__ void gemv_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// lds: fp8_gemv_lds_total(G, rmax, K / ks) bytes, the plan loaded; total workgroup tiles.
// QC column quads (4 x 32 columns each) per workgroup tile, NB 256-wide K blocks per slice
// (K / ks = 256 NB), D blocks in the weight ring (D divides NB).  Block t of a tile is K
// block t % NB of quad t / NB: each quad's 32 weight rows are streamed through in turn
// (measured on MI355X, 9 x 4096 x 7168: 32.5 us in this order against 43 us when every K
// block visits all four quads first), one accumulator per quad.  A ring deeper than a
// quad's slice (D = 2 NB) streams the quads in passes of D / NB, each pass with its own
// accumulators, stored as soon as the pass's last block has landed.
// COH (the persistent kernel): the outputs -- linear1 partial sums, linear2 rows -- are
// stored device-coherently, and linear2's activation scales (an h-scale line holds rows
// finished by different waves) are copied at device scope.
template <bool LIN1, int QC, int NB, int D, bool COH = false>
__device__ __forceinline__ void fp8_gemv_run(const DecArgs &a, int rmax, const int32_t *plan, uint8_t *lds,
                                             int total) {
    constexpr int KC = NB * 256, RS = KC + 16, NSC = KC / 128, NBT = QC * NB;
    constexpr int LPB = 5;  // global loads per weight block: four 16-byte code loads, one 8-byte scale load
    static_assert(NB == 4 || NB == 8, "K slices of 1024 or 2048");
    static_assert((NB % D == 0 || (D % NB == 0 && QC % (D / NB) == 0)) && D >= 2, "ring slot of block t is t % D");
    const int P = gridDim.x, b0 = blockIdx.x;
    if (b0 >= total) return;
    const int ntile = (total - 1 - b0) / P + 1;
    const int lane = lane_id(), kh = lane >> 5, r = lane & 31, wave = threadIdx.x >> 6;
    const size_t BUF = fp8_gemv_buf(rmax, KC), SCA = (size_t)rmax * RS;
    int32_t *srcb = (int32_t *)(lds + fp8_gemv_off_src(a.G));
    uint8_t *buf0 = lds + fp8_gemv_off_buf(a.G);
    const long tk = (long)a.T * a.k;

    // the row_to_slot entries of tile n's rows into srcb[n % 2] (lanes past the rows and
    // 32..63 re-read the first row)
    auto copy_src = [&](int n, const GemvTile &t) {
        if (LIN1 && wave == 0) {
            const long rr = t.row0 + (r < t.nrows ? r : 0);
            lds_dma4_hidden(a.row_to_slot + (rr < tk ? rr : 0), (uint8_t *)(srcb + (n & 1) * 64));
        }
    };
    // token feeding row rw of tile n (rows of the shared expert follow the routed ones);
    // clamped as row_token clamps.  The first tile's entries come from one load per lane
    // (raw0, lane r: row r) -- no copy to wait for before the tile's own copies -- later
    // tiles' from the entries staged in LDS.
    int raw0 = 0;
    auto src_of = [&](int n, const GemvTile &t, int rw) -> long {
        const long rr = (long)t.row0 + rw;
        if (!LIN1) return rr;
        long tok;
        if (rr < tk) {
            long s = n == 0 ? __shfl(raw0, rw, 64) : srcb[(n & 1) * 64 + rw];
            s = s < 0 ? 0 : (s >= tk ? tk - 1 : s);
            tok = s / a.k;
        } else {
            tok = rr - tk;
        }
        return tok < 0 ? 0 : (tok >= a.T ? a.T - 1 : tok);
    };
    // tile n's activation rows (1 KB copies, rows dealt to waves) and scales (64 per copy)
    // into buffer n % 2
    auto copy_act = [&](int n, const GemvTile &t) {
        uint8_t *la = buf0 + (n & 1) * BUF;
        const int kbeg = t.ksl * KC;
        for (int rw = wave; rw < t.nrows; rw += 4) {
            const long s = src_of(n, t, rw);
            const int shi = __builtin_amdgcn_readfirstlane((int)(s >> 32)),
                      slo = __builtin_amdgcn_readfirstlane((int)s);
            const long src = ((long)shi << 32) | (uint32_t)slo;
#pragma unroll
            for (int c = 0; c < KC / 1024; ++c)
                lds_dma16_hidden(a.A + (size_t)src * a.K + kbeg + c * 1024 + lane * 16, la + rw * RS + c * 1024);
        }
        const int nsc = t.nrows * NSC;
        float *lsa = (float *)(la + SCA);
        for (int q = wave; q * 64 < nsc; q += 4) {
            const int idx = q * 64 + lane < nsc ? q * 64 + lane : 0;
            const long src = src_of(n, t, idx / NSC);
            if (COH && !LIN1)
                lds_dma4_hidden_sc1(a.As + src * (a.K / 128) + kbeg / 128 + idx % NSC, (uint8_t *)(lsa + q * 64));
            else
                lds_dma4_hidden(a.As + src * (a.K / 128) + kbeg / 128 + idx % NSC, (uint8_t *)(lsa + q * 64));
        }
    };
    const long qsb = 128L * (a.K / 2), qss = 128L * (a.K / 32);  // the next quad: 128 columns on
    // this lane's weight codes and scales in quad 0 of a tile
    auto wptr = [&](const GemvTile &t, const uint8_t *&pb, const uint8_t *&ps) {
        const long n0 = (long)(4 * t.qc * QC + wave) * 32 + r;
        const int kbeg = t.ksl * KC;
        pb = a.B + ((long)t.g * a.N + n0) * (a.K / 2) + kbeg / 2 + 16 * kh;
        ps = a.Bs + ((long)t.g * a.N + n0) * (a.K / 32) + kbeg / 32;
    };

    // after the last tile the "next" blocks re-read the last quad's blocks NB - D .. NB - 2,
    // read moments before (in bounds, cached, unused); a ring deeper than a quad re-reads the
    // tile's first D - 1 blocks instead
    const uint8_t *pbC, *psC, *pbN, *psN;
    auto wptr_last = [&](const uint8_t *&pb, const uint8_t *&ps) {
        if constexpr (D > NB) {
            pb = pbC;
            ps = psC;
        } else {
            pb = pbC + (QC - 1) * qsb + (NB - D) * 128;
            ps = psC + (QC - 1) * qss + (NB - D) * 8;
        }
    };
    i32x4 bq[D][4];
    uint2 sbw[D];
    // block tl of the stream position: tl < NBT the current tile's block tl, else the next
    // tile's block tl - NBT
#define GEMV_LOAD(slot, tl_)                                                                      \
    do {                                                                                          \
        int tl = (tl_);                                                                           \
        asm volatile("" : "+v"(tl)); /* opaque: the loads issue here, are not hoisted */          \
        const bool nx_ = tl >= NBT;                                                               \
        const int tt_ = nx_ ? tl - NBT : tl;                                                      \
        const int c_ = tt_ / NB, i_ = tt_ % NB;                                                   \
        const uint8_t *pb_ = (nx_ ? pbN : pbC) + c_ * qsb + i_ * 128;                             \
        const uint8_t *ps_ = (nx_ ? psN : psC) + c_ * qss + i_ * 8;                               \
        _Pragma("unroll") for (int u = 0; u < 4; ++u) bq[slot][u] = *(const i32x4 *)(pb_ + 32 * u); \
        sbw[slot] = *(const uint2 *)ps_;                                                          \
    } while (0)

    GemvTile cur = gemv_tile<QC>(plan, a.G, a.ks, rmax, b0);
    GemvTile nxt = ntile > 1 ? gemv_tile<QC>(plan, a.G, a.ks, rmax, b0 + P) : cur;
    if (LIN1) {
        const long rr = cur.row0 + (r < cur.nrows ? r : 0);
        raw0 = a.row_to_slot[rr < tk ? rr : 0];
    }
    copy_act(0, cur);
    if (ntile > 1) copy_src(1, nxt);
    wptr(cur, pbC, psC);
    if (ntile > 1) wptr(nxt, pbN, psN);
    else wptr_last(pbN, psN);
#pragma unroll
    for (int j = 0; j < D - 1; ++j) GEMV_LOAD(j, j);
    // tile 0's copies and tile 1's row_to_slot entries landed: everything older than the
    // ring's loads
    wait_vmcnt<(D - 1) * LPB>();
    gemv_barrier();

    for (int n = 0; n < ntile; ++n) {
        // the next tile's activations (their row_to_slot entries landed before this tile
        // began), then the row_to_slot entries of the tile after it into the set this tile's
        // copies are done with
        GemvTile nn = nxt;
        if (n + 1 < ntile) {
            copy_act(n + 1, nxt);
            if (n + 2 < ntile) {
                nn = gemv_tile<QC>(plan, a.G, a.ks, rmax, b0 + (n + 2) * P);
                copy_src(n + 2, nn);
            }
        }
        const uint8_t *la = buf0 + (n & 1) * BUF;
        const int rr = r < cur.nrows ? r : 0;
        const uint8_t *arow = la + rr * RS;
        const float *asr = (const float *)(la + SCA) + rr * NSC;
        if constexpr (D <= NB) {
        f32x16 acc[QC];
#pragma unroll
        for (int c = 0; c < QC; ++c) acc[c] = (f32x16){};
        // an opaque trip count keeps the K loop a loop: unrolled over a whole tile, the
        // compiler hoists the ring's loads and runs out of registers
        int nbr = NB;
        asm volatile("" : "+s"(nbr));
#pragma unroll
        for (int c = 0; c < QC; ++c) {
            for (int i0 = 0; i0 < nbr; i0 += D) {
#pragma unroll
                for (int j = 0; j < D; ++j) {
                    const int i = i0 + j, t = c * NB + i;
                    GEMV_LOAD((j + D - 1) % D, t + D - 1);  // into the slot block t - 1 freed
                    wait_vmcnt<(D - 1) * LPB>();             // block t landed: LPB loads per block, in order
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const i32x4 lo4 = *(const i32x4 *)(arow + i * 256 + 64 * u + 16 * kh);
                        const i32x4 hi4 = *(const i32x4 *)(arow + i * 256 + 64 * u + 32 + 16 * kh);
                        i32x8 av = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
                        i32x8 bv = {bq[j][u][0], bq[j][u][1], bq[j][u][2], bq[j][u][3], 0, 0, 0, 0};
                        const uint32_t sw = (u >> 1) ? sbw[j].y : sbw[j].x;
                        const int sb = (int)((sw >> (8 * (2 * (u & 1) + kh))) & 0xFF);
                        const int sa = (int)((__float_as_uint(asr[2 * i + (u >> 1)]) >> 23) & 0xFF);
                        acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc[c], 0, 4, 0, sa, 0, sb);
                    }
                }
            }
        }
        // this tile's last block landed, and with it every copy issued before it (the next
        // tile's activations); the stores below come after the wait
        wait_vmcnt<(D - 1) * LPB>();
#pragma unroll
        for (int c = 0; c < QC; ++c) {
            const long ncol = (long)(4 * cur.qc * QC + wave) * 32 + r + (long)c * 128;
#pragma unroll
            for (int qq = 0; qq < 16; ++qq) {
                const int row = 8 * (qq >> 2) + 4 * kh + (qq & 3);
                if (row >= cur.nrows) continue;
                const long orow = cur.row0 + row;
                if constexpr (COH) {
                    if (LIN1) stc<true>(a.part + ((long)cur.ksl * a.rows + orow) * a.N + ncol, acc[c][qq]);
                    else stc16<true>(a.Y, (size_t)(orow * a.N + ncol), f32_to_bf16(acc[c][qq]));
                } else {
                    if (LIN1) a.part[((long)cur.ksl * a.rows + orow) * a.N + ncol] = acc[c][qq];
                    else a.Y[orow * a.N + ncol] = f32_to_bf16(acc[c][qq]);
                }
            }
        }
        } else {
            // the four MFMAs of K block i (256 wide) of a quad, weights from ring slot j
            auto mma_block = [&](f32x16 &acc_, int i, int j) {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const i32x4 lo4 = *(const i32x4 *)(arow + i * 256 + 64 * u + 16 * kh);
                    const i32x4 hi4 = *(const i32x4 *)(arow + i * 256 + 64 * u + 32 + 16 * kh);
                    i32x8 av = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
                    i32x8 bv = {bq[j][u][0], bq[j][u][1], bq[j][u][2], bq[j][u][3], 0, 0, 0, 0};
                    const uint32_t sw = (u >> 1) ? sbw[j].y : sbw[j].x;
                    const int sb = (int)((sw >> (8 * (2 * (u & 1) + kh))) & 0xFF);
                    const int sa = (int)((__float_as_uint(asr[2 * i + (u >> 1)]) >> 23) & 0xFF);
                    acc_ = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc_, 0, 4, 0, sa, 0, sb);
                }
            };
            // the rows of quad c's 32 columns
            auto store_quad = [&](const f32x16 &acc_, int c) {
                const long ncol = (long)(4 * cur.qc * QC + wave) * 32 + r + (long)c * 128;
#pragma unroll
                for (int qq = 0; qq < 16; ++qq) {
                    const int row = 8 * (qq >> 2) + 4 * kh + (qq & 3);
                    if (row >= cur.nrows) continue;
                    const long orow = cur.row0 + row;
                    if (LIN1) stc<COH>(a.part + ((long)cur.ksl * a.rows + orow) * a.N + ncol, acc_[qq]);
                    else stc16<COH>(a.Y, (size_t)(orow * a.N + ncol), f32_to_bf16(acc_[qq]));
                }
            };
            // passes of D / NB quads: block t = p D + j sits in ring slot j
            constexpr int QPR = D / NB;
            int npass = QC / QPR;
            asm volatile("" : "+s"(npass));  // a loop, not unrolled (see above)
            for (int p = 0; p < npass; ++p) {
                f32x16 accp[QPR];
#pragma unroll
                for (int c2 = 0; c2 < QPR; ++c2) accp[c2] = (f32x16){};
#pragma unroll
                for (int j = 0; j < D; ++j) {
                    GEMV_LOAD((j + D - 1) % D, p * D + j + D - 1);  // into the slot block t - 1 freed
                    wait_vmcnt<(D - 1) * LPB>();                      // block t landed
                    mma_block(accp[j / NB], j % NB, j);
                }
                // the pass's last block landed, and with it every copy issued before it
#pragma unroll
                for (int c2 = 0; c2 < QPR; ++c2) store_quad(accp[c2], p * QPR + c2);
            }
        }
        cur = nxt;
        nxt = nn;
        pbC = pbN;
        psC = psN;
        if (n + 2 < ntile) wptr(nxt, pbN, psN);
        else wptr_last(pbN, psN);
        gemv_barrier();  // every wave's copies for the next tile landed; this tile's buffer is free
    }
    wait_vmcnt<0>();
#undef GEMV_LOAD
}

// Sums the K slices of linear1 in order, applies SwiGLU and quantises h to e4m3 with one
// power-of-two scale per 128 columns.  One wave per (row, 128-column block): wid = row *
// (F / 128) + block.
template <bool COH>
__device__ __forceinline__ void decode_swiglu_wave(const float *__restrict__ part, long rows, int F, int ks,
                                                  uint8_t *__restrict__ hq, float *__restrict__ hs, long wid) {
    const int lane = lane_id();
    const int nfb = F / 128;
    const long r = wid / nfb;
    const int fb = (int)(wid % nfb), f = fb * 128 + 2 * lane;
    float gsum[2] = {0.0f, 0.0f}, usum[2] = {0.0f, 0.0f};
    for (int q = 0; q < ks; ++q) {
        const float *p = part + ((long)q * rows + r) * (2L * F);
        gsum[0] += ldc<COH>(p + f); gsum[1] += ldc<COH>(p + f + 1);
        usum[0] += ldc<COH>(p + F + f); usum[1] += ldc<COH>(p + F + f + 1);
    }
    float h[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) h[i] = swiglu(gsum[i], usum[i]);
    float amax = fmaxf(fabsf(h[0]), fabsf(h[1]));
    amax = wave_max(amax);
    const int e = e4m3_block_exponent(amax);
    const float inv = ldexpf(1.0f, -e);
    const uint32_t c = cvt_e4m3x2(h[0] * inv, h[1] * inv);
    stc16<COH>((uint16_t *)hq, (size_t)((r * F + f) / 2), (uint16_t)c);
    if (lane == 0) stc<COH>(hs + r * nfb + fb, ldexpf(1.0f, e));
}

}  // namespace moe
