// Expert FFN work items over dispatched rows (S8-S9), bf16 and fp32: linear1 (gate+up)
// with SwiGLU in the epilogue, then linear2, as grouped GEMMs over ragged expert groups.
//
// MoE lesson (factory.pai-world.com, "Mixture of Experts", "FFN swap"): each expert
// is an independent FFN, usually SwiGLU.  Mega MoE blog (donniechu.com, spec table)
// and Mega MoE wiki ("One-line definition"): linear1, SwiGLU and linear2 are the
// middle of the fused chain.  SwiGLU is read as silu(x Wg^T) * (x Wu^T), with
// W1 = [Wg; Wu] stacked along its output rows.
//
// Tiles: a group g of n_g rows is cut into ceil(n_g / BM) row tiles times the N
// tiles; a planning step writes the exclusive prefix of tiles per group, and each
// tile finds its (group, row tile, N tile) by binary search.  Within a group, row
// tiles vary fastest so that the tiles sharing one weight tile are neighbours, and
// neighbouring tiles are dealt to the same XCD (and its L2).
#pragma once

#include "common.hpp"

namespace moe {

// ---- bf16 grouped GEMM ----------------------------------------------------------
//
// C[rows, N] = A[rows, K] * B_g[N, K]^T per group, bf16 inputs, fp32 accumulation on
// v_mfma_f32_32x32x16_bf16.  256 threads = 2 x 2 waves, each owning a (BM/2) x (BN/2)
// block of 32x32 MFMA tiles.
//
// SWIGLU (linear1): the BN columns of a tile are BN/2 gate rows f0.. of W1 followed
// by the BN/2 up rows F+f0..; each wave holds matching gate and up accumulators,
// and the epilogue writes h = silu(gate) * up as bf16 [rows, F].
// Otherwise (linear2): the epilogue writes C as bf16 [rows, ldc].

struct GemmArgs {
    const uint16_t *A;           // linear1: x [T, K] (gathered by row); linear2: h [rows, K]
    const int32_t *row_to_slot;  // linear1 only
    const uint16_t *B;           // [G, Ntot, K]
    uint16_t *C;                 // linear1: h [rows, F]; linear2: y_perm [rows, ldc]
    const int32_t *offsets;      // [G+1]
    const int32_t *tile_start;   // [G+1]
    int T, k, K, Ntot, ldc, G, F;
};

template <int BM, int BN>
constexpr size_t bf16_tile_lds() { return 4 * (size_t)(BM + BN) * 64; }  // 4 stages of BK = 32

// ---- bf16 grouped GEMM, LDS DMA with a mid-stage barrier -----------------------------
//
// BK = 32 (two k16 MFMA steps per stage), NS = 4 LDS stages, DMA issued PD = 3 stages
// ahead.  Fragments are double-buffered in registers.  The one barrier per stage sits
// between the two k16 steps and publishes stage kt+1 (every wave has waited for its own
// DMA of it), so the first fragments of stage kt+1 are read while the second half of
// stage kt runs on the MFMAs.  Buffer (kt+3) % 4 held stage kt-1, whose last fragments
// were read before the barrier of iteration kt-1, which every wave has passed when it
// issues the DMA at the start of iteration kt.
//
// The wave is the only one on its SIMD and issues in order, so a burst of LDS reads or
// DMA instructions would leave the MFMA pipe idle.  Each k16 step is therefore issued
// as groups {one DMA instruction, one fragment read, TM*TN/(TM+TN) MFMAs}, pinned with
// scheduling barriers.  The loop body has no branches: past the last stage the DMA
// re-reads the last stage into the free buffer, which is never read again.
//
// One tile per call; lds holds bf16_tile_lds<BM, BN>() bytes.  Every wave has waited for
// its own DMAs when it returns, but other waves may still read fragments: callers that
// reuse lds must pass a workgroup barrier first.
template <int BM, int BN, bool SWIGLU, bool GATHER>
__device__ __forceinline__ void bf16_tile(const GemmArgs &a, int tile, uint8_t *lds) {
    constexpr int BK = 32, PD = 3, NS = PD + 1;
    constexpr int TM = BM / 64, TN = BN / 64;
    constexpr int CPR = BK / 8, RPI = 64 / CPR;
    constexpr int IA = BM / (4 * RPI), IB = BN / (4 * RPI);
    constexpr int PER = IA + IB;
    constexpr int ROWB = BK * 2;
    constexpr int STAGE = (BM + BN) * ROWB;
    static_assert(IA >= 1 && IB >= 1 && (BN / 2) % (RPI * IB) == 0, "tile shape");

    const TileInfo ti = decode_tile(tile, a.tile_start, a.offsets, a.G, BM);

    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int lrow = lane / CPR, lphys = lane % CPR;

    const uint16_t *pa[IA];
#pragma unroll
    for (int q = 0; q < IA; ++q) {
        int r = RPI * (wave * IA + q) + lrow;
        long grow = ti.row0 + (r < ti.nrows ? r : 0);
        long src = GATHER ? row_token(grow, a.row_to_slot, a.T, a.k) : grow;
        pa[q] = a.A + src * a.K + ((lphys ^ swz_key<BK>(r)) * 8);
    }
    const int f0 = ti.nt * (BN / 2), n0 = ti.nt * BN;
    const uint16_t *pb[IB];
#pragma unroll
    for (int q = 0; q < IB; ++q) {
        int r = RPI * (wave * IB + q) + lrow;
        long wrow = SWIGLU ? (r < BN / 2 ? f0 + r : a.F + f0 + r - BN / 2) : n0 + r;
        pb[q] = a.B + ((long)ti.g * a.Ntot + wrow) * a.K + ((lphys ^ swz_key<BK>(r)) * 8);
    }

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = (f32x16){};

    // LDS byte offsets of this lane's fragment rows, for both k16 halves of a stage
    int aoff[2][TM], boff[2][TN];
    const int khalf = lane >> 5;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int i = 0; i < TM; ++i) aoff[h][i] = swz_off<BK>(wm * (BM / 2) + i * 32 + (lane & 31), h * 2 + khalf);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            int base;
            if (SWIGLU) {
                constexpr int TNh = TN / 2;
                base = j < TNh ? wn * (BN / 4) + j * 32 : BN / 2 + wn * (BN / 4) + (j - TNh) * 32;
            } else {
                base = wn * (BN / 2) + j * 32;
            }
            boff[h][j] = BM * ROWB + swz_off<BK>(base + (lane & 31), h * 2 + khalf);
        }
    }
    const int nk = a.K / BK;

#define MOE_BARRIER()                          \
    do {                                       \
        asm volatile("" ::: "memory");         \
        __builtin_amdgcn_s_barrier();          \
        asm volatile("" ::: "memory");         \
    } while (0)

    bf16x8 fr0[TM + TN], fr1[TM + TN];  // A fragments then B fragments
    // one DMA instruction q (< PER) of stage kt_ into buffer stg
#define MOE_DMA1(q, stg, kt_)                                                                    \
    do {                                                                                         \
        uint8_t *s_ = lds + (stg) * STAGE;                                                       \
        const int ko_ = (kt_) * BK;                                                              \
        if ((q) < IA) lds_dma16(pa[(q) < IA ? (q) : 0] + ko_, s_ + (wave * IA + (q)) * 1024);    \
        else lds_dma16(pb[(q) >= IA ? (q) - IA : 0] + ko_, s_ + BM * ROWB + (wave * IB + (q) - IA) * 1024); \
    } while (0)
#define MOE_FRAG1(F, u, stg, h)                                                                  \
    do {                                                                                         \
        const uint8_t *s_ = lds + (stg) * STAGE;                                                 \
        F[u] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(s_ + ((u) < TM ? aoff[h][(u) < TM ? (u) : 0] \
                                                                  : boff[h][(u) >= TM ? (u) - TM : 0]))); \
    } while (0)
#define MOE_MFMA1(F, m)                                                                          \
    acc[(m) / TN][(m) % TN] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F[(m) / TN], F[TM + (m) % TN], \
                                                                      acc[(m) / TN][(m) % TN], 0, 0, 0)

    constexpr int NF = TM + TN;          // fragments per k16 step
    constexpr int NM = TM * TN;          // MFMAs per k16 step
    static_assert(NF == PER, "one DMA and one fragment read per MFMA group");

    // prologue: stages 0 and 1 in flight, stage 0 published, its first fragments read
#pragma unroll
    for (int s0 = 0; s0 < PD; ++s0)
#pragma unroll
        for (int q = 0; q < PER; ++q) MOE_DMA1(q, s0, s0 < nk ? s0 : nk - 1);
    wait_vmcnt<(PD - 1) * PER>();
    MOE_BARRIER();
#pragma unroll
    for (int u = 0; u < NF; ++u) MOE_FRAG1(fr0, u, 0, 0);

    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt % NS, nxt = (kt + 1) % NS, pre = (kt + PD) % NS;
        const int kpre = kt + PD < nk ? kt + PD : nk - 1;  // past the end: a harmless copy into the free buffer
        wait_lgkmcnt0();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < NF; ++u) {
            MOE_DMA1(u, pre, kpre);
            MOE_FRAG1(fr1, u, cur, 1);
#pragma unroll
            for (int m = u * NM / NF; m < (u + 1) * NM / NF; ++m) MOE_MFMA1(fr0, m);
            __builtin_amdgcn_sched_barrier(0);
        }
        wait_lgkmcnt0();
        wait_vmcnt<(PD - 1) * PER>();
        MOE_BARRIER();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < NF; ++u) {
            MOE_FRAG1(fr0, u, nxt, 0);
#pragma unroll
            for (int m = u * NM / NF; m < (u + 1) * NM / NF; ++m) MOE_MFMA1(fr1, m);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    wait_vmcnt<0>();
#undef MOE_DMA1
#undef MOE_FRAG1
#undef MOE_MFMA1
#undef MOE_BARRIER

    // epilogue
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = wm * (BM / 2) + i * 32 + 8 * (r >> 2) + 4 * khalf + (r & 3);
            if (row >= ti.nrows) continue;
            const long grow = ti.row0 + row;
            if (SWIGLU) {
                constexpr int TNh = TN / 2;
#pragma unroll
                for (int j = 0; j < TNh; ++j) {
                    float gv = acc[i][j][r], uv = acc[i][j + TNh][r];
                    float h = swiglu(gv, uv);
                    int f = f0 + wn * (BN / 4) + j * 32 + (lane & 31);
                    a.C[grow * a.F + f] = f32_to_bf16(h);
                }
            } else {
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    int col = n0 + wn * (BN / 2) + j * 32 + (lane & 31);
                    a.C[grow * a.ldc + col] = f32_to_bf16(acc[i][j][r]);
                }
            }
        }
    }
}

// ---- bf16 grouped GEMM, 8 waves on a 256 x 256 tile ------------------------------------
//
// Two waves per SIMD (512 threads), each owning a 128 x 64 block of 32x32 MFMA tiles
// (linear1: 32 gate and the matching 32 up columns), so that one wave's MFMAs fill the
// pipe while the other waits on LDS or a barrier.  BK = 32, NS = 5 LDS stages of 32 KB
// (the whole 160 KB), all of them in flight: stage s is published by the barrier of pass
// s - 1, so its DMA has NS - 1 passes to land.
//
// Each pass multiplies the k16 half h = 0 of stage kt (fragments in F0) while reading the
// h = 1 fragments into F1, waits for its own loads, passes the one barrier (stage kt + 1
// published, every wave done with stage kt), then multiplies F1 while reading the h = 0
// fragments of stage kt + 1 into F0.  Measured on MI355X, a burst of 4 DMA instructions
// per wave right after the barrier saturated the per-CU address path for ~400 cycles and
// stalled both waves of a SIMD; each stage is therefore loaded in two halves of 2
// instructions: its B rows in the first half of pass s - NS + 1 and its A rows in the
// second half of pass s - NS, each into the buffer freed by the barrier of pass s - NS.
// Fragment reads, DMAs and MFMAs are interleaved with scheduling group barriers.  The
// accumulation order over k is that of bf16_tile, so results are identical bit for bit.
//
// One tile per call; lds holds bf16_tile8_lds() bytes; same caller contract as bf16_tile.
constexpr size_t bf16_tile8_lds() { return 5 * (size_t)(256 + 256) * 64; }

// The core takes the tile's rows and N tile (ti), the row stride of A and B in elements
// (lda), and the K range [k0, k0 + 32 nk).  F32OUT (not with SWIGLU) writes fp32 C.
//
// TM = 32-row blocks per wave: 4 for tiles of up to 256 rows; a group's last, partial
// tile runs with TM = 2 (up to 128 rows) or 1 (up to 64), which keeps the wave grid and
// the LDS layout, loads only the first 128 A rows and multiplies only TM blocks: MFMA work
// shrinks with the rows present and stays balanced over the SIMDs.
// COH: fp32 outputs go out as device-coherent stores (a consumer in the same launch reads
// them after a counter hand-off, with no fence)
template <bool SWIGLU, bool GATHER, bool F32OUT, int TM, bool COH = false>
__device__ __forceinline__ void bf16_tile8_core(const GemmArgs &a, const TileInfo &ti, long lda, int k0, int nk,
                                                uint8_t *lds) {
    constexpr int BM = 256, BN = 256, BK = 32, NS = 5;
    static_assert(!(SWIGLU && F32OUT), "SwiGLU writes bf16 h");
    static_assert(TM == 4 || TM == 2 || TM == 1, "row blocks per wave");
    constexpr int TN = 2;                                  // wave block (32 TM) x 64
    constexpr int CPR = BK / 8, RPI = 64 / CPR;            // 16 rows per DMA instruction
    constexpr int IA = TM == 4 ? 2 : 1, IB = BN / (8 * RPI);  // A and B DMA instructions per wave and stage
    constexpr int PER = IA + IB;
    constexpr int ROWB = BK * 2;
    constexpr int STAGE = (BM + BN) * ROWB;
    static_assert(IB == 2, "interleave pattern assumes two B instructions");

    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int lrow = lane / CPR, lphys = lane % CPR;

    const uint16_t *pa[IA];
#pragma unroll
    for (int q = 0; q < IA; ++q) {
        const int r = RPI * (wave * IA + q) + lrow;
        const long grow = ti.row0 + (r < ti.nrows ? r : 0);
        const long src = GATHER ? row_token(grow, a.row_to_slot, a.T, a.k) : grow;
        pa[q] = a.A + src * lda + k0 + ((lphys ^ swz_key<BK>(r)) * 8);
    }
    const int f0 = ti.nt * (BN / 2), n0 = ti.nt * BN;
    const uint16_t *pb[IB];
#pragma unroll
    for (int q = 0; q < IB; ++q) {
        const int r = RPI * (wave * IB + q) + lrow;
        const long wrow = SWIGLU ? (r < BN / 2 ? f0 + r : a.F + f0 + r - BN / 2) : n0 + r;
        pb[q] = a.B + ((long)ti.g * a.Ntot + wrow) * lda + k0 + ((lphys ^ swz_key<BK>(r)) * 8);
    }

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = (f32x16){};

    int aoff[2][TM], boff[2][TN];
    const int khalf = lane >> 5;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int i = 0; i < TM; ++i) aoff[h][i] = swz_off<BK>(wm * (32 * TM) + i * 32 + (lane & 31), h * 2 + khalf);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int base = SWIGLU ? (j == 0 ? wn * 32 : BN / 2 + wn * 32) : wn * 64 + j * 32;
            boff[h][j] = BM * ROWB + swz_off<BK>(base + (lane & 31), h * 2 + khalf);
        }
    }

#define MOE_BARRIER()                          \
    do {                                       \
        asm volatile("" ::: "memory");         \
        __builtin_amdgcn_s_barrier();          \
        asm volatile("" ::: "memory");         \
    } while (0)
    // DMA of the A (resp. B) rows of stage s into buffer s % NS; past the last stage it
    // re-reads the last one into a free buffer that is never read again
#define MOE_DMA_A(s)                                                                             \
    do {                                                                                         \
        const int s_ = (s);                                                                      \
        uint8_t *st_ = lds + (s_ % NS) * STAGE;                                                  \
        const int ko_ = (s_ < nk ? s_ : nk - 1) * BK;                                            \
        _Pragma("unroll") for (int q = 0; q < IA; ++q) lds_dma16(pa[q] + ko_, st_ + (wave * IA + q) * 1024); \
    } while (0)
#define MOE_DMA_B(s)                                                                             \
    do {                                                                                         \
        const int s_ = (s);                                                                      \
        uint8_t *st_ = lds + (s_ % NS) * STAGE;                                                  \
        const int ko_ = (s_ < nk ? s_ : nk - 1) * BK;                                            \
        _Pragma("unroll") for (int q = 0; q < IB; ++q)                                           \
            lds_dma16(pb[q] + ko_, st_ + BM * ROWB + (wave * IB + q) * 1024);                    \
    } while (0)
#define MOE_READ(F, s, h)                                                                        \
    do {                                                                                         \
        const uint8_t *st_ = lds + ((s) % NS) * STAGE;                                           \
        _Pragma("unroll") for (int i = 0; i < TM; ++i)                                           \
            F[i] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(st_ + aoff[h][i]));               \
        _Pragma("unroll") for (int j = 0; j < TN; ++j)                                           \
            F[TM + j] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(st_ + boff[h][j]));          \
    } while (0)
#define MOE_MMA(F)                                                                               \
    do {                                                                                         \
        _Pragma("unroll") for (int i = 0; i < TM; ++i)                                           \
            _Pragma("unroll") for (int j = 0; j < TN; ++j)                                       \
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F[i], F[TM + j], acc[i][j], 0, 0, 0); \
    } while (0)
    // per half pass with TM = 4: 8 MFMAs, 6 fragment reads and 2 DMA instructions, as
    // {3 x (read, MFMA), (DMA, MFMA)} twice; smaller TM: (DMA?, reads, MFMA) per MFMA
#define MOE_INTERLEAVE(ND)                                                                       \
    do {                                                                                         \
        if constexpr (TM == 4) {                                                                 \
            _Pragma("unroll") for (int r_ = 0; r_ < 2; ++r_) {                                   \
                _Pragma("unroll") for (int q_ = 0; q_ < 3; ++q_) {                               \
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                           \
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                           \
                }                                                                                \
                __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);                               \
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                               \
            }                                                                                    \
        } else {                                                                                 \
            _Pragma("unroll") for (int m_ = 0; m_ < TM * TN; ++m_) {                             \
                if (m_ < (ND)) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);                \
                __builtin_amdgcn_sched_group_barrier(0x100, (TM + TN + TM * TN - 1) / (TM * TN), 0); \
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                               \
            }                                                                                    \
        }                                                                                        \
        __builtin_amdgcn_sched_barrier(0);                                                       \
    } while (0)

    bf16x8 F0[TM + TN], F1[TM + TN];
    // prologue: stages 0 .. NS-2 whole and the A rows of stage NS-1; stage 0 published
#pragma unroll
    for (int s0 = 0; s0 < NS - 1; ++s0) {
        MOE_DMA_A(s0);
        MOE_DMA_B(s0);
    }
    MOE_DMA_A(NS - 1);
    wait_vmcnt<(NS - 2) * PER + IA>();
    MOE_BARRIER();
    MOE_READ(F0, 0, 0);
    wait_lgkmcnt0();
    for (int kt = 0; kt < nk; ++kt) {
        MOE_READ(F1, kt, 1);
        MOE_DMA_B(kt + NS - 1);
        MOE_MMA(F0);
        MOE_INTERLEAVE(IB);
        wait_vmcnt<(NS - 2) * PER>();  // own loads of stage kt+1 landed (kt+2 .. kt+NS-1 may fly)
        wait_lgkmcnt0();
        MOE_BARRIER();
        __builtin_amdgcn_sched_barrier(0);
        MOE_DMA_A(kt + NS);
        MOE_READ(F0, (kt + 1 < nk ? kt + 1 : kt), 0);  // the last pass re-reads a published stage
        MOE_MMA(F1);
        MOE_INTERLEAVE(IA);
        wait_lgkmcnt0();
    }
    wait_vmcnt<0>();
#undef MOE_BARRIER
#undef MOE_DMA_A
#undef MOE_DMA_B
#undef MOE_READ
#undef MOE_MMA
#undef MOE_INTERLEAVE

#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = wm * (32 * TM) + i * 32 + 8 * (r >> 2) + 4 * khalf + (r & 3);
            if (row >= ti.nrows) continue;
            const long grow = ti.row0 + row;
            if (SWIGLU) {
                const float gv = acc[i][0][r], uv = acc[i][1][r];
                const float h = swiglu(gv, uv);
                a.C[grow * a.F + f0 + wn * 32 + (lane & 31)] = f32_to_bf16(h);
            } else if (F32OUT) {
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    stc<COH>((float *)a.C + grow * a.ldc + n0 + wn * 64 + j * 32 + (lane & 31), acc[i][j][r]);
            } else {
#pragma unroll
                for (int j = 0; j < TN; ++j) a.C[grow * a.ldc + n0 + wn * 64 + j * 32 + (lane & 31)] = f32_to_bf16(acc[i][j][r]);
            }
        }
    }
}

// the core sized to the tile's rows
template <bool SWIGLU, bool GATHER, bool F32OUT, bool COH = false>
__device__ __forceinline__ void bf16_tile8_rows(const GemmArgs &a, const TileInfo &ti, long lda, int k0, int nk,
                                                uint8_t *lds) {
    if (ti.nrows > 128) bf16_tile8_core<SWIGLU, GATHER, F32OUT, 4, COH>(a, ti, lda, k0, nk, lds);
    else if (ti.nrows > 64) bf16_tile8_core<SWIGLU, GATHER, F32OUT, 2, COH>(a, ti, lda, k0, nk, lds);
    else bf16_tile8_core<SWIGLU, GATHER, F32OUT, 1, COH>(a, ti, lda, k0, nk, lds);
}

// half: -1 the whole tile, 0 / 1 its rows 0..127 / 128..255 (an empty half returns at once);
// every output element takes the same k order either way, so the bits do not change
template <bool SWIGLU, bool GATHER>
__device__ __forceinline__ void bf16_tile8(const GemmArgs &a, int tile, uint8_t *lds, int half = -1) {
    TileInfo ti = decode_tile_grouped<kTileGroup>(tile, a.tile_start, a.offsets, a.G, 256);
    if (half >= 0) {
        ti.row0 += 128 * half;
        ti.nrows = half ? ti.nrows - 128 : min(ti.nrows, 128);
        if (ti.nrows <= 0) return;
    }
    bf16_tile8_rows<SWIGLU, GATHER, false>(a, ti, a.K, 0, a.K / 32, lds);
}

// ---- fp32 path: one lane per output element ------------------------------------

__device__ __forceinline__ int group_of_row(long r, const int32_t *__restrict__ offsets, int G) {
    int lo = 0, hi = G - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (offsets[mid] <= r) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// linear1 + SwiGLU, one output element h[r, f] per lane; gid = r * F + f
__device__ __forceinline__ void ffn1_f32_lane(const float *__restrict__ x, const int32_t *__restrict__ r2s,
                                              const float *__restrict__ w1, const int32_t *__restrict__ offsets,
                                              int G, int T, int k, int d, int F, long rows, float *__restrict__ h,
                                              long gid) {
    if (gid >= rows * F) return;
    const long r = gid / F;
    const int f = (int)(gid % F);
    const int g = group_of_row(r, offsets, G);
    const long t = row_token(r, r2s, T, k);
    const float *xr = x + t * d;
    const float *wg = w1 + ((long)g * 2 * F + f) * d, *wu = w1 + ((long)g * 2 * F + F + f) * d;
    float ug = 0.0f, uu = 0.0f;
    for (int i = 0; i < d; ++i) {
        ug = fmaf(xr[i], wg[i], ug);
        uu = fmaf(xr[i], wu[i], uu);
    }
    h[r * F + f] = ug / (1.0f + expf(-ug)) * uu;
}

// linear2, one output element y[r, c] per lane; gid = r * d + c
__device__ __forceinline__ void ffn2_f32_lane(const float *__restrict__ h, const float *__restrict__ w2,
                                              const int32_t *__restrict__ offsets, int G, int d, int F, long rows,
                                              float *__restrict__ y, long gid) {
    if (gid >= rows * d) return;
    const long r = gid / d;
    const int c = (int)(gid % d);
    const int g = group_of_row(r, offsets, G);
    const float *hr = h + r * F, *wr = w2 + ((long)g * d + c) * F;
    float s = 0.0f;
    for (int f = 0; f < F; ++f) s = fmaf(hr[f], wr[f], s);
    y[r * d + c] = s;
}

}  // namespace moe
