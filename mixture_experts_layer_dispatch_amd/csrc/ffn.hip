// Expert FFNs over dispatched rows (S8-S9): linear1 (gate+up) with SwiGLU in the
// epilogue, then linear2, as grouped GEMMs over ragged expert groups.
//
// MoE lesson (factory.pai-world.com, "Mixture of Experts", "FFN swap"): each expert
// is an independent FFN, usually SwiGLU.  Mega MoE blog (donniechu.com, spec table)
// and Mega MoE wiki ("One-line definition"): linear1, SwiGLU and linear2 are the
// middle of the fused chain.  SwiGLU is read as silu(x Wg^T) * (x Wu^T), with
// W1 = [Wg; Wu] stacked along its output rows.
//
// Tiles: a group g of n_g rows is cut into ceil(n_g / BM) row tiles times the N
// tiles; a tiny planning kernel writes the exclusive prefix of tiles per group,
// and each GEMM workgroup finds its (group, row tile, N tile) by binary search.
// Within a group, row tiles vary fastest so that the tiles sharing one weight tile
// are neighbours, and neighbouring tiles are dealt to the same XCD (and its L2).
#include <cstdlib>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// ---- tile plan ----------------------------------------------------------------

__global__ __launch_bounds__(1024) void tile_plan_kernel(const int32_t *__restrict__ offsets, int G, int bm1,
                                                        int ntn1, int bm2, int ntn2, int32_t *__restrict__ ts1,
                                                        int32_t *__restrict__ ts2) {
    __shared__ int32_t s1[1024], s2[1024];
    const int tid = threadIdx.x;
    int a1[2] = {0, 0}, a2[2] = {0, 0};
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        int g = 2 * tid + u;
        if (g < G) {
            int c = offsets[g + 1] - offsets[g];
            a1[u] = (c + bm1 - 1) / bm1 * ntn1;
            a2[u] = (c + bm2 - 1) / bm2 * ntn2;
        }
    }
    s1[tid] = a1[0] + a1[1];
    s2[tid] = a2[0] + a2[1];
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        int v1 = tid >= off ? s1[tid - off] : 0, v2 = tid >= off ? s2[tid - off] : 0;
        __syncthreads();
        s1[tid] += v1;
        s2[tid] += v2;
        __syncthreads();
    }
    int e1 = s1[tid] - a1[0] - a1[1], e2 = s2[tid] - a2[0] - a2[1];
    if (2 * tid < G) { ts1[2 * tid] = e1; ts2[2 * tid] = e2; }
    if (2 * tid + 1 < G) { ts1[2 * tid + 1] = e1 + a1[0]; ts2[2 * tid + 1] = e2 + a2[0]; }
    if (tid == 1023) { ts1[G] = s1[1023]; ts2[G] = s2[1023]; }
}

// Tile of this workgroup, or -1.  Workgroup b runs on XCD b % 8; the tiles are
// split into 8 contiguous ranges, range x going to the workgroups of XCD x.
__device__ __forceinline__ int pick_tile(int total) {
    const int b = blockIdx.x, xcd = b & 7, j = b >> 3;
    const int per = (total + 7) >> 3;
    const int t = xcd * per + j;
    return (j < per && t < total) ? t : -1;
}

struct TileInfo {
    int g, row0, nrows, nt;
};

__device__ __forceinline__ TileInfo decode_tile(int tile, const int32_t *__restrict__ ts, const int32_t *__restrict__ offsets,
                                                int G, int BM) {
    int lo = 0, hi = G - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (ts[mid] <= tile) lo = mid; else hi = mid - 1;
    }
    TileInfo ti;
    ti.g = lo;
    const int rb = offsets[lo], cnt = offsets[lo + 1] - rb;
    const int mtiles = (cnt + BM - 1) / BM;
    const int local = tile - ts[lo];
    const int mt = local % mtiles;
    ti.nt = local / mtiles;
    ti.row0 = rb + mt * BM;
    ti.nrows = min(BM, cnt - mt * BM);
    return ti;
}

// Token feeding dispatched row r: routed rows carry slot = t*k + j, the shared
// expert's rows are T*k + t.  Clamped so that corrupt inputs cannot read outside x.
__device__ __forceinline__ long row_token(long r, const int32_t *__restrict__ row_to_slot, int T, int k) {
    long tk = (long)T * k;
    long t;
    if (r < tk) {
        long s = row_to_slot[r];
        s = s < 0 ? 0 : (s >= tk ? tk - 1 : s);
        t = s / k;
    } else {
        t = r - tk;
    }
    return t < 0 ? 0 : (t >= T ? T - 1 : t);
}

// ---- bf16 grouped GEMM ----------------------------------------------------------
//
// C[rows, N] = A[rows, K] * B_g[N, K]^T per group, bf16 inputs, fp32 accumulation on
// v_mfma_f32_32x32x16_bf16.  256 threads = 2 x 2 waves, each owning a
// (BM/2) x (BN/2) block of 32x32 MFMA tiles.  K advances 64 per stage; stages are
// double-buffered in LDS (one barrier per stage), filled from registers loaded one
// stage ahead.  LDS rows are 128 bytes whose 16-byte chunks are XOR-swizzled with
// (row & 7), so both the 16-byte stores and the MFMA fragment reads are free of
// bank conflicts.
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

constexpr int kBK = 64;

// 128-byte LDS rows of 16-byte chunks.  gfx950 serves ds_read_b128 from 64 banks
// (a 256-byte window per 16 lanes): rows r..r+15 read at one logical chunk must land in
// 16 distinct 16-byte slots of that window, hence the key (row >> 1) & 7 (odd and even
// rows fill the two 128-byte halves).
__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4); }

template <int BM, int BN, bool SWIGLU, bool GATHER>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmArgs a) {
    constexpr int TM = BM / 64, TN = BN / 64;  // 32x32 tiles per wave along M and N
    constexpr int LA = BM / 32, LB = BN / 32;  // 16-byte loads per thread per stage
    constexpr int STAGE = (BM + BN) * 128;     // bytes per stage
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];  // 2 stages

    const int total = a.tile_start[a.G];
    const int tile = pick_tile(total);
    if (tile < 0) return;
    const TileInfo ti = decode_tile(tile, a.tile_start, a.offsets, a.G, BM);

    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int ch = tid & 7, r8 = tid >> 3;

    // global sources of this thread's 16-byte chunks (rows r8 + 32 i)
    const uint16_t *pa[LA];
#pragma unroll
    for (int i = 0; i < LA; ++i) {
        int r = r8 + 32 * i;
        long grow = ti.row0 + (r < ti.nrows ? r : 0);
        long src = GATHER ? row_token(grow, a.row_to_slot, a.T, a.k) : grow;
        pa[i] = a.A + src * a.K + ch * 8;
    }
    const int f0 = ti.nt * (BN / 2), n0 = ti.nt * BN;
    const uint16_t *pb0, *pb1;  // first and second half of the B tile rows
    {
        const long g0 = (long)ti.g * a.Ntot;
        long w0 = SWIGLU ? f0 + r8 : n0 + r8;
        long w1 = SWIGLU ? a.F + f0 + r8 : n0 + BN / 2 + r8;
        pb0 = a.B + (g0 + w0) * a.K + ch * 8;
        pb1 = a.B + (g0 + w1) * a.K + ch * 8;
    }
    const long bstep = 32L * a.K;  // 32 rows

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = (f32x16){};

    // LDS offsets of this wave's fragment rows (without the stage and chunk)
    int arow[TM], brow[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) arow[i] = wm * (BM / 2) + i * 32 + (lane & 31);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        int base;
        if (SWIGLU) {
            constexpr int TNh = TN / 2;
            base = j < TNh ? wn * (BN / 4) + j * 32 : BN / 2 + wn * (BN / 4) + (j - TNh) * 32;
        } else {
            base = wn * (BN / 2) + j * 32;
        }
        brow[j] = base + (lane & 31);
    }
    const int khalf = lane >> 5;
    int st_off[LA > LB ? LA : LB];  // swizzled LDS store offsets (row r8 + 32 i)
#pragma unroll
    for (int i = 0; i < (LA > LB ? LA : LB); ++i) st_off[i] = swz(r8 + 32 * i, ch);

    u32x4 ra[LA], rb[LB];
    const int nk = a.K / kBK;

    // prologue: stage 0
#pragma unroll
    for (int i = 0; i < LA; ++i) ra[i] = *(const u32x4 *)(pa[i]);
#pragma unroll
    for (int i = 0; i < LB / 2; ++i) {
        rb[i] = *(const u32x4 *)(pb0 + i * bstep);
        rb[LB / 2 + i] = *(const u32x4 *)(pb1 + i * bstep);
    }
#pragma unroll
    for (int i = 0; i < LA; ++i) *(u32x4 *)(lds + st_off[i]) = ra[i];
#pragma unroll
    for (int i = 0; i < LB; ++i) *(u32x4 *)(lds + BM * 128 + st_off[i]) = rb[i];
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
        const int stage = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) {
            const int ko = (kt + 1) * kBK;
#pragma unroll
            for (int i = 0; i < LA; ++i) ra[i] = *(const u32x4 *)(pa[i] + ko);
#pragma unroll
            for (int i = 0; i < LB / 2; ++i) {
                rb[i] = *(const u32x4 *)(pb0 + i * bstep + ko);
                rb[LB / 2 + i] = *(const u32x4 *)(pb1 + i * bstep + ko);
            }
        }
        const uint8_t *sa = lds + stage * STAGE, *sb = sa + BM * 128;
#pragma unroll
        for (int kk = 0; kk < kBK / 16; ++kk) {
            bf16x8 fa[TM], fb[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i)
                fa[i] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(sa + swz(arow[i], kk * 2 + khalf)));
#pragma unroll
            for (int j = 0; j < TN; ++j)
                fb[j] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(sb + swz(brow[j], kk * 2 + khalf)));
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
        if (more) {
            uint8_t *da = lds + (stage ^ 1) * STAGE, *db = da + BM * 128;
#pragma unroll
            for (int i = 0; i < LA; ++i) *(u32x4 *)(da + st_off[i]) = ra[i];
#pragma unroll
            for (int i = 0; i < LB; ++i) *(u32x4 *)(db + st_off[i]) = rb[i];
        }
        __syncthreads();
    }

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
                    float h = gv / (1.0f + __expf(-gv)) * uv;
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

// ---- bf16 grouped GEMM, direct global->LDS loads ---------------------------------
//
// Same tiling, fragment layout and epilogues as gemm_bf16_kernel, but the tiles are
// moved by global_load_lds_dwordx4 (gfx950): each lane's 16 bytes land in LDS at
// (M0 base + 16 * lane), with no staging registers, so the next stage streams in
// while the current one feeds the MFMAs.  One instruction fills 8 rows x 128 bytes;
// lane L of it owns row L/8 and physical chunk L%8, and therefore loads logical
// chunk (L%8) ^ (L/8) -- the XOR swizzle the fragment reads expect.

__device__ __forceinline__ void lds_dma16(const void *g, uint8_t *lds_block) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)g,
                                     (__attribute__((address_space(3))) void *)lds_block, 16, 0, 0);
}

// LDS tile rows hold BK bf16 (BK * 2 bytes) as 16-byte chunks.  Physical chunk =
// logical chunk XOR a key of the row, chosen so that the 16 lanes of one ds_read_b128
// phase (rows r..r+15 at one logical chunk) hit 16 distinct 16-byte slots of the
// 256-byte window of gfx950's 64 LDS banks: (row >> 1) & 7 for 128-byte rows,
// (row >> 2) & 3 for 64-byte rows.  (Measured: 0 bank-conflict cycles; keyed on
// the low row bits instead, half of the LDS cycles are conflicts.)
template <int BK>
__device__ __forceinline__ int swz_key(int row) {
    return BK == 64 ? ((row >> 1) & 7) : ((row >> 2) & 3);
}
template <int BK>
__device__ __forceinline__ int swz_off(int row, int chunk) {
    return row * (BK * 2) + ((chunk ^ swz_key<BK>(row)) << 4);
}

// s_waitcnt lgkmcnt(0) with vmcnt and expcnt left at their maxima.
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// s_waitcnt vmcnt(n) (n < 64) with expcnt and lgkmcnt left at their maxima.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

template <int BM, int BN, int BK, int NS, bool SWIGLU, bool GATHER>
__global__ __launch_bounds__(256) void gemm_bf16_dma_kernel(GemmArgs a) {
    constexpr int TM = BM / 64, TN = BN / 64;
    constexpr int CPR = BK / 8;            // 16-byte chunks per LDS row
    constexpr int RPI = 64 / CPR;          // rows filled by one DMA instruction (1 KB)
    constexpr int IA = BM / (4 * RPI), IB = BN / (4 * RPI);  // DMA instructions per wave per stage
    constexpr int PER = IA + IB;
    constexpr int ROWB = BK * 2;
    constexpr int STAGE = (BM + BN) * ROWB;
    static_assert(IA >= 1 && IB >= 1 && (BN / 2) % (RPI * IB) == 0, "tile shape");
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    const int total = a.tile_start[a.G];
    const int tile = pick_tile(total);
    if (tile < 0) return;
    const TileInfo ti = decode_tile(tile, a.tile_start, a.offsets, a.G, BM);

    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int lrow = lane / CPR;   // row within a DMA block
    const int lphys = lane % CPR;  // physical chunk this lane fills

    // A: the logical chunk follows from the absolute tile row (its swizzle key)
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
        int r = RPI * (wave * IB + q) + lrow;  // tile row; never straddles the gate/up split per wave
        long wrow = SWIGLU ? (r < BN / 2 ? f0 + r : a.F + f0 + r - BN / 2) : n0 + r;
        pb[q] = a.B + ((long)ti.g * a.Ntot + wrow) * a.K + ((lphys ^ swz_key<BK>(r)) * 8);
    }

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = (f32x16){};

    int arow[TM], brow[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) arow[i] = wm * (BM / 2) + i * 32 + (lane & 31);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        int base;
        if (SWIGLU) {
            constexpr int TNh = TN / 2;
            base = j < TNh ? wn * (BN / 4) + j * 32 : BN / 2 + wn * (BN / 4) + (j - TNh) * 32;
        } else {
            base = wn * (BN / 2) + j * 32;
        }
        brow[j] = base + (lane & 31);
    }
    const int khalf = lane >> 5;
    const int nk = a.K / BK;

#define MOE_ISSUE_STAGE(stg, kt_)                                                            \
    do {                                                                                     \
        uint8_t *sa_ = lds + (stg) * STAGE, *sb_ = sa_ + BM * ROWB;                          \
        const int ko_ = (kt_) * BK;                                                          \
        _Pragma("unroll") for (int q = 0; q < IA; ++q)                                       \
            lds_dma16(pa[q] + ko_, sa_ + (wave * IA + q) * 1024);                            \
        _Pragma("unroll") for (int q = 0; q < IB; ++q)                                       \
            lds_dma16(pb[q] + ko_, sb_ + (wave * IB + q) * 1024);                            \
    } while (0)

    // prologue: stages 0 .. NS-2 in flight
#pragma unroll
    for (int s0 = 0; s0 < NS - 1; ++s0)
        if (s0 < nk) MOE_ISSUE_STAGE(s0, s0);

    for (int kt = 0; kt < nk; ++kt) {
        // stage kt landed: later stages (at most NS-2 of them) may still be in flight
        const int later = min(NS - 2, nk - 1 - kt);
        if (NS >= 4 && later >= 2) wait_vmcnt<(NS >= 4 ? 2 : 0) * PER>();
        else if (NS >= 3 && later >= 1) wait_vmcnt<(NS >= 3 ? 1 : 0) * PER>();
        else wait_vmcnt<0>();
        // Every wave has its own part of stage kt in LDS and has consumed stage kt-1
        // (its MFMAs used the fragments it read), so a bare barrier suffices: a fenced
        // one would also drain the later stages still in flight.
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (kt + NS - 1 < nk) MOE_ISSUE_STAGE((kt + NS - 1) % NS, kt + NS - 1);
        const uint8_t *sa = lds + (kt % NS) * STAGE, *sb = sa + BM * ROWB;
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            bf16x8 fa[TM], fb[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i)
                fa[i] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(sa + swz_off<BK>(arow[i], kk * 2 + khalf)));
#pragma unroll
            for (int j = 0; j < TN; ++j)
                fb[j] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(sb + swz_off<BK>(brow[j], kk * 2 + khalf)));
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
    }
#undef MOE_ISSUE_STAGE

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
                    float h = gv / (1.0f + __expf(-gv)) * uv;
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
template <int BM, int BN, bool SWIGLU, bool GATHER>
__global__ __launch_bounds__(256) void gemm_bf16_pipe_kernel(GemmArgs a) {
    constexpr int BK = 32, PD = 3, NS = PD + 1;
    constexpr int TM = BM / 64, TN = BN / 64;
    constexpr int CPR = BK / 8, RPI = 64 / CPR;
    constexpr int IA = BM / (4 * RPI), IB = BN / (4 * RPI);
    constexpr int PER = IA + IB;
    constexpr int ROWB = BK * 2;
    constexpr int STAGE = (BM + BN) * ROWB;
    static_assert(IA >= 1 && IB >= 1 && (BN / 2) % (RPI * IB) == 0, "tile shape");
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    const int total = a.tile_start[a.G];
    const int tile = pick_tile(total);
    if (tile < 0) return;
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
                    float h = gv / (1.0f + __expf(-gv)) * uv;
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

// ---- fp32 path: one thread per output element ------------------------------------

__device__ __forceinline__ int group_of_row(long r, const int32_t *__restrict__ offsets, int G) {
    int lo = 0, hi = G - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (offsets[mid] <= r) lo = mid; else hi = mid - 1;
    }
    return lo;
}

__global__ __launch_bounds__(256) void ffn1_f32_kernel(const float *__restrict__ x, const int32_t *__restrict__ r2s,
                                                      const float *__restrict__ w1, const int32_t *__restrict__ offsets,
                                                      int G, int T, int k, int d, int F, long rows,
                                                      float *__restrict__ h) {
    const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
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

__global__ __launch_bounds__(256) void ffn2_f32_kernel(const float *__restrict__ h, const float *__restrict__ w2,
                                                      const int32_t *__restrict__ offsets, int G, int d, int F,
                                                      long rows, float *__restrict__ y) {
    const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= rows * d) return;
    const long r = gid / d;
    const int c = (int)(gid % d);
    const int g = group_of_row(r, offsets, G);
    const float *hr = h + r * F, *wr = w2 + ((long)g * d + c) * F;
    float s = 0.0f;
    for (int f = 0; f < F; ++f) s = fmaf(hr[f], wr[f], s);
    y[r * d + c] = s;
}

// ---- launch ------------------------------------------------------------------------

FfnPlan ffn_plan(const Shape &s) {
    FfnPlan p;
    const long rows = s.rows();
    const double per_group = (double)rows / s.G();
    p.decode = s.mode == MODE_FP8 && per_group <= 48.0;
    if (p.decode) {
        // one 64-lane wave per (group, 32-row tile, 32 output columns, K slice)
        p.ks = rows <= 32 && (s.d / 128) % 4 == 0 ? 4 : 1;
        p.bm1 = p.bm2 = 32;
        p.bn1 = p.bn2 = 32;
        p.ntn1 = (2 * s.F / 32) * p.ks;
        p.ntn2 = s.d / 32;
        return p;
    }
    p.ks = 1;
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

static int gemm_variant() {
    static int v = -1;
    if (v < 0) {
        const char *e = getenv("MOE_GEMM_VARIANT");  // 0: register-staged; 1: DMA, 4 stages; 2: DMA, 2 stages; 3: DMA, mid-stage barrier (default)
        v = e ? atoi(e) : 3;
    }
    return v;
}

template <int BM, int BN, bool SWIGLU, bool GATHER>
static hipError_t launch_gemm(const char *name, dim3 grid, const GemmArgs &a, hipStream_t st) {
    constexpr size_t lds0 = 2 * (size_t)(BM + BN) * 128;       // BK 64, 2 stages
    constexpr size_t lds1 = 4 * (size_t)(BM + BN) * 64;        // BK 32, 4 stages
    constexpr size_t lds3 = 4 * (size_t)(BM + BN) * 64;        // BK 32, 4 stages, mid-stage barrier
    static bool attr = false;
    if (!attr) {
        hipError_t e = hipFuncSetAttribute((const void *)gemm_bf16_kernel<BM, BN, SWIGLU, GATHER>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds0);
        if (e == hipSuccess)
            e = hipFuncSetAttribute((const void *)gemm_bf16_dma_kernel<BM, BN, 32, 4, SWIGLU, GATHER>,
                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds1);
        if (e == hipSuccess)
            e = hipFuncSetAttribute((const void *)gemm_bf16_dma_kernel<BM, BN, 64, 2, SWIGLU, GATHER>,
                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds0);
        if (e == hipSuccess)
            e = hipFuncSetAttribute((const void *)gemm_bf16_pipe_kernel<BM, BN, SWIGLU, GATHER>,
                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds3);
        if (e != hipSuccess) return e;
        attr = true;
    }
    switch (gemm_variant()) {
        case 0: MOE_LAUNCH(name, (gemm_bf16_kernel<BM, BN, SWIGLU, GATHER>), grid, dim3(256), lds0, st, a); break;
        case 1: MOE_LAUNCH(name, (gemm_bf16_dma_kernel<BM, BN, 32, 4, SWIGLU, GATHER>), grid, dim3(256), lds1, st, a); break;
        case 2: MOE_LAUNCH(name, (gemm_bf16_dma_kernel<BM, BN, 64, 2, SWIGLU, GATHER>), grid, dim3(256), lds0, st, a); break;
        default: MOE_LAUNCH(name, (gemm_bf16_pipe_kernel<BM, BN, SWIGLU, GATHER>), grid, dim3(256), lds3, st, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_fp8_ffn(const Shape &s, const FfnPlan &p, const uint8_t *w1, const uint8_t *w1s,
                          const uint8_t *w2, const uint8_t *w2s, const uint8_t *xq, const float *xs,
                          const int32_t *offsets, const int32_t *row_to_slot, uint8_t *h, float *hs, void *y_perm,
                          const int32_t *ts1, const int32_t *ts2, float *upart, hipStream_t st);

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
    MOE_LAUNCH("tile_plan", tile_plan_kernel, dim3(1), dim3(1024), 0, st, offsets, G, p.bm1, ntn1, p.bm2, ntn2, ts1, ts2);
    if (s.mode == MODE_FP8)
        return launch_fp8_ffn(s, p, (const uint8_t *)w1, (const uint8_t *)w1s, (const uint8_t *)w2,
                              (const uint8_t *)w2s, xq, xs, offsets, row_to_slot, (uint8_t *)h, hs, y_perm, ts1, ts2,
                              upart, st);
    auto grid_for = [&](int bm, int ntn) {
        long ub = (rows / bm + G) * (long)ntn;
        return dim3((unsigned)((ub + 7) / 8 * 8));
    };
    GemmArgs a1 = {(const uint16_t *)x, row_to_slot, (const uint16_t *)w1, (uint16_t *)h, offsets, ts1,
                   s.T, s.k, s.d, 2 * s.F, s.F, G, s.F};
    GemmArgs a2 = {(const uint16_t *)h, nullptr, (const uint16_t *)w2, (uint16_t *)y_perm, offsets, ts2,
                   s.T, s.k, s.F, s.d, s.d, G, s.F};
    hipError_t e;
    if (p.bm1 == 256) e = launch_gemm<256, 256, true, true>("linear1", grid_for(p.bm1, ntn1), a1, st);
    else e = launch_gemm<128, 256, true, true>("linear1", grid_for(p.bm1, ntn1), a1, st);
    if (e != hipSuccess) return e;
    if (p.bm2 == 256 && p.bn2 == 256) e = launch_gemm<256, 256, false, false>("linear2", grid_for(p.bm2, ntn2), a2, st);
    else if (p.bn2 == 256) e = launch_gemm<128, 256, false, false>("linear2", grid_for(p.bm2, ntn2), a2, st);
    else if (p.bm2 == 256) e = launch_gemm<256, 128, false, false>("linear2", grid_for(p.bm2, ntn2), a2, st);
    else e = launch_gemm<128, 128, false, false>("linear2", grid_for(p.bm2, ntn2), a2, st);
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

}  // namespace moe
