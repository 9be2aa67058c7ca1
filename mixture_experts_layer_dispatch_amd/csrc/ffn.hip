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

__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

template <int BM, int BN, bool SWIGLU, bool GATHER>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmArgs a) {
    constexpr int TM = BM / 64, TN = BN / 64;  // 32x32 tiles per wave along M and N
    constexpr int LA = BM / 32, LB = BN / 32;  // 16-byte loads per thread per stage
    constexpr int STAGE = (BM + BN) * 128;     // bytes per stage
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE];

    const int total = a.tile_start[a.G];
    const int tile = pick_tile(total);
    if (tile < 0) return;
    const TileInfo ti = decode_tile(tile, a.tile_start, a.offsets, a.G, BM);

    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int ch = tid & 7, r8 = tid >> 3;

    // global sources of this thread's 16-byte chunks
    const uint16_t *pa[LA];
    const uint16_t *pb[LB];
#pragma unroll
    for (int i = 0; i < LA; ++i) {
        int r = r8 + 32 * i;
        long grow = ti.row0 + (r < ti.nrows ? r : 0);
        long src = GATHER ? row_token(grow, a.row_to_slot, a.T, a.k) : grow;
        pa[i] = a.A + src * a.K + ch * 8;
    }
    const int f0 = ti.nt * (BN / 2), n0 = ti.nt * BN;
#pragma unroll
    for (int i = 0; i < LB; ++i) {
        int c = r8 + 32 * i;
        long wrow = SWIGLU ? (c < BN / 2 ? f0 + c : a.F + f0 + c - BN / 2) : n0 + c;
        pb[i] = a.B + ((long)ti.g * a.Ntot + wrow) * a.K + ch * 8;
    }

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = (f32x16){};

    uint4 ra[LA], rb[LB];
    auto gload = [&](int kt) {
#pragma unroll
        for (int i = 0; i < LA; ++i) ra[i] = *(const uint4 *)(pa[i] + kt * kBK);
#pragma unroll
        for (int i = 0; i < LB; ++i) rb[i] = *(const uint4 *)(pb[i] + kt * kBK);
    };
    auto lstore = [&](int stage) {
        uint8_t *sa = lds + stage * STAGE, *sb = sa + BM * 128;
#pragma unroll
        for (int i = 0; i < LA; ++i) *(uint4 *)(sa + swz(r8 + 32 * i, ch)) = ra[i];
#pragma unroll
        for (int i = 0; i < LB; ++i) *(uint4 *)(sb + swz(r8 + 32 * i, ch)) = rb[i];
    };

    // LDS rows of this wave's fragments
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

    const int nk = a.K / kBK;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int stage = kt & 1;
        if (kt + 1 < nk) gload(kt + 1);
        const uint8_t *sa = lds + stage * STAGE, *sb = sa + BM * 128;
#pragma unroll
        for (int kk = 0; kk < kBK / 16; ++kk) {
            bf16x8 fa[TM], fb[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i)
                fa[i] = __builtin_bit_cast(bf16x8, *(const uint4 *)(sa + swz(arow[i], kk * 2 + khalf)));
#pragma unroll
            for (int j = 0; j < TN; ++j)
                fb[j] = __builtin_bit_cast(bf16x8, *(const uint4 *)(sb + swz(brow[j], kk * 2 + khalf)));
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) lstore(stage ^ 1);
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
    p.bm1 = 128; p.bn1 = 128;
    p.bm2 = 128; p.bn2 = 128;
    return p;
}

hipError_t launch_fp8_ffn(const Shape &s, const FfnPlan &p, const uint8_t *w1, const uint8_t *w1s,
                          const uint8_t *w2, const uint8_t *w2s, const uint8_t *xq, const float *xs,
                          const int32_t *offsets, const int32_t *row_to_slot, uint8_t *h, float *hs, void *y_perm,
                          const int32_t *ts1, const int32_t *ts2, hipStream_t st);

hipError_t launch_ffn(const Shape &s, const FfnPlan &p, const void *w1, const void *w1s, const void *w2,
                      const void *w2s, const void *x, const uint8_t *xq, const float *xs, const int32_t *offsets,
                      const int32_t *row_to_slot, void *h, float *hs, void *y_perm, int32_t *tile_start,
                      hipStream_t st) {
    if (s.T == 0) return hipSuccess;
    const long rows = s.rows();
    const int G = s.G();
    if (s.mode == MODE_F32) {
        long n1 = rows * s.F, n2 = rows * s.d;
        hipLaunchKernelGGL(ffn1_f32_kernel, dim3((unsigned)((n1 + 255) / 256)), dim3(256), 0, st, (const float *)x,
                           row_to_slot, (const float *)w1, offsets, G, s.T, s.k, s.d, s.F, rows, (float *)h);
        hipLaunchKernelGGL(ffn2_f32_kernel, dim3((unsigned)((n2 + 255) / 256)), dim3(256), 0, st, (const float *)h,
                           (const float *)w2, offsets, G, s.d, s.F, rows, (float *)y_perm);
        return hipGetLastError();
    }
    int32_t *ts1 = tile_start, *ts2 = tile_start + (G + 1);
    const int ntn1 = s.F / (p.bn1 / 2), ntn2 = s.d / p.bn2;
    hipLaunchKernelGGL(tile_plan_kernel, dim3(1), dim3(1024), 0, st, offsets, G, p.bm1, ntn1, p.bm2, ntn2, ts1, ts2);
    if (s.mode == MODE_FP8)
        return launch_fp8_ffn(s, p, (const uint8_t *)w1, (const uint8_t *)w1s, (const uint8_t *)w2,
                              (const uint8_t *)w2s, xq, xs, offsets, row_to_slot, (uint8_t *)h, hs, y_perm, ts1, ts2,
                              st);
    auto grid_for = [&](int bm, int ntn) {
        long ub = (rows / bm + G) * (long)ntn;
        return dim3((unsigned)((ub + 7) / 8 * 8));
    };
    GemmArgs a1 = {(const uint16_t *)x, row_to_slot, (const uint16_t *)w1, (uint16_t *)h, offsets, ts1,
                   s.T, s.k, s.d, 2 * s.F, s.F, G, s.F};
    hipLaunchKernelGGL((gemm_bf16_kernel<128, 128, true, true>), grid_for(p.bm1, ntn1), dim3(256), 0, st, a1);
    GemmArgs a2 = {(const uint16_t *)h, nullptr, (const uint16_t *)w2, (uint16_t *)y_perm, offsets, ts2,
                   s.T, s.k, s.F, s.d, s.d, G, s.F};
    hipLaunchKernelGGL((gemm_bf16_kernel<128, 128, false, false>), grid_for(p.bm2, ntn2), dim3(256), 0, st, a2);
    return hipGetLastError();
}

}  // namespace moe
