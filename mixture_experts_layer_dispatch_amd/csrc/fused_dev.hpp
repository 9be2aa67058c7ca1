// The persistent layer kernel (S11): router, dispatch, both expert GEMMs and the combine
// in one launch.
//
// Mega MoE wiki (aiki.softdaddy-o.com, "One-line definition", "How it works") and Mega
// MoE blog (donniechu.com, "TL;DR", "What's new"): the whole dispatch -> linear1 ->
// SwiGLU -> linear2 -> combine chain runs as one persistent kernel, so the time lost to
// launch gaps between the steps disappears and one step's tail overlaps the next one's
// head.  On one GPU there is no inter-GPU traffic to overlap; the kernel instead
// schedules tiles over the ragged expert groups and lets a linear2 tile start as soon as
// the linear1 tiles of its rows are done.
//
// Scheduling.  Work items are numbered in step order: FP8 activation blocks, router
// items, (split-K router) token selections, dispatch histograms, the plan (one item:
// scan + tile plans), dispatch scatters, then linear1 tiles, linear2 tiles and combine
// items.  Item i goes to workgroup i % P (P = co-resident workgroups, a multiple of 8, so
// item i runs on XCD i % 8 and the GEMM tiles keep the XCD-aware order of the stand-alone
// kernels).  An item waits only on items with smaller numbers, which are either done or
// held by running workgroups that never wait on larger numbers -- so with the whole grid
// resident (a cooperative launch) every wait ends.  Waits are still bounded in time:
// after 2 s a wait sets the timeout error and gives up, and so does every later wait.
//
// Decode (FP8 x FP4, few rows per group): after the plan, items are single waves --
// weight-streaming tiles of linear1 (K slices), then of linear2, then combine chunks.
// The wave that completes the last linear1 slice of a 32-row tile adds the slices,
// applies SwiGLU and quantises h for those rows, and then opens the tile to linear2.
//
// Memory ordering.  A producer makes its writes visible with an agent-scope release
// fence (every wave) before one lane bumps the counter; a consumer spins on the counter
// with relaxed agent-scope atomic loads and then issues an agent-scope acquire fence.
// Each wait is made once per workgroup or wave and remembered.
#pragma once

#include "combine_dev.hpp"
#include "common.hpp"
#include "dispatch_dev.hpp"
#include "gemm_bf16_dev.hpp"
#include "gemm_fp8_dev.hpp"
#include "kernels.hpp"
#include "route_dev.hpp"

namespace moe {

constexpr uint64_t kSpinTicks = 200000000ull;  // 2 s of the 100 MHz real-time counter

__device__ __forceinline__ int atomic_ld(const int32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Lane 0 spins until *p >= target, or until a timeout is (or was) reported.
__device__ __forceinline__ void spin_until(const int32_t *p, int target, int32_t *err) {
    if (lane_id() == 0 && atomic_ld(p) < target) {
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        while (atomic_ld(p) < target) {
            if (atomic_ld(err) == DEVERR_TIMEOUT) break;
            if (__builtin_amdgcn_s_memrealtime() - t0 > kSpinTicks) {
                set_error(err, DEVERR_TIMEOUT);
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
    }
}

// Workgroup-wide wait: wave 0 spins, then every wave acquires.
__device__ __forceinline__ void wg_wait(const int32_t *p, int target, int32_t *err) {
    if (threadIdx.x < kWave) spin_until(p, target, err);
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// Workgroup-wide release of everything written so far, then counter += v.
__device__ __forceinline__ void wg_release_add(int32_t *ctr, int v) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_fetch_add(ctr, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void wave_wait(const int32_t *p, int target, int32_t *err) {
    spin_until(p, target, err);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// Wave release, then counter += 1; returns the counter's previous value.
__device__ __forceinline__ int wave_release_add(int32_t *ctr) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    int old = 0;
    if (lane_id() == 0) old = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return __shfl(old, 0, kWave);
}

__device__ __forceinline__ long round8(long n) { return (n + 7) / 8 * 8; }

// Global index of a row tile: ts[g] / ntn row tiles precede group g.
__device__ __forceinline__ int row_tile_index(const TileInfo &ti, const int32_t *ts, int ntn) {
    return ts[ti.g] / ntn + ti.mt;
}

// ---- items of the steps before the GEMMs (workgroup items, 256 threads) ----------------

template <int MODE>
__device__ __forceinline__ void front_item(const FusedArgs &a, long i, uint8_t *lds, bool &routed) {
    if (i < a.b_r) {  // FP8 activations: 64 blocks of 128 per item
        const long nblocks = (long)a.T * a.d / 128;
#pragma unroll
        for (int pass = 0; pass < 4; ++pass)
            quant_x_lane((const uint16_t *)a.x, nblocks, a.xq, a.xs, (i * 4 + pass) * 256 + threadIdx.x);
        wg_release_add(a.sync + SYNC_QUANT, 1);
    } else if (i < a.b_sel) {  // router
        const int b = (int)(i - a.b_r);
        float *lg = (float *)lds;
        if (a.router == ROUTER_SPLITK) {
            const long w = (long)b * 4 + (threadIdx.x >> 6);
            if (w < (long)(a.E / 32) * a.nks * ((a.T + 31) / 32))
                route_splitk_wave((const uint16_t *)a.x, (const uint16_t *)a.wr, a.T, a.d, a.E, a.nks, w, a.rpart);
        } else if (a.router == ROUTER_MFMA) {
            if constexpr (MODE != MODE_F32)
                route_mfma_block((const uint16_t *)a.x, (const uint16_t *)a.wr, a.bias, a.T, a.d, a.E, a.k, a.gating, b,
                             lg, a.idx, a.gate, nullptr, nullptr, a.err);
        } else if (a.router == ROUTER_VALU8) {
            route_valu_block<MODE == MODE_F32, 8>(a.x, a.wr, a.bias, a.T, a.d, a.E, a.k, a.gating, b, lg, a.idx,
                                                   a.gate, nullptr, nullptr, a.err);
        } else {
            route_valu_block<MODE == MODE_F32, 32>(a.x, a.wr, a.bias, a.T, a.d, a.E, a.k, a.gating, b, lg, a.idx,
                                                    a.gate, nullptr, nullptr, a.err);
        }
        wg_release_add(a.sync + SYNC_ROUTE, 1);
    } else if (i < a.b_cnt) {  // split-K router: one token's selection
        if (!routed) {
            wg_wait(a.sync + SYNC_ROUTE, (int)(a.b_sel - a.b_r), a.err);
            routed = true;
        }
        route_sum_select(a.rpart, a.nks, a.T, a.E, a.k, a.gating, a.bias, i - a.b_sel, (float *)lds, a.idx, a.gate,
                         nullptr, nullptr, a.err);
        wg_release_add(a.sync + SYNC_SELECT, 1);
    } else if (i < a.b_plan) {  // dispatch histogram of one block
        wg_wait(a.router == ROUTER_SPLITK ? a.sync + SYNC_SELECT : a.sync + SYNC_ROUTE,
                (int)(a.router == ROUTER_SPLITK ? a.T : a.b_sel - a.b_r), a.err);
        count_block(a.idx, a.T, a.k, a.E, (int)(i - a.b_cnt), (unsigned long long *)lds, a.blockcounts, a.err);
        wg_release_add(a.sync + SYNC_COUNT, 1);
    } else if (i == a.b_plan) {  // scan, tile plans, cleared row-tile counters
        wg_wait(a.sync + SYNC_COUNT, a.nblk, a.err);
        int32_t *sh = (int32_t *)lds;
        dispatch_scan_block(a.blockcounts, a.nblk, a.T, a.E, a.S, a.counts, a.offsets, sh);
        tile_plan_block(a.offsets, a.G, a.bm, a.ntn1, a.bm, a.ntn2, a.ts1, a.ts2, sh);
        for (int m = threadIdx.x; m < a.nm; m += blockDim.x) a.done1[m] = 0;
        wg_release_add(a.sync + SYNC_PLAN, 1);
    } else if (i < a.b_plan + 1 + a.nblk) {  // dispatch scatter of one block
        wg_wait(a.sync + SYNC_PLAN, 1, a.err);
        scatter_block(a.idx, a.T, a.k, a.E, (int)(i - a.b_plan - 1), a.blockcounts, a.s2r, a.r2s,
                      (unsigned long long *)lds);
        wg_release_add(a.sync + SYNC_SCATTER, 1);
    }
    // [b_plan + 1 + nblk, b_end): padding to a multiple of 8
}

// Workgroup exit: the last one out clears the counters for the next launch.
__device__ __forceinline__ void fused_exit(const FusedArgs &a) {
    __syncthreads();
    if (threadIdx.x == 0) {
        const int old = __hip_atomic_fetch_add(a.sync + SYNC_EXIT, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (old == (int)gridDim.x - 1) {
            for (int w = 0; w < SYNC_WORDS; ++w)
                __hip_atomic_store(a.sync + w, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// ---- tiled variants (bf16, FP8 x FP4, fp32): every item is a workgroup item ------------

template <int MODE, int BM, int BN2>
__device__ __forceinline__ void fused_tiled(const FusedArgs &a, uint8_t *lds) {
    const long P = gridDim.x;
    long i = blockIdx.x;
    bool routed = false;
    for (; i < a.b_end; i += P) {
        __syncthreads();  // the previous item may still read its LDS
        front_item<MODE>(a, i, lds, routed);
    }
    wg_wait(a.sync + SYNC_PLAN, 1, a.err);
    const long N1 = MODE == MODE_F32 ? a.n1 : a.ts1[a.G], N2 = MODE == MODE_F32 ? a.n2 : a.ts2[a.G];
    const long e1 = a.b_end + round8(N1), e2 = e1 + round8(N2), e3 = e2 + a.ncb;
    bool scattered = false, lin1_all = false, lin2_all = false;
    for (; i < e3; i += P) {
        __syncthreads();
        if (i < e1) {  // linear1
            if (!scattered) {
                wg_wait(a.sync + SYNC_SCATTER, a.nblk, a.err);
                if constexpr (MODE == MODE_FP8) wg_wait(a.sync + SYNC_QUANT, (int)a.b_r, a.err);
                scattered = true;
            }
            const long j = i - a.b_end;
            if constexpr (MODE == MODE_F32) {
                if (j < N1) {
                    ffn1_f32_lane((const float *)a.x, a.r2s, (const float *)a.w1, a.offsets, a.G, a.T, a.k, a.d, a.F,
                                  a.rows, (float *)a.h, j * 256 + threadIdx.x);
                    wg_release_add(a.sync + SYNC_LIN1, 1);
                }
                continue;
            }
            const int tile = pick_tile((int)j, (int)N1);
            if (tile < 0) continue;
            if constexpr (MODE == MODE_BF16) {
                GemmArgs g = {(const uint16_t *)a.x, a.r2s, (const uint16_t *)a.w1, (uint16_t *)a.h, a.offsets, a.ts1,
                              a.T, a.k, a.d, 2 * a.F, a.F, a.G, a.F};
                bf16_tile<BM, 256, true, true>(g, tile, lds);
            } else {
                Fp8Args g = {a.xq, a.xs, a.r2s, (const uint8_t *)a.w1, (const uint8_t *)a.w1s, a.h, a.hs, a.offsets,
                             a.ts1, a.T, a.k, a.d, 2 * a.F, a.F, a.G, a.F};
                fp8_tile<BM, 256, 4, true, true>(g, tile, lds);
            }
            const TileInfo ti = decode_tile(tile, a.ts1, a.offsets, a.G, BM);
            wg_release_add(a.done1 + row_tile_index(ti, a.ts1, a.ntn1), 1);
        } else if (i < e2) {  // linear2
            const long j = i - e1;
            if constexpr (MODE == MODE_F32) {
                if (j < N2) {
                    if (!lin1_all) {
                        wg_wait(a.sync + SYNC_LIN1, (int)N1, a.err);
                        lin1_all = true;
                    }
                    ffn2_f32_lane((const float *)a.h, (const float *)a.w2, a.offsets, a.G, a.d, a.F, a.rows,
                                  (float *)a.yperm, j * 256 + threadIdx.x);
                    wg_release_add(a.sync + SYNC_LIN2, 1);
                }
                continue;
            }
            const int tile = pick_tile((int)j, (int)N2);
            if (tile < 0) continue;
            const TileInfo ti = decode_tile(tile, a.ts2, a.offsets, a.G, BM);
            wg_wait(a.done1 + row_tile_index(ti, a.ts2, a.ntn2), a.ntn1, a.err);
            if constexpr (MODE == MODE_BF16) {
                GemmArgs g = {(const uint16_t *)a.h, nullptr, (const uint16_t *)a.w2, (uint16_t *)a.yperm, a.offsets,
                              a.ts2, a.T, a.k, a.F, a.d, a.d, a.G, a.F};
                bf16_tile<BM, BN2, false, false>(g, tile, lds);
            } else {
                Fp8Args g = {(const uint8_t *)a.h, a.hs, nullptr, (const uint8_t *)a.w2, (const uint8_t *)a.w2s,
                             a.yperm, nullptr, a.offsets, a.ts2, a.T, a.k, a.F, a.d, a.d, a.G, a.F};
                fp8_tile<BM, BN2, 2, false, false>(g, tile, lds);
            }
            wg_release_add(a.sync + SYNC_LIN2, 1);
        } else {  // combine
            if (!lin2_all) {
                wg_wait(a.sync + SYNC_LIN2, (int)N2, a.err);
                lin2_all = true;
            }
            combine_lane<MODE == MODE_F32>(a.yperm, a.s2r, a.gate, a.y, a.T, a.k, a.d, a.S,
                                           (i - e2) * 256 + threadIdx.x);
        }
    }
    fused_exit(a);
}

// ---- decode variant (FP8 x FP4, few rows per group): wave items after the plan --------

__device__ __forceinline__ void fused_decode(const FusedArgs &a, uint8_t *lds) {
    const long P = gridDim.x;
    long i = blockIdx.x;
    bool routed = false;
    for (; i < a.b_end; i += P) {
        __syncthreads();
        front_item<MODE_FP8>(a, i, lds, routed);
    }
    wg_wait(a.sync + SYNC_PLAN, 1, a.err);
    const long N1 = a.ts1[a.G], N2 = a.ts2[a.G];
    const long e1 = N1, e2 = e1 + N2, e3 = e2 + a.ncb;
    const int lane = lane_id();
    bool ready = false, lin2_all = false;
    const DecArgs d1 = {a.xq, a.xs, a.r2s, a.offsets, a.ts1, (const uint8_t *)a.w1, (const uint8_t *)a.w1s,
                        a.upart, nullptr, a.rows, a.T, a.k, a.d, 2 * a.F, a.G, a.ks};
    const DecArgs d2 = {(const uint8_t *)a.h, a.hs, nullptr, a.offsets, a.ts2, (const uint8_t *)a.w2,
                        (const uint8_t *)a.w2s, nullptr, (uint16_t *)a.yperm, a.rows, a.T, a.k, a.F, a.d, a.G, 1};
    const int nfb = a.F / 128;
    for (long w = (long)blockIdx.x * 4 + (threadIdx.x >> 6); w < e3; w += 4 * P) {
        if (w < e1) {  // linear1 K slice of a (32 rows x 32 columns) tile
            if (!ready) {
                wave_wait(a.sync + SYNC_SCATTER, a.nblk, a.err);
                wave_wait(a.sync + SYNC_QUANT, (int)a.b_r, a.err);
                ready = true;
            }
            const int tile = (int)w;
            fp8_decode_tile<true>(d1, tile);
            const TileInfo ti = decode_tile(tile, a.ts1, a.offsets, a.G, 32);
            int32_t *ctr = a.done1 + row_tile_index(ti, a.ts1, a.ntn1);
            if (wave_release_add(ctr) == a.ntn1 - 1) {
                // last slice of this row tile: SwiGLU + e4m3 for its rows, then open it to linear2
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                for (long q = 0; q < (long)ti.nrows * nfb; ++q)
                    decode_swiglu_wave(a.upart, a.rows, a.F, a.ks, (uint8_t *)a.h, a.hs,
                                       (long)ti.row0 * nfb + q);
                wave_release_add(ctr);
            }
        } else if (w < e2) {  // linear2 tile
            const int tile = (int)(w - e1);
            const TileInfo ti = decode_tile(tile, a.ts2, a.offsets, a.G, 32);
            wave_wait(a.done1 + row_tile_index(ti, a.ts2, a.ntn2), a.ntn1 + 1, a.err);
            fp8_decode_tile<false>(d2, tile);
            wave_release_add(a.sync + SYNC_LIN2);
        } else {  // combine: 64 lanes x 8 columns
            if (!lin2_all) {
                wave_wait(a.sync + SYNC_LIN2, (int)N2, a.err);
                lin2_all = true;
            }
            combine_lane<false>(a.yperm, a.s2r, a.gate, a.y, a.T, a.k, a.d, a.S, (w - e2) * kWave + lane);
        }
    }
    fused_exit(a);
}

template <int MODE, int BM, int BN2, bool DEC>
__global__ __launch_bounds__(256) void fused_layer_kernel(FusedArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    if constexpr (DEC) fused_decode(a, lds);
    else fused_tiled<MODE, BM, BN2>(a, lds);
}

// Host side: a cooperative launch of as many workgroups as fit on the device at once
// (at most cu_limit CUs' worth when cu_limit > 0).
template <int MODE, int BM, int BN2, bool DEC>
hipError_t launch_fused_kernel(FusedArgs &a, size_t lds, int cu_limit, hipStream_t st) {
    const void *fn = (const void *)fused_layer_kernel<MODE, BM, BN2, DEC>;
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 256, lds);
    if (e != hipSuccess) return e;
    if (per_cu < 1) return hipErrorInvalidConfiguration;
    if (cu_limit > 0 && cu_limit < cus) cus = cu_limit;
    int P = cus * per_cu;
    if (P >= 8) P -= P % 8;  // item i then runs on XCD i % 8
    void *args[] = {&a};
    prof_begin(st);
    e = hipLaunchCooperativeKernel(fn, dim3(P), dim3(256), args, (unsigned)lds, st);
    prof_end("layer_fused", st);
    return e;
}

}  // namespace moe
