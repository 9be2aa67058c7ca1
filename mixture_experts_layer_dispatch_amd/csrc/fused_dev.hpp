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
// Hand-offs.  An agent-scope fence costs microseconds per wave on MI355X and its acquire
// half invalidates the XCD's whole L2, so fences are kept off the per-item path.  The
// small data of the steps before the GEMMs (routing, histograms, plan, permutation, FP8
// activations) moves through device-coherent (sc1) loads and stores, handed over by
// counters alone.  The GEMM phases read it, and the GEMM outputs, with ordinary cached
// loads; there each workgroup makes one acquire before linear1, one release after its
// last linear1 tile, one acquire before its first linear2 tile, and the same again around
// the combine.
//
// Decode (FP8 x FP4, few rows per group): from two tokens on, where the shapes allow, the
// linear phases are the stand-alone kernels' workgroup weight streams, separated by
// workgroup counts (linear1, SwiGLU, linear2).  Otherwise items are single waves --
// weight-streaming tiles of linear1 (K slices), then of linear2, then combine chunks --
// and every hand-off is coherent: the wave that completes the last linear1 slice of a
// 32-row tile adds the slices, applies SwiGLU and quantises h for those rows, and then
// opens the tile to linear2.  The plan is cached in LDS once per workgroup.
#pragma once

#include "combine_dev.hpp"
#include "common.hpp"
#include "dispatch_dev.hpp"
#include "gemm_bf16_dev.hpp"
#include "gemm_fp8_dev.hpp"
#include "gemm_fp8x8_dev.hpp"
#include "kernels.hpp"
#include "route_dev.hpp"

namespace moe {

constexpr uint64_t kSpinTicks = 200000000ull;  // 2 s of the 100 MHz real-time counter

__device__ __forceinline__ int atomic_ld(const int32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int atomic_add(int32_t *p, int v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// Timeouts.  The sticky error word err[0] keeps the first error of any kind; err[1] is
// raised by every wait that expires, so the later waits of the launch give up at once
// even when err[0] already held another code.  A wait also gives up when err[0] reads
// DEVERR_TIMEOUT.  The launch's last workgroup clears err[1] on its way out.
__device__ __forceinline__ bool timed_out(const int32_t *err) {
    return atomic_ld(err + 1) != 0 || atomic_ld(err) == DEVERR_TIMEOUT;
}
__device__ __forceinline__ void report_timeout(int32_t *err) {
    set_error(err, DEVERR_TIMEOUT);
    __hip_atomic_store(err + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Lane 0 spins until *p >= target, or until a timeout is (or was) reported.  The sleep
// between polls doubles up to MAXSLEEP x 8 x 64 cycles: many waves polling one word at
// full rate would starve the memory channel that serves it, and with it the very
// producers they wait for; a word with few pollers keeps a short sleep (low latency).
template <int MAXSLEEP>
__device__ __forceinline__ void spin_until(const int32_t *p, int target, int32_t *err) {
    if (lane_id() == 0 && atomic_ld(p) < target) {
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        int backoff = 1;
        for (unsigned n = 1; atomic_ld(p) < target; ++n) {
            if ((n & 15) == 0) {
                if (timed_out(err)) break;
                if (__builtin_amdgcn_s_memrealtime() - t0 > kSpinTicks) {
                    report_timeout(err);
                    break;
                }
            }
            for (int z = 0; z < backoff; ++z) __builtin_amdgcn_s_sleep(8);
            backoff = backoff < MAXSLEEP ? 2 * backoff : MAXSLEEP;
        }
    }
    compiler_fence();
}

// ---- spread counters and replicated flags ----------------------------------------------

__device__ __forceinline__ int32_t *counter_sub(int32_t *sync, int c, long id) {
    return sync + ((long)c * kSpread + id % kSpread) * kSlot;
}
__device__ __forceinline__ int32_t *flag_replica(int32_t *sync, int f, long id) {
    return sync + ((long)(NUM_COUNTERS + f) * kSpread + id % kSpread) * kSlot;
}

// Sum of a spread counter, in every lane of the calling wave (one load per lane).
__device__ __forceinline__ int counter_sum(int32_t *sync, int c) {
    int v = atomic_ld(counter_sub(sync, c, lane_id()));
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
    return v;
}

// The calling wave polls a spread counter until its sum reaches target (bounded, with
// the same back-off as spin_until).
template <int MAXSLEEP>
__device__ __forceinline__ void counter_wait(int32_t *sync, int c, int target, int32_t *err) {
    if (counter_sum(sync, c) < target) {
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        int backoff = 1;
        for (unsigned n = 1; counter_sum(sync, c) < target; ++n) {
            if ((n & 15) == 0) {
                if (__shfl((int)timed_out(err), 0, kWave)) break;
                if (__builtin_amdgcn_s_memrealtime() - t0 > kSpinTicks) {
                    if (lane_id() == 0) report_timeout(err);
                    break;
                }
            }
            for (int z = 0; z < backoff; ++z) __builtin_amdgcn_s_sleep(8);
            backoff = backoff < MAXSLEEP ? 2 * backoff : MAXSLEEP;
        }
    }
    compiler_fence();
}

// One wave raises a flag: all replicas (the wave's stores done first).
__device__ __forceinline__ void flag_raise(int32_t *sync, int f) {
    wait_vmcnt<0>();
    compiler_fence();
    __hip_atomic_store(flag_replica(sync, f, lane_id()), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- coherent hand-offs (data moved with sc1 accesses) --------------------------------

// Producer workgroup item id: every wave's sc1 stores complete, then counter c += 1.
__device__ __forceinline__ void wg_count(int32_t *sync, int c, long id) {
    wait_vmcnt<0>();
    compiler_fence();
    __syncthreads();
    if (threadIdx.x == 0) atomic_add(counter_sub(sync, c, id), 1);
}
// (the steps before the GEMMs have a few waiting workgroups: a short sleep by default)
template <int MAXSLEEP = 1>
__device__ __forceinline__ void wg_counter_wait(int32_t *sync, int c, int target, int32_t *err) {
    if (threadIdx.x < kWave) counter_wait<MAXSLEEP>(sync, c, target, err);
    __syncthreads();
    compiler_fence();
}
// (every workgroup polls: kSpread replicas keep each word to a few pollers)
__device__ __forceinline__ void wg_flag_wait(int32_t *sync, int f, int32_t *err) {
    if (threadIdx.x < kWave) spin_until<2>(flag_replica(sync, f, blockIdx.x), 1, err);
    __syncthreads();
    compiler_fence();
}
// Producer workgroup raising a flag once its (and every wave's) stores are done.
__device__ __forceinline__ void wg_flag_raise(int32_t *sync, int f) {
    wait_vmcnt<0>();
    compiler_fence();
    __syncthreads();
    if (threadIdx.x < kWave) flag_raise(sync, f);
}

// ---- fenced hand-offs (data moved with ordinary cached accesses) ------------------------

__device__ __forceinline__ void wg_release_count(int32_t *sync, int c) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    if (threadIdx.x == 0) atomic_add(counter_sub(sync, c, blockIdx.x), 1);
}
// (every workgroup waits: the long sleep)
__device__ __forceinline__ void wg_counter_wait_acquire(int32_t *sync, int c, int target, int32_t *err) {
    wg_counter_wait<16>(sync, c, target, err);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

__device__ __forceinline__ long round8(long n) { return (n + 7) / 8 * 8; }

// ---- items of the steps before the GEMMs (workgroup items) -------------------------------
//
// Each item does the work of 256 threads; in the 512-thread kernel the upper 256 only take
// part in the barriers.

static __device__ __noinline__ void route_tile8_call(const uint16_t *x, const uint16_t *wr, int T, int d, int E, int nks,
                                             int b, float *part);

// W8: the 512-thread kernel's items (the tiled router runs only there)
// KIND: -1 every kind of item (inlined callers), else only that kind's code (0 FP8
// activations, 1 router, 2 selection, 3 histogram, 4 plan, 5 scatter), so that each
// out-of-line instantiation is a compact function of its own.
template <int MODE, bool W8 = false, int KIND = -1>
__device__ __forceinline__ void front_item(const FusedArgs &a, long i, uint8_t *lds, bool &routed) {
    constexpr bool ALL = KIND < 0;
    const int nr = (int)(a.b_sel - a.b_r);
    if ((ALL || KIND == 0) && i < a.b_r) {  // FP8 activations: a contiguous range of 128-value blocks per item
        // Coarse items (a counter hand-off each), every thread of the workgroup with 16 loads in
        // flight per lane, device-coherent stores (no fence).
        const long nblocks = (long)a.T * a.d / 128;
        const long per = (nblocks + a.b_r - 1) / a.b_r, blk0 = i * per;
        const long blk1 = blk0 + per < nblocks ? blk0 + per : nblocks;
        const long nth = blockDim.x;
        for (long gid = blk0 * 16 + threadIdx.x; gid - threadIdx.x < blk1 * 16; gid += 16 * nth)
            quant_x_batch<16, true>((const uint16_t *)a.x, blk1, a.xq, a.xs, gid, nth);
        wg_count(a.sync, CNT_QUANT, i);
    } else if ((ALL || KIND == 1) && i < a.b_sel) {  // router
        const int b = (int)(i - a.b_r);
        float *lg = (float *)lds;
        if (W8 && a.router == ROUTER_TILE) {
            // one 256 x 256 tile of one K slice; its partial logits go out with device-coherent
            // stores, complete before the count (selection reads them with coherent loads)
            if constexpr (W8 && MODE != MODE_F32)
                route_tile8_call((const uint16_t *)a.x, (const uint16_t *)a.wr, a.T, a.d, a.E, a.nks, b, a.rpart);
        } else if (a.router == ROUTER_SPLITK) {
            const long w = (long)b * 4 + (threadIdx.x >> 6);
            if (threadIdx.x < 256 && w < (long)(a.E / 32) * a.nks * ((a.T + 31) / 32))
                route_splitk_wave<true>((const uint16_t *)a.x, (const uint16_t *)a.wr, a.T, a.d, a.E, a.nks, w,
                                        a.rpart);
        } else if (a.router == ROUTER_MFMA) {
            if constexpr (MODE != MODE_F32)
                route_mfma_block<true>((const uint16_t *)a.x, (const uint16_t *)a.wr, a.bias, a.T, a.d, a.E, a.k,
                                       a.gating, b, lg, a.idx, a.gate, nullptr, nullptr, a.err);
        } else {
            route_valu_block<MODE == MODE_F32, 8, true>(a.x, a.wr, a.bias, a.T, a.d, a.E, a.k, a.gating, b, lg,
                                                        a.idx, a.gate, nullptr, nullptr, a.err);
        }
        wg_count(a.sync, CNT_ROUTE, b);
    } else if ((ALL || KIND == 2) && i < a.b_cnt) {  // sliced router: selection, sel4 tokens or one
        if (!routed) {
            wg_counter_wait(a.sync, CNT_ROUTE, nr, a.err);
            routed = true;
        }
        if (a.sel4) {
            // sel4 tokens per item, a wave each in turn (every wave of the workgroup)
            const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
            const long t0 = (i - a.b_sel) * a.sel4, t1 = t0 + a.sel4 < a.T ? t0 + a.sel4 : a.T;
            for (long t = t0 + wave; t < t1; t += nw)
                route_sum_select_wave<true>(a.rpart, a.nks, a.T, a.E, a.k, a.gating, a.bias, t,
                                            (float *)lds + wave * a.E, a.idx, a.gate, nullptr, nullptr, a.err);
        } else {
            route_sum_select<true>(a.rpart, a.nks, a.T, a.E, a.k, a.gating, a.bias, i - a.b_sel, (float *)lds, a.idx,
                                   a.gate, nullptr, nullptr, a.err);
        }
        wg_count(a.sync, CNT_SELECT, i - a.b_sel);
    } else if ((ALL || KIND == 3) && i < a.b_plan) {  // dispatch histogram of one block
        if (router_in_slices(a.router)) wg_counter_wait(a.sync, CNT_SELECT, (int)(a.b_cnt - a.b_sel), a.err);
        else wg_counter_wait(a.sync, CNT_ROUTE, nr, a.err);
        count_block<true>(a.idx, a.T, a.k, a.E, (int)(i - a.b_cnt), (unsigned long long *)lds, a.blockcounts,
                          a.err);
        wg_count(a.sync, CNT_COUNT, i - a.b_cnt);
    } else if ((ALL || KIND == 4) && i == a.b_plan) {  // scan, tile plans, cleared row-tile counters
        int32_t *sh = (int32_t *)lds;
        if (a.nblk == 1) {
            // one dispatch block: histogram, scan and scatter through LDS, then the plan
            if (router_in_slices(a.router)) wg_counter_wait(a.sync, CNT_SELECT, (int)(a.b_cnt - a.b_sel), a.err);
            else wg_counter_wait(a.sync, CNT_ROUTE, nr, a.err);
            dispatch_single_block<true>(a.idx, a.T, a.k, a.E, a.S, a.counts, a.offsets, a.s2r, a.r2s, a.err, lds);
            wait_vmcnt<0>();
            __syncthreads();
        } else {
            wg_counter_wait(a.sync, CNT_COUNT, a.nblk, a.err);
            dispatch_scan_block<true>(a.blockcounts, a.nblk, a.T, a.E, a.S, a.counts, a.offsets, sh);
        }
        tile_plan_block<true>(a.offsets, a.G, a.bm, a.ntn1, a.bm, a.ntn2, a.ts1, a.ts2, sh);
        for (long m = threadIdx.x; m < (long)a.nm * kRowTileSlots; m += blockDim.x) stc<true>(a.done1 + m * kSlot, 0);
        if (a.nblk == 1) {
            wg_counter_wait(a.sync, CNT_QUANT, (int)a.b_r, a.err);
            wg_flag_raise(a.sync, FLAG_FRONT);
        } else {
            wg_flag_raise(a.sync, FLAG_PLAN);
        }
    } else if ((ALL || KIND == 5) && a.nblk > 1 && i < a.b_plan + 1 + a.nblk) {  // dispatch scatter of one block
        wg_flag_wait(a.sync, FLAG_PLAN, a.err);
        scatter_block<true>(a.idx, a.T, a.k, a.E, (int)(i - a.b_plan - 1), a.blockcounts, a.s2r, a.r2s,
                            (unsigned long long *)lds);
        // the last scatter block also waits for the activations, then opens linear1
        wait_vmcnt<0>();
        compiler_fence();
        __syncthreads();
        int *last = (int *)lds;
        if (threadIdx.x == 0) *last = atomic_add(a.sync + kSyncTopScatter, 1) == a.nblk - 1;
        __syncthreads();
        if (*last) {
            wg_counter_wait(a.sync, CNT_QUANT, (int)a.b_r, a.err);
            wg_flag_raise(a.sync, FLAG_FRONT);
        }
    }
    // the rest up to b_end: padding to a multiple of 8
}

// Workgroup exit: the last one out clears the synchronisation words for the next launch
// (a two-level count: one sub-counter per 64 workgroups, then a top counter).
__device__ __forceinline__ void fused_exit(const FusedArgs &a, uint8_t *lds) {
    __syncthreads();
    int *last = (int *)lds;
    if (threadIdx.x == 0) {
        const int P = (int)gridDim.x, sub = (int)(blockIdx.x % kSpread);
        const int nsub = P < kSpread ? P : kSpread, per = (P - sub + kSpread - 1) / kSpread;
        int l = 0;
        if (atomic_add(counter_sub(a.sync, CNT_EXIT, sub), 1) == per - 1)
            l = atomic_add(a.sync + kSyncTopExit, 1) == nsub - 1;
        *last = l;
    }
    __syncthreads();
    if (*last) {
        for (int w = threadIdx.x; w < (NUM_COUNTERS + NUM_FLAGS) * kSpread; w += blockDim.x)
            __hip_atomic_store(a.sync + (long)w * kSlot, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (threadIdx.x == 0) {
            __hip_atomic_store(a.sync + kSyncTopExit, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(a.sync + kSyncTopScatter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(a.err + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// ---- 8-wave GEMM tiles, called out of line -----------------------------------------------
//
// The persistent kernel is one large function: inlined into it, the 8-wave tiles (about 200
// VGPRs each at two waves per SIMD) would share its register allocation and spill.  Called
// out of line they keep their own, and the call saves the caller's live registers once per
// tile.  Arguments arrive in vector registers, so they are read back as uniform values, and
// the tiles take the kernel's dynamic LDS directly.
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
template <typename P>
__device__ __forceinline__ P *unip(P *p) {
    const uint64_t u = (uint64_t)p;
    return (P *)(((uint64_t)(uint32_t)uni((int)(u >> 32)) << 32) | (uint32_t)uni((int)(uint32_t)u));
}
template <typename Args>
__device__ __forceinline__ void uniform_ints(Args &a) {
    a.T = uni(a.T); a.k = uni(a.k); a.K = uni(a.K); a.Ntot = uni(a.Ntot);
    a.ldc = uni(a.ldc); a.G = uni(a.G); a.F = uni(a.F);
}

template <bool SWIGLU>
__device__ __noinline__ void bf16_tile8_call(GemmArgs a, int tile, int half) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds_dyn[];
    a.A = unip(a.A); a.row_to_slot = unip(a.row_to_slot); a.B = unip(a.B); a.C = unip(a.C);
    a.offsets = unip(a.offsets); a.tile_start = unip(a.tile_start);
    uniform_ints(a);
    bf16_tile8<SWIGLU, SWIGLU>(a, uni(tile), lds_dyn, uni(half));
}

template <bool SWIGLU>
__device__ __noinline__ void fp8_tile8_call(Fp8Args a, int tile, int half) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds_dyn[];
    a.A = unip(a.A); a.As = unip(a.As); a.row_to_slot = unip(a.row_to_slot); a.B = unip(a.B);
    a.Bs = unip(a.Bs); a.C = unip(a.C); a.Cs = unip(a.Cs); a.offsets = unip(a.offsets);
    a.tile_start = unip(a.tile_start);
    uniform_ints(a);
    fp8_tile8<1, 8, SWIGLU, SWIGLU>(a, uni(tile), lds_dyn, uni(half));
}

// Router tile b of the tiled router (the stand-alone path's route_tile_kernel without its
// XCD-aware order: slice b / per, then the 256-token tile fastest and the 256-expert tile).
static __device__ __noinline__ void route_tile8_call(const uint16_t *x, const uint16_t *wr, int T, int d, int E, int nks,
                                             int b, float *part) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds_dyn[];
    x = unip(x);
    wr = unip(wr);
    part = unip(part);
    T = uni(T);
    d = uni(d);
    E = uni(E);
    nks = uni(nks);
    b = uni(b);
    const int mtn = (T + 255) / 256, per = mtn * (E / 256);
    const int ks = b / per, rem = b % per;
    TileInfo ti;
    ti.g = 0;
    ti.mt = rem % mtn;
    ti.nt = rem / mtn;
    ti.row0 = ti.mt * 256;
    ti.nrows = min(256, T - ti.row0);
    GemmArgs g = {x, nullptr, wr, (uint16_t *)(part + (long)ks * T * E), nullptr, nullptr, T, 1, d, E, E, 1, 0};
    const int kchunk = d / nks;
    bf16_tile8_rows<false, false, true, true>(g, ti, d, ks * kchunk, kchunk / 32, lds_dyn);
}

// The steps before the GEMMs, out of line in the 512-thread and decode kernels (inlined
// there, they would share those kernels' register allocation and spill); the kernel
// arguments are read back as uniform values.  W8: the 512-thread kernel's items.
template <int MODE, bool W8, int KIND>
__device__ __noinline__ int front_item_call(FusedArgs a, long i, int routed) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds_dyn[];
    static_assert(sizeof(FusedArgs) % 4 == 0, "argument words");
    FusedArgs u;
    const int32_t *src = (const int32_t *)&a;
    int32_t *dst = (int32_t *)&u;
#pragma unroll
    for (int w = 0; w < (int)(sizeof(FusedArgs) / 4); ++w) dst[w] = uni(src[w]);
    const long iu = ((long)uni((int)(i >> 32)) << 32) | (uint32_t)uni((int)i);
    bool r = uni(routed) != 0;
    front_item<MODE, W8, KIND>(u, iu, lds_dyn, r);
    return r ? 1 : 0;
}

// Item i's kind (see front_item), -1 for the padding items; each kind runs in a function of
// its own: one function holding every kind measured ~10 us per call even for a padding item
// (a padding item now makes no call).
__device__ __forceinline__ int front_kind(const FusedArgs &a, long i) {
    if (i < a.b_r) return 0;
    if (i < a.b_sel) return 1;
    if (i < a.b_cnt) return 2;
    if (i < a.b_plan) return 3;
    if (i == a.b_plan) return 4;
    return a.nblk > 1 && i < a.b_plan + 1 + a.nblk ? 5 : -1;
}
template <int MODE, bool W8>
__device__ __forceinline__ bool front_item_out(const FusedArgs &a, long i, bool routed) {
    const int r = routed ? 1 : 0;
    switch (front_kind(a, i)) {
        case 0: return front_item_call<MODE, W8, 0>(a, i, r) != 0;
        case 1: return front_item_call<MODE, W8, 1>(a, i, r) != 0;
        case 2: return front_item_call<MODE, W8, 2>(a, i, r) != 0;
        case 3: return front_item_call<MODE, W8, 3>(a, i, r) != 0;
        case 4: return front_item_call<MODE, W8, 4>(a, i, r) != 0;
        case 5: return front_item_call<MODE, W8, 5>(a, i, r) != 0;
        default: return routed;
    }
}

// ---- tiled variants (bf16, FP8 x FP4, fp32): every item is a workgroup item ------------
//
// W8: 512 threads, and the GEMM items run the 8-wave 256 x 256 tiles of the stand-alone
// kernels (same k order per output element, so the same bits).

template <int MODE, int BM, int BN2, bool W8 = false>
__device__ __forceinline__ void fused_tiled(const FusedArgs &a, uint8_t *lds) {
    static_assert(!W8 || (MODE != MODE_F32 && BM == 256 && BN2 == 256), "8-wave tiles are 256 x 256");
    const long P = gridDim.x;
    long i = blockIdx.x;
    bool routed = false;
    for (; i < a.b_end; i += P) {
        __syncthreads();  // the previous item may still read its LDS
        if constexpr (W8) routed = front_item_out<MODE, true>(a, i, routed);
        else front_item<MODE>(a, i, lds, routed);
    }
    // everything before linear1, then one acquire: the GEMMs read it with cached loads
    wg_flag_wait(a.sync, FLAG_FRONT, a.err);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    const long N1 = MODE == MODE_F32 ? a.n1 : a.ts1[a.G], N2 = MODE == MODE_F32 ? a.n2 : a.ts2[a.G];
    const long e1 = a.b_end + round8(N1), e2 = e1 + round8(N2), e3 = e2 + a.ncb;
    if constexpr (W8) {
        // GEMM tiles vary in cost (a group's last row tile holds few rows), so they are
        // taken from queues as workgroups free up instead of dealt round robin: queue
        // b % 8 hands workgroup b the items q * 8 + b % 8 (its XCD's tiles under the
        // XCD-aware tile order), linear1 before linear2.  A workgroup leaves linear1 (and
        // counts itself past it) when it first takes a linear2 item or runs out; linear2
        // waits for every workgroup past linear1 -- which each reaches, as linear1 items
        // wait on nothing.  The taken index is broadcast through LDS between tiles.  Indices
        // map to tiles as block indices do in the stand-alone kernels, tail split included
        // (a queue's short last round of 256-row tiles as 128-row halves; C = workgroups
        // per queue).
        const int nq = P % 8 == 0 ? 8 : 1, qid = (int)(blockIdx.x % nq);
        const int C = (int)(P / 8 > 0 ? P / 8 : 1);
        int32_t *queue = counter_sub(a.sync, CNT_QUEUE, qid);
        const long n1 = 8L * ((N1 + 7) / 8 + C / 2), n12 = n1 + 8L * ((N2 + 7) / 8 + C / 2);
        bool past1 = false, open2 = false;
        int *slot = (int *)lds;
        for (;;) {
            __syncthreads();  // the previous tile is done with the LDS
            if (threadIdx.x == 0) *slot = atomic_add(queue, 1);
            __syncthreads();
            const long j = (long)*slot * nq + qid;
            __syncthreads();  // every thread has the index before a tile reuses the LDS
            if (j >= n12) break;
            int half;
            if (j < n1) {
                const int tile = pick_tile_split((int)j, (int)N1, C, half);
                if (tile < 0) continue;
                if constexpr (MODE == MODE_BF16) {
                    GemmArgs g = {(const uint16_t *)a.x, a.r2s, (const uint16_t *)a.w1, (uint16_t *)a.h, a.offsets,
                                  a.ts1, a.T, a.k, a.d, 2 * a.F, a.F, a.G, a.F};
                    bf16_tile8_call<true>(g, tile, half);
                } else {
                    Fp8Args g = {a.xq, a.xs, a.r2s, (const uint8_t *)a.w1, (const uint8_t *)a.w1s, a.h, a.hs,
                                 a.offsets, a.ts1, a.T, a.k, a.d, 2 * a.F, a.F, a.G, a.F};
                    fp8_tile8_call<true>(g, tile, half);
                }
            } else {
                if (!past1) {
                    wg_release_count(a.sync, CNT_LIN1);
                    past1 = true;
                }
                if (!open2) {
                    wg_counter_wait_acquire(a.sync, CNT_LIN1, (int)P, a.err);
                    open2 = true;
                }
                const int tile = pick_tile_split((int)(j - n1), (int)N2, C, half);
                if (tile < 0) continue;
                if constexpr (MODE == MODE_BF16) {
                    GemmArgs g = {(const uint16_t *)a.h, nullptr, (const uint16_t *)a.w2, (uint16_t *)a.yperm,
                                  a.offsets, a.ts2, a.T, a.k, a.F, a.d, a.d, a.G, a.F};
                    bf16_tile8_call<false>(g, tile, half);
                } else {
                    Fp8Args g = {(const uint8_t *)a.h, a.hs, nullptr, (const uint8_t *)a.w2, (const uint8_t *)a.w2s,
                                 a.yperm, nullptr, a.offsets, a.ts2, a.T, a.k, a.F, a.d, a.d, a.G, a.F};
                    fp8_tile8_call<false>(g, tile, half);
                }
            }
        }
        if (!past1) wg_release_count(a.sync, CNT_LIN1);
        i = e2 + blockIdx.x;  // the combine items stay dealt round robin
    }
    if constexpr (!W8) {  // GEMM items dealt round robin
        for (; i < e1; i += P) {  // linear1
            __syncthreads();
            const long j = i - a.b_end;
            if constexpr (MODE == MODE_F32) {
                if (j < N1)
                    ffn1_f32_lane((const float *)a.x, a.r2s, (const float *)a.w1, a.offsets, a.G, a.T, a.k, a.d,
                                  a.F, a.rows, (float *)a.h, j * 256 + threadIdx.x);
            } else {
                const int tile = pick_tile((int)j, (int)N1);
                if (tile < 0) continue;
                if constexpr (MODE == MODE_BF16) {
                    GemmArgs g = {(const uint16_t *)a.x, a.r2s, (const uint16_t *)a.w1, (uint16_t *)a.h, a.offsets,
                                  a.ts1, a.T, a.k, a.d, 2 * a.F, a.F, a.G, a.F};
                    bf16_tile<BM, 256, true, true>(g, tile, lds);
                } else if constexpr (MODE == MODE_FP8X8) {
                    Fp8Args g = {a.xq, a.xs, a.r2s, (const uint8_t *)a.w1, (const uint8_t *)a.w1s, a.h, a.hs,
                                 a.offsets, a.ts1, a.T, a.k, a.d, 2 * a.F, a.F, a.G, a.F};
                    fp8x8_tile<true, true, 256>(g, tile, lds);
                } else {
                    Fp8Args g = {a.xq, a.xs, a.r2s, (const uint8_t *)a.w1, (const uint8_t *)a.w1s, a.h, a.hs,
                                 a.offsets, a.ts1, a.T, a.k, a.d, 2 * a.F, a.F, a.G, a.F};
                    fp8_tile<BM, 256, 4, true, true>(g, tile, lds);
                }
            }
        }
        wg_release_count(a.sync, CNT_LIN1);
        bool open2 = false;
        for (; i < e2; i += P) {  // linear2
            if (!open2) {
                wg_counter_wait_acquire(a.sync, CNT_LIN1, (int)P, a.err);
                open2 = true;
            }
            __syncthreads();
            const long j = i - e1;
            if constexpr (MODE == MODE_F32) {
                if (j < N2)
                    ffn2_f32_lane((const float *)a.h, (const float *)a.w2, a.offsets, a.G, a.d, a.F, a.rows,
                                  (float *)a.yperm, j * 256 + threadIdx.x);
            } else {
                const int tile = pick_tile((int)j, (int)N2);
                if (tile < 0) continue;
                if constexpr (MODE == MODE_BF16) {
                    GemmArgs g = {(const uint16_t *)a.h, nullptr, (const uint16_t *)a.w2, (uint16_t *)a.yperm,
                                  a.offsets, a.ts2, a.T, a.k, a.F, a.d, a.d, a.G, a.F};
                    bf16_tile<BM, BN2, false, false>(g, tile, lds);
                } else if constexpr (MODE == MODE_FP8X8) {
                    Fp8Args g = {(const uint8_t *)a.h, a.hs, nullptr, (const uint8_t *)a.w2, (const uint8_t *)a.w2s,
                                 a.yperm, nullptr, a.offsets, a.ts2, a.T, a.k, a.F, a.d, a.d, a.G, a.F};
                    fp8x8_tile<false, false, BN2>(g, tile, lds);
                } else {
                    Fp8Args g = {(const uint8_t *)a.h, a.hs, nullptr, (const uint8_t *)a.w2, (const uint8_t *)a.w2s,
                                 a.yperm, nullptr, a.offsets, a.ts2, a.T, a.k, a.F, a.d, a.d, a.G, a.F};
                    fp8_tile<BM, BN2, 2, false, false>(g, tile, lds);
                }
            }
        }
    }
    wg_release_count(a.sync, CNT_LIN2);
    bool waited = false;
    for (; i < e3; i += P) {  // combine
        if (!waited) {
            wg_counter_wait_acquire(a.sync, CNT_LIN2, (int)P, a.err);
            waited = true;
        }
        if constexpr (W8) {  // the upper 256 threads take the next round's item
            const long item = threadIdx.x < 256 ? i : i + P;
            if (item < e3)
                combine_lane<false, false>(a.yperm, a.s2r, a.gate, a.y, a.T, a.k, a.d, a.S,
                                           (item - e2) * 256 + (threadIdx.x & 255));
            i += P;
        } else if (threadIdx.x < 256) {
            combine_lane<MODE == MODE_F32, false>(a.yperm, a.s2r, a.gate, a.y, a.T, a.k, a.d, a.S,
                                                  (i - e2) * 256 + threadIdx.x);
        }
    }
    fused_exit(a, lds);
}

// ---- decode variant (FP8 x FP4, few rows per group): wave items after the plan --------

// One weight-streaming tile, out of line (its own register allocation: two blocks of
// weights in flight per wave), with the plan read from the kernel's LDS.
template <bool LIN1>
__device__ __noinline__ void fp8_decode_tile_call(DecArgs d, int tile, int G) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds_dyn[];
    const int32_t *lts = (const int32_t *)lds_dyn + (LIN1 ? 0 : uni(G) + 1), *loffs = (const int32_t *)lds_dyn + 2 * (uni(G) + 1);
    d.A = unip(d.A); d.As = unip(d.As); d.row_to_slot = unip(d.row_to_slot); d.offsets = unip(d.offsets);
    d.tile_start = unip(d.tile_start); d.B = unip(d.B); d.Bs = unip(d.Bs); d.part = unip(d.part); d.Y = unip(d.Y);
    d.T = uni(d.T); d.k = uni(d.k); d.K = uni(d.K); d.N = uni(d.N); d.G = uni(d.G); d.ks = uni(d.ks);
    d.rows = ((long)uni((int)(d.rows >> 32)) << 32) | (uint32_t)uni((int)d.rows);
    fp8_decode_tile<LIN1, true, true>(d, uni(tile), lts, loffs);
}

// ---- decode with workgroup weight streams ----------------------------------------------
//
// The linear phases are the stand-alone kernels' workgroup weight streams (fp8_gemv_run:
// a row tile's activations staged in LDS once for all of the workgroup's column tiles),
// with coherent outputs; the phases are separated by workgroup counts (linear1, SwiGLU,
// linear2, each waited for by every workgroup), so every hand-off is a coherent one and no
// fence is needed.  Same tiles, same K slices, same k order per output element as the
// stand-alone kernels: the same bits.

// One workgroup's stream over the tile plan in LDS, out of line (its own register
// allocation); the arguments are read back as uniform values.
template <bool LIN1, int QC, int NB, int D>
__device__ __noinline__ void gemv_stream_call(DecArgs d, int rmax, int total) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds_dyn[];
    d.A = unip(d.A); d.As = unip(d.As); d.row_to_slot = unip(d.row_to_slot); d.offsets = unip(d.offsets);
    d.tile_start = unip(d.tile_start); d.B = unip(d.B); d.Bs = unip(d.Bs); d.part = unip(d.part); d.Y = unip(d.Y);
    d.T = uni(d.T); d.k = uni(d.k); d.K = uni(d.K); d.N = uni(d.N); d.G = uni(d.G); d.ks = uni(d.ks);
    d.rows = ((long)uni((int)(d.rows >> 32)) << 32) | (uint32_t)uni((int)d.rows);
    fp8_gemv_run<LIN1, QC, NB, D, true>(d, uni(rmax), (const int32_t *)lds_dyn, lds_dyn, uni(total));
}

// linear1 streams 1024-wide K slices (NB = 4), linear2 2048-wide ones (NB = 8); qc column
// quads per workgroup tile (4, else 1), dd weight blocks in flight per wave (8 at one
// workgroup per CU, else 4)
template <bool LIN1>
__device__ __forceinline__ void gemv_stream(const DecArgs &d, int rmax, int total, int qc, int dd) {
    constexpr int NB = LIN1 ? 4 : 8;
    if (qc == 4) {
        if (dd == 8) gemv_stream_call<LIN1, 4, NB, 8>(d, rmax, total);
        else gemv_stream_call<LIN1, 4, NB, 4>(d, rmax, total);
    } else {
        if constexpr (!LIN1) {
            if (dd == 8) {
                gemv_stream_call<LIN1, 1, NB, 8>(d, rmax, total);
                return;
            }
        }
        gemv_stream_call<LIN1, 1, NB, 4>(d, rmax, total);
    }
}

// After the steps before the GEMMs (the front flag seen).  LDS: the current phase's tile
// plan (tile starts, then group offsets, loaded from the workspace), then the stream's
// staging buffers.
__device__ __forceinline__ void fused_decode_stream(const FusedArgs &a, uint8_t *lds) {
    const long P = gridDim.x;
    const int G = a.G, lane = lane_id(), wave = threadIdx.x >> 6;
    const int rmax = a.T < 32 ? a.T : 32;
    int32_t *plan = (int32_t *)lds;
    auto load_plan = [&](const int32_t *ts) {
        __syncthreads();  // the previous phase is done with the LDS
        for (int g = threadIdx.x; g <= G; g += blockDim.x) {
            plan[g] = ldc<true>(ts + g);
            plan[G + 1 + g] = ldc<true>(a.offsets + g);
        }
        __syncthreads();
    };
    load_plan(a.ts1);
    const DecArgs d1 = {a.xq, a.xs, a.r2s, a.offsets, a.ts1, (const uint8_t *)a.w1, (const uint8_t *)a.w1s,
                        a.upart, nullptr, a.rows, a.T, a.k, a.d, 2 * a.F, G, a.ks};
    gemv_stream<true>(d1, rmax, plan[G] / (4 * a.sq1), a.sq1, a.sd1);
    wg_count(a.sync, CNT_LIN1, blockIdx.x);
    // SwiGLU and h's e4m3 codes: one wave per (row, 128-column block)
    wg_counter_wait<16>(a.sync, CNT_LIN1, (int)P, a.err);
    const long nsw = a.rows * (a.F / 128);
    for (long w = blockIdx.x * 4 + wave; w < nsw; w += 4 * P)
        decode_swiglu_wave<true>(a.upart, a.rows, a.F, a.ks, (uint8_t *)a.h, a.hs, w);
    wg_count(a.sync, CNT_SWIGLU, blockIdx.x);
    wg_counter_wait<16>(a.sync, CNT_SWIGLU, (int)P, a.err);
    load_plan(a.ts2);
    const DecArgs d2 = {(const uint8_t *)a.h, a.hs, nullptr, a.offsets, a.ts2, (const uint8_t *)a.w2,
                        (const uint8_t *)a.w2s, nullptr, (uint16_t *)a.yperm, a.rows, a.T, a.k, a.F, a.d, G, 1};
    gemv_stream<false>(d2, rmax, plan[G] / (4 * a.sq2), a.sq2, a.sd2);
    wg_count(a.sync, CNT_LIN2, blockIdx.x);
    // combine: 64 lanes x 8 columns per wave item; y_perm lines were written by two
    // linear2 tiles each, all finished before this read
    wg_counter_wait<16>(a.sync, CNT_LIN2, (int)P, a.err);
    for (long w = blockIdx.x * 4 + wave; w < a.ncb; w += 4 * P)
        combine_lane<false, false>(a.yperm, a.s2r, a.gate, a.y, a.T, a.k, a.d, a.S, w * kWave + lane);
    fused_exit(a, lds);
}

__device__ __forceinline__ void fused_decode(const FusedArgs &a, uint8_t *lds) {
    const long P = gridDim.x;
    long i = blockIdx.x;
    bool routed = false;
    for (; i < a.b_end; i += P) {
        __syncthreads();
        routed = front_item_out<MODE_FP8, false>(a, i, routed);
    }
    wg_flag_wait(a.sync, FLAG_FRONT, a.err);
    if (a.sq1 > 0) {
        fused_decode_stream(a, lds);
        return;
    }
    // the plan in LDS: tile prefixes of both GEMMs and the group offsets
    const int G = a.G;
    int32_t *lts1 = (int32_t *)lds, *lts2 = lts1 + (G + 1), *loffs = lts2 + (G + 1);
    __syncthreads();
    for (int g = threadIdx.x; g <= G; g += blockDim.x) {
        lts1[g] = ldc<true>(a.ts1 + g);
        lts2[g] = ldc<true>(a.ts2 + g);
        loffs[g] = ldc<true>(a.offsets + g);
    }
    __syncthreads();
    const long N1 = lts1[G], N2 = lts2[G];
    const int nfb = a.F / 128;
    const long MT = N1 / a.ntn1;  // row tiles
    const long e1 = N1, es = e1 + MT * nfb, e2 = es + N2, e3 = e2 + a.ncb;
    const int lane = lane_id();
    bool lin2_all = false;
    const DecArgs d1 = {a.xq, a.xs, a.r2s, a.offsets, a.ts1, (const uint8_t *)a.w1, (const uint8_t *)a.w1s,
                        a.upart, nullptr, a.rows, a.T, a.k, a.d, 2 * a.F, G, a.ks};
    const DecArgs d2 = {(const uint8_t *)a.h, a.hs, nullptr, a.offsets, a.ts2, (const uint8_t *)a.w2,
                        (const uint8_t *)a.w2s, nullptr, (uint16_t *)a.yperm, a.rows, a.T, a.k, a.F, a.d, G, 1};
    auto row_tile = [&](long m) { return a.done1 + m * kRowTileSlots * kSlot; };
    for (long w = (long)blockIdx.x * 4 + (threadIdx.x >> 6); w < e3; w += 4 * P) {
        if (w < e1) {  // linear1 K slice of a (32 rows x 32 columns) tile
            const int tile = (int)w;
            fp8_decode_tile_call<true>(d1, tile, G);
            const TileInfo ti = decode_tile(tile, lts1, loffs, G, 32);
            int32_t *rt = row_tile(lts1[ti.g] / a.ntn1 + ti.mt);
            // two-level count of this row tile's linear1 items: sub-counter (item % 8), then
            // top; the last one opens the tile's SwiGLU blocks
            wait_vmcnt<0>();
            compiler_fence();
            int done = 0;
            if (lane == 0 && atomic_add(rt + (ti.nt % 8) * kSlot, 1) == a.ntn1 / 8 - 1)
                done = atomic_add(rt + 8 * kSlot, 1) == 7;
            if (__shfl(done, 0, kWave) && lane < 8)
                __hip_atomic_store(rt + (9 + lane) * kSlot, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else if (w < es) {  // SwiGLU + e4m3 of one 128-column block of a row tile
            const long m = (w - e1) / nfb;
            const int fb = (int)((w - e1) % nfb);
            int lo = 0, hi = G - 1;  // group of row tile m
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (lts1[mid] <= m * a.ntn1) lo = mid; else hi = mid - 1;
            }
            const int mt = (int)(m - lts1[lo] / a.ntn1);
            const int row0 = loffs[lo] + 32 * mt, nrows = min(32, loffs[lo + 1] - loffs[lo] - 32 * mt);
            int32_t *rt = row_tile(m);
            spin_until<2>(rt + (9 + (int)(w % 8)) * kSlot, 1, a.err);
            for (int r = 0; r < nrows; ++r)
                decode_swiglu_wave<true>(a.upart, a.rows, a.F, a.ks, (uint8_t *)a.h, a.hs, (long)(row0 + r) * nfb + fb);
            wait_vmcnt<0>();
            compiler_fence();
            int done = 0;
            if (lane == 0) done = atomic_add(rt + 17 * kSlot, 1) == nfb - 1;
            if (__shfl(done, 0, kWave) && lane < 8)
                __hip_atomic_store(rt + (18 + lane) * kSlot, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else if (w < e2) {  // linear2 tile
            const int tile = (int)(w - es);
            const TileInfo ti = decode_tile(tile, lts2, loffs, G, 32);
            spin_until<4>(row_tile(lts2[ti.g] / a.ntn2 + ti.mt) + (18 + (int)(w % 8)) * kSlot, 1, a.err);
            fp8_decode_tile_call<false>(d2, tile, G);
            wait_vmcnt<0>();
            compiler_fence();
            if (lane == 0) atomic_add(counter_sub(a.sync, CNT_LIN2, w), 1);
        } else {  // combine: 64 lanes x 8 columns
            if (!lin2_all) {
                counter_wait<4>(a.sync, CNT_LIN2, (int)N2, a.err);
                lin2_all = true;
            }
            // y_perm lines are written by two linear2 tiles each, all finished before this read
            combine_lane<false, false>(a.yperm, a.s2r, a.gate, a.y, a.T, a.k, a.d, a.S, (w - e2) * kWave + lane);
        }
    }
    fused_exit(a, lds);
}

template <int MODE, int BM, int BN2>
__global__ __launch_bounds__(256) void fused_layer_kernel(FusedArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    fused_tiled<MODE, BM, BN2>(a, lds);
}

// 512 threads, 8-wave 256 x 256 GEMM tiles (bf16 or FP8 x FP4)
template <int MODE>
__global__ __launch_bounds__(512) void fused_layer_kernel8(FusedArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    fused_tiled<MODE, 256, 256, true>(a, lds);
}

// The decode variant streams weights: two waves per SIMD, its weight-streaming tiles (two
// blocks in flight per wave) and the steps before them called out of line, each with its
// own register allocation.
template <int UNUSED = 0>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void fused_decode_kernel(FusedArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    fused_decode(a, lds);
}

// Workgroups per CU of a kernel at (threads, lds) on device dev, and the device's CU
// count: queried once per (kernel, device, threads, LDS bytes) and kept, together with
// the kernel's LDS attribute, so a launch makes no runtime query.
hipError_t fused_occupancy(const void *fn, int dev, int threads, size_t lds, int &cus, int &per_cu);

// Host side: a cooperative launch of as many workgroups as fit on the device at once
// (at most cu_limit CUs' worth when cu_limit > 0).
inline hipError_t launch_fused_fn(const void *fn, FusedArgs &a, size_t lds, int cu_limit, hipStream_t st,
                                  int threads = 256) {
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = fused_occupancy(fn, dev, threads, lds, cus, per_cu);
    if (e != hipSuccess) return e;
    if (per_cu < 1) return hipErrorInvalidConfiguration;
    if (cu_limit > 0 && cu_limit < cus) cus = cu_limit;
    int P = cus * per_cu;
    if (P >= 8) P -= P % 8;  // item i then runs on XCD i % 8
    void *args[] = {&a};
    prof_begin(st);
    e = hipLaunchCooperativeKernel(fn, dim3(P), dim3(threads), args, (unsigned)lds, st);
    prof_end("layer_fused", st);
    return e;
}

template <int MODE, int BM, int BN2>
hipError_t launch_fused_kernel(FusedArgs &a, size_t lds, int cu_limit, hipStream_t st) {
    return launch_fused_fn((const void *)fused_layer_kernel<MODE, BM, BN2>, a, lds, cu_limit, st);
}

template <int MODE>
hipError_t launch_fused_kernel8(FusedArgs &a, size_t lds, int cu_limit, hipStream_t st) {
    return launch_fused_fn((const void *)fused_layer_kernel8<MODE>, a, lds, cu_limit, st, 512);
}

}  // namespace moe
