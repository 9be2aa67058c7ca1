// Dispatch work items (S5-S7): group the T*k (token, choice) slots by expert, and the
// FP8 activation stage.
//
// Mega MoE wiki (aiki.softdaddy-o.com, "How it works") and Mega MoE blog
// (donniechu.com, "What's new"): dispatch sends each token to its chosen experts
// before the expert MLPs.  On one GPU this is a permutation into expert-contiguous
// rows.  Rows of one expert keep ascending token order, so the permutation is
// unique and the result deterministic: a per-block histogram, one scan over
// (expert, block), then a scatter whose in-block rank comes from 64-bit lane masks
// (population counts), never from the order of atomics.
//
// Workgroup-level items do the work of 256 threads; in a larger workgroup the threads past
// 256 only take part in the barriers.
#pragma once

#include "common.hpp"

namespace moe {

constexpr int kDispTok = 256;  // tokens per dispatch block (4 waves x 64)
constexpr int kMaxChoices = 16;

// Token t's k choices, loaded together (clamped, unconditional loads: a load under a
// branch would be waited for before the branch joins), with a bit per usable choice:
// in range and not a repeat of an earlier choice of the same token.
template <bool COH>
__device__ __forceinline__ uint32_t load_choices(const int32_t *__restrict__ idx, long t, int k, int E,
                                                 int ids[kMaxChoices], bool &bad_index, bool &dup) {
#pragma unroll
    for (int j = 0; j < kMaxChoices; ++j) ids[j] = ldc<COH>(idx + t * k + (j < k ? j : k - 1));
    uint32_t ok = 0;
    bad_index = dup = false;
#pragma unroll
    for (int j = 0; j < kMaxChoices; ++j) {
        if (j < k) {
            const int e = ids[j];
            bool d = false;
#pragma unroll
            for (int jj = 0; jj < j; ++jj) d |= ids[jj] == e;
            const bool inr = e >= 0 && e < E;
            bad_index |= !inr;
            dup |= inr && d;
            if (inr && !d) ok |= 1u << j;
        }
    }
    return ok;
}

// Builds masks[w][e] for dispatch block blk: bit `lane` set when token
// (blk*256 + w*64 + lane) chose e.  Invalid choices are reported (when err) and skipped.
template <bool COH>
__device__ __forceinline__ void build_masks(const int32_t *__restrict__ idx, int T, int k, int E, int blk,
                                            unsigned long long *masks, int32_t *err) {
    const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
    for (int i = tid; i < 4 * E; i += blockDim.x) masks[i] = 0ull;
    __syncthreads();
    const long t = (long)blk * kDispTok + tid;
    if (tid < kDispTok && t < T) {
        int ids[kMaxChoices];
        bool bad, dup;
        const uint32_t ok = load_choices<COH>(idx, t, k, E, ids, bad, dup);
        if (bad) set_error(err, DEVERR_INDEX);
        if (dup) set_error(err, DEVERR_DUP);
#pragma unroll
        for (int j = 0; j < kMaxChoices; ++j)
            if (ok >> j & 1u) atomicOr(&masks[wave * E + ids[j]], 1ull << lane);
    }
    __syncthreads();
}

// Per-expert histogram of block blk: blockcounts[blk][e].  masks: 4*E words of LDS.
template <bool COH>
__device__ __forceinline__ void count_block(const int32_t *__restrict__ idx, int T, int k, int E, int blk,
                                            unsigned long long *masks, int32_t *__restrict__ blockcounts,
                                            int32_t *err) {
    build_masks<COH>(idx, T, k, E, blk, masks, err);
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        int c = __popcll(masks[e]) + __popcll(masks[E + e]) + __popcll(masks[2 * E + e]) + __popcll(masks[3 * E + e]);
        stc<COH>(blockcounts + (long)blk * E + e, c);
    }
}

// In-place exclusive scan of v[0..n) in LDS by 256 threads (n <= 256 * 8); returns the
// total.  tmp: 256 ints of LDS.
__device__ __forceinline__ int block_exclusive_scan(int32_t *v, int n, int32_t *tmp) {
    const int tid = threadIdx.x;
    const bool act = tid < 256;  // threads past 256 only meet the barriers
    const int C = (n + 255) / 256, b0 = tid * C;
    int loc = 0;
    if (act) {
        for (int i = 0; i < C; ++i)
            if (b0 + i < n) loc += v[b0 + i];
        tmp[tid] = loc;
    }
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
        int a = act && tid >= off ? tmp[tid - off] : 0;
        __syncthreads();
        if (act) tmp[tid] += a;
        __syncthreads();
    }
    const int total = tmp[255];
    if (act) {
        int run = tmp[tid] - loc;
        for (int i = 0; i < C; ++i)
            if (b0 + i < n) {
                int c = v[b0 + i];
                v[b0 + i] = run;
                run += c;
            }
    }
    __syncthreads();
    return total;
}

// One workgroup: per-expert totals, the exclusive scan over experts (counts, offsets),
// and each block's base row per expert, written over the block counts.  sh: 1024 + 256
// ints of LDS.  Column loads go 16 blocks at a time, all in flight together.
template <bool COH>
__device__ __forceinline__ void dispatch_scan_block(int32_t *__restrict__ blockcounts, int nblk, int T, int E,
                                                    int S, int32_t *__restrict__ counts,
                                                    int32_t *__restrict__ offsets, int32_t *sh) {
    constexpr int CH = 16;
    int32_t *tot = sh, *tmp = sh + 1024;
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        int s = 0;
        for (int b0 = 0; b0 < nblk; b0 += CH) {
            int c[CH];
#pragma unroll
            for (int u = 0; u < CH; ++u) c[u] = ldc<COH>(blockcounts + (long)min(b0 + u, nblk - 1) * E + e);
#pragma unroll
            for (int u = 0; u < CH; ++u)
                if (b0 + u < nblk) s += c[u];
        }
        tot[e] = s;
        stc<COH>(counts + e, s);
    }
    __syncthreads();
    const int routed = block_exclusive_scan(tot, E, tmp);  // tot[e] = offsets[e] now
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        int s = tot[e];
        stc<COH>(offsets + e, s);
        for (int b0 = 0; b0 < nblk; b0 += CH) {
            int c[CH];
#pragma unroll
            for (int u = 0; u < CH; ++u) c[u] = ldc<COH>(blockcounts + (long)min(b0 + u, nblk - 1) * E + e);
#pragma unroll
            for (int u = 0; u < CH; ++u)
                if (b0 + u < nblk) {
                    stc<COH>(blockcounts + (long)(b0 + u) * E + e, s);
                    s += c[u];
                }
        }
    }
    if (threadIdx.x == 0) {
        stc<COH>(offsets + E, routed);
        if (S) {
            stc<COH>(counts + E, T);
            stc<COH>(offsets + E + 1, routed + T);
        }
    }
    __syncthreads();
}

// One workgroup: tile_start prefixes of both GEMMs over the G groups (ragged row tiles
// times N tiles per group).  sh: 2 * 1032 + 256 ints of LDS.
template <bool COH>
__device__ __forceinline__ void tile_plan_block(const int32_t *__restrict__ offsets, int G, int bm1, int ntn1,
                                                int bm2, int ntn2, int32_t *__restrict__ ts1,
                                                int32_t *__restrict__ ts2, int32_t *sh) {
    int32_t *v1 = sh, *v2 = sh + 1032, *tmp = sh + 2064;
    for (int g = threadIdx.x; g < G; g += blockDim.x) {
        const int c = ldc<COH>(offsets + g + 1) - ldc<COH>(offsets + g);
        v1[g] = (c + bm1 - 1) / bm1 * ntn1;
        v2[g] = (c + bm2 - 1) / bm2 * ntn2;
    }
    __syncthreads();
    const int n1 = block_exclusive_scan(v1, G, tmp);
    const int n2 = block_exclusive_scan(v2, G, tmp);
    for (int g = threadIdx.x; g < G; g += blockDim.x) {
        stc<COH>(ts1 + g, v1[g]);
        stc<COH>(ts2 + g, v2[g]);
    }
    if (threadIdx.x == 0) {
        stc<COH>(ts1 + G, n1);
        stc<COH>(ts2 + G, n2);
    }
    __syncthreads();
}

// Rows of block blk: slot_to_row and row_to_slot from the block bases.
template <bool COH>
__device__ __forceinline__ void scatter_block(const int32_t *__restrict__ idx, int T, int k, int E, int blk,
                                              const int32_t *__restrict__ bases, int32_t *__restrict__ slot_to_row,
                                              int32_t *__restrict__ row_to_slot, unsigned long long *masks) {
    build_masks<COH>(idx, T, k, E, blk, masks, nullptr);  // errors were reported by the count pass
    const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
    const long t = (long)blk * kDispTok + tid;
    if (tid >= kDispTok || t >= T) return;
    const unsigned long long below = (1ull << lane) - 1ull;
    int ids[kMaxChoices];
    bool bad, dup;
    const uint32_t ok = load_choices<COH>(idx, t, k, E, ids, bad, dup);
#pragma unroll
    for (int j = 0; j < kMaxChoices; ++j) {
        if (!(ok >> j & 1u)) continue;
        const int e = ids[j];
        int rank = __popcll(masks[wave * E + e] & below);
        for (int w = 0; w < wave; ++w) rank += __popcll(masks[w * E + e]);
        int row = ldc<COH>(bases + (long)blk * E + e) + rank;
        stc<COH>(slot_to_row + t * k + j, row);
        stc<COH>(row_to_slot + row, (int32_t)(t * k + j));
    }
}

// One dispatch block (T <= 256) by one workgroup: histogram, scan and scatter with the
// per-expert counts and bases kept in LDS, so the choices are loaded once (kept in
// registers) and counts, offsets and both permutations are stored once -- no global
// round trip between the steps.  Same results as count_block + dispatch_scan_block +
// scatter_block on one block.  lds: 4 E words of masks, then E + 256 ints.
template <bool COH>
__device__ __forceinline__ void dispatch_single_block(const int32_t *__restrict__ idx, int T, int k, int E, int S,
                                                      int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
                                                      int32_t *__restrict__ slot_to_row,
                                                      int32_t *__restrict__ row_to_slot, int32_t *err,
                                                      uint8_t *lds) {
    unsigned long long *masks = (unsigned long long *)lds;
    int32_t *base = (int32_t *)(masks + 4 * E), *tmp = base + E;
    const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
    const bool live = tid < T && tid < kDispTok;
    int ids[kMaxChoices];
    uint32_t ok = 0;
    if (live) {
        bool bad, dup;
        ok = load_choices<COH>(idx, tid, k, E, ids, bad, dup);
        if (bad) set_error(err, DEVERR_INDEX);
        if (dup) set_error(err, DEVERR_DUP);
    }
    for (int i = tid; i < 4 * E; i += blockDim.x) masks[i] = 0ull;
    __syncthreads();
    if (live) {
#pragma unroll
        for (int j = 0; j < kMaxChoices; ++j)
            if (ok >> j & 1u) atomicOr(&masks[wave * E + ids[j]], 1ull << lane);
    }
    __syncthreads();
    for (int e = tid; e < E; e += blockDim.x) {
        const int c = __popcll(masks[e]) + __popcll(masks[E + e]) + __popcll(masks[2 * E + e]) +
                      __popcll(masks[3 * E + e]);
        base[e] = c;
        stc<COH>(counts + e, c);
    }
    __syncthreads();
    const int routed = block_exclusive_scan(base, E, tmp);  // base[e] = offsets[e] now
    for (int e = tid; e < E; e += blockDim.x) stc<COH>(offsets + e, base[e]);
    if (tid == 0) {
        stc<COH>(offsets + E, routed);
        if (S) {
            stc<COH>(counts + E, T);
            stc<COH>(offsets + E + 1, routed + T);
        }
    }
    if (!live) return;
    const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
    for (int j = 0; j < kMaxChoices; ++j) {
        if (!(ok >> j & 1u)) continue;
        const int e = ids[j];
        int rank = __popcll(masks[wave * E + e] & below);
        for (int w = 0; w < wave; ++w) rank += __popcll(masks[w * E + e]);
        const int row = base[e] + rank;
        stc<COH>(slot_to_row + (long)tid * k + j, row);
        stc<COH>(row_to_slot + row, (int32_t)((long)tid * k + j));
    }
}

// ---- the capacity variant (expert capacity with token dropping) -------------------------
//
// MoE lesson (factory.pai-world.com, "The load-balancing problem", item 2): each routed
// expert takes at most `cap` of the slots that chose it, the first ones in slot order (the
// dropless dispatch's ascending token order); the rest skip the layer.  Layout: rows
// 0 .. D-1 hold the D dropped slots, expert by expert in slot order (dbase[e] = the first
// of expert e's); expert e's kept rows start at offsets[e] = D + (kept rows of the experts
// before it), so offsets[E] = T*k and the shared expert keeps rows T*k + t.  A kept slot's
// slot_to_row is its row, a dropped one's -1; row_to_slot covers every row.

// One workgroup: per-expert totals n_e, kept min(n_e, cap) and dropped counts, both scans,
// and each block's first rank among its expert's slots (written over the block counts).
// sh: 2048 + 256 ints of LDS.
__device__ __forceinline__ void dispatch_scan_cap_block(int32_t *__restrict__ blockcounts, int nblk, int T, int E,
                                                        int S, int cap, int32_t *__restrict__ counts,
                                                        int32_t *__restrict__ dropped,
                                                        int32_t *__restrict__ offsets, int32_t *__restrict__ dbase,
                                                        int32_t *sh) {
    int32_t *kept = sh, *drop = sh + 1024, *tmp = sh + 2048;
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        int n = 0;
        for (int b = 0; b < nblk; ++b) {
            const int c = blockcounts[(long)b * E + e];
            blockcounts[(long)b * E + e] = n;  // the block's first rank within expert e
            n += c;
        }
        const int kp = n < cap ? n : cap;
        kept[e] = kp;
        drop[e] = n - kp;
        counts[e] = kp;
        dropped[e] = n - kp;
    }
    __syncthreads();
    const int nk = block_exclusive_scan(kept, E, tmp);  // kept[e] = kept rows before expert e
    const int D = block_exclusive_scan(drop, E, tmp);   // drop[e] = dropped rows before expert e
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        offsets[e] = D + kept[e];
        dbase[e] = drop[e];
    }
    if (threadIdx.x == 0) {
        offsets[E] = D + nk;
        if (S) {
            counts[E] = T;
            offsets[E + 1] = D + nk + T;
        }
    }
}

// Rows of dispatch block blk under the capacity: a slot's rank among its expert's slots is
// the block's first rank plus the lanes below it (lane masks, as scatter_block).
__device__ __forceinline__ void scatter_cap_block(const int32_t *__restrict__ idx, int T, int k, int E, int blk, int cap,
                                                  const int32_t *__restrict__ ranks,
                                                  const int32_t *__restrict__ offsets,
                                                  const int32_t *__restrict__ dbase,
                                                  int32_t *__restrict__ slot_to_row,
                                                  int32_t *__restrict__ row_to_slot, unsigned long long *masks) {
    build_masks<false>(idx, T, k, E, blk, masks, nullptr);  // errors were reported by the count pass
    const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
    const long t = (long)blk * kDispTok + tid;
    if (tid >= kDispTok || t >= T) return;
    const unsigned long long below = (1ull << lane) - 1ull;
    int ids[kMaxChoices];
    bool bad, dup;
    const uint32_t ok = load_choices<false>(idx, t, k, E, ids, bad, dup);
#pragma unroll
    for (int j = 0; j < kMaxChoices; ++j) {
        if (!(ok >> j & 1u)) continue;
        const int e = ids[j];
        int rank = __popcll(masks[wave * E + e] & below);
        for (int w = 0; w < wave; ++w) rank += __popcll(masks[w * E + e]);
        rank += ranks[(long)blk * E + e];
        const bool keep = rank < cap;
        const int row = keep ? offsets[e] + rank : dbase[e] + (rank - cap);
        slot_to_row[t * k + j] = keep ? row : -1;
        row_to_slot[row] = (int32_t)(t * k + j);
    }
}

// ---- FP8 activation stage: x (bf16) -> e4m3 codes + power-of-two scale per 1x128 ----
//
// 16 lanes own one 128-value block (8 values each, one 16-byte load); gid is the global
// lane index, block gid / 16.
template <bool COH>
__device__ __forceinline__ void quant_x_lane(const uint16_t *__restrict__ x, long nblocks, uint8_t *__restrict__ xq,
                                             float *__restrict__ xs, long gid) {
    const long blk = gid >> 4;
    const int sub = (int)(gid & 15);
    const bool live = blk < nblocks;
    uint4 q = live ? *(const uint4 *)(x + blk * 128 + sub * 8) : make_uint4(0, 0, 0, 0);
    const uint16_t *h = (const uint16_t *)&q;
    float v[8];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        v[i] = bf16_to_f32(h[i]);
        amax = fmaxf(amax, fabsf(v[i]));
    }
    amax = row16_max(amax);
    if (!live) return;
    const int e = e4m3_block_exponent(amax);
    const float inv = ldexpf(1.0f, -e);
    uint2 out;
    out.x = cvt_e4m3x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
    out.y = cvt_e4m3x4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
    stc<COH>((uint64_t *)(xq + blk * 128 + sub * 8), (uint64_t)out.x | ((uint64_t)out.y << 32));
    if (sub == 0) stc<COH>(xs + blk, ldexpf(1.0f, e));
}

// NB lane tasks gid0 + u * stride (u < NB, stride a multiple of 16) of quant_x_lane, every
// load issued before the first conversion: a few workgroups looping over many blocks keep NB
// loads in flight per lane instead of one.  COH: device-coherent stores, as quant_x_lane.
template <int NB, bool COH>
__device__ __forceinline__ void quant_x_batch(const uint16_t *__restrict__ x, long nblocks, uint8_t *__restrict__ xq,
                                              float *__restrict__ xs, long gid0, long stride) {
    uint4 q[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
        const long blk = (gid0 + u * stride) >> 4;
        const int sub = (int)((gid0 + u * stride) & 15);
        q[u] = blk < nblocks ? *(const uint4 *)(x + blk * 128 + sub * 8) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < NB; ++u) {
        const long blk = (gid0 + u * stride) >> 4;
        const int sub = (int)((gid0 + u * stride) & 15);
        const uint16_t *h = (const uint16_t *)&q[u];
        float v[8];
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            v[i] = bf16_to_f32(h[i]);
            amax = fmaxf(amax, fabsf(v[i]));
        }
        amax = row16_max(amax);
        if (blk < nblocks) {
            const int e = e4m3_block_exponent(amax);
            const float inv = ldexpf(1.0f, -e);
            uint2 out;
            out.x = cvt_e4m3x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
            out.y = cvt_e4m3x4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
            stc<COH>((uint64_t *)(xq + blk * 128 + sub * 8), (uint64_t)out.x | ((uint64_t)out.y << 32));
            if (sub == 0) stc<COH>(xs + blk, ldexpf(1.0f, e));
        }
    }
}

// The same quantiser over fp32 values: 16 lanes per 128-value block, 8 values (two 16-byte
// loads) each.
__device__ __forceinline__ void quant_f32_lane(const float *__restrict__ v, long nblocks, uint8_t *__restrict__ q,
                                               float *__restrict__ qs, long gid) {
    const long blk = gid >> 4;
    const int sub = (int)(gid & 15);
    const bool live = blk < nblocks;
    float4 a = live ? *(const float4 *)(v + blk * 128 + sub * 8) : make_float4(0.f, 0.f, 0.f, 0.f);
    float4 b = live ? *(const float4 *)(v + blk * 128 + sub * 8 + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
    float amax = fmaxf(fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))),
                       fmaxf(fmaxf(fabsf(b.x), fabsf(b.y)), fmaxf(fabsf(b.z), fabsf(b.w))));
    amax = row16_max(amax);
    if (!live) return;
    const int e = e4m3_block_exponent(amax);
    const float inv = ldexpf(1.0f, -e);
    uint2 out;
    out.x = cvt_e4m3x4(a.x * inv, a.y * inv, a.z * inv, a.w * inv);
    out.y = cvt_e4m3x4(b.x * inv, b.y * inv, b.z * inv, b.w * inv);
    *(uint2 *)(q + blk * 128 + sub * 8) = out;
    if (sub == 0) qs[blk] = ldexpf(1.0f, e);
}

}  // namespace moe
