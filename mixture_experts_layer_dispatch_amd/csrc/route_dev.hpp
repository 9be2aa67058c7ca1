// Router work items (S1-S4): router GEMM, selection keys, top-k and gates.
//
// MoE lesson (factory.pai-world.com, "Mixture of Experts"): "FFN swap" gives the
// router as one linear layer producing an (N_tokens, E) score matrix and a top-k
// per token; "The load-balancing problem" and "Build it, Step 1: router" add the
// per-expert bias to the scores for selection only, order by descending biased
// score with a stable sort, and take the gates from the unbiased scores (softmax over
// the chosen ones).  MoE playbook (molayo1419.me, "How it works") gives the same
// score / select / weighted-sum steps.
//
// Each function is one work item with its index passed in, so the stand-alone
// kernels and the persistent layer kernel run the very same code.
#pragma once

#include "common.hpp"

namespace moe {

constexpr int kMaxKeysPerLane = 16;  // E <= 1024 over 64 lanes
constexpr int kMaxK = 16;

__device__ __forceinline__ float sigmoidf_(float l) { return 1.0f / (1.0f + expf(-l)); }

// One wave selects the top-k of token t whose E logits sit in LDS (lg[0..E)).
// Keys for expert e live in lane e % 64, slot e / 64.
template <bool COH>
__device__ __forceinline__ void select_token(const float *lg, int E, int k, int gating, const float *bias, long t,
                                             int32_t *idx, float *gate, float *logits, float *keys, int32_t *err) {
    const int lane = lane_id();
    const int nper = (E + kWave - 1) / kWave;
    float key[kMaxKeysPerLane];
    uint32_t taken = 0;  // bit i: slot i unavailable
    bool bad = false;
#pragma unroll
    for (int i = 0; i < kMaxKeysPerLane; ++i) {
        int e = lane + kWave * i;
        key[i] = -INFINITY;
        if (i < nper && e < E) {
            float l = lg[e];
            float s = gating == GATE_SIGMOID ? sigmoidf_(l) : l;
            float kk = s + (bias ? bias[e] : 0.0f);
            key[i] = kk;
            bad |= !isfinite(kk);
            if (logits) logits[t * E + e] = l;
            if (keys) keys[t * E + e] = kk;
        } else {
            taken |= 1u << i;
        }
    }
    if (__any(bad) && lane == 0) set_error(err, DEVERR_NONFINITE);

    int sel[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
        sel[j] = 0;
        if (j < k) {
            float bk = -INFINITY;
            int bi = 0x7fffffff;
#pragma unroll
            for (int i = 0; i < kMaxKeysPerLane; ++i) {
                int e = lane + kWave * i;
                bool ok = !(taken >> i & 1u);
                if (ok && (key[i] > bk || (key[i] == bk && e < bi))) { bk = key[i]; bi = e; }
            }
#pragma unroll
            for (int m = 32; m >= 1; m >>= 1) {
                float ok_ = __shfl_xor(bk, m, kWave);
                int oi = __shfl_xor(bi, m, kWave);
                if (ok_ > bk || (ok_ == bk && oi < bi)) { bk = ok_; bi = oi; }
            }
            if (bi == 0x7fffffff) bi = 0;  // only with non-finite keys (error already flagged)
            if ((bi & (kWave - 1)) == lane) taken |= 1u << (bi / kWave);
            sel[j] = bi;
        }
    }

    // gates from the unbiased scores of the chosen experts
    float v[kMaxK];
    float m = -INFINITY, sum = 0.0f;
    if (gating == GATE_SIGMOID) {
#pragma unroll
        for (int j = 0; j < kMaxK; ++j)
            if (j < k) { v[j] = sigmoidf_(lg[sel[j]]); sum += v[j]; }
    } else {
#pragma unroll
        for (int j = 0; j < kMaxK; ++j)
            if (j < k) m = fmaxf(m, lg[sel[j]]);
#pragma unroll
        for (int j = 0; j < kMaxK; ++j)
            if (j < k) { v[j] = expf(lg[sel[j]] - m); sum += v[j]; }
    }
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
        if (j < k && lane == j) {
            stc<COH>(idx + t * k + j, sel[j]);
            stc<COH>(gate + t * k + j, v[j] / sum);
        }
}

// ---- VALU router: one wave per token (small E, or fp32 activations) ----------
//
// Writes the E logits of token t into lg (LDS); lane 0 stores each dot product.
template <bool F32, int CH>
__device__ __forceinline__ void route_valu_token(const void *__restrict__ xv, const void *__restrict__ wv, int d,
                                                 int E, long t, float *lg) {
    const int lane = lane_id();
    constexpr int V = F32 ? 4 : 8;  // elements per 16-byte load
    for (int e0 = 0; e0 < E; e0 += CH) {
        float acc[CH];
#pragma unroll
        for (int c = 0; c < CH; ++c) acc[c] = 0.0f;
        for (int i0 = lane * V; i0 < d; i0 += kWave * V) {
            float xs[V];
            if (F32) {
                float4 q = *(const float4 *)((const float *)xv + t * d + i0);
                xs[0] = q.x; xs[1] = q.y; xs[2] = q.z; xs[3] = q.w;
            } else {
                uint4 q = *(const uint4 *)((const uint16_t *)xv + t * d + i0);
                const uint16_t *h = (const uint16_t *)&q;
#pragma unroll
                for (int u = 0; u < V; ++u) xs[u] = bf16_to_f32(h[u]);
            }
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                int e = e0 + c;
                if (e < E) {
                    float ws[V];
                    if (F32) {
                        float4 q = *(const float4 *)((const float *)wv + (long)e * d + i0);
                        ws[0] = q.x; ws[1] = q.y; ws[2] = q.z; ws[3] = q.w;
                    } else {
                        uint4 q = *(const uint4 *)((const uint16_t *)wv + (long)e * d + i0);
                        const uint16_t *h = (const uint16_t *)&q;
#pragma unroll
                        for (int u = 0; u < V; ++u) ws[u] = bf16_to_f32(h[u]);
                    }
#pragma unroll
                    for (int u = 0; u < V; ++u) acc[c] = fmaf(xs[u], ws[u], acc[c]);
                }
            }
        }
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            float s = wave_sum(acc[c]);
            if (lane == 0 && e0 + c < E) lg[e0 + c] = s;
        }
    }
}

// 256 threads: tokens 4 b .. 4 b + 3, one wave each; lds holds [4][E] floats.
template <bool F32, int CH, bool COH>
__device__ __forceinline__ void route_valu_block(const void *x, const void *wr, const float *bias, int T, int d,
                                                 int E, int k, int gating, int b, float *lds, int32_t *idx,
                                                 float *gate, float *logits, float *keys, int32_t *err) {
    const int wave = threadIdx.x / kWave;
    const long t = (long)b * 4 + wave;
    float *lg = lds + wave * E;
    if (t < T) route_valu_token<F32, CH>(x, wr, d, E, t, lg);
    __syncthreads();
    if (t < T) select_token<COH>(lg, E, k, gating, bias, t, idx, gate, logits, keys, err);
}

// ---- MFMA router (bf16, E a multiple of 32): 32 tokens per workgroup ----------
//
// v_mfma_f32_32x32x16_bf16: lane l holds A[row l%32][k 8*(l/32)..+8] and
// B[k 8*(l/32)..+8][col l%32]; result register r of lane l is
// C[row 8*(r/4) + 4*(l/32) + r%4][col l%32].  Rows are tokens, columns experts.
constexpr int kRouteTok = 32;

// 256 threads: tokens 32 b .. 32 b + 31; lds holds [32][E] floats.  Passes of 8 expert
// tiles: wave w owns tiles p + w and p + w + 4 of pass p (two accumulators).
template <bool COH>
__device__ __forceinline__ void route_mfma_block(const uint16_t *__restrict__ x, const uint16_t *__restrict__ wr,
                                                 const float *__restrict__ bias, int T, int d, int E, int k,
                                                 int gating, int b, float *lds, int32_t *idx, float *gate,
                                                 float *logits, float *keys, int32_t *err) {
    const int wave = threadIdx.x / kWave, lane = lane_id();
    const int ntile = E / 32;
    const long t0 = (long)b * kRouteTok;
    long trow = t0 + (lane & 31);
    if (trow >= T) trow = T - 1;
    const uint16_t *xa = x + trow * d + 8 * (lane >> 5);
    for (int p = 0; p < ntile; p += 8) {
        const int nt0 = p + wave, nt1 = p + wave + 4;
        const bool has0 = nt0 < ntile, has1 = nt1 < ntile;
        const uint16_t *wb0 = wr + (long)((has0 ? nt0 : 0) * 32 + (lane & 31)) * d + 8 * (lane >> 5);
        const uint16_t *wb1 = wr + (long)((has1 ? nt1 : 0) * 32 + (lane & 31)) * d + 8 * (lane >> 5);
        f32x16 acc0 = (f32x16){}, acc1 = (f32x16){};
        if (has0) {
            for (int k0 = 0; k0 < d; k0 += 64) {
                uint4 av[4], bv[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    av[u] = *(const uint4 *)(xa + k0 + 16 * u);
                    bv[u] = *(const uint4 *)(wb0 + k0 + 16 * u);
                }
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[u]),
                                                                   __builtin_bit_cast(bf16x8, bv[u]), acc0, 0, 0, 0);
                if (has1) {
#pragma unroll
                    for (int u = 0; u < 4; ++u) bv[u] = *(const uint4 *)(wb1 + k0 + 16 * u);
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[u]),
                                                                       __builtin_bit_cast(bf16x8, bv[u]), acc1, 0, 0,
                                                                       0);
                }
            }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = 8 * (r / 4) + 4 * (lane >> 5) + (r % 4);
            if (has0) lds[row * E + nt0 * 32 + (lane & 31)] = acc0[r];
            if (has1) lds[row * E + nt1 * 32 + (lane & 31)] = acc1[r];
        }
    }
    __syncthreads();
    for (int tr = wave; tr < kRouteTok; tr += 4) {
        long t = t0 + tr;
        if (t < T) select_token<COH>(lds + tr * E, E, k, gating, bias, t, idx, gate, logits, keys, err);
    }
}

// ---- split-K router for few tokens: one wave owns 32 tokens x 32 experts x a K slice ----
//
// With few tokens the router is a GEMV over W_r; spreading it over (expert tile, K slice,
// token tile) waves streams W_r once across the whole chip.  Partial logits land in
// part[ks][t][e] and route_sum_select adds them in ks order (fixed, so deterministic).
// Wave item w = (tt * nks + ks) * (E / 32) + et.
template <bool COH>
__device__ __forceinline__ void route_splitk_wave(const uint16_t *__restrict__ x, const uint16_t *__restrict__ wr,
                                                  int T, int d, int E, int nks, long w, float *__restrict__ part) {
    const int lane = lane_id();
    const int ntile = E / 32;
    const int et = (int)(w % ntile), ks = (int)((w / ntile) % nks);
    const long tt = w / ((long)ntile * nks);
    const int kchunk = d / nks;
    long trow = tt * 32 + (lane & 31);
    if (trow >= T) trow = T - 1;
    const int k0 = ks * kchunk;
    const uint16_t *xa = x + trow * d + k0 + 8 * (lane >> 5);
    const uint16_t *wb = wr + (long)(et * 32 + (lane & 31)) * d + k0 + 8 * (lane >> 5);
    f32x16 acc = (f32x16){};
    for (int kk = 0; kk < kchunk; kk += 64) {
        u32x4 av[4], bv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            av[u] = *(const u32x4 *)(xa + kk + 16 * u);
            bv[u] = *(const u32x4 *)(wb + kk + 16 * u);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[u]),
                                                          __builtin_bit_cast(bf16x8, bv[u]), acc, 0, 0, 0);
    }
    // acc[r] = logit partial of token 8(r/4) + 4(lane/32) + r%4 of the tile, expert lane%32
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        long t = tt * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (t < T) stc<COH>(part + ((long)ks * T + t) * E + et * 32 + (lane & 31), acc[r]);
    }
}

// 256 threads, token t: thread e adds expert e's K slices in slice order, 16 loads in
// flight at a time (unconditional, clamped loads: a load under a branch would be waited
// for before the branch joins, serialising the slices); then wave 0 selects.  lg: E
// floats of LDS.
template <bool COH>
__device__ __forceinline__ void route_sum_select(const float *__restrict__ part, int nks, int T, int E, int k,
                                                 int gating, const float *__restrict__ bias, long t, float *lg,
                                                 int32_t *idx, float *gate, float *logits, float *keys,
                                                 int32_t *err) {
    constexpr int CH = 16;
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        float s = 0.0f;
        for (int q0 = 0; q0 < nks; q0 += CH) {
            float v[CH];
#pragma unroll
            for (int q = 0; q < CH; ++q) v[q] = ldc<COH>(part + ((long)min(q0 + q, nks - 1) * T + t) * E + e);
#pragma unroll
            for (int q = 0; q < CH; ++q)
                if (q0 + q < nks) s += v[q];
        }
        lg[e] = s;
    }
    __syncthreads();
    if (threadIdx.x < kWave) select_token<COH>(lg, E, k, gating, bias, t, idx, gate, logits, keys, err);
}

}  // namespace moe
