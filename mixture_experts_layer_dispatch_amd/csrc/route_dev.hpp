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


__device__ __forceinline__ float sigmoidf_(float l) { return 1.0f / (1.0f + expf(-l)); }

// Order-preserving 64-bit key: the float key's bits mapped so that unsigned order is float
// order (-0 taken as +0, so the two compare equal), then the complemented expert index, so
// that the larger of two packed keys is the larger key and, on equal keys, the lower expert
// index.  0 lies below every real key.
__device__ __forceinline__ uint64_t pack_key(float key, int e) {
    uint32_t u = __float_as_uint(key == 0.0f ? 0.0f : key);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)u << 32) | (uint32_t)~(uint32_t)e;
}

// v moved across lanes by one DPP control (lanes the control leaves out, or whose source
// is out of range, keep their own value)
template <int CTRL, int ROWMASK = 0xF>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
    const int lo = (int)(uint32_t)v, hi = (int)(uint32_t)(v >> 32);
    const uint32_t l2 = (uint32_t)__builtin_amdgcn_update_dpp(lo, lo, CTRL, ROWMASK, 0xF, false);
    const uint32_t h2 = (uint32_t)__builtin_amdgcn_update_dpp(hi, hi, CTRL, ROWMASK, 0xF, false);
    return ((uint64_t)h2 << 32) | l2;
}
__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Wave-wide maximum, in every lane: within quads (quad_perm swaps), half rows
// (row_half_mirror) and rows (row_mirror), then row 0 -> 1 and 2 -> 3 (row_bcast:15 into
// rows 1 and 3), rows 0-1 -> 2-3 (row_bcast:31 into rows 2 and 3); lane 63 then holds the
// maximum, read out as a uniform value.  The maximum is exact, so the order is free.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    v = max_u64(v, dpp_u64<0xB1>(v));        // quad_perm [1, 0, 3, 2]
    v = max_u64(v, dpp_u64<0x4E>(v));        // quad_perm [2, 3, 0, 1]
    v = max_u64(v, dpp_u64<0x141>(v));       // row_half_mirror
    v = max_u64(v, dpp_u64<0x140>(v));       // row_mirror
    v = max_u64(v, dpp_u64<0x142, 0xA>(v));  // row_bcast:15
    v = max_u64(v, dpp_u64<0x143, 0xC>(v));  // row_bcast:31
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
    return ((uint64_t)hi << 32) | lo;
}

// One wave selects the top-k of token t whose E logits sit in LDS (lg[0..E)); expert e
// lives in lane e % 64, slot e / 64 (NPER slots per lane).  Each of the k rounds takes the
// wave-wide maximum of the packed keys -- a stable descending order with ties to the lower
// expert index -- and lane j keeps the j-th choice, then works out its gate.
template <int NPER, bool COH>
__device__ __forceinline__ void select_token_n(const float *lg, int E, int k, int gating, const float *bias, long t,
                                               int32_t *idx, float *gate, float *logits, float *keys,
                                               int32_t *err) {
    const int lane = lane_id();
    uint64_t pk[NPER];
    bool bad = false;
#pragma unroll
    for (int i = 0; i < NPER; ++i) {
        const int e = lane + kWave * i;
        pk[i] = 0;
        if (e < E) {
            const float l = lg[e];
            const float s = gating == GATE_SIGMOID ? sigmoidf_(l) : l;
            const float kk = s + (bias ? bias[e] : 0.0f);
            bad |= !isfinite(kk);
            if (logits) logits[t * E + e] = l;
            if (keys) keys[t * E + e] = kk;
            pk[i] = pack_key(kk, e);
        }
    }
    if (__any(bad) && lane == 0) set_error(err, DEVERR_NONFINITE);

    int mine = 0;  // lane j < k: the j-th choice
    for (int j = 0; j < k; ++j) {
        uint64_t best = pk[0];
#pragma unroll
        for (int i = 1; i < NPER; ++i) best = pk[i] > best ? pk[i] : best;
        best = wave_max_u64(best);
        // only non-finite keys leave nothing above 0 (an error already reported): expert 0
        const int e = best ? (int)~(uint32_t)best : 0;
#pragma unroll
        for (int i = 0; i < NPER; ++i)
            if (lane + kWave * i == e) pk[i] = 0;
        mine = lane == j ? e : mine;
    }

    // gates from the unbiased scores of the chosen experts (lanes 0 .. k-1)
    const bool chosen = lane < k;
    const float l = lg[chosen ? mine : 0];
    float v;
    if (gating == GATE_SIGMOID) {
        v = chosen ? sigmoidf_(l) : 0.0f;
    } else {
        float m = chosen ? l : -INFINITY;
#pragma unroll
        for (int s = 32; s >= 1; s >>= 1) m = fmaxf(m, __shfl_xor(m, s, kWave));
        v = chosen ? expf(l - m) : 0.0f;
    }
    float sum = v;
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) sum += __shfl_xor(sum, s, kWave);
    if (chosen) {
        stc<COH>(idx + t * k + lane, mine);
        stc<COH>(gate + t * k + lane, v / sum);
    }
}

template <bool COH>
__device__ __forceinline__ void select_token(const float *lg, int E, int k, int gating, const float *bias, long t,
                                             int32_t *idx, float *gate, float *logits, float *keys, int32_t *err) {
    if (E <= 64) select_token_n<1, COH>(lg, E, k, gating, bias, t, idx, gate, logits, keys, err);
    else if (E <= 128) select_token_n<2, COH>(lg, E, k, gating, bias, t, idx, gate, logits, keys, err);
    else if (E <= 256) select_token_n<4, COH>(lg, E, k, gating, bias, t, idx, gate, logits, keys, err);
    else if (E <= 512) select_token_n<8, COH>(lg, E, k, gating, bias, t, idx, gate, logits, keys, err);
    else select_token_n<16, COH>(lg, E, k, gating, bias, t, idx, gate, logits, keys, err);
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
            // unconditional loads (rows past E re-read row E-1 into accumulators that are
            // dropped), so that all CH loads of a step are in flight together
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                const int e = e0 + c < E ? e0 + c : E - 1;
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
    const bool act = wave < 4 && t < T;  // waves past 4 (a larger workgroup) only meet the barrier
    float *lg = lds + (wave & 3) * E;
    if (act) route_valu_token<F32, CH>(x, wr, d, E, t, lg);
    __syncthreads();
    if (act) select_token<COH>(lg, E, k, gating, bias, t, idx, gate, logits, keys, err);
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
    for (int p = 0; p < (wave < 4 ? ntile : 0); p += 8) {  // waves past 4 only meet the barrier
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
    for (int tr = wave; tr < (wave < 4 ? kRouteTok : 0); tr += 4) {
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
    // the next 64-wide step's loads are issued before this step's MFMAs
    u32x4 av[2][4], bv[2][4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        av[0][u] = *(const u32x4 *)(xa + 16 * u);
        bv[0][u] = *(const u32x4 *)(wb + 16 * u);
    }
    for (int kk = 0; kk < kchunk; kk += 128) {
        const int k1 = kk + 64 < kchunk ? kk + 64 : kk;  // an odd last step re-reads (unused)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            av[1][u] = *(const u32x4 *)(xa + k1 + 16 * u);
            bv[1][u] = *(const u32x4 *)(wb + k1 + 16 * u);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[0][u]),
                                                          __builtin_bit_cast(bf16x8, bv[0][u]), acc, 0, 0, 0);
        if (kk + 64 >= kchunk) break;
        const int k2 = kk + 128 < kchunk ? kk + 128 : kk;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            av[0][u] = *(const u32x4 *)(xa + k2 + 16 * u);
            bv[0][u] = *(const u32x4 *)(wb + k2 + 16 * u);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[1][u]),
                                                          __builtin_bit_cast(bf16x8, bv[1][u]), acc, 0, 0, 0);
    }
    // acc[r] = logit partial of token 8(r/4) + 4(lane/32) + r%4 of the tile, expert lane%32
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        long t = tt * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (t < T) stc<COH>(part + ((long)ks * T + t) * E + et * 32 + (lane & 31), acc[r]);
    }
}

// Thread e's sum of expert e's K slices, in slice order, CH loads in flight at a time
// (unconditional, clamped loads: a load under a branch would be waited for before the
// branch joins, serialising the slices).
template <bool COH, int CH>
__device__ __forceinline__ float sum_slices(const float *__restrict__ part, int nks, int T, int E, long t, int e) {
    float s = 0.0f;
    for (int q0 = 0; q0 < nks; q0 += CH) {
        float v[CH];
#pragma unroll
        for (int q = 0; q < CH; ++q) v[q] = ldc<COH>(part + ((long)min(q0 + q, nks - 1) * T + t) * E + e);
#pragma unroll
        for (int q = 0; q < CH; ++q)
            if (q0 + q < nks) s += v[q];
    }
    return s;
}

// One wave, token t (E <= 256, at most QS K slices): lane l adds the slices of experts l,
// l + 64, l + 128, l + 192 in slice order into lg, every load (clamped) in flight together.
template <bool COH, int QS>
__device__ __forceinline__ void wave_sum_slices(const float *__restrict__ part, int nks, int T, int E, long t,
                                                float *lg) {
    const int lane = lane_id();
    float v[4][QS];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = lane + kWave * i < E ? lane + kWave * i : E - 1;
#pragma unroll
        for (int q = 0; q < QS; ++q) v[i][q] = ldc<COH>(part + ((long)(q < nks ? q : nks - 1) * T + t) * E + e);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float sum = 0.0f;
#pragma unroll
        for (int q = 0; q < QS; ++q)
            if (q < nks) sum += v[i][q];
        if (lane + kWave * i < E) lg[lane + kWave * i] = sum;
    }
}

// One wave, token t: lane l adds the K slices of experts l, l + 64, ... into lg (this
// wave's E floats of LDS), then selects (E <= 256, at most 16 slices); used when the slices are few, so that all four
// waves of a workgroup select (four tokens at a time).  Same sums, same order, same bits
// as route_sum_select.
template <bool COH>
__device__ __forceinline__ void route_sum_select_wave(const float *__restrict__ part, int nks, int T, int E, int k,
                                                      int gating, const float *__restrict__ bias, long t, float *lg,
                                                      int32_t *idx, float *gate, float *logits, float *keys,
                                                      int32_t *err) {
    if (nks <= 4) wave_sum_slices<COH, 4>(part, nks, T, E, t, lg);
    else wave_sum_slices<COH, 16>(part, nks, T, E, t, lg);
    __builtin_amdgcn_wave_barrier();  // the wave reads back its own LDS stores
    select_token<COH>(lg, E, k, gating, bias, t, idx, gate, logits, keys, err);
}

// 256 threads, token t: thread e adds expert e's K slices (all of them in one round trip
// when there are more than 16) and copies the expert's bias beside them (its load in flight
// with the slices', not after them), then wave 0 selects.  lg: 2 E floats of LDS.
template <bool COH>
__device__ __forceinline__ void route_sum_select(const float *__restrict__ part, int nks, int T, int E, int k,
                                                 int gating, const float *__restrict__ bias, long t, float *lg,
                                                 int32_t *idx, float *gate, float *logits, float *keys,
                                                 int32_t *err) {
    float *lb = lg + E;
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        const float b = bias ? bias[e] : 0.0f;
        lg[e] = nks > 16 ? sum_slices<COH, 64>(part, nks, T, E, t, e) : sum_slices<COH, 16>(part, nks, T, E, t, e);
        lb[e] = b;
    }
    __syncthreads();
    if (threadIdx.x < kWave) select_token<COH>(lg, E, k, gating, bias ? lb : nullptr, t, idx, gate, logits, keys, err);
}

}  // namespace moe
