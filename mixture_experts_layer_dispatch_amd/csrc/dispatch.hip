// Dispatch (S5-S6): group the T*k (token, choice) slots by expert, and the FP8
// activation stage (S7).
//
// Mega MoE wiki (aiki.softdaddy-o.com, "How it works") and Mega MoE blog
// (donniechu.com, "What's new"): dispatch sends each token to its chosen experts
// before the expert MLPs.  On one GPU this is a permutation into expert-contiguous
// rows.  Rows of one expert keep ascending token order, so the permutation is
// unique and the result deterministic: a per-block histogram, one scan over
// (expert, block), then a scatter whose in-block rank comes from 64-bit lane masks
// (population counts), never from the order of atomics.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kDispTok = 256;  // tokens per dispatch block (4 waves x 64)

int dispatch_blocks(int T) { return (T + kDispTok - 1) / kDispTok; }

// Builds masks[w][e]: bit `lane` set when token (block*256 + w*64 + lane) chose e.
// Validates indices; invalid ones are reported and skipped.
__device__ void build_masks(const int32_t *__restrict__ idx, int T, int k, int E, unsigned long long *masks,
                            int32_t *err) {
    const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
    for (int i = tid; i < 4 * E; i += blockDim.x) masks[i] = 0ull;
    __syncthreads();
    const long t = (long)blockIdx.x * kDispTok + tid;
    if (t < T) {
        for (int j = 0; j < k; ++j) {
            int e = idx[t * k + j];
            if (e < 0 || e >= E) { set_error(err, DEVERR_INDEX); continue; }
            bool dup = false;
            for (int jj = 0; jj < j; ++jj) dup |= idx[t * k + jj] == e;
            if (dup) { set_error(err, DEVERR_DUP); continue; }
            atomicOr(&masks[wave * E + e], 1ull << lane);
        }
    }
    __syncthreads();
}

__global__ __launch_bounds__(256) void dispatch_count_kernel(const int32_t *__restrict__ idx, int T, int k, int E,
                                                            int32_t *__restrict__ blockcounts, int32_t *err) {
    extern __shared__ unsigned long long masks[];  // [4][E]
    build_masks(idx, T, k, E, masks, err);
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        int c = __popcll(masks[e]) + __popcll(masks[E + e]) + __popcll(masks[2 * E + e]) + __popcll(masks[3 * E + e]);
        blockcounts[(long)blockIdx.x * E + e] = c;
    }
}

// One workgroup: per-expert totals, the exclusive scan over experts, and each
// block's base row per expert (written over the block counts).
__global__ __launch_bounds__(1024) void dispatch_scan_kernel(int32_t *__restrict__ blockcounts, int nblk, int T,
                                                            int k, int E, int S, int32_t *__restrict__ counts,
                                                            int32_t *__restrict__ offsets) {
    __shared__ int32_t tot[1024];
    __shared__ int32_t scan[1024];
    const int e = threadIdx.x;
    int s = 0;
    if (e < E) {
        for (int b = 0; b < nblk; ++b) {
            int c = blockcounts[(long)b * E + e];
            blockcounts[(long)b * E + e] = s;
            s += c;
        }
    }
    tot[e] = e < E ? s : 0;
    scan[e] = tot[e];
    __syncthreads();
    // inclusive Hillis-Steele scan over 1024 entries
    for (int off = 1; off < 1024; off <<= 1) {
        int v = e >= off ? scan[e - off] : 0;
        __syncthreads();
        scan[e] += v;
        __syncthreads();
    }
    const int excl = scan[e] - tot[e];
    if (e < E) {
        counts[e] = tot[e];
        offsets[e] = excl;
        for (int b = 0; b < nblk; ++b) blockcounts[(long)b * E + e] += excl;
    }
    if (e == 0) {
        int routed = scan[1023];
        offsets[E] = routed;
        if (S) {
            counts[E] = T;
            offsets[E + 1] = routed + T;
        }
    }
}

__global__ __launch_bounds__(256) void dispatch_scatter_kernel(const int32_t *__restrict__ idx, int T, int k, int E,
                                                              const int32_t *__restrict__ bases,
                                                              int32_t *__restrict__ slot_to_row,
                                                              int32_t *__restrict__ row_to_slot, int32_t *err) {
    extern __shared__ unsigned long long masks[];  // [4][E]
    build_masks(idx, T, k, E, masks, nullptr);  // errors were reported by the count pass
    const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
    const long t = (long)blockIdx.x * kDispTok + tid;
    if (t >= T) return;
    const unsigned long long below = (1ull << lane) - 1ull;
    for (int j = 0; j < k; ++j) {
        int e = idx[t * k + j];
        if (e < 0 || e >= E) continue;
        bool dup = false;
        for (int jj = 0; jj < j; ++jj) dup |= idx[t * k + jj] == e;
        if (dup) continue;
        int rank = __popcll(masks[wave * E + e] & below);
        for (int w = 0; w < wave; ++w) rank += __popcll(masks[w * E + e]);
        int row = bases[(long)blockIdx.x * E + e] + rank;
        slot_to_row[t * k + j] = row;
        row_to_slot[row] = (int32_t)(t * k + j);
    }
}

hipError_t launch_dispatch(const Shape &s, const int32_t *idx, int32_t *blockcounts, int32_t *counts,
                           int32_t *offsets, int32_t *slot_to_row, int32_t *row_to_slot, int32_t *err,
                           hipStream_t st) {
    if (s.T == 0) return hipSuccess;
    const int nblk = dispatch_blocks(s.T);
    const size_t lds = (size_t)4 * s.E * sizeof(unsigned long long);
    MOE_LAUNCH("dispatch_count", dispatch_count_kernel, dim3(nblk), dim3(256), lds, st, idx, s.T, s.k, s.E, blockcounts, err);
    MOE_LAUNCH("dispatch_scan", dispatch_scan_kernel, dim3(1), dim3(1024), 0, st, blockcounts, nblk, s.T, s.k, s.E, s.S,
                       counts, offsets);
    MOE_LAUNCH("dispatch_scatter", dispatch_scatter_kernel, dim3(nblk), dim3(256), lds, st, idx, s.T, s.k, s.E,
                       (const int32_t *)blockcounts, slot_to_row, row_to_slot, err);
    return hipGetLastError();
}

// ---- FP8 activation stage: x (bf16) -> e4m3 codes + power-of-two scale per 1x128 ----
//
// 16 lanes own one 128-value block (8 values each, one 16-byte load).
__global__ __launch_bounds__(256) void quant_x_kernel(const uint16_t *__restrict__ x, long nblocks,
                                                     uint8_t *__restrict__ xq, float *__restrict__ xs) {
    const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
    const long blk = gid >> 4;
    const int sub = (int)(gid & 15);
    if (blk >= nblocks) return;
    uint4 q = *(const uint4 *)(x + blk * 128 + sub * 8);
    const uint16_t *h = (const uint16_t *)&q;
    float v[8];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        v[i] = bf16_to_f32(h[i]);
        amax = fmaxf(amax, fabsf(v[i]));
    }
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 16));
    const int e = e4m3_block_exponent(amax);
    const float inv = ldexpf(1.0f, -e);
    uint2 out;
    out.x = cvt_e4m3x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
    out.y = cvt_e4m3x4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
    *(uint2 *)(xq + blk * 128 + sub * 8) = out;
    if (sub == 0) xs[blk] = ldexpf(1.0f, e);
}

hipError_t launch_quant_x(const Shape &s, const uint16_t *x, uint8_t *xq, float *xs, hipStream_t st) {
    const long nblocks = (long)s.T * s.d / 128;
    if (nblocks == 0) return hipSuccess;
    const long threads = nblocks * 16;
    MOE_LAUNCH("quant_x", quant_x_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, x, nblocks, xq, xs);
    return hipGetLastError();
}

}  // namespace moe
