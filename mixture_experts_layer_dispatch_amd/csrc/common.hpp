// Internal device helpers for the gfx950 MoE kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

enum Mode { MODE_F32 = 0, MODE_BF16 = 1, MODE_FP8 = 2 };
enum Gating { GATE_SOFTMAX = 0, GATE_SIGMOID = 1 };
enum DevErr { DEVERR_NONE = 0, DEVERR_INDEX = 1, DEVERR_DUP = 2, DEVERR_NONFINITE = 3, DEVERR_TIMEOUT = 4 };

constexpr int kWave = 64;

// ---- bf16 <-> fp32 (raw bits in uint16) ---------------------------------

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round to nearest even; finite inputs (NaN keeps a quiet payload).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// ---- sticky device error word -------------------------------------------

__device__ __forceinline__ void set_error(int32_t *err, int32_t code) {
    if (err) atomicCAS(err, 0, code);
}

// ---- wave helpers ---------------------------------------------------------

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int mask) {
    return __shfl_xor(v, mask, kWave);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
    return v;
}

// ---- e4m3 block quantisation (power-of-two scale per 128 values) ---------
//
// e = smallest integer with amax <= 448 * 2^e, clamped to [-127, 127]; amax == 0
// gives e = 0.  With amax = m * 2^p, m in [0.5, 1): e = p - 9, plus one when
// m > 0.875 (448 = 0.875 * 2^9).  Exact integer logic, no rounding involved.
__device__ __forceinline__ int e4m3_block_exponent(float amax) {
    if (!(amax > 0.0f)) return 0;
    int p;
    float m = frexpf(amax, &p);
    int e = p - 9 + (m > 0.875f ? 1 : 0);
    return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Two fp32 -> two e4m3 (OCP E4M3FN) codes, round to nearest even, in the low 16 bits.
__device__ __forceinline__ uint32_t cvt_e4m3x2(float a, float b) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
}

// Four fp32 -> four e4m3 codes packed in a dword (a in the low byte).
__device__ __forceinline__ uint32_t cvt_e4m3x4(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

// Map a linear workgroup id so that ids landing on one XCD (ids are dealt to the
// 8 XCDs round-robin) become a contiguous range.  n must be a multiple of 8.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
    if (n % 8) return bid;
    return (bid % 8) * (n / 8) + bid / 8;
}

}  // namespace moe
