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

// MODE_FP8: FP8 e4m3 activations x MXFP4 weights; MODE_FP8X8: e4m3 x e4m3 (1x128 scales)
enum Mode { MODE_F32 = 0, MODE_BF16 = 1, MODE_FP8 = 2, MODE_FP8X8 = 3 };
__host__ __device__ inline bool fp8_act(int mode) { return mode == MODE_FP8 || mode == MODE_FP8X8; }
enum Gating { GATE_SOFTMAX = 0, GATE_SIGMOID = 1 };
enum DevErr {
    DEVERR_NONE = 0,
    DEVERR_INDEX = 1,
    DEVERR_DUP = 2,
    DEVERR_NONFINITE = 3,
    DEVERR_TIMEOUT = 4,
    DEVERR_OVERFLOW = 5  // received rows exceed the receive buffer (or a negative count)
};

constexpr int kWave = 64;

// ---- bf16 <-> fp32 (raw bits in uint16) ---------------------------------

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Round to nearest even: gfx950's packed conversion (v_cvt_pk_bf16_f32), two at a time.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return (uint16_t)pack_bf16x2(f, f); }

// SwiGLU of one (gate, up) pair, silu(g) * u with silu(g) = g * sigmoid(g): the sigmoid's
// reciprocal is the hardware one (v_rcp_f32, 1 ulp) rather than an IEEE division.
__device__ __forceinline__ float swiglu(float g, float u) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u; }

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

// ---- lane reductions with DPP -------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Maximum over each row of 16 lanes, left in every lane of the row: quad swaps, then the
// half-row and row mirrors (max is exact, so any pairing gives the same value).
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp_f32<0xB1>(v));     // quad_perm [1, 0, 3, 2]
    v = fmaxf(v, dpp_f32<0x4E>(v));     // quad_perm [2, 3, 0, 1]
    v = fmaxf(v, dpp_f32<0x141>(v));    // row_half_mirror
    return fmaxf(v, dpp_f32<0x140>(v));  // row_mirror
}

// Maximum over each half-wave (lanes 0-31, 32-63): the rows, then one swap across them.
__device__ __forceinline__ float half_wave_max(float v) {
    v = row16_max(v);
    return fmaxf(v, __shfl_xor(v, 16, kWave));
}

// ---- LDS DMA, counted waits and LDS swizzles (shared by the GEMM tiles) ----------

// global_load_lds_dwordx4 / _dword (gfx950): lane L's bytes land in LDS at (M0 base +
// size * L), with no staging registers.
__device__ __forceinline__ void lds_dma16(const void *g, uint8_t *lds_block) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)g,
                                     (__attribute__((address_space(3))) void *)lds_block, 16, 0, 0);
}
__device__ __forceinline__ void lds_dma4(const void *g, uint8_t *lds_block) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)g,
                                     (__attribute__((address_space(3))) void *)lds_block, 4, 0, 0);
}

// s_waitcnt lgkmcnt(0) with vmcnt and expcnt left at their maxima.
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// s_waitcnt vmcnt(n) (n < 64) with expcnt and lgkmcnt left at their maxima.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// LDS tile rows of BK bf16 (BK * 2 bytes: 128 or 64) as 16-byte chunks.  Physical chunk
// = logical chunk XOR a key of the row, chosen so that the 16 lanes of one ds_read_b128
// phase (rows r..r+15 at one logical chunk) hit 16 distinct 16-byte slots of the
// 256-byte window of gfx950's 64 LDS banks: (row >> 1) & 7 for 128-byte rows,
// (row >> 2) & 3 for 64-byte rows.  (Measured: 0 bank-conflict cycles; keyed on the
// low row bits instead, half of the LDS cycles are conflicts.)
template <int BK>
__device__ __forceinline__ int swz_key(int row) {
    return BK == 64 ? ((row >> 1) & 7) : ((row >> 2) & 3);
}
template <int BK>
__device__ __forceinline__ int swz_off(int row, int chunk) {
    return row * (BK * 2) + ((chunk ^ swz_key<BK>(row)) << 4);
}

// ---- device-coherent accesses ----------------------------------------------------------
//
// Data that one workgroup writes and another reads inside the persistent layer kernel
// moves through device-scope (sc1) loads and stores: on gfx950 these are coherent across
// the XCDs' L2 caches, so they need no cache write-back or invalidation (an agent-scope
// fence costs microseconds per wave and invalidates the whole L2).  The hand-off is then
// s_waitcnt vmcnt(0) on the producer (its sc1 stores have reached the device coherence
// point) followed by a relaxed device-scope counter update, and a spin on that counter on
// the consumer, whose later sc1 loads are issued in order after the spin.  COH = false
// gives plain accesses: the stand-alone kernels, where launches order everything.

template <bool COH>
__device__ __forceinline__ int32_t ldc(const int32_t *p) {
    if constexpr (COH) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else return *p;
}
template <bool COH>
__device__ __forceinline__ float ldc(const float *p) {
    if constexpr (COH) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else return *p;
}
template <bool COH>
__device__ __forceinline__ void stc(int32_t *p, int32_t v) {
    if constexpr (COH) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else *p = v;
}
template <bool COH>
__device__ __forceinline__ void stc(float *p, float v) {
    if constexpr (COH) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else *p = v;
}
template <bool COH>
__device__ __forceinline__ void stc(uint64_t *p, uint64_t v) {
    if constexpr (COH) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else *p = v;
}

// Raw buffer resource over [base, base + 2 GiB): base must be wave-uniform.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, 0x7fffffff, 0x00020000);
}
constexpr int kCpolSc1 = 16;  // cache policy: device scope

// 16 bytes at base + off (the coherent form needs off < 2^31).
template <bool COH>
__device__ __forceinline__ i32x4 ldc16(const void *base, size_t off) {
    if constexpr (COH) return __builtin_amdgcn_raw_buffer_load_b128(buffer_rsrc(base), (uint32_t)off, 0, kCpolSc1);
    else return *(const i32x4 *)((const uint8_t *)base + off);
}
// 2 bytes at base + 2 i (the coherent form needs 2 i < 2^31).
template <bool COH>
__device__ __forceinline__ void stc16(uint16_t *base, size_t i, uint16_t v) {
    if constexpr (COH) __builtin_amdgcn_raw_buffer_store_b16(v, buffer_rsrc(base), (uint32_t)(2 * i), 0, kCpolSc1);
    else base[i] = v;
}

// Token feeding dispatched row r: routed rows carry slot = t*k + j, the shared
// expert's rows are T*k + t.  Clamped so that corrupt inputs cannot read outside x.
template <bool COH = false>
__device__ __forceinline__ long row_token(long r, const int32_t *__restrict__ row_to_slot, int T, int k) {
    long tk = (long)T * k;
    long t;
    if (r < tk) {
        long s = ldc<COH>(row_to_slot + r);
        s = s < 0 ? 0 : (s >= tk ? tk - 1 : s);
        t = s / k;
    } else {
        t = r - tk;
    }
    return t < 0 ? 0 : (t >= T ? T - 1 : t);
}

// ---- tiles over ragged expert groups ------------------------------------------------
//
// A group g of n_g rows is cut into ceil(n_g / BM) row tiles times the N tiles; ts[g] is
// the exclusive prefix of tiles per group (ts[G] the total).  Within a group, row tiles
// vary fastest so that the tiles sharing one weight tile are neighbours.

// Tile of workgroup slot b (of a multiple of 8 slots), or -1.  Slot b runs on XCD b % 8;
// the tiles are split into 8 contiguous ranges, range x going to the slots of XCD x.
__device__ __forceinline__ int pick_tile(int b, int total) {
    const int xcd = b & 7, j = b >> 3;
    const int per = (total + 7) >> 3;
    const int t = xcd * per + j;
    return (j < per && t < total) ? t : -1;
}

// Tail split of a launch of 256-row tiles.  Workgroups are dealt to the eight XCDs round
// robin (block b runs on XCD b % 8) and pick_tile gives each XCD a contiguous chunk of the
// tiles.  An XCD runs C such workgroups at a time (one per CU), so a chunk of n tiles takes
// ceil(n / C) rounds and a last round of n % C tiles leaves CUs idle.  When that round has
// at most C / 2 tiles, each of them runs as two 128-row halves instead: still one round,
// but a shorter one.  Returns the tile, or -1, and sets half to -1 (the whole tile), 0 (its
// rows 0..127) or 1 (its rows 128..255).  Blocks needed per XCD: at most ceil(total / 8) +
// C / 2.
__host__ __device__ __forceinline__ int pick_tile_split(int b, int total, int C, int &half) {
    const int xcd = b & 7, j = b >> 3;
    const int per = (total + 7) >> 3;
    const int base = xcd * per, n = per < total - base ? per : total - base;
    half = -1;
    if (n <= 0) return -1;
    const int r = n % C, full = n - r;
    if (j < full) return base + j;
    if (2 * r <= C) {
        const int q = j - full;
        if (q >= 2 * r) return -1;
        half = q & 1;
        return base + full + (q >> 1);
    }
    return j < n ? base + j : -1;
}

struct TileInfo {
    int g, row0, nrows, nt, mt;  // group, first row, valid rows, N tile, row tile within the group
};

constexpr int kTileGroup = 8;  // row tiles per run of the grouped tile order

// Grouped order of a group's (row tile, N tile) pairs: runs of GM row tiles take every N
// tile in turn (row tile fastest within a run), so the tiles an XCD runs together share a
// few activation row tiles and a few weight column tiles, and each activation tile is
// fetched about ntn / (tiles in flight / GM) times instead of ntn times.  A bijection on
// [0, mtiles * ntn).
template <int GM>
__host__ __device__ __forceinline__ void grouped_tile(int local, int mtiles, int ntn, int &mt, int &nt) {
    const int per = GM * ntn, grp = local / per, first = grp * GM;
    const int gsz = mtiles - first < GM ? mtiles - first : GM;
    const int in = local - grp * per;
    mt = first + in % gsz;
    nt = in / gsz;
}

// As decode_tile, with the grouped order within each group (ts[g + 1] - ts[g] = mtiles x
// N tiles).
template <int GM>
__device__ __forceinline__ TileInfo decode_tile_grouped(int tile, const int32_t *__restrict__ ts,
                                                        const int32_t *__restrict__ offsets, int G, int BM) {
    int lo = 0, hi = G - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (ts[mid] <= tile) lo = mid; else hi = mid - 1;
    }
    TileInfo ti;
    ti.g = lo;
    const int rb = offsets[lo], cnt = offsets[lo + 1] - rb;
    const int mtiles = (cnt + BM - 1) / BM;
    grouped_tile<GM>(tile - ts[lo], mtiles, (ts[lo + 1] - ts[lo]) / mtiles, ti.mt, ti.nt);
    ti.row0 = rb + ti.mt * BM;
    ti.nrows = min(BM, cnt - ti.mt * BM);
    return ti;
}

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
    ti.mt = mt;
    ti.nt = local / mtiles;
    ti.row0 = rb + mt * BM;
    ti.nrows = min(BM, cnt - mt * BM);
    return ti;
}

}  // namespace moe
