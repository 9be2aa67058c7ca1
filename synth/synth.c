/*
 * Seeded synthetic inputs for the MoE-layer forward.
 *
 * This module only draws numbers; it holds none of the layer's arithmetic.
 * Both the CPU oracle and the GPU path receive the arrays it writes.
 *
 * Random source: Philox4x32-10, the counter-based generator of Salmon, Moraes,
 * Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3" (SC'11).
 * Element i of tensor (seed, tensor_id) is taken from the Philox block with
 * counter (i/4 low, i/4 high, tensor_id, 0) and key (seed, SYNTH_KEY1), so any
 * sub-range of a tensor can be drawn on its own and equals the same range of the
 * whole tensor, whatever the thread count.
 *
 * Normals: Box-Muller on the two 32-bit pairs of each Philox block.
 * bf16: round-to-nearest-even of the fp32 value.
 * MXFP4 (OCP Microscaling Formats v1.0): per block of 32 values along K, shared
 * exponent floor(log2(amax)) - 2 stored as e8m0, elements e2m1 with
 * round-to-nearest-even and saturation at 6.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>
#include <unistd.h>

#define SYNTH_KEY1 0x4d6f4521u

/* ---- Philox4x32-10 ---------------------------------------------------- */

static inline void mulhilo32(uint32_t a, uint32_t b, uint32_t *hi, uint32_t *lo) {
    uint64_t p = (uint64_t)a * (uint64_t)b;
    *hi = (uint32_t)(p >> 32);
    *lo = (uint32_t)p;
}

void synth_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int r = 0; r < 10; ++r) {
        uint32_t hi0, lo0, hi1, lo1;
        mulhilo32(0xD2511F53u, c0, &hi0, &lo0);
        mulhilo32(0xCD9E8D57u, c2, &hi1, &lo1);
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

static inline void block_bits(uint64_t seed, uint32_t tensor_id, uint64_t block, uint32_t out[4]) {
    uint32_t ctr[4] = {(uint32_t)block, (uint32_t)(block >> 32), tensor_id, (uint32_t)(seed >> 32)};
    uint32_t key[2] = {(uint32_t)seed, SYNTH_KEY1};
    synth_philox4x32_10(ctr, key, out);
}

/* Four standard normals from one Philox block (two Box-Muller pairs). */
static inline void block_normals(uint64_t seed, uint32_t tensor_id, uint64_t block, float z[4]) {
    uint32_t r[4];
    block_bits(seed, tensor_id, block, r);
    for (int p = 0; p < 2; ++p) {
        double u1 = ((double)r[2 * p] + 1.0) * (1.0 / 4294967296.0);   /* (0, 1] */
        double u2 = (double)r[2 * p + 1] * (1.0 / 4294967296.0);       /* [0, 1) */
        double rad = sqrt(-2.0 * log(u1));
        double ang = 6.283185307179586476925286766559 * u2;
        z[2 * p] = (float)(rad * cos(ang));
        z[2 * p + 1] = (float)(rad * sin(ang));
    }
}

static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* ---- thread pool helper ------------------------------------------------- */

typedef void (*range_fn)(void *ctx, uint64_t lo, uint64_t hi);
typedef struct { range_fn fn; void *ctx; uint64_t lo, hi; } range_job;

static void *range_thread(void *p) {
    range_job *j = (range_job *)p;
    j->fn(j->ctx, j->lo, j->hi);
    return NULL;
}

/* Runs fn over [0, n) split into contiguous chunks aligned to `align`. */
static void parallel_range(range_fn fn, void *ctx, uint64_t n, uint64_t align, int nthreads) {
    if (nthreads <= 0) {
        long c = sysconf(_SC_NPROCESSORS_ONLN);
        nthreads = c > 0 ? (int)c : 1;
    }
    if (nthreads > 64) nthreads = 64;
    uint64_t units = (n + align - 1) / align;
    if ((uint64_t)nthreads > units) nthreads = units ? (int)units : 1;
    if (nthreads <= 1) { fn(ctx, 0, n); return; }
    pthread_t th[64];
    int ok[64];
    range_job jobs[64];
    uint64_t per = (units + nthreads - 1) / nthreads;
    for (int t = 0; t < nthreads; ++t) {
        uint64_t lo = (uint64_t)t * per * align, hi = lo + per * align;
        ok[t] = 0;
        if (lo >= n) continue;
        if (hi > n) hi = n;
        jobs[t] = (range_job){fn, ctx, lo, hi};
        if (pthread_create(&th[t], NULL, range_thread, &jobs[t]) == 0) ok[t] = 1;
        else fn(ctx, lo, hi);
    }
    for (int t = 0; t < nthreads; ++t)
        if (ok[t]) pthread_join(th[t], NULL);
}

/* ---- normals ------------------------------------------------------------ */

typedef struct {
    uint64_t seed, offset;
    uint32_t tensor_id;
    float sigma;
    float *out_f32;
    uint16_t *out_bf16;
} normal_ctx;

static void normal_range(void *p, uint64_t lo, uint64_t hi) {
    normal_ctx *c = (normal_ctx *)p;
    uint64_t i = lo;
    while (i < hi) {
        uint64_t g = c->offset + i;
        uint64_t blk = g >> 2;
        float z[4];
        block_normals(c->seed, c->tensor_id, blk, z);
        for (uint64_t lane = g & 3; lane < 4 && i < hi; ++lane, ++i) {
            float v = z[lane] * c->sigma;
            if (c->out_f32) c->out_f32[i] = v;
            if (c->out_bf16) c->out_bf16[i] = f32_to_bf16_rne(v);
        }
    }
}

/* out[i] = sigma * N(0,1) drawn for element (offset + i) of tensor (seed, tensor_id). */
void synth_normal_f32(uint64_t seed, uint32_t tensor_id, uint64_t offset, uint64_t n, float sigma,
                      float *out, int nthreads) {
    normal_ctx c = {seed, offset, tensor_id, sigma, out, NULL};
    parallel_range(normal_range, &c, n, 1024, nthreads);
}

/* Same values as synth_normal_f32, rounded to bf16 (RNE); returns raw bf16 bits. */
void synth_normal_bf16(uint64_t seed, uint32_t tensor_id, uint64_t offset, uint64_t n, float sigma,
                       uint16_t *out, int nthreads) {
    normal_ctx c = {seed, offset, tensor_id, sigma, NULL, out};
    parallel_range(normal_range, &c, n, 1024, nthreads);
}

/* Uniform integers in [lo, hi] (inclusive) as float, for exact-arithmetic grids. */
typedef struct { uint64_t seed, offset; uint32_t tensor_id; int lo, hi; float *out_f32; uint16_t *out_bf16; } grid_ctx;

static void grid_range(void *p, uint64_t a, uint64_t b) {
    grid_ctx *c = (grid_ctx *)p;
    uint32_t span = (uint32_t)(c->hi - c->lo + 1);
    for (uint64_t i = a; i < b; ++i) {
        uint64_t g = c->offset + i;
        uint32_t r[4];
        block_bits(c->seed, c->tensor_id, g >> 2, r);
        int v = c->lo + (int)(r[g & 3] % span);
        float f = (float)v;
        if (c->out_f32) c->out_f32[i] = f;
        if (c->out_bf16) c->out_bf16[i] = f32_to_bf16_rne(f);
    }
}

void synth_intgrid_f32(uint64_t seed, uint32_t tensor_id, uint64_t offset, uint64_t n, int lo, int hi,
                       float *out, int nthreads) {
    grid_ctx c = {seed, offset, tensor_id, lo, hi, out, NULL};
    parallel_range(grid_range, &c, n, 1024, nthreads);
}

void synth_intgrid_bf16(uint64_t seed, uint32_t tensor_id, uint64_t offset, uint64_t n, int lo, int hi,
                        uint16_t *out, int nthreads) {
    grid_ctx c = {seed, offset, tensor_id, lo, hi, NULL, out};
    parallel_range(grid_range, &c, n, 1024, nthreads);
}

/* Raw 32-bit words, for permutations and other integer draws. */
void synth_u32(uint64_t seed, uint32_t tensor_id, uint64_t offset, uint64_t n, uint32_t *out) {
    for (uint64_t i = 0; i < n; ++i) {
        uint64_t g = offset + i;
        uint32_t r[4];
        block_bits(seed, tensor_id, g >> 2, r);
        out[i] = r[g & 3];
    }
}

/* ---- MXFP4 (OCP MX v1.0) weight quantiser -------------------------------- */

/* e2m1 code (sign in bit 3) of v, round-to-nearest-even, saturating at 6. */
static inline uint8_t e2m1_rne_sat(float v) {
    uint8_t s = signbit(v) ? 8 : 0;
    float a = fabsf(v);
    /* grid: 0, 0.5, 1, 1.5, 2, 3, 4, 6 (codes 0..7); midpoints go to the even code */
    uint8_t c;
    if (a <= 0.25f) c = 0;            /* 0.25 ties to code 0 */
    else if (a < 0.75f) c = 1;
    else if (a <= 1.25f) c = 2;       /* 0.75 -> 2 (even), 1.25 -> 2 (even) */
    else if (a < 1.75f) c = 3;
    else if (a <= 2.5f) c = 4;        /* 1.75 -> 4, 2.5 -> 4 */
    else if (a < 3.5f) c = 5;
    else if (a <= 5.0f) c = 6;        /* 3.5 -> 6, 5 -> 6 */
    else c = 7;                       /* saturate */
    return (uint8_t)(s | c);
}

typedef struct {
    uint64_t seed;
    uint32_t tensor_id;
    uint64_t row0, K;
    float sigma;
    int grid_lo, grid_hi, use_grid; /* integer-grid mode: values drawn as ints, scale 2^0 */
    uint8_t *codes, *scales;
} mx_ctx;

static void mx_rows(void *p, uint64_t r0, uint64_t r1) {
    mx_ctx *c = (mx_ctx *)p;
    uint64_t K = c->K;
    float v[32];
    for (uint64_t r = r0; r < r1; ++r) {
        uint64_t grow = c->row0 + r;
        for (uint64_t kb = 0; kb < K / 32; ++kb) {
            uint64_t base = grow * K + kb * 32;
            if (c->use_grid) {
                grid_ctx g = {c->seed, base, c->tensor_id, c->grid_lo, c->grid_hi, v, NULL};
                grid_range(&g, 0, 32);
            } else {
                normal_ctx n = {c->seed, base, c->tensor_id, c->sigma, v, NULL};
                normal_range(&n, 0, 32);
            }
            int e;
            if (c->use_grid) {
                e = 0;
            } else {
                float amax = 0.f;
                for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
                if (amax == 0.f) {
                    e = -127;
                } else {
                    int p2;
                    frexpf(amax, &p2);      /* amax = m * 2^p2, m in [0.5, 1) */
                    e = (p2 - 1) - 2;       /* floor(log2(amax)) - emax(e2m1) */
                    if (e < -127) e = -127;
                    if (e > 127) e = 127;
                }
            }
            c->scales[r * (K / 32) + kb] = (uint8_t)(e + 127);
            float inv = ldexpf(1.0f, -e);
            uint8_t *dst = c->codes + r * (K / 2) + kb * 16;
            for (int i = 0; i < 16; ++i) {
                uint8_t lo = e2m1_rne_sat(v[2 * i] * inv);
                uint8_t hi = e2m1_rne_sat(v[2 * i + 1] * inv);
                dst[i] = (uint8_t)(lo | (hi << 4));
            }
        }
    }
}

/*
 * Draws rows [row0, row0+rows) of a [*, K] weight from N(0, sigma^2) and quantises
 * them to MXFP4: codes [rows, K/2] (two per byte, even K index in the low nibble),
 * e8m0 scales [rows, K/32]. K must be a multiple of 32.
 */
void synth_mxfp4(uint64_t seed, uint32_t tensor_id, uint64_t row0, uint64_t rows, uint64_t K, float sigma,
                 uint8_t *codes, uint8_t *scales, int nthreads) {
    mx_ctx c = {seed, tensor_id, row0, K, sigma, 0, 0, 0, codes, scales};
    parallel_range(mx_rows, &c, rows, 1, nthreads);
}

/* Integer-grid MXFP4: values drawn from [lo, hi] (must lie on the e2m1 grid), scale 2^0. */
void synth_mxfp4_intgrid(uint64_t seed, uint32_t tensor_id, uint64_t row0, uint64_t rows, uint64_t K,
                         int lo, int hi, uint8_t *codes, uint8_t *scales, int nthreads) {
    mx_ctx c = {seed, tensor_id, row0, K, 0.f, lo, hi, 1, codes, scales};
    parallel_range(mx_rows, &c, rows, 1, nthreads);
}

/* ---- FP8 e4m3 rows with one power-of-two scale per 128 (OCP MX v1.0, E4M3 elements) ---- */

/* OCP E4M3FN code of v, round-to-nearest-even, saturating at 448 (code 0x7E). */
static inline uint8_t e4m3_rne_sat(float v) {
    uint8_t s = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    if (!(a < 448.0)) return (uint8_t)(s | 0x7E);
    int code;
    if (a < ldexp(1.0, -6)) {                 /* subnormals: multiples of 2^-9 */
        double q = a * 512.0, f = floor(q);
        int m = (int)f;
        if (q - f > 0.5 || (q - f == 0.5 && (m & 1))) ++m;
        code = m;                             /* m == 8 is the smallest normal, code 0x08 */
    } else {
        int ex;
        double m = frexp(a, &ex);             /* a = m 2^ex, m in [0.5, 1) */
        int E = ex - 1;                       /* a = (2m) 2^E, 2m in [1, 2) */
        double q = (2.0 * m - 1.0) * 8.0, f = floor(q);
        int mant = (int)f;
        if (q - f > 0.5 || (q - f == 0.5 && (mant & 1))) ++mant;
        if (mant == 8) { mant = 0; ++E; }
        code = ((E + 7) << 3) | mant;
        if (code > 0x7E) code = 0x7E;
    }
    return (uint8_t)(s | code);
}

typedef struct {
    uint64_t seed;
    uint32_t tensor_id;
    uint64_t row0, K;
    float sigma;
    int grid_lo, grid_hi, use_grid;
    uint8_t *codes;
    float *scales;
} f8_ctx;

static void f8_rows(void *p, uint64_t r0, uint64_t r1) {
    f8_ctx *c = (f8_ctx *)p;
    uint64_t K = c->K;
    float v[128];
    for (uint64_t r = r0; r < r1; ++r) {
        uint64_t grow = c->row0 + r;
        for (uint64_t kb = 0; kb < K / 128; ++kb) {
            uint64_t base = grow * K + kb * 128;
            if (c->use_grid) {
                grid_ctx g = {c->seed, base, c->tensor_id, c->grid_lo, c->grid_hi, v, NULL};
                grid_range(&g, 0, 128);
            } else {
                normal_ctx n = {c->seed, base, c->tensor_id, c->sigma, v, NULL};
                normal_range(&n, 0, 128);
            }
            int e = 0;
            if (!c->use_grid) {
                float amax = 0.f;
                for (int i = 0; i < 128; ++i) amax = fmaxf(amax, fabsf(v[i]));
                if (amax > 0.f) {
                    int p2;
                    frexpf(amax, &p2);
                    e = (p2 - 1) - 8;          /* floor(log2(amax)) - emax(e4m3) */
                    if (e < -127) e = -127;
                    if (e > 127) e = 127;
                }
            }
            c->scales[r * (K / 128) + kb] = ldexpf(1.0f, e);
            float inv = ldexpf(1.0f, -e);
            for (int i = 0; i < 128; ++i) c->codes[r * K + kb * 128 + i] = e4m3_rne_sat(v[i] * inv);
        }
    }
}

/*
 * Draws rows [row0, row0+rows) of a [*, K] tensor from N(0, sigma^2) and encodes them as
 * FP8 e4m3 with one power-of-two fp32 scale per 128 consecutive values: the OCP MX v1.0
 * scale rule with E4M3 elements (shared exponent floor(log2 amax) - 8, elements rounded to
 * nearest even and saturated at 448).  codes [rows, K], scales [rows, K/128].  K must be a
 * multiple of 128.
 */
void synth_fp8_rows(uint64_t seed, uint32_t tensor_id, uint64_t row0, uint64_t rows, uint64_t K, float sigma,
                    uint8_t *codes, float *scales, int nthreads) {
    f8_ctx c = {seed, tensor_id, row0, K, sigma, 0, 0, 0, codes, scales};
    parallel_range(f8_rows, &c, rows, 1, nthreads);
}

/* Integer-grid FP8 rows: values drawn from [lo, hi] (|v| <= 16, exact in e4m3), scale 1. */
void synth_fp8_rows_intgrid(uint64_t seed, uint32_t tensor_id, uint64_t row0, uint64_t rows, uint64_t K, int lo,
                            int hi, uint8_t *codes, float *scales, int nthreads) {
    f8_ctx c = {seed, tensor_id, row0, K, 0.f, lo, hi, 1, codes, scales};
    parallel_range(f8_rows, &c, rows, 1, nthreads);
}
