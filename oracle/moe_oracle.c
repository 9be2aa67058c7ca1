/*
 * CPU oracle for the forward pass of one Mixture-of-Experts layer.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this library. The GPU library
 * never links it, includes it or calls it, and shares no code with it.
 *
 * It is written to be read against the pages, not to be fast: plain loops in
 * the order the definitions give, fp64 accumulation, one token at a time.
 * Threads only split the token list; every token is computed independently.
 *
 * Sources (page title, then section):
 *  - MoE lesson: factory.pai-world.com, "Mixture of Experts" (Phase 7, lesson 11).
 *    "FFN swap": the MoE block; router scores (N_tokens, E); top-k per token;
 *    output h + sum over the chosen experts of gate * Expert_e(x).
 *    "Load balancing": DeepSeek-V3's per-expert bias enters selection only;
 *    gate probabilities use the unbiased scores.
 *    "Shared expert": every token also passes through the shared expert.
 *    "Build it, Step 1: router": one linear layer, bias added for selection,
 *    a stable descending sort picks k, softmax (max subtracted) over the chosen
 *    raw scores gives the gates.
 *  - MoE playbook: molayo1419.me, "How it works": scores = softmax(x W_router),
 *    keep top-k, combine y = sum_i g_i Expert_i(x); shared expert is always on.
 *  - Mega MoE wiki (aiki.softdaddy-o.com) "One-line definition" and Mega MoE blog
 *    (donniechu.com) spec table: the fused chain dispatch -> linear1 -> SwiGLU ->
 *    linear2 -> combine, both linears FP8 x FP4.
 *
 * Readings where the pages are silent (each one is listed in the design notes):
 *  - SwiGLU expert: h = silu(x Wg^T) * (x Wu^T), out = h Wd^T, no biases;
 *    W1 = [Wg; Wu] stacked along the output dimension (gate rows first).
 *  - Sigmoid gating (the DeepSeek-V3-shaped workload): s = sigmoid(logit),
 *    key = s + bias, gate = s_j / sum of chosen s.
 *  - Ties in the selection key go to the lower expert index (stable sort).
 *  - FP8 activations: e4m3 (OCP E4M3FN, max 448) with one power-of-two fp32
 *    scale per 1x128 block, 2^e with e the smallest integer such that
 *    amax <= 448 * 2^e; codes are round-to-nearest-even of v * 2^-e.
 *  - MXFP4 weights are dequantised exactly: e2m1 value * 2^(e8m0 - 127).
 *  - FP8 e4m3 x e4m3 mode: weights are e4m3 codes with one power-of-two fp32 scale per
 *    1x128 block along K (the activations' format), dequantised exactly; activations
 *    and h are quantised as in the FP8 x MXFP4 mode.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_FP8_MXFP4 = 2, ORC_FP8_FP8 = 3 };
enum { ORC_SOFTMAX = 0, ORC_SIGMOID = 1 };
enum { ORC_OK = 0, ORC_BAD_INDEX = 1, ORC_DUP_INDEX = 2, ORC_NONFINITE = 3, ORC_SHAPE = 4 };

typedef struct {
    int32_t T, d, E, k, F, S; /* tokens, width, routed experts, top-k, expert hidden, shared */
    int32_t gating;           /* ORC_SOFTMAX or ORC_SIGMOID */
    int32_t mode;             /* ORC_F32, ORC_BF16, ORC_FP8_MXFP4, ORC_FP8_FP8 */
} oracle_cfg;

/* ---- number formats --------------------------------------------------- */

static double bf16_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* OCP E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa; S.1111.111 is NaN; no inf. */
double oracle_e4m3_decode(uint8_t c) {
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    double v = (e == 0) ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

/* OCP E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa; values 0,.5,1,1.5,2,3,4,6. */
double oracle_e2m1_decode(uint8_t c) {
    int s = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
    double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -v : v;
}

/* E8M0: 2^(c - 127); 0xFF is NaN. */
double oracle_e8m0_decode(uint8_t c) {
    if (c == 0xFF) return NAN;
    return ldexp(1.0, (int)c - 127);
}

/*
 * fp32 -> E4M3FN, round to nearest (ties to even) over the finite grid, values
 * beyond the largest finite magnitude saturate to 448. Written from the format
 * definition: enumerate the 127 non-negative finite codes and pick the closest.
 */
uint8_t oracle_e4m3_encode(float v) {
    if (isnan(v)) return 0x7F;
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    if (a >= 448.0) return (uint8_t)(sign | 0x7E);
    int best = 0;
    double bestd = INFINITY;
    for (int c = 0; c <= 0x7E; ++c) {
        double d = fabs(oracle_e4m3_decode((uint8_t)c) - a);
        if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) { bestd = d; best = c; }
    }
    return (uint8_t)(sign | best);
}

/*
 * Power-of-two block scale exponent for an fp32 block with max magnitude amax:
 * the smallest integer e with amax <= 448 * 2^e, clamped to the e8m0 range.
 * amax == 0 gives e = 0.
 */
int oracle_e4m3_block_exponent(float amax) {
    if (!(amax > 0.0f)) return 0;
    int e = (int)ceil(log2((double)amax / 448.0));
    /* guard the floating-point log against an off-by-one at exact powers */
    while (ldexp(448.0, e - 1) >= (double)amax) --e;
    while (ldexp(448.0, e) < (double)amax) ++e;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

/*
 * Quantise n values (n a multiple of 128) to e4m3 codes with one power-of-two
 * fp32 scale per 128 consecutive values.
 */
void oracle_quant_e4m3_b128(const float *v, int64_t n, uint8_t *codes, float *scales) {
    for (int64_t b = 0; b < n / 128; ++b) {
        float amax = 0.0f;
        for (int i = 0; i < 128; ++i) {
            float a = fabsf(v[b * 128 + i]);
            if (a > amax) amax = a;
        }
        int e = oracle_e4m3_block_exponent(amax);
        scales[b] = (float)ldexp(1.0, e);
        float inv = (float)ldexp(1.0, -e);
        for (int i = 0; i < 128; ++i) codes[b * 128 + i] = oracle_e4m3_encode(v[b * 128 + i] * inv);
    }
}

/* ---- S1: router logits ---------------------------------------------------- */

static double elem(const void *p, int64_t i, int mode_is_f32) {
    return mode_is_f32 ? (double)((const float *)p)[i] : bf16_to_double(((const uint16_t *)p)[i]);
}

/* logits[t,e] = sum_i x[t,i] W_r[e,i]; fp64 sum, rounded once to fp32. */
void oracle_logits_token(const oracle_cfg *c, const void *x, const void *wr, int64_t t, float *out) {
    int f32 = c->mode == ORC_F32;
    for (int e = 0; e < c->E; ++e) {
        double s = 0.0;
        for (int i = 0; i < c->d; ++i)
            s += elem(x, t * (int64_t)c->d + i, f32) * elem(wr, (int64_t)e * c->d + i, f32);
        out[e] = (float)s;
    }
}

/* ---- S2: selection keys --------------------------------------------------- */

static float sigmoid_f32(float l) { return (float)(1.0 / (1.0 + exp(-(double)l))); }

/* softmax gating: key = logit + bias; sigmoid gating: key = sigmoid(logit) + bias (fp32 adds). */
void oracle_keys_token(const oracle_cfg *c, const float *logits, const float *bias, float *keys) {
    for (int e = 0; e < c->E; ++e) {
        float s = c->gating == ORC_SIGMOID ? sigmoid_f32(logits[e]) : logits[e];
        keys[e] = s + (bias ? bias[e] : 0.0f);
    }
}

/* ---- S3: top-k ------------------------------------------------------------ */

/*
 * The k experts with the largest keys, in descending key order; equal keys keep
 * ascending expert order (a stable sort of 0..E-1 by descending key, first k).
 */
int oracle_topk_token(const oracle_cfg *c, const float *keys, int32_t *idx) {
    int E = c->E;
    int32_t *order = (int32_t *)malloc(sizeof(int32_t) * E);
    for (int e = 0; e < E; ++e) {
        if (!isfinite(keys[e])) { free(order); return ORC_NONFINITE; }
        order[e] = e;
    }
    /* stable insertion sort by descending key */
    for (int i = 1; i < E; ++i) {
        int32_t cur = order[i];
        int j = i - 1;
        while (j >= 0 && keys[order[j]] < keys[cur]) { order[j + 1] = order[j]; --j; }
        order[j + 1] = cur;
    }
    for (int j = 0; j < c->k; ++j) idx[j] = order[j];
    free(order);
    return ORC_OK;
}

/* ---- S4: gates ------------------------------------------------------------ */

/*
 * softmax: g_j = exp(l_j - m) / sum_i exp(l_i - m) over the chosen raw logits;
 * sigmoid: g_j = s_j / sum_i s_i over the chosen s = sigmoid(l). The bias never
 * enters. Computed in fp64, rounded to fp32.
 */
void oracle_gates_token(const oracle_cfg *c, const float *logits, const int32_t *idx, float *gates) {
    int k = c->k;
    double v[64];
    if (c->gating == ORC_SIGMOID) {
        double sum = 0.0;
        for (int j = 0; j < k; ++j) { v[j] = 1.0 / (1.0 + exp(-(double)logits[idx[j]])); sum += v[j]; }
        for (int j = 0; j < k; ++j) gates[j] = (float)(v[j] / sum);
    } else {
        double m = -INFINITY, sum = 0.0;
        for (int j = 0; j < k; ++j) if ((double)logits[idx[j]] > m) m = (double)logits[idx[j]];
        for (int j = 0; j < k; ++j) { v[j] = exp((double)logits[idx[j]] - m); sum += v[j]; }
        for (int j = 0; j < k; ++j) gates[j] = (float)(v[j] / sum);
    }
}

/* ---- S1-S4 over all tokens ------------------------------------------------ */

typedef struct {
    const oracle_cfg *c;
    const void *x, *wr;
    const float *bias;
    int32_t *idx;
    float *gates, *logits, *keys;
    int status;
} route_ctx;

static void route_range(route_ctx *r, int64_t t0, int64_t t1) {
    const oracle_cfg *c = r->c;
    float *l = (float *)malloc(sizeof(float) * c->E), *kk = (float *)malloc(sizeof(float) * c->E);
    for (int64_t t = t0; t < t1; ++t) {
        oracle_logits_token(c, r->x, r->wr, t, l);
        oracle_keys_token(c, l, r->bias, kk);
        int st = oracle_topk_token(c, kk, r->idx + t * c->k);
        if (st) {
            /* no valid selection: report it and leave a harmless placeholder */
            r->status = st;
            for (int j = 0; j < c->k; ++j) { r->idx[t * c->k + j] = j; r->gates[t * c->k + j] = NAN; }
        } else {
            oracle_gates_token(c, l, r->idx + t * c->k, r->gates + t * c->k);
        }
        if (r->logits) memcpy(r->logits + t * c->E, l, sizeof(float) * c->E);
        if (r->keys) memcpy(r->keys + t * c->E, kk, sizeof(float) * c->E);
    }
    free(l);
    free(kk);
}

/* ---- thread split over a token list --------------------------------------- */

typedef struct { void (*fn)(void *, int64_t, int64_t); void *ctx; int64_t lo, hi; } job;
static void *job_main(void *p) { job *j = (job *)p; j->fn(j->ctx, j->lo, j->hi); return NULL; }

static void run_split(void (*fn)(void *, int64_t, int64_t), void *ctx, int64_t n, int nthreads) {
    if (nthreads <= 0) { long cpus = sysconf(_SC_NPROCESSORS_ONLN); nthreads = cpus > 0 ? (int)cpus : 1; }
    if (nthreads > 256) nthreads = 256;
    if (nthreads > n) nthreads = n > 0 ? (int)n : 1;
    if (nthreads <= 1) { fn(ctx, 0, n); return; }
    pthread_t th[256];
    job jobs[256];
    int ok[256];
    for (int i = 0; i < nthreads; ++i) {
        jobs[i] = (job){fn, ctx, n * i / nthreads, n * (i + 1) / nthreads};
        ok[i] = pthread_create(&th[i], NULL, job_main, &jobs[i]) == 0;
        if (!ok[i]) fn(ctx, jobs[i].lo, jobs[i].hi);
    }
    for (int i = 0; i < nthreads; ++i) if (ok[i]) pthread_join(th[i], NULL);
}

static void route_thunk(void *p, int64_t a, int64_t b) { route_ctx *r = (route_ctx *)p; route_range(r, a, b); }

/* Routes all T tokens: topk_idx [T,k], topk_gate [T,k], optional logits/keys [T,E]. */
int oracle_route(const oracle_cfg *c, const void *x, const void *wr, const float *bias, int32_t *idx,
                 float *gates, float *logits, float *keys, int nthreads) {
    if (c->k < 1 || c->k > c->E || c->k > 64) return ORC_SHAPE;
    route_ctx r = {c, x, wr, bias, idx, gates, logits, keys, ORC_OK};
    run_split(route_thunk, &r, c->T, nthreads);
    return r.status;
}

/* Top-k and gates from given logits and keys (e.g. exported by another implementation). */
int oracle_topk_gates_from(const oracle_cfg *c, const float *logits, const float *keys, int32_t *idx,
                           float *gates) {
    if (c->k < 1 || c->k > c->E || c->k > 64) return ORC_SHAPE;
    for (int64_t t = 0; t < c->T; ++t) {
        int st = oracle_topk_token(c, keys + t * c->E, idx + t * c->k);
        if (st) return st;
        oracle_gates_token(c, logits + t * c->E, idx + t * c->k, gates + t * c->k);
    }
    return ORC_OK;
}

/* ---- S5-S6: dispatch -------------------------------------------------------- */

/*
 * Counting sort of the T*k slots (slot = t*k + j) by expert, stable in slot
 * order, so rows of one expert are in ascending token order. Group E is the
 * shared expert (when S = 1): rows T*k + t, one per token, in token order.
 * counts [E+S], offsets [E+S+1], slot_to_row [T*k], row_to_slot [T*k].
 */
int oracle_dispatch(const oracle_cfg *c, const int32_t *idx, int32_t *counts, int32_t *offsets,
                    int32_t *slot_to_row, int32_t *row_to_slot) {
    int64_t T = c->T;
    int k = c->k, E = c->E, G = c->E + c->S;
    for (int64_t t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            int32_t e = idx[t * k + j];
            if (e < 0 || e >= E) return ORC_BAD_INDEX;
            for (int jj = 0; jj < j; ++jj) if (idx[t * k + jj] == e) return ORC_DUP_INDEX;
        }
    for (int g = 0; g < G; ++g) counts[g] = 0;
    for (int64_t s = 0; s < T * k; ++s) counts[idx[s]]++;
    if (c->S) counts[E] = (int32_t)T;
    offsets[0] = 0;
    for (int g = 0; g < G; ++g) offsets[g + 1] = offsets[g] + counts[g];
    int32_t *cursor = (int32_t *)calloc((size_t)G, sizeof(int32_t));
    for (int64_t s = 0; s < T * k; ++s) {
        int32_t e = idx[s];
        int32_t row = offsets[e] + cursor[e]++;
        slot_to_row[s] = row;
        row_to_slot[row] = (int32_t)s;
    }
    free(cursor);
    return ORC_OK;
}

/* ---- S7-S9: one expert on one token ----------------------------------------- */

typedef struct {
    const void *w1, *w1s, *w2, *w2s; /* per mode: f32 / bf16 values, or MXFP4 codes + e8m0 scales */
} oracle_weights;

/* Weight element W[g][r][i] of a [G, R, K] matrix, dequantised exactly. */
static double weight(const oracle_cfg *c, const void *w, const void *ws, int g, int64_t R, int64_t K,
                     int64_t r, int64_t i) {
    int64_t flat = ((int64_t)g * R + r) * K + i;
    if (c->mode == ORC_F32) return (double)((const float *)w)[flat];
    if (c->mode == ORC_BF16) return bf16_to_double(((const uint16_t *)w)[flat]);
    if (c->mode == ORC_FP8_FP8) /* e4m3 code times its 1x128 block's fp32 scale */
        return oracle_e4m3_decode(((const uint8_t *)w)[flat]) *
               (double)((const float *)ws)[((int64_t)g * R + r) * (K / 128) + i / 128];
    uint8_t byte = ((const uint8_t *)w)[flat >> 1];
    uint8_t code = (flat & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15);
    uint8_t sc = ((const uint8_t *)ws)[((int64_t)g * R + r) * (K / 32) + i / 32];
    return oracle_e2m1_decode(code) * oracle_e8m0_decode(sc);
}

/*
 * out[c] = sum_f h_f W2[g][c][f], h = silu(u_gate) * u_up, u = W1[g] xin.
 * xin is the (already dequantised, in FP8 mode) input row. In FP8 mode h is
 * rounded to fp32 and quantised to e4m3 per 1x128 block before linear2, since
 * linear2 consumes FP8 activations; h_out (optional) receives h before that.
 */
void oracle_expert_row(const oracle_cfg *c, const oracle_weights *w, int g, const double *xin, double *out,
                       double *h_out) {
    int64_t d = c->d, F = c->F;
    double *h = (double *)malloc(sizeof(double) * F);
    for (int64_t f = 0; f < F; ++f) {
        double ug = 0.0, uu = 0.0;
        for (int64_t i = 0; i < d; ++i) ug += xin[i] * weight(c, w->w1, w->w1s, g, 2 * F, d, f, i);
        for (int64_t i = 0; i < d; ++i) uu += xin[i] * weight(c, w->w1, w->w1s, g, 2 * F, d, F + f, i);
        h[f] = ug / (1.0 + exp(-ug)) * uu;
    }
    if (h_out) memcpy(h_out, h, sizeof(double) * F);
    if (c->mode == ORC_FP8_MXFP4 || c->mode == ORC_FP8_FP8) {
        float *hf = (float *)malloc(sizeof(float) * F);
        uint8_t *hc = (uint8_t *)malloc((size_t)F);
        float *hs = (float *)malloc(sizeof(float) * (F / 128));
        for (int64_t f = 0; f < F; ++f) hf[f] = (float)h[f];
        oracle_quant_e4m3_b128(hf, F, hc, hs);
        for (int64_t f = 0; f < F; ++f) h[f] = oracle_e4m3_decode(hc[f]) * (double)hs[f / 128];
        free(hf); free(hc); free(hs);
    }
    for (int64_t o = 0; o < d; ++o) {
        double s = 0.0;
        for (int64_t f = 0; f < F; ++f) s += h[f] * weight(c, w->w2, w->w2s, g, d, F, o, f);
        out[o] = s;
    }
    free(h);
}

/* The expert input row of token t: x itself, or its FP8 e4m3 b128 dequantisation. */
void oracle_input_row(const oracle_cfg *c, const void *x, int64_t t, double *xin) {
    int64_t d = c->d;
    if (c->mode == ORC_F32) { for (int64_t i = 0; i < d; ++i) xin[i] = ((const float *)x)[t * d + i]; return; }
    if (c->mode == ORC_BF16) { for (int64_t i = 0; i < d; ++i) xin[i] = bf16_to_double(((const uint16_t *)x)[t * d + i]); return; }
    float *xf = (float *)calloc((size_t)d, sizeof(float));
    if (!xf) return;
    uint8_t *q = (uint8_t *)malloc((size_t)d);
    float *s = (float *)malloc(sizeof(float) * (d / 128));
    for (int64_t i = 0; i < d; ++i) xf[i] = (float)bf16_to_double(((const uint16_t *)x)[t * d + i]);
    oracle_quant_e4m3_b128(xf, d, q, s);
    for (int64_t i = 0; i < d; ++i) xin[i] = oracle_e4m3_decode(q[i]) * (double)s[i / 128];
    free(xf); free(q); free(s);
}

/* ---- S10 + the whole layer ------------------------------------------------------ */

typedef struct {
    const oracle_cfg *c;
    const void *x, *wr;
    const float *bias;
    oracle_weights w;
    const int32_t *idx_in;
    const float *gates_in;
    const int64_t *tokens;
    double *y;
    int32_t *idx_out;
    float *gates_out;
    int status;
    const uint8_t *keep; /* [T*k] or NULL: a slot with keep 0 was dropped (capacity variant) */
} layer_ctx;

static void layer_range(void *p, int64_t a, int64_t b) {
    layer_ctx *L = (layer_ctx *)p;
    const oracle_cfg *c = L->c;
    int64_t d = c->d;
    int k = c->k;
    double *xin = (double *)malloc(sizeof(double) * d), *o = (double *)malloc(sizeof(double) * d);
    float *lg = (float *)malloc(sizeof(float) * c->E), *ky = (float *)malloc(sizeof(float) * c->E);
    int32_t idx[64];
    float g[64];
    for (int64_t n = a; n < b; ++n) {
        int64_t t = L->tokens[n];
        if (L->idx_in) {
            for (int j = 0; j < k; ++j)
                if (L->idx_in[t * k + j] < 0 || L->idx_in[t * k + j] >= c->E) { L->status = ORC_BAD_INDEX; goto next; }
            memcpy(idx, L->idx_in + t * k, sizeof(int32_t) * k);
            memcpy(g, L->gates_in + t * k, sizeof(float) * k);
        } else {
            oracle_logits_token(c, L->x, L->wr, t, lg);
            oracle_keys_token(c, lg, L->bias, ky);
            int st = oracle_topk_token(c, ky, idx);
            if (st) { L->status = st; goto next; }
            oracle_gates_token(c, lg, idx, g);
        }
        if (L->idx_out) memcpy(L->idx_out + n * k, idx, sizeof(int32_t) * k);
        if (L->gates_out) memcpy(L->gates_out + n * k, g, sizeof(float) * k);
        oracle_input_row(c, L->x, t, xin);
        double *y = L->y + n * d;
        for (int64_t i = 0; i < d; ++i) y[i] = 0.0;
        /* fixed order: routed experts j = 0..k-1 in selection order, then the shared expert */
        for (int j = 0; j < k; ++j) {
            if (L->keep && !L->keep[t * k + j]) continue; /* a dropped slot skips the layer */
            oracle_expert_row(c, &L->w, idx[j], xin, o, NULL);
            for (int64_t i = 0; i < d; ++i) y[i] += (double)g[j] * o[i];
        }
        for (int s = 0; s < c->S; ++s) {
            oracle_expert_row(c, &L->w, c->E + s, xin, o, NULL);
            for (int64_t i = 0; i < d; ++i) y[i] += o[i];
        }
        continue;
    next:
        for (int64_t i = 0; i < d; ++i) L->y[n * d + i] = NAN;
    }
    free(xin); free(o); free(lg); free(ky);
}

/*
 * y[n, :] for each token t = tokens[n]: sum_j g_j Expert_{idx_j}(x_t) + Expert_shared(x_t),
 * in fp64. Routing is computed here unless idx_in/gates_in ([T,k]) are given, in
 * which case that routing is used (to compare outputs under identical routing).
 * idx_out/gates_out ([ntok,k], optional) receive the routing used.
 */
int oracle_layer(const oracle_cfg *c, const void *x, const void *wr, const float *bias, const void *w1,
                 const void *w1s, const void *w2, const void *w2s, const int32_t *idx_in,
                 const float *gates_in, const int64_t *tokens, int64_t ntok, double *y, int32_t *idx_out,
                 float *gates_out, int nthreads) {
    if (c->k < 1 || c->k > c->E || c->k > 64) return ORC_SHAPE;
    if ((c->mode == ORC_FP8_MXFP4 || c->mode == ORC_FP8_FP8) && (c->d % 128 || c->F % 128)) return ORC_SHAPE;
    layer_ctx L = {c, x, wr, bias, {w1, w1s, w2, w2s}, idx_in, gates_in, tokens, y, idx_out, gates_out, ORC_OK, NULL};
    run_split(layer_range, &L, ntok, nthreads);
    return L.status;
}

/*
 * The layer under the capacity variant: as oracle_layer with the given routing
 * (idx_in, gates_in [T,k]), except that a slot whose keep[t*k + j] is 0 was dropped
 * and contributes nothing -- its token skips that expert (MoE lesson, "The
 * load-balancing problem", item 2: tokens over an expert's capacity skip the layer).
 * The remaining gates are not renormalised; the shared expert always applies.
 */
int oracle_layer_dropping(const oracle_cfg *c, const void *x, const void *w1, const void *w1s, const void *w2,
                          const void *w2s, const int32_t *idx_in, const float *gates_in, const uint8_t *keep,
                          const int64_t *tokens, int64_t ntok, double *y, int nthreads) {
    if (c->k < 1 || c->k > c->E || c->k > 64 || !idx_in || !gates_in || !keep) return ORC_SHAPE;
    if ((c->mode == ORC_FP8_MXFP4 || c->mode == ORC_FP8_FP8) && (c->d % 128 || c->F % 128)) return ORC_SHAPE;
    layer_ctx L = {c, x, NULL, NULL, {w1, w1s, w2, w2s}, idx_in, gates_in, tokens, y, NULL, NULL, ORC_OK, keep};
    run_split(layer_range, &L, ntok, nthreads);
    return L.status;
}

/* ---- the capacity variant of the dispatch ----------------------------------------- */

/*
 * Expert capacity with token dropping (MoE lesson, "The load-balancing problem",
 * item 2): each routed expert takes at most `capacity` of the slots that chose it;
 * the others are dropped.  Which ones: the slots of one expert in slot order (that is,
 * ascending token order, the order of the dropless dispatch); the first `capacity` are
 * kept.  The shared expert has no capacity.
 *
 * Outputs, with kept_e = min(n_e, capacity), dropped_e = n_e - kept_e and
 * D = sum of dropped_e:
 *  counts[e] = kept_e (counts[E] = T when S = 1); dropped[e] = dropped_e;
 *  offsets[0] = D, offsets[e + 1] = offsets[e] + kept_e, so offsets[E] = T*k and the
 *  shared group keeps rows T*k + t;
 *  rows 0 .. D-1 list the dropped slots, expert by expert, in slot order;
 *  slot_to_row[s] = the kept row of slot s, or -1 when s was dropped;
 *  row_to_slot[r] = the slot of row r (kept and dropped rows alike).
 */
int oracle_dispatch_capacity(const oracle_cfg *c, const int32_t *idx, int32_t capacity, int32_t *counts,
                             int32_t *dropped, int32_t *offsets, int32_t *slot_to_row, int32_t *row_to_slot) {
    int64_t T = c->T;
    int k = c->k, E = c->E, G = c->E + c->S;
    if (capacity < 0) return ORC_SHAPE;
    for (int64_t t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            int32_t e = idx[t * k + j];
            if (e < 0 || e >= E) return ORC_BAD_INDEX;
            for (int jj = 0; jj < j; ++jj) if (idx[t * k + jj] == e) return ORC_DUP_INDEX;
        }
    int32_t *n = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    int32_t *drop_base = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    int32_t *seen = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    for (int64_t s = 0; s < T * k; ++s) n[idx[s]]++;
    int32_t D = 0;
    for (int e = 0; e < E; ++e) {
        counts[e] = n[e] < capacity ? n[e] : capacity;
        dropped[e] = n[e] - counts[e];
        drop_base[e] = D;
        D += dropped[e];
    }
    if (c->S) counts[E] = (int32_t)T;
    offsets[0] = D;
    for (int g = 0; g < G; ++g) offsets[g + 1] = offsets[g] + counts[g];
    for (int64_t s = 0; s < T * k; ++s) {
        int32_t e = idx[s];
        int32_t rank = seen[e]++;  /* position of slot s among expert e's slots, in slot order */
        int32_t row;
        if (rank < capacity) {
            row = offsets[e] + rank;
            slot_to_row[s] = row;
        } else {
            row = drop_base[e] + (rank - capacity);
            slot_to_row[s] = -1;
        }
        row_to_slot[row] = (int32_t)s;
    }
    free(n);
    free(drop_base);
    free(seen);
    return ORC_OK;
}

/* ---- aux-loss-free load balancing ------------------------------------------------ */

/*
 * One update of the per-expert selection bias (MoE lesson, "The load-balancing
 * problem", the DeepSeek-V3 scheme, and "Build it -- Step 2: route 100 tokens"):
 * after a step, an expert used more than its target gets -gamma, one used less gets
 * +gamma.  The target is the mean load over the E routed experts, sum(counts) / E; an
 * expert exactly on target keeps its bias (compared exactly, as counts[e] * E against
 * the total).  The addition is an fp32 add, as the bias is fp32.
 */
void oracle_bias_update(int32_t E, const int32_t *counts, float *bias, float gamma) {
    int64_t total = 0;
    for (int e = 0; e < E; ++e) total += counts[e];
    for (int e = 0; e < E; ++e) {
        int64_t scaled = (int64_t)counts[e] * E;
        if (scaled > total) bias[e] = bias[e] - gamma;
        else if (scaled < total) bias[e] = bias[e] + gamma;
    }
}

/* One expert applied to given input rows (already in the mode's input precision). */
void oracle_expert_rows(const oracle_cfg *c, const void *w1, const void *w1s, const void *w2, const void *w2s,
                        int g, const double *xin, int64_t nrows, double *out, double *h_out) {
    oracle_weights w = {w1, w1s, w2, w2s};
    for (int64_t r = 0; r < nrows; ++r)
        oracle_expert_row(c, &w, g, xin + r * c->d, out + r * c->d, h_out ? h_out + r * c->F : NULL);
}

/* Selection keys for all T tokens from given logits [T,E] (e.g. another implementation's). */
void oracle_keys_from(const oracle_cfg *c, const float *logits, const float *bias, float *keys) {
    for (int64_t t = 0; t < c->T; ++t) oracle_keys_token(c, logits + t * c->E, bias, keys + t * c->E);
}

/*
 * linear2 alone: out[r][c] = sum_f hhat[r][f] W2[g][c][f] for given rows hhat [nrows, F]
 * (fp64; in FP8 mode the dequantised e4m3 h rows, code * scale). It lets a caller project
 * the very h codes another implementation produced, as the MXFP4 weights are dequantised
 * exactly and the sum is taken in fp64 in f order.
 */
void oracle_down_rows(const oracle_cfg *c, const void *w2, const void *w2s, int g, const double *hhat,
                      int64_t nrows, double *out) {
    int64_t d = c->d, F = c->F;
    for (int64_t r = 0; r < nrows; ++r)
        for (int64_t o = 0; o < d; ++o) {
            double s = 0.0;
            for (int64_t f = 0; f < F; ++f) s += hhat[r * F + f] * weight(c, w2, w2s, g, d, F, o, f);
            out[r * d + o] = s;
        }
}

/* ---- FP8 operands given as codes ----------------------------------------------------- */

/* Rows of e4m3 codes [n, K] with fp32 scales per 128 [n, K/128] -> fp64 values code * scale. */
void oracle_dequant_e4m3_rows(const uint8_t *codes, const float *scales, int64_t n, int64_t K, double *out) {
    for (int64_t r = 0; r < n; ++r)
        for (int64_t i = 0; i < K; ++i)
            out[r * K + i] = oracle_e4m3_decode(codes[r * K + i]) * (double)scales[r * (K / 128) + i / 128];
}

/*
 * The dense FP8 x MXFP4 GEMM that ships next to the fused MoE kernel (Mega MoE blog,
 * "What's new"): C[m][n] = sum_k A[m][k] B[n][k], A given as e4m3 codes [M, K] with fp32
 * scales per 1x128 [M, K/128], B as MXFP4 (e2m1 codes [N, K/2], even k in the low nibble,
 * e8m0 scales [N, K/32]); every operand dequantised exactly, the sum in fp64 in k order.
 */
void oracle_gemm_fp8_mxfp4(int64_t M, int64_t N, int64_t K, const uint8_t *a, const float *as, const uint8_t *b,
                           const uint8_t *bs, double *c) {
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double av = oracle_e4m3_decode(a[m * K + k]) * (double)as[m * (K / 128) + k / 128];
                uint8_t byte = b[(n * K + k) >> 1];
                uint8_t code = (k & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15);
                double bv = oracle_e2m1_decode(code) * oracle_e8m0_decode(bs[n * (K / 32) + k / 32]);
                s += av * bv;
            }
            c[m * N + n] = s;
        }
}
