/*
 * moe.h -- C ABI of libmoe.so: the forward pass of one Mixture-of-Experts layer
 * on an AMD Instinct MI355X (gfx950).
 *
 * The layer (MoE lesson, factory.pai-world.com "Mixture of Experts", section
 * "FFN swap"; MoE playbook, molayo1419.me, section "How it works"):
 *
 *   logits = x W_r^T                       router, one linear layer   (moe_route)
 *   idx    = top-k of the selection keys    bias enters selection only (moe_route)
 *   g      = gates over the chosen experts  unbiased scores            (moe_route)
 *   rows   = tokens grouped by expert       dispatch                   (moe_dispatch)
 *   h      = silu(x Wg^T) * (x Wu^T)        linear1 + SwiGLU           (moe_ffn)
 *   o      = h Wd^T                         linear2                    (moe_ffn)
 *   y      = sum_j g_j o_j + o_shared       gate-weighted combine      (moe_combine)
 *
 * moe_layer_fused runs the whole chain in one persistent launch, the one-GPU
 * counterpart of the single mega-kernel that fuses dispatch, linear1, SwiGLU,
 * linear2 and combine (Mega MoE wiki, aiki.softdaddy-o.com, "One-line
 * definition"; Mega MoE blog, donniechu.com, spec table "Ops fused in 1 kernel").
 *
 * Conventions shared by every entry point:
 *  - Pointers named x, y, w*, idx, gate, counts, offsets, *_row, *_slot, ws are
 *    DEVICE pointers; moe_cfg and moe_weights structs are HOST memory read only
 *    during the call.  The caller allocates and owns every buffer; the library
 *    never allocates device memory and keeps no state between calls.
 *  - Every call is asynchronous and stream-ordered on `stream`.  The return value
 *    reports host-side validation and launch errors only.  Errors found by a
 *    kernel (bad or duplicate expert indices, non-finite keys, an expired bounded
 *    wait) set a sticky word at the start of the workspace; read it with
 *    moe_read_device_error.
 *  - All device pointers must be 16-byte aligned.
 *  - Outputs are bitwise deterministic: identical inputs give identical bits.
 *    No floating-point atomics are used.
 *  - T == 0 is a valid no-op (MOE_OK, nothing launched).
 *  - Calls that share a workspace must not overlap on the device.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_NULL = 1,      /* a required pointer is NULL */
    MOE_ERR_SHAPE = 2,     /* shape outside the supported limits (see moe_cfg) */
    MOE_ERR_MODE = 3,      /* unknown mode or gating */
    MOE_ERR_ALIGN = 4,     /* a device pointer is not 16-byte aligned */
    MOE_ERR_WORKSPACE = 5, /* ws is NULL or smaller than moe_workspace_bytes() */
    MOE_ERR_LAUNCH = 6,    /* a HIP launch or runtime call failed */
    MOE_ERR_ARCH = 7,      /* the current device is not gfx950 */
    MOE_ERR_DEVICE = 8     /* a kernel reported an error (moe_read_device_error) */
} moe_status;

/*
 * Arithmetic modes.
 *  MOE_MODE_F32:       x, W_r, W1, W2, y fp32; y_perm fp32; fp32 accumulation.
 *  MOE_MODE_BF16:      x, W_r, W1, W2, y bf16; fp32 accumulation; h and y_perm bf16.
 *  MOE_MODE_FP8_MXFP4: x, W_r, y bf16. The router runs in bf16 with fp32 sums.
 *                      Expert inputs x and h are quantised in-layer to FP8 e4m3
 *                      (OCP E4M3FN) with one power-of-two fp32 scale per 1x128
 *                      block along K; W1, W2 are MXFP4 (OCP MX v1.0): e2m1 codes,
 *                      two per byte, even K index in the low nibble, plus one e8m0
 *                      scale byte per 32 consecutive K.  Both linears are FP8 x FP4
 *                      (Mega MoE blog, donniechu.com, spec table), fp32
 *                      accumulation; y_perm bf16.
 *  MOE_MODE_FP8_FP8:   as MOE_MODE_FP8_MXFP4, with FP8 weights as well: W1, W2 are e4m3
 *                      codes, one byte each, with one power-of-two fp32 scale per 1x128
 *                      block along K (the activations' format).  Both linears e4m3 x e4m3.
 */
typedef enum { MOE_MODE_F32 = 0, MOE_MODE_BF16 = 1, MOE_MODE_FP8_MXFP4 = 2, MOE_MODE_FP8_FP8 = 3 } moe_mode;

/*
 * Gating (MoE lesson "Build it, Step 1: router" and "Load balancing"; the
 * sigmoid form is the reading taken for the DeepSeek-V3-shaped workload):
 *  MOE_GATE_SOFTMAX: key = logit + bias;          gate_j = softmax over the chosen raw logits.
 *  MOE_GATE_SIGMOID: key = sigmoid(logit) + bias; gate_j = s_j / sum of the chosen s.
 * Top-k orders experts by descending key; equal keys go to the lower expert index.
 */
typedef enum { MOE_GATE_SOFTMAX = 0, MOE_GATE_SIGMOID = 1 } moe_gating;

/*
 * Shapes.  T tokens, d model width, E routed experts, k experts per token, F
 * expert hidden width, n_shared in {0, 1} always-on shared experts (MoE lesson,
 * "Shared expert").  G = E + n_shared expert groups; the shared expert is group E.
 * Limits: 0 <= T <= 2^20, 1 <= k <= min(E, 16), E <= 1024, d and F multiples of
 * 128 (every mode), T*(k+n_shared) < 2^31.
 * cu_limit caps the number of compute units the persistent kernels spread over
 * (0 = all).
 */
typedef struct {
    int32_t T, d, E, k, F, n_shared;
    int32_t gating;   /* moe_gating */
    int32_t mode;     /* moe_mode */
    int32_t cu_limit; /* 0 = all compute units */
    int32_t reserved; /* must be 0 */
} moe_cfg;

/*
 * Expert weights, canonical layout (out x in, K contiguous), G groups:
 *  w1 [G, 2F, d]: rows 0..F-1 are W_gate, rows F..2F-1 are W_up.
 *  w2 [G, d, F]:  W_down.
 *  fp32 / bf16 modes: values; w1_scale = w2_scale = NULL.
 *  FP8 x MXFP4 mode:  w1 [G, 2F, d/2] and w2 [G, d, F/2] bytes of e2m1 codes;
 *                     w1_scale [G, 2F, d/32], w2_scale [G, d, F/32] e8m0 bytes.
 *  FP8 x FP8 mode:    w1 [G, 2F, d] and w2 [G, d, F] e4m3 codes; w1_scale [G, 2F, d/128],
 *                     w2_scale [G, d, F/128] fp32 powers of two.
 */
typedef struct {
    const void *w1, *w1_scale, *w2, *w2_scale;
} moe_weights;

/* Device error codes stored in the workspace's sticky word (first error wins). */
#define MOE_DEVERR_NONE 0
#define MOE_DEVERR_INDEX 1     /* an expert index outside [0, E) */
#define MOE_DEVERR_DUP 2       /* a token chose the same expert twice */
#define MOE_DEVERR_NONFINITE 3 /* a selection key is NaN or infinite */
#define MOE_DEVERR_TIMEOUT 4   /* a bounded wait in the persistent kernel expired */
#define MOE_DEVERR_OVERFLOW 5  /* moe_ep_ffn: received rows exceed the receive buffer, or a count < 0 */

/* Human-readable name of a status code (static string). */
const char *moe_status_str(moe_status s);

/* Checks that the current HIP device is gfx950. MOE_OK or MOE_ERR_ARCH / MOE_ERR_LAUNCH. */
moe_status moe_device_check(void);

/*
 * Bytes of device workspace every call with this configuration needs (the same
 * size serves all entry points).  0 if cfg is invalid.  The workspace holds the
 * sticky error word, dispatch block counts, the tile plan, the intermediate h
 * (and its FP8 scales), and the persistent kernel's counters.
 */
size_t moe_workspace_bytes(const moe_cfg *cfg);

/*
 * Where an intermediate result lives in a workspace, for verification tools (the
 * layout is otherwise private and may change between versions of the library).
 *  MOE_WS_ERROR:   the error words (256 bytes; the sticky error word first).
 *  MOE_WS_H:       h, the SwiGLU output per dispatched row [T*k + n_shared*T, F]: fp32
 *                  (F32 mode), bf16 (BF16 mode) or e4m3 codes (FP8 x MXFP4 mode).
 *  MOE_WS_H_SCALE: FP8 x MXFP4 mode: h's power-of-two fp32 scales [rows, F/128]
 *                  (0 bytes in the other modes).
 * moe_ffn and moe_layer_fused leave h there; row r is dispatched row r.
 * *offset and *bytes (host memory) receive the region's byte offset from the start of
 * the workspace and its size.  MOE_ERR_SHAPE for an unknown region.
 */
#define MOE_WS_ERROR 0
#define MOE_WS_H 1
#define MOE_WS_H_SCALE 2
moe_status moe_workspace_region(const moe_cfg *cfg, int32_t region, size_t *offset, size_t *bytes);

/*
 * Clears the sticky error word and the persistent kernel's synchronisation words
 * (stream-ordered).  A workspace must be zero-filled, or cleared by this call, before
 * its first moe_layer_fused; every moe_layer_fused launch leaves those words zero
 * again (also after a timeout), so one clear per workspace suffices.
 */
moe_status moe_clear_device_error(const moe_cfg *cfg, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Copies the sticky error word to *code_out (host memory) and synchronises
 * `stream`.  Returns MOE_ERR_DEVICE if the word is non-zero.
 */
moe_status moe_read_device_error(const moe_cfg *cfg, const void *ws, int32_t *code_out, hipStream_t stream);

/*
 * Router, selection and gates (MoE lesson "FFN swap" and "Build it, Step 1:
 * router"; MoE playbook "How it works", score and select).
 *  x [T, d]        activations (fp32 in F32 mode, else bf16)
 *  w_router [E, d] router weight (same dtype as x)
 *  bias [E]        fp32 selection bias, or NULL for zeros (MoE lesson "Load balancing")
 *  topk_idx [T, k]  int32 out: chosen experts, descending key, ties to the lower index
 *  topk_gate [T, k] fp32 out: gates
 *  logits [T, E]    fp32 out or NULL: x W_r^T
 *  keys [T, E]      fp32 out or NULL: selection keys
 *  ws: workspace (the error word and the split-K partial logits).
 */
moe_status moe_route(const moe_cfg *cfg, const void *x, const void *w_router, const float *bias,
                     int32_t *topk_idx, float *topk_gate, float *logits, float *keys, void *ws,
                     size_t ws_bytes, hipStream_t stream);

/*
 * Dispatch: group the T*k (token, choice) slots by expert (Mega MoE wiki,
 * "How it works": tokens are sent to their experts before the expert MLPs).
 * Slot s = t*k + j.  Rows of expert e are offsets[e] .. offsets[e+1]-1, in
 * ascending token order; the shared expert (group E) owns rows T*k + t.
 *  topk_idx [T, k]     int32 in
 *  x [T, d]            activations (read only in FP8 x MXFP4 mode, else may be NULL)
 *  counts [G]          int32 out: rows per group (counts[E] = T when n_shared)
 *  offsets [G + 1]     int32 out: exclusive prefix of counts
 *  slot_to_row [T*k]   int32 out
 *  row_to_slot [T*k]   int32 out: inverse permutation
 *  xq [T, d]           FP8 mode: uint8 e4m3 codes out (token order; gathered on load)
 *  xq_scale [T, d/128] FP8 mode: fp32 power-of-two scales out
 * Indices outside [0, E) or repeated within a token set the device error word
 * (MOE_DEVERR_INDEX / MOE_DEVERR_DUP); the outputs are then unspecified.
 */
moe_status moe_dispatch(const moe_cfg *cfg, const int32_t *topk_idx, const void *x, int32_t *counts,
                        int32_t *offsets, int32_t *slot_to_row, int32_t *row_to_slot, uint8_t *xq,
                        float *xq_scale, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * The capacity variant of the dispatch: expert capacity with token dropping (MoE
 * lesson, factory.pai-world.com, "The load-balancing problem", item 2: each expert takes
 * at most C x N / E tokens and the rest skip the layer).  `capacity` is that bound in
 * slots per routed expert -- for a capacity factor C, floor(C * T * k / E), the N of the
 * lesson's bound being the T*k routed slots (with k = 1, the tokens).  Of the slots that
 * chose expert e, the first `capacity` in slot order (ascending token order, as in the
 * dropless dispatch) are kept; the shared expert has no capacity.  Row layout, with
 * D = the number of dropped slots:
 *  rows 0 .. D-1         the dropped slots, expert by expert, in slot order (never computed);
 *  rows offsets[e] ..    expert e's kept slots, offsets[0] = D, offsets[E] = T*k;
 *  rows T*k + t          the shared expert (as in moe_dispatch).
 * So moe_ffn runs unchanged on these offsets (only kept rows belong to a group), and
 * moe_combine leaves dropped slots out: their slot_to_row is -1 (their gates are not
 * renormalised).
 *  capacity            >= 0 (0 drops every routed slot)
 *  counts [G]          int32 out: kept rows per group (counts[E] = T when n_shared)
 *  dropped [E]         int32 out: dropped slots per routed expert (the overflow)
 *  offsets [G + 1]     int32 out: first row of each group, as above
 *  slot_to_row [T*k]   int32 out: the row of a kept slot, -1 for a dropped one
 *  row_to_slot [T*k]   int32 out: the slot of every row (dropped rows included)
 *  x, xq, xq_scale     as in moe_dispatch (the FP8 activation stage)
 * Bad or duplicate indices set the device error word as in moe_dispatch.
 */
moe_status moe_dispatch_capacity(const moe_cfg *cfg, const int32_t *topk_idx, const void *x, int32_t capacity,
                                 int32_t *counts, int32_t *dropped, int32_t *offsets, int32_t *slot_to_row,
                                 int32_t *row_to_slot, uint8_t *xq, float *xq_scale, void *ws, size_t ws_bytes,
                                 hipStream_t stream);

/*
 * Aux-loss-free load balancing, one update of the per-expert selection bias that
 * moe_route adds to the keys (MoE lesson, "The load-balancing problem", the DeepSeek-V3
 * scheme, and "Build it -- Step 2: route 100 tokens"): after a step, bias[e] -= gamma
 * for a routed expert used more than the mean load, bias[e] += gamma for one used less,
 * unchanged for one exactly on it (compared in integers: counts[e] * E against the sum
 * of the E counts).  fp32 additions, on device, stream-ordered.
 *  counts [>= E]  int32 in: routed slots per expert -- the counts moe_dispatch writes (or,
 *                 under the capacity variant, counts + dropped: the load the router asked
 *                 for); only the first E entries are read
 *  bias [E]       fp32 in/out
 *  gamma          >= 0
 */
moe_status moe_bias_update(const moe_cfg *cfg, const int32_t *counts, float *bias, float gamma, hipStream_t stream);

/*
 * moe_dispatch for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  Same arguments,
 * kernels and results as moe_dispatch, without a workspace: the per-(dispatch block,
 * expert) counts those kernels need live in a fixed 1 MiB device array of the library
 * (one per GPU, held until the process ends), so dispatch_blocks(T) * E * 4 bytes must
 * fit -- (T + 255) / 256 * E <= 262144, e.g. T <= 262144 at E = 256; larger shapes
 * return MOE_ERR_WORKSPACE.  The call allocates nothing.
 *  err: device pointer to one int32, the sticky error word for bad or duplicate indices
 *       (first error wins; the caller clears it), or NULL to skip the checks' report.
 * Every call on a GPU shares that GPU's array: calls that overlap on one GPU (two
 * streams, two threads) race and must be serialised by the caller.  Each call writes
 * every array word it reads first, so nothing needs clearing between calls.
 */
moe_status moe_dispatch_noalloc(const moe_cfg *cfg, const int32_t *topk_idx, const void *x, int32_t *counts,
                                int32_t *offsets, int32_t *slot_to_row, int32_t *row_to_slot, uint8_t *xq,
                                float *xq_scale, int32_t *err, hipStream_t stream);

/*
 * The FP8 activation quantiser on its own: rows of K values (K a multiple of 128) to
 * e4m3 codes with one power-of-two fp32 scale per 1x128 block along K -- the rule the
 * FP8 x MXFP4 mode applies to x (moe_dispatch) and to h (the linear1 epilogue), with the
 * same conversion instructions.  Scale 2^e, e the smallest integer with
 * max|v| <= 448 * 2^e over the block (clamped to [-127, 127]; an all-zero block has
 * e = 0); code_i = e4m3 round-to-nearest-even of v_i * 2^-e (Mega MoE blog,
 * donniechu.com, spec table: FP8 activations).  Feeds moe_gemm_fp8_mxfp4.
 *  in [rows, K]         fp32 (in_dtype MOE_QUANT_IN_F32) or bf16 (MOE_QUANT_IN_BF16)
 *  codes [rows, K]      uint8 out
 *  scales [rows, K/128] fp32 out
 * Inputs must be finite.  rows == 0 is a no-op.
 */
#define MOE_QUANT_IN_F32 0
#define MOE_QUANT_IN_BF16 1
moe_status moe_quant_e4m3(const void *in, int32_t in_dtype, int64_t rows, int32_t K, uint8_t *codes, float *scales,
                          hipStream_t stream);

/*
 * The dense FP8 x MXFP4 GEMM that ships alongside the fused MoE kernel (Mega MoE blog,
 * donniechu.com, "What's new"), on the same scaled-MFMA tiles as the expert linears:
 *   C[M, N] = A[M, K] . B[N, K]^T,  fp32 accumulation, C rounded to bf16 (nearest even).
 *  a [M, K]        uint8 e4m3 codes (OCP E4M3FN), a_scale [M, K/128] fp32 power-of-two scales
 *                  per 1x128 block (e.g. from moe_quant_e4m3)
 *  b [N, K/2]      uint8 MXFP4: e2m1 codes, even K index in the low nibble; b_scale [N, K/32]
 *                  e8m0 bytes (the PyTorch Linear layout, out x in)
 *  c [M, N]        bf16 out
 *  ws              MOE_GEMM_WORKSPACE_BYTES of device scratch (the tile plan)
 * Limits: 0 <= M < 2^31, N and K multiples of 128 up to 65536.  M == 0 is a no-op.
 */
#define MOE_GEMM_WORKSPACE_BYTES 256
moe_status moe_gemm_fp8_mxfp4(int64_t M, int32_t N, int32_t K, const uint8_t *a, const float *a_scale,
                              const uint8_t *b, const uint8_t *b_scale, void *c, void *ws, size_t ws_bytes,
                              hipStream_t stream);

/*
 * One expert-parallel rank's share of the layer (Mega MoE wiki, aiki.softdaddy-o.com,
 * "Why it matters": EP8 with per-rank batches; Mega MoE blog, "What's new": the dispatch
 * sends each token's FP8 row to the ranks that own its experts, and the expert outputs go
 * back for the combine).  The rank owns cfg->E local experts (plus the replicated shared
 * expert when cfg->n_shared = 1) and runs them over the rows it received, then the shared
 * expert over its own cfg->T tokens; the outputs are left in receive order, ready to go
 * back.  Receive buffer layout: the rows of local expert e from source rank s form block
 * (e, s), blocks in expert-major order (expert 0: sources 0, 1, ..; then expert 1 ..),
 * each block's rows in the source's token order; recv_counts [E, n_src] (device int32)
 * holds the block sizes.  Same tile plan and kernels as moe_ffn's FP8 x MXFP4 path, the
 * rows read in place (no gather).
 *  cfg             mode MOE_MODE_FP8_MXFP4; E = local experts; T = the rank's own tokens
 *                  (shared expert rows; k is not used)
 *  w               the local experts' weights, canonical layout, G = E + n_shared groups
 *                  (the shared expert last)
 *  recv_capacity   rows the receive buffers hold (host value); the received rows
 *                  (sum of recv_counts) must fit, else MOE_DEVERR_OVERFLOW and the rows past
 *                  the capacity are not computed
 *  recv_xq [recv_capacity, d] uint8 e4m3 codes, recv_xs [recv_capacity, d/128] fp32 scales
 *  y_recv [recv_capacity, d] bf16 out: each received row's expert output, same row order
 *  xq [T, d], xs [T, d/128]: the rank's own tokens in FP8 (moe_quant_e4m3 or moe_dispatch)
 *  y_shared [T, d] bf16 out: the shared expert's output per own token
 *  ws              moe_ep_workspace_bytes(cfg, recv_capacity) bytes (error word first:
 *                  moe_read_device_error(cfg, ws, ...) reads it)
 */
size_t moe_ep_workspace_bytes(const moe_cfg *cfg, int64_t recv_capacity);
moe_status moe_ep_ffn(const moe_cfg *cfg, const moe_weights *w, int32_t n_src, const int32_t *recv_counts,
                      int64_t recv_capacity, const uint8_t *recv_xq, const float *recv_xs, void *y_recv,
                      const uint8_t *xq, const float *xs, void *y_shared, void *ws, size_t ws_bytes,
                      hipStream_t stream);

/*
 * Expert FFNs over the dispatched rows: linear1 (gate+up) with SwiGLU fused in
 * its epilogue, then linear2 (Mega MoE blog, donniechu.com, spec table).
 * Row r of group g reads token row_to_slot[r] / k (routed) or r - T*k (shared).
 *  w               weights (moe_weights, canonical layout)
 *  x [T, d]        activations (F32 / BF16 modes)
 *  xq, xq_scale    FP8 codes and scales from moe_dispatch (FP8 x MXFP4 mode)
 *  offsets [G+1], row_to_slot [T*k]: from moe_dispatch
 *  y_perm [T*k + n_shared*T, d] out: expert output per row (fp32 in F32 mode, else bf16)
 */
moe_status moe_ffn(const moe_cfg *cfg, const moe_weights *w, const void *x, const uint8_t *xq,
                   const float *xq_scale, const int32_t *offsets, const int32_t *row_to_slot, void *y_perm,
                   void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Gate-weighted combine (MoE playbook "How it works", combine step; MoE lesson
 * "Shared expert"):  y[t] = (((g_0 o_0 + g_1 o_1) + ...) + g_{k-1} o_{k-1}) + o_shared
 * in fp32 in exactly that order, then rounded to nearest even to y's dtype.  A slot
 * whose slot_to_row is negative (dropped by moe_dispatch_capacity) is left out.
 *  y_perm [T*k + n_shared*T, d], slot_to_row [T*k], topk_gate [T, k] in;  y [T, d] out.
 */
moe_status moe_combine(const moe_cfg *cfg, const void *y_perm, const int32_t *slot_to_row,
                       const float *topk_gate, void *y, hipStream_t stream);

/*
 * The whole layer in one persistent launch (Mega MoE wiki, "One-line definition":
 * the dispatch -> linear1 -> SwiGLU -> linear2 -> combine chain as one kernel): route,
 * dispatch, linear1 + SwiGLU, linear2 and combine, chained on device through
 * counters in the workspace with bounded waits.  A cooperative launch of every
 * workgroup the device (or cfg->cu_limit CUs) can hold at once; MOE_ERR_LAUNCH if the
 * runtime cannot make it co-resident.  A wait that exceeds 2 s sets
 * MOE_DEVERR_TIMEOUT (if the error word is still clear) and raises a second word
 * of the workspace's error region, so every later wait of the launch gives up at
 * once, whatever code the error word holds; a wait also gives up at once while the
 * error word reads MOE_DEVERR_TIMEOUT.  The call's outputs are then unspecified, and
 * the launch still clears its synchronisation words (and that second word) on exit.  Bitwise equal to
 * moe_route -> moe_dispatch -> moe_ffn -> moe_combine on the same inputs.
 *  x [T, d], w_router [E, d], bias [E] or NULL, w: as above; y [T, d] out.
 *  topk_idx_out [T, k], topk_gate_out [T, k], counts_out [G]: optional copies (NULL to skip).
 */
moe_status moe_layer_fused(const moe_cfg *cfg, const moe_weights *w, const void *x, const void *w_router,
                           const float *bias, void *y, int32_t *topk_idx_out, float *topk_gate_out,
                           int32_t *counts_out, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Kernel timing for measurement tools (not needed to run the layer).  While
 * enabled (on != 0), every kernel the library launches is bracketed by two HIP
 * events recorded on that launch's own stream, so timings include no host gaps.
 * Returns MOE_OK.
 */
moe_status moe_profile_enable(int on);

/*
 * Synchronises on the recorded events, writes one line "name launches total_ms\n"
 * per kernel name (in first-launch order) into the host buffer buf (NUL-terminated,
 * truncated to n bytes), clears the records and returns the full length of the
 * report in bytes.  buf may be NULL to clear the records only.
 */
int moe_profile_report(char *buf, size_t n);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
