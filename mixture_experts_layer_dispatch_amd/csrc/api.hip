// C ABI of libmoe.so: validation, workspace layout and launches.
#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>

#include "../../include/moe.h"

#include "kernels.hpp"

using namespace moe;

namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// FP8 activations (x and h quantised in-layer): the FP8 x MXFP4 and FP8 x FP8 modes
bool fp8_mode(const moe_cfg *c) { return c->mode == MOE_MODE_FP8_MXFP4 || c->mode == MOE_MODE_FP8_FP8; }

moe_status validate(const moe_cfg *c) {
    if (!c) return MOE_ERR_NULL;
    if (c->mode < MOE_MODE_F32 || c->mode > MOE_MODE_FP8_FP8) return MOE_ERR_MODE;
    if (c->gating < MOE_GATE_SOFTMAX || c->gating > MOE_GATE_SIGMOID) return MOE_ERR_MODE;
    if (c->T < 0 || c->T > (1 << 20)) return MOE_ERR_SHAPE;
    if (c->E < 1 || c->E > 1024 || c->k < 1 || c->k > 16 || c->k > c->E) return MOE_ERR_SHAPE;
    if (c->d < 128 || c->d % 128 || c->d > 65536 || c->F < 128 || c->F % 128 || c->F > 65536) return MOE_ERR_SHAPE;
    if (c->n_shared != 0 && c->n_shared != 1) return MOE_ERR_SHAPE;
    if (c->reserved != 0 || c->cu_limit < 0) return MOE_ERR_SHAPE;
    if ((long long)c->T * (c->k + c->n_shared) >= (1LL << 31)) return MOE_ERR_SHAPE;
    return MOE_OK;
}

Shape shape_of(const moe_cfg *c) {
    return Shape{c->T, c->d, c->E, c->k, c->F, c->n_shared, c->gating, c->mode};
}

// Workspace regions (byte offsets, each aligned to 256).
struct Layout {
    size_t err, blockcounts, dbase, tiles, h, hs, rpart, upart;      // every path
    size_t idx, gate, counts, offsets, s2r, r2s, xq, xs, yperm, sync, done1;  // fused path
    size_t total;
};

Layout layout_of(const moe_cfg *c) {
    Layout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off += (bytes + 255) & ~(size_t)255;
        return o;
    };
    const size_t T = c->T, k = c->k, E = c->E, G = c->E + c->n_shared, d = c->d, F = c->F;
    const size_t rows = T * k + c->n_shared * T;
    const bool fp8 = fp8_mode(c), f32 = c->mode == MOE_MODE_F32;
    L.err = take(256);  // sticky error word
    L.blockcounts = take((size_t)dispatch_blocks(c->T) * E * 4);
    L.dbase = take(E * 4);  // capacity variant: first dropped row per expert
    L.tiles = take(2 * (G + 1) * 4);
    L.h = take(rows * F * (f32 ? 4 : fp8 ? 1 : 2));
    L.hs = fp8 ? take(rows * (F / 128) * 4) : 0;
    {
        const Shape s = Shape{c->T, c->d, c->E, c->k, c->F, c->n_shared, c->gating, c->mode};
        L.rpart = take((size_t)route_splitk_slices(s) * T * E * 4);
        L.upart = take(ffn_partial_bytes(s));
    }
    L.idx = take(T * k * 4);
    L.gate = take(T * k * 4);
    L.counts = take(G * 4);
    L.offsets = take((G + 1) * 4);
    L.s2r = take(T * k * 4);
    L.r2s = take(T * k * 4);
    L.xq = fp8 ? take(T * d) : 0;
    L.xs = fp8 ? take(T * (d / 128) * 4) : 0;
    L.yperm = take(rows * d * (f32 ? 4 : 2));
    {
        const Shape s = Shape{c->T, c->d, c->E, c->k, c->F, c->n_shared, c->gating, c->mode};
        L.sync = take(kSyncInts * 4);
        L.done1 = take((size_t)fused_row_tiles(s, ffn_plan(s)) * kRowTileSlots * kSlot * 4);
    }
    L.total = off;
    return L;
}

template <typename T>
T *at(void *ws, size_t off) {
    return (T *)((uint8_t *)ws + off);
}

moe_status check_ws(const moe_cfg *c, const void *ws, size_t ws_bytes) {
    if (!ws) return MOE_ERR_WORKSPACE;
    if (!aligned16(ws)) return MOE_ERR_ALIGN;
    if (ws_bytes < layout_of(c).total) return MOE_ERR_WORKSPACE;
    return MOE_OK;
}

moe_status launched(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH; }

// gfx950 check, cached per device.
std::mutex g_arch_mu;
int g_arch_ok[64];  // 0 unknown, 1 ok, 2 not gfx950

moe_status arch_check() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_LAUNCH;
    if (dev < 0 || dev >= 64) return MOE_ERR_ARCH;
    std::lock_guard<std::mutex> lk(g_arch_mu);
    if (g_arch_ok[dev] == 0) {
        hipDeviceProp_t p;
        if (hipGetDeviceProperties(&p, dev) != hipSuccess) return MOE_ERR_LAUNCH;
        g_arch_ok[dev] = std::strncmp(p.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    }
    return g_arch_ok[dev] == 1 ? MOE_OK : MOE_ERR_ARCH;
}

__global__ void zero_words_kernel(int32_t *p, int n) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0;
}

}  // namespace

#define MOE_TRY(expr)                    \
    do {                                 \
        moe_status _s = (expr);          \
        if (_s != MOE_OK) return _s;     \
    } while (0)

extern "C" {

const char *moe_status_str(moe_status s) {
    switch (s) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_NULL: return "MOE_ERR_NULL: a required pointer is NULL";
        case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE: shape outside the supported limits";
        case MOE_ERR_MODE: return "MOE_ERR_MODE: unknown mode or gating";
        case MOE_ERR_ALIGN: return "MOE_ERR_ALIGN: device pointer not 16-byte aligned";
        case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing or too small";
        case MOE_ERR_LAUNCH: return "MOE_ERR_LAUNCH: HIP launch or runtime call failed";
        case MOE_ERR_ARCH: return "MOE_ERR_ARCH: current device is not gfx950";
        case MOE_ERR_DEVICE: return "MOE_ERR_DEVICE: a kernel reported an error";
    }
    return "unknown moe_status";
}

moe_status moe_device_check(void) { return arch_check(); }

moe_status moe_profile_enable(int on) {
    g_prof_on.store(on ? 1 : 0);
    return MOE_OK;
}

int moe_profile_report(char *buf, size_t n) { return prof_report(buf, n); }

size_t moe_workspace_bytes(const moe_cfg *cfg) {
    if (validate(cfg) != MOE_OK) return 0;
    return layout_of(cfg).total;
}

moe_status moe_workspace_region(const moe_cfg *cfg, int32_t region, size_t *offset, size_t *bytes) {
    MOE_TRY(validate(cfg));
    if (!offset || !bytes) return MOE_ERR_NULL;
    const Layout L = layout_of(cfg);
    const size_t rows = (size_t)cfg->T * cfg->k + (size_t)cfg->n_shared * cfg->T;
    const bool fp8 = fp8_mode(cfg), f32 = cfg->mode == MOE_MODE_F32;
    switch (region) {
        case MOE_WS_ERROR: *offset = L.err; *bytes = 256; return MOE_OK;
        case MOE_WS_H: *offset = L.h; *bytes = rows * cfg->F * (f32 ? 4 : fp8 ? 1 : 2); return MOE_OK;
        case MOE_WS_H_SCALE: *offset = L.hs; *bytes = fp8 ? rows * (cfg->F / 128) * 4 : 0; return MOE_OK;
        default: return MOE_ERR_SHAPE;
    }
}

moe_status moe_clear_device_error(const moe_cfg *cfg, void *ws, size_t ws_bytes, hipStream_t stream) {
    MOE_TRY(validate(cfg));
    MOE_TRY(check_ws(cfg, ws, ws_bytes));
    MOE_TRY(arch_check());
    // the error word and the persistent kernel's synchronisation words
    const Layout L = layout_of(cfg);
    MOE_LAUNCH("clear_error", zero_words_kernel, dim3(1), dim3(64), 0, stream, at<int32_t>(ws, L.err), 64);
    MOE_LAUNCH("clear_error", zero_words_kernel, dim3((unsigned)((kSyncInts + 255) / 256)), dim3(256), 0, stream,
               at<int32_t>(ws, L.sync), (int)kSyncInts);
    return launched(hipGetLastError());
}

moe_status moe_read_device_error(const moe_cfg *cfg, const void *ws, int32_t *code_out, hipStream_t stream) {
    MOE_TRY(validate(cfg));
    if (!ws || !code_out) return MOE_ERR_NULL;
    int32_t v = 0;
    if (hipMemcpyAsync(&v, ws, sizeof(v), hipMemcpyDeviceToHost, stream) != hipSuccess) return MOE_ERR_LAUNCH;
    if (hipStreamSynchronize(stream) != hipSuccess) return MOE_ERR_LAUNCH;
    *code_out = v;
    return v == 0 ? MOE_OK : MOE_ERR_DEVICE;
}

moe_status moe_quant_e4m3(const void *in, int32_t in_dtype, int64_t rows, int32_t K, uint8_t *codes, float *scales,
                          hipStream_t stream) {
    if (in_dtype != MOE_QUANT_IN_F32 && in_dtype != MOE_QUANT_IN_BF16) return MOE_ERR_MODE;
    if (rows < 0 || K < 128 || K % 128 || (double)rows * K >= 9.0e18) return MOE_ERR_SHAPE;
    if (rows == 0) return MOE_OK;
    if (!in || !codes || !scales) return MOE_ERR_NULL;
    for (const void *p : {in, (const void *)codes, (const void *)scales})
        if (!aligned16(p)) return MOE_ERR_ALIGN;
    MOE_TRY(arch_check());
    return launched(launch_quant_e4m3(in, in_dtype == MOE_QUANT_IN_F32, (long)(rows * (K / 128)), codes, scales,
                                      stream));
}

moe_status moe_gemm_fp8_mxfp4(int64_t M, int32_t N, int32_t K, const uint8_t *a, const float *a_scale,
                              const uint8_t *b, const uint8_t *b_scale, void *c, void *ws, size_t ws_bytes,
                              hipStream_t stream) {
    if (M < 0 || M > (1L << 31) - 1 || N < 128 || N % 128 || N > 65536 || K < 128 || K % 128 || K > 65536)
        return MOE_ERR_SHAPE;
    if (M == 0) return MOE_OK;
    if (!a || !a_scale || !b || !b_scale || !c || !ws) return MOE_ERR_NULL;
    for (const void *p : {(const void *)a, (const void *)a_scale, (const void *)b, (const void *)b_scale, (const void *)c,
                          (const void *)ws})
        if (!aligned16(p)) return MOE_ERR_ALIGN;
    if (ws_bytes < MOE_GEMM_WORKSPACE_BYTES) return MOE_ERR_WORKSPACE;
    MOE_TRY(arch_check());
    return launched(launch_gemm_fp8_dense(M, N, K, a, a_scale, b, b_scale, c, (int32_t *)ws, stream));
}

namespace {
struct EpLayout {
    size_t err, plan, h, hs, total;
};
EpLayout ep_layout(const moe_cfg *c, int64_t cap) {
    EpLayout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off += (bytes + 255) & ~(size_t)255;
        return o;
    };
    const size_t rows = (size_t)cap + (size_t)c->n_shared * c->T;
    L.err = take(256);
    L.plan = take((3 * ((size_t)c->E + 1) + 6) * 4);
    L.h = take(rows * c->F);
    L.hs = take(rows * (c->F / 128) * 4);
    L.total = off;
    return L;
}
moe_status ep_validate(const moe_cfg *cfg, int64_t cap) {
    MOE_TRY(validate(cfg));
    if (cfg->mode != MOE_MODE_FP8_MXFP4) return MOE_ERR_MODE;
    if (cap < 0 || cap + (int64_t)cfg->n_shared * cfg->T >= (1LL << 31)) return MOE_ERR_SHAPE;
    return MOE_OK;
}
}  // namespace

size_t moe_ep_workspace_bytes(const moe_cfg *cfg, int64_t recv_capacity) {
    if (ep_validate(cfg, recv_capacity) != MOE_OK) return 0;
    return ep_layout(cfg, recv_capacity).total;
}

moe_status moe_ep_ffn(const moe_cfg *cfg, const moe_weights *w, int32_t n_src, const int32_t *recv_counts,
                      int64_t recv_capacity, const uint8_t *recv_xq, const float *recv_xs, void *y_recv,
                      const uint8_t *xq, const float *xs, void *y_shared, void *ws, size_t ws_bytes,
                      hipStream_t stream) {
    MOE_TRY(ep_validate(cfg, recv_capacity));
    if (n_src < 1 || n_src > 4096) return MOE_ERR_SHAPE;
    const bool routed = recv_capacity > 0, shared = cfg->n_shared && cfg->T > 0;
    if (!routed && !shared) return MOE_OK;
    if (!w || !w->w1 || !w->w1_scale || !w->w2 || !w->w2_scale || !ws) return MOE_ERR_NULL;
    if (routed && (!recv_counts || !recv_xq || !recv_xs || !y_recv)) return MOE_ERR_NULL;
    if (shared && (!xq || !xs || !y_shared)) return MOE_ERR_NULL;
    for (const void *p : {w->w1, w->w1_scale, w->w2, w->w2_scale, (const void *)recv_counts, (const void *)recv_xq,
                          (const void *)recv_xs, (const void *)y_recv, (const void *)xq, (const void *)xs,
                          (const void *)y_shared, (const void *)ws})
        if (p && !aligned16(p)) return MOE_ERR_ALIGN;
    const EpLayout L = ep_layout(cfg, recv_capacity);
    if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    MOE_TRY(arch_check());
    return launched(launch_ep_ffn(shape_of(cfg), n_src, recv_counts, recv_capacity, recv_xq, recv_xs,
                                  (const uint8_t *)w->w1, (const uint8_t *)w->w1_scale, (const uint8_t *)w->w2,
                                  (const uint8_t *)w->w2_scale, y_recv, xq, xs, y_shared, at<int32_t>(ws, L.plan),
                                  at<uint8_t>(ws, L.h), at<float>(ws, L.hs), at<int32_t>(ws, L.err), stream));
}

moe_status moe_route(const moe_cfg *cfg, const void *x, const void *w_router, const float *bias, int32_t *topk_idx,
                     float *topk_gate, float *logits, float *keys, void *ws, size_t ws_bytes, hipStream_t stream) {
    MOE_TRY(validate(cfg));
    if (cfg->T == 0) return MOE_OK;
    if (!x || !w_router || !topk_idx || !topk_gate) return MOE_ERR_NULL;
    for (const void *p : {x, w_router, (const void *)bias, (const void *)topk_idx, (const void *)topk_gate,
                          (const void *)logits, (const void *)keys})
        if (p && !aligned16(p)) return MOE_ERR_ALIGN;
    MOE_TRY(check_ws(cfg, ws, ws_bytes));
    MOE_TRY(arch_check());
    const Layout L = layout_of(cfg);
    return launched(launch_route(shape_of(cfg), x, w_router, bias, topk_idx, topk_gate, logits, keys,
                                 at<int32_t>(ws, L.err), at<float>(ws, L.rpart), stream));
}

moe_status moe_dispatch(const moe_cfg *cfg, const int32_t *topk_idx, const void *x, int32_t *counts,
                        int32_t *offsets, int32_t *slot_to_row, int32_t *row_to_slot, uint8_t *xq, float *xq_scale,
                        void *ws, size_t ws_bytes, hipStream_t stream) {
    MOE_TRY(validate(cfg));
    if (cfg->T == 0) return MOE_OK;
    const bool fp8 = fp8_mode(cfg);
    if (!topk_idx || !counts || !offsets || !slot_to_row || !row_to_slot) return MOE_ERR_NULL;
    if (fp8 && (!x || !xq || !xq_scale)) return MOE_ERR_NULL;
    for (const void *p : {(const void *)topk_idx, x, (const void *)counts, (const void *)offsets,
                          (const void *)slot_to_row, (const void *)row_to_slot, (const void *)xq,
                          (const void *)xq_scale})
        if (p && !aligned16(p)) return MOE_ERR_ALIGN;
    MOE_TRY(check_ws(cfg, ws, ws_bytes));
    MOE_TRY(arch_check());
    const Layout L = layout_of(cfg);
    const Shape s = shape_of(cfg);
    // FP8 mode: the activations are quantised by the same launch (an independent job)
    return launched(launch_dispatch(s, topk_idx, at<int32_t>(ws, L.blockcounts), counts, offsets, slot_to_row,
                                    row_to_slot, at<int32_t>(ws, L.err), fp8 ? (const uint16_t *)x : nullptr,
                                    fp8 ? xq : nullptr, fp8 ? xq_scale : nullptr, stream));
}

moe_status moe_dispatch_capacity(const moe_cfg *cfg, const int32_t *topk_idx, const void *x, int32_t capacity,
                                 int32_t *counts, int32_t *dropped, int32_t *offsets, int32_t *slot_to_row,
                                 int32_t *row_to_slot, uint8_t *xq, float *xq_scale, void *ws, size_t ws_bytes,
                                 hipStream_t stream) {
    MOE_TRY(validate(cfg));
    if (capacity < 0) return MOE_ERR_SHAPE;
    if (cfg->T == 0) return MOE_OK;
    const bool fp8 = fp8_mode(cfg);
    if (!topk_idx || !counts || !dropped || !offsets || !slot_to_row || !row_to_slot) return MOE_ERR_NULL;
    if (fp8 && (!x || !xq || !xq_scale)) return MOE_ERR_NULL;
    for (const void *p : {(const void *)topk_idx, x, (const void *)counts, (const void *)dropped,
                          (const void *)offsets, (const void *)slot_to_row, (const void *)row_to_slot,
                          (const void *)xq, (const void *)xq_scale})
        if (p && !aligned16(p)) return MOE_ERR_ALIGN;
    MOE_TRY(check_ws(cfg, ws, ws_bytes));
    MOE_TRY(arch_check());
    const Layout L = layout_of(cfg);
    return launched(launch_dispatch_capacity(shape_of(cfg), topk_idx, capacity, at<int32_t>(ws, L.blockcounts),
                                             counts, dropped, offsets, at<int32_t>(ws, L.dbase), slot_to_row,
                                             row_to_slot, at<int32_t>(ws, L.err), fp8 ? (const uint16_t *)x : nullptr,
                                             fp8 ? xq : nullptr, fp8 ? xq_scale : nullptr, stream));
}

moe_status moe_bias_update(const moe_cfg *cfg, const int32_t *counts, float *bias, float gamma, hipStream_t stream) {
    MOE_TRY(validate(cfg));
    if (!counts || !bias) return MOE_ERR_NULL;
    if (!aligned16(counts) || !aligned16(bias)) return MOE_ERR_ALIGN;
    if (!(gamma >= 0.0f) || gamma > 3.0e38f) return MOE_ERR_SHAPE;
    MOE_TRY(arch_check());
    return launched(launch_bias_update(counts, cfg->E, bias, gamma, stream));
}

moe_status moe_ffn(const moe_cfg *cfg, const moe_weights *w, const void *x, const uint8_t *xq, const float *xq_scale,
                   const int32_t *offsets, const int32_t *row_to_slot, void *y_perm, void *ws, size_t ws_bytes,
                   hipStream_t stream) {
    MOE_TRY(validate(cfg));
    if (cfg->T == 0) return MOE_OK;
    const bool fp8 = fp8_mode(cfg);
    if (!w || !w->w1 || !w->w2 || !offsets || !row_to_slot || !y_perm) return MOE_ERR_NULL;
    if (fp8 && (!w->w1_scale || !w->w2_scale || !xq || !xq_scale)) return MOE_ERR_NULL;
    if (!fp8 && !x) return MOE_ERR_NULL;
    for (const void *p : {w->w1, w->w2, w->w1_scale, w->w2_scale, x, (const void *)xq, (const void *)xq_scale,
                          (const void *)offsets, (const void *)row_to_slot, (const void *)y_perm})
        if (p && !aligned16(p)) return MOE_ERR_ALIGN;
    MOE_TRY(check_ws(cfg, ws, ws_bytes));
    MOE_TRY(arch_check());
    const Layout L = layout_of(cfg);
    const Shape s = shape_of(cfg);
    return launched(launch_ffn(s, ffn_plan(s), w->w1, w->w1_scale, w->w2, w->w2_scale, x, xq, xq_scale, offsets,
                               row_to_slot, at<void>(ws, L.h), fp8 ? at<float>(ws, L.hs) : nullptr, y_perm,
                               at<int32_t>(ws, L.tiles), at<float>(ws, L.upart), stream));
}

moe_status moe_combine(const moe_cfg *cfg, const void *y_perm, const int32_t *slot_to_row, const float *topk_gate,
                       void *y, hipStream_t stream) {
    MOE_TRY(validate(cfg));
    if (cfg->T == 0) return MOE_OK;
    if (!y_perm || !slot_to_row || !topk_gate || !y) return MOE_ERR_NULL;
    for (const void *p : {y_perm, (const void *)slot_to_row, (const void *)topk_gate, (const void *)y})
        if (!aligned16(p)) return MOE_ERR_ALIGN;
    MOE_TRY(arch_check());
    return launched(launch_combine(shape_of(cfg), y_perm, slot_to_row, topk_gate, y, stream));
}

moe_status moe_layer_fused(const moe_cfg *cfg, const moe_weights *w, const void *x, const void *w_router,
                           const float *bias, void *y, int32_t *topk_idx_out, float *topk_gate_out,
                           int32_t *counts_out, void *ws, size_t ws_bytes, hipStream_t stream) {
    MOE_TRY(validate(cfg));
    if (cfg->T == 0) return MOE_OK;
    const bool fp8 = fp8_mode(cfg);
    if (!w || !w->w1 || !w->w2 || !x || !w_router || !y) return MOE_ERR_NULL;
    if (fp8 && (!w->w1_scale || !w->w2_scale)) return MOE_ERR_NULL;
    for (const void *p : {w->w1, w->w2, w->w1_scale, w->w2_scale, x, w_router, (const void *)bias, (const void *)y,
                          (const void *)topk_idx_out, (const void *)topk_gate_out, (const void *)counts_out})
        if (p && !aligned16(p)) return MOE_ERR_ALIGN;
    MOE_TRY(check_ws(cfg, ws, ws_bytes));
    MOE_TRY(arch_check());
    const Layout L = layout_of(cfg);
    const Shape s = shape_of(cfg);
    int32_t *err = at<int32_t>(ws, L.err);
    int32_t *idx = topk_idx_out ? topk_idx_out : at<int32_t>(ws, L.idx);
    float *gate = topk_gate_out ? topk_gate_out : at<float>(ws, L.gate);
    int32_t *counts = counts_out ? counts_out : at<int32_t>(ws, L.counts);
    FusedArgs a{};
    a.x = x;
    a.wr = w_router;
    a.bias = bias;
    a.w1 = w->w1;
    a.w1s = w->w1_scale;
    a.w2 = w->w2;
    a.w2s = w->w2_scale;
    a.y = y;
    a.idx = idx;
    a.gate = gate;
    a.counts = counts;
    a.err = err;
    a.sync = at<int32_t>(ws, L.sync);
    a.done1 = at<int32_t>(ws, L.done1);
    a.blockcounts = at<int32_t>(ws, L.blockcounts);
    a.offsets = at<int32_t>(ws, L.offsets);
    a.s2r = at<int32_t>(ws, L.s2r);
    a.r2s = at<int32_t>(ws, L.r2s);
    a.ts1 = at<int32_t>(ws, L.tiles);
    a.ts2 = a.ts1 + (s.G() + 1);
    a.xq = fp8 ? at<uint8_t>(ws, L.xq) : nullptr;
    a.xs = fp8 ? at<float>(ws, L.xs) : nullptr;
    a.h = at<void>(ws, L.h);
    a.hs = fp8 ? at<float>(ws, L.hs) : nullptr;
    a.yperm = at<void>(ws, L.yperm);
    a.rpart = at<float>(ws, L.rpart);
    a.upart = at<float>(ws, L.upart);
    return launched(launch_layer_fused(s, ffn_plan(s), a, cfg->cu_limit, stream));
}

}  // extern "C"
