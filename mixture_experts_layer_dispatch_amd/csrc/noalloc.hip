// moe_dispatch_noalloc: the dispatch (S5-S7) for callers that cannot allocate device
// memory -- code under HIP graph capture, tight serving loops, harnesses that forbid
// allocation.  It runs the very kernels of moe_dispatch; the only scratch those kernels
// need, the per-(dispatch block, expert) counts and bases, lives in a fixed device array
// of this library instead of a caller workspace.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/moe.h"

#include "kernels.hpp"

namespace {

// Per-(dispatch block, expert) counts, rewritten in place into the blocks' base rows.
// Every word a call reads was written earlier by the same call, so nothing needs
// clearing between calls.  One copy per GPU, held until the process ends.
constexpr size_t kScratchBytes = (size_t)1 << 20;
static __device__ __align__(256) int32_t scratch[kScratchBytes / sizeof(int32_t)];

// Device address of `scratch` per device.  In host code the array's name is only a
// host-side stand-in: kernels get this address instead.
std::mutex g_mu;
void *g_scratch[64];

moe_status scratch_of(void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_LAUNCH;
    if (dev < 0 || dev >= 64) return MOE_ERR_LAUNCH;
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_LAUNCH;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return MOE_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

extern "C" moe_status moe_dispatch_noalloc(const moe_cfg *cfg, const int32_t *topk_idx, const void *x,
                                           int32_t *counts, int32_t *offsets, int32_t *slot_to_row,
                                           int32_t *row_to_slot, uint8_t *xq, float *xq_scale, int32_t *err,
                                           hipStream_t stream) {
    // shape and mode checks of moe_dispatch (a zero-sized workspace query fails on a bad cfg)
    if (!cfg) return MOE_ERR_NULL;
    if (moe_workspace_bytes(cfg) == 0) {
        if (cfg->mode < MOE_MODE_F32 || cfg->mode > MOE_MODE_FP8_FP8 || cfg->gating < MOE_GATE_SOFTMAX ||
            cfg->gating > MOE_GATE_SIGMOID)
            return MOE_ERR_MODE;
        return MOE_ERR_SHAPE;
    }
    if (cfg->T == 0) return MOE_OK;
    const bool fp8 = cfg->mode == MOE_MODE_FP8_MXFP4 || cfg->mode == MOE_MODE_FP8_FP8;
    if (!topk_idx || !counts || !offsets || !slot_to_row || !row_to_slot) return MOE_ERR_NULL;
    if (fp8 && (!x || !xq || !xq_scale)) return MOE_ERR_NULL;
    for (const void *p : {(const void *)topk_idx, x, (const void *)counts, (const void *)offsets,
                          (const void *)slot_to_row, (const void *)row_to_slot, (const void *)xq,
                          (const void *)xq_scale})
        if (p && !aligned16(p)) return MOE_ERR_ALIGN;
    if (err && ((uintptr_t)err & 3u)) return MOE_ERR_ALIGN;
    // the scratch holds dispatch_blocks(T) x E block counts
    const size_t need = (size_t)moe::dispatch_blocks(cfg->T) * cfg->E * sizeof(int32_t);
    if (need > kScratchBytes) return MOE_ERR_WORKSPACE;
    moe_status st = moe_device_check();
    if (st != MOE_OK) return st;
    void *buf = nullptr;
    st = scratch_of(&buf);
    if (st != MOE_OK) return st;
    const moe::Shape s{cfg->T, cfg->d, cfg->E, cfg->k, cfg->F, cfg->n_shared, cfg->gating, cfg->mode};
    const hipError_t e = moe::launch_dispatch(s, topk_idx, (int32_t *)buf, counts, offsets, slot_to_row, row_to_slot,
                                              err, fp8 ? (const uint16_t *)x : nullptr, fp8 ? xq : nullptr,
                                              fp8 ? xq_scale : nullptr, stream);
    return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}
