// Launchers for the gfx950 MoE kernels; called by the C ABI in api.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace moe {

// per-kernel timing hooks (prof.hip)
void prof_begin(hipStream_t st);
void prof_end(const char *name, hipStream_t st);
int prof_report(char *buf, size_t n);
extern std::atomic<int> g_prof_on;

// hipLaunchKernelGGL bracketed by the timing hooks
#define MOE_LAUNCH(name, kernel, grid, block, lds, stream, ...)                  \
    do {                                                                        \
        ::moe::prof_begin(stream);                                              \
        hipLaunchKernelGGL(kernel, grid, block, lds, stream, __VA_ARGS__);      \
        ::moe::prof_end(name, stream);                                          \
    } while (0)

struct Shape {
    int T, d, E, k, F, S, gating, mode;
    int G() const { return E + S; }
    long rows() const { return (long)T * k + (long)S * T; }
};

// router: logits, keys, top-k, gates.  part: fp32 scratch of route_splitk_slices(s) * T * E
// partial logits (few-token split-K path), or nullptr to always use the one-pass kernels.
constexpr int kRouteSplitMaxT = 128;
int route_splitk_slices(const Shape &s);
hipError_t launch_route(const Shape &s, const void *x, const void *wr, const float *bias, int32_t *idx,
                        float *gate, float *logits, float *keys, int32_t *err, float *part, hipStream_t st);

// dispatch: block histogram, scan, scatter; FP8 activation quantisation
hipError_t launch_dispatch(const Shape &s, const int32_t *idx, int32_t *blockcounts, int32_t *counts,
                           int32_t *offsets, int32_t *slot_to_row, int32_t *row_to_slot, int32_t *err,
                           hipStream_t st);
hipError_t launch_quant_x(const Shape &s, const uint16_t *x, uint8_t *xq, float *xs, hipStream_t st);
int dispatch_blocks(int T);

// expert FFN
struct FfnPlan {
    int bm1, bn1, bm2, bn2;  // tile shapes of linear1 (N = 2F) and linear2 (N = d)
    int ntn1, ntn2;          // tiles along N per row tile (incl. K slices on the decode path)
    bool decode;             // FP8 x FP4 with few rows per group: weight-streaming kernels
    int ks;                  // decode: K slices of linear1
};
FfnPlan ffn_plan(const Shape &s);
size_t ffn_partial_bytes(const Shape &s);  // decode: fp32 linear1 partials [ks][rows][2F]
hipError_t launch_ffn(const Shape &s, const FfnPlan &p, const void *w1, const void *w1s, const void *w2,
                      const void *w2s, const void *x, const uint8_t *xq, const float *xs, const int32_t *offsets,
                      const int32_t *row_to_slot, void *h, float *hs, void *y_perm, int32_t *tile_start,
                      float *upart, hipStream_t st);

// combine
hipError_t launch_combine(const Shape &s, const void *y_perm, const int32_t *slot_to_row, const float *gate,
                          void *y, hipStream_t st);

}  // namespace moe
