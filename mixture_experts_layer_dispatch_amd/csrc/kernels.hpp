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
// partial logits (split-K and tiled paths), or nullptr to always use the one-pass kernels.
// route_tile_slices(s) > 0: the unfused router runs as a tiled GEMM over that many slices.
int route_splitk_slices(const Shape &s);
int route_tile_slices(const Shape &s);
long route_splitk_waves(const Shape &s, int nks);
hipError_t launch_route(const Shape &s, const void *x, const void *wr, const float *bias, int32_t *idx,
                        float *gate, float *logits, float *keys, int32_t *err, float *part, hipStream_t st);

// dispatch: block histogram, scan, scatter; FP8 activation quantisation
hipError_t launch_dispatch(const Shape &s, const int32_t *idx, int32_t *blockcounts, int32_t *counts,
                           int32_t *offsets, int32_t *slot_to_row, int32_t *row_to_slot, int32_t *err,
                           const uint16_t *x, uint8_t *xq, float *xs, hipStream_t st);
int dispatch_blocks(int T);
// the capacity variant: at most cap slots per routed expert (dbase: E ints of scratch)
hipError_t launch_dispatch_capacity(const Shape &s, const int32_t *idx, int cap, int32_t *blockcounts,
                                    int32_t *counts, int32_t *dropped, int32_t *offsets, int32_t *dbase,
                                    int32_t *slot_to_row, int32_t *row_to_slot, int32_t *err, const uint16_t *x,
                                    uint8_t *xq, float *xs, hipStream_t st);
// aux-loss-free bias update from routed per-expert counts
hipError_t launch_bias_update(const int32_t *counts, int E, float *bias, float gamma, hipStream_t st);
// stand-alone FP8 quantiser of fp32 (f32) or bf16 rows: nblocks 128-value blocks
hipError_t launch_quant_e4m3(const void *in, bool f32, long nblocks, uint8_t *q, float *qs, hipStream_t st);
int xcd_cus();  // CUs per XCD of the current device

// expert FFN
struct FfnPlan {
    int bm1, bn1, bm2, bn2;  // tile shapes of linear1 (N = 2F) and linear2 (N = d)
    int ntn1, ntn2;          // tiles along N per row tile (incl. K slices on the decode path)
    bool decode;             // FP8 x FP4 below 20 rows per group: weight-streaming kernels
    int ks;                  // decode: K slices of linear1
};
FfnPlan ffn_plan(const Shape &s);
size_t ffn_partial_bytes(const Shape &s);  // decode: fp32 linear1 partials [ks][rows][2F]
// FP8 decode: the workgroup kernels run (and need no tile plan from tile_plan)
bool fp8_gemv_ok(const Shape &s, const FfnPlan &p);
// column quads per workgroup tile of the workgroup decode kernels (1, 2 or 4), for the
// 32-column tiles ntn per row tile of linear1 (lin1) or linear2
int fp8_gemv_qc(const Shape &s, int ntn);
hipError_t launch_ffn(const Shape &s, const FfnPlan &p, const void *w1, const void *w1s, const void *w2,
                      const void *w2s, const void *x, const uint8_t *xq, const float *xs, const int32_t *offsets,
                      const int32_t *row_to_slot, void *h, float *hs, void *y_perm, int32_t *tile_start,
                      float *upart, hipStream_t st);

// dense FP8 x MXFP4 GEMM: c [M, N] bf16 = a [M, K] . b [N, K]^T; plan: 6 ints of scratch
hipError_t launch_gemm_fp8_dense(long M, int N, int K, const uint8_t *a, const float *as, const uint8_t *b,
                                 const uint8_t *bs, void *c, int32_t *plan, hipStream_t st);
// one expert-parallel rank's experts over its receive buffer (s.E local experts, s.T own tokens
// for the shared expert); plan: 3 (E + 1) + 6 ints; h, hs: (cap + S T) rows
hipError_t launch_ep_ffn(const Shape &s, int nsrc, const int32_t *recv_counts, long cap, const uint8_t *rq,
                         const float *rs, const uint8_t *w1, const uint8_t *w1s, const uint8_t *w2,
                         const uint8_t *w2s, void *y_recv, const uint8_t *xq, const float *xs, void *y_shared,
                         int32_t *plan, uint8_t *h, float *hs, int32_t *err, hipStream_t st);

// combine
hipError_t launch_combine(const Shape &s, const void *y_perm, const int32_t *slot_to_row, const float *gate,
                          void *y, hipStream_t st);

// Selection after the split-K router by one wave per token (else one workgroup per token)
inline bool route_select_by_wave(int E, int nks) { return E <= 256 && nks <= 16; }

// ---- persistent layer kernel -------------------------------------------------------
//
// One launch runs every step of the layer.  Work items are numbered in step order and
// dealt round-robin to co-resident workgroups (waves, on the decode path); an item waits
// only on items with smaller numbers, through counters in the workspace, so every wait
// ends once the grid is resident.

// Synchronisation words, in a workspace region of kSyncInts ints that must be zero before
// the first launch (every launch leaves it zero).  Same-address atomics serialise at the
// memory (about 12 ns each on MI355X), so a counter bumped by many items is spread over
// kSpread sub-counters, and a flag polled by many waves is written to kSpread replicas;
// every one sits in its own 128-byte slot.
constexpr int kSpread = 64;
constexpr int kSlot = 32;  // ints per 128-byte slot
enum SyncCounter {
    CNT_QUANT = 0,  // FP8 activation items done
    CNT_ROUTE,      // router items done
    CNT_SELECT,     // split-K router: selection items done
    CNT_COUNT,      // dispatch histogram blocks done
    CNT_SCATTER,    // dispatch scatter blocks done
    CNT_LIN1,       // tiled path: workgroups past linear1
    CNT_LIN2,       // linear2 items (decode) or workgroups past linear2 (tiled) done
    CNT_EXIT,       // workgroups finished
    CNT_QUEUE,      // 512-thread tiled path: GEMM items taken, one sub-counter per queue
    CNT_SWIGLU,     // decode with weight streams: workgroups past SwiGLU
    NUM_COUNTERS
};
enum SyncFlag {
    FLAG_PLAN = 0,  // scan and tile plans published
    FLAG_FRONT,     // everything before linear1 done: activations, plan, permutation
    NUM_FLAGS
};
constexpr int kSyncTopExit = (NUM_COUNTERS + NUM_FLAGS) * kSpread * kSlot;  // single counters
constexpr int kSyncTopScatter = kSyncTopExit + kSlot;
constexpr size_t kSyncInts = (size_t)kSyncTopScatter + kSlot;
// decode path, per 32-row tile: 8 sub-counters of its linear1 items (slots 0-7), their
// top counter (8), 8 replicas of its "partial sums ready" flag (9-16), the counter of its
// SwiGLU blocks (17) and 8 replicas of its "h ready" flag (18-25)
constexpr int kRowTileSlots = 26;

enum RouterKind { ROUTER_SPLITK = 0, ROUTER_MFMA = 1, ROUTER_VALU8 = 2, ROUTER_VALU32 = 3, ROUTER_TILE = 4 };
// routers that leave K-slice partial logits for separate selection items
__host__ __device__ inline bool router_in_slices(int kind) { return kind == ROUTER_SPLITK || kind == ROUTER_TILE; }

struct FusedArgs {
    int T, d, E, k, F, S, G, gating;
    const void *x, *wr;
    const float *bias;
    const void *w1, *w1s, *w2, *w2s;
    void *y;
    int32_t *idx;
    float *gate;
    int32_t *counts;
    // workspace
    int32_t *err, *sync, *done1, *blockcounts, *offsets, *s2r, *r2s, *ts1, *ts2;
    uint8_t *xq;
    float *xs;
    void *h;
    float *hs;
    void *yperm;
    float *rpart, *upart;
    // plan
    int router, nks, nblk;
    int sel4;  // split-K router: tokens per selection item (a wave each in turn), or 0: one token per item
    int bm, ntn1, ntn2, ks;
    long rows;
    int nm;   // row tiles bound (kRowTileSlots slots each in done1)
    // workgroup item ranges: [0, b_r) quant, [b_r, b_sel) router, [b_sel, b_cnt) select,
    // [b_cnt, b_plan) histogram, b_plan plan, [b_plan + 1, b_end) scatter, then the GEMMs
    long b_r, b_sel, b_cnt, b_plan, b_end;
    long n1, n2;  // fp32 path: linear1 and linear2 items
    long ncb;     // combine items (workgroups of 256 lanes; waves of 64 on the decode path)
    // decode with workgroup weight streams: column quads per workgroup tile and weight blocks
    // in flight per wave of linear1 and linear2 (0: the decode path's per-wave tiles)
    int sq1, sd1, sq2, sd2;
};

size_t fused_lds_bytes(const Shape &s, const FfnPlan &p);
int fused_row_tiles(const Shape &s, const FfnPlan &p);  // bound of row tiles (counters needed)
hipError_t launch_layer_fused(const Shape &s, const FfnPlan &p, FusedArgs &a, int cu_limit, hipStream_t st);

}  // namespace moe
