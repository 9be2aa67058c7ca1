// Host planning of the persistent layer kernel: router kind, item ranges, LDS size, and
// the launch of the matching instantiation (fp32 here; bf16 and FP8 in their own files).
#include "dispatch_dev.hpp"
#include "fused_dev.hpp"
#include "kernels.hpp"

#include <mutex>
#include <vector>

namespace moe {

hipError_t launch_fused_bf16(FusedArgs &a, int bm, int bn2, size_t lds, int cu_limit, hipStream_t st);
hipError_t launch_fused_fp8(FusedArgs &a, bool decode, int bm, int bn2, bool w8, size_t lds, int cu_limit,
                            hipStream_t st);
hipError_t launch_fused_fp8x8(FusedArgs &a, int bn2, size_t lds, int cu_limit, hipStream_t st);

namespace {

int router_kind(const Shape &s, int nks) {
    if (nks > 0) return ROUTER_SPLITK;
    if (s.mode != MODE_F32 && s.E % 32 == 0) return ROUTER_MFMA;
    return s.E <= 8 ? ROUTER_VALU8 : ROUTER_VALU32;
}

size_t router_lds(const Shape &s, int kind) {
    switch (kind) {
        case ROUTER_SPLITK: return (size_t)4 * s.E * 4;
        case ROUTER_MFMA: return (size_t)kRouteTok * s.E * 4;
        default: return (size_t)4 * s.E * 4;
    }
}

// FP8 8-wave tiles: their A operands (x codes, h codes) addressed with 32-bit byte offsets
bool fp8_w8(const Shape &s) { return (long)s.T * s.d < (1L << 32) && s.rows() * (long)s.F < (1L << 32); }

// the 512-thread kernel with the 8-wave tiles runs
bool fused_w8(const Shape &s, const FfnPlan &p) {
    if (s.mode == MODE_F32 || p.decode || p.bm1 != 256 || p.bn2 != 256) return false;
    return s.mode == MODE_BF16 || fp8_w8(s);
}

size_t gemm_lds(const Shape &s, const FfnPlan &p) {
    if (s.mode == MODE_F32 || p.decode) return 0;
    if (s.mode == MODE_FP8X8) return fp8x8_tile_lds<256>();
    const bool b256 = p.bm1 == 256, n256 = p.bn2 == 256;
    if (b256 && n256 && s.mode == MODE_BF16) return bf16_tile8_lds();
    if (b256 && n256 && fp8_w8(s)) return fp8_tile8_lds();
    if (s.mode == MODE_BF16) {
        const size_t l1 = b256 ? bf16_tile_lds<256, 256>() : bf16_tile_lds<128, 256>();
        const size_t l2 = b256 ? (n256 ? bf16_tile_lds<256, 256>() : bf16_tile_lds<256, 128>())
                               : (n256 ? bf16_tile_lds<128, 256>() : bf16_tile_lds<128, 128>());
        return l1 > l2 ? l1 : l2;
    }
    const size_t l1 = b256 ? fp8_tile_lds<256, 256>() : fp8_tile_lds<128, 256>();
    const size_t l2 = b256 ? (n256 ? fp8_tile_lds<256, 256>() : fp8_tile_lds<256, 128>())
                           : (n256 ? fp8_tile_lds<128, 256>() : fp8_tile_lds<128, 128>());
    return l1 > l2 ? l1 : l2;
}

// The decode variant runs the stand-alone kernels' workgroup weight streams as its linear
// phases: the shapes whose streams it instantiates (1024-wide K slices of linear1, 2048-wide
// rows of W2, whole quads of column tiles in every group), from two tokens on.  With one
// token its per-wave tiles and per-row-tile hand-offs were the faster ones (DeepSeek-V3
// shape: 142 against 149 us); from 64 tokens the streams are (1.38 against 1.99 ms).
bool fused_stream_ok(const Shape &s, const FfnPlan &p) {
    if (s.mode != MODE_FP8 || !p.decode || !fp8_gemv_ok(s, p) || s.T < 2) return false;
    return s.d / p.ks == 1024 && s.F == 2048 && (p.ntn1 / 4) % 4 == 0 && (p.ntn2 / 4) % 4 == 0;
}

}  // namespace

int fused_row_tiles(const Shape &s, const FfnPlan &p) {
    const long rows = s.rows(), G = s.G();
    return (int)((rows + p.bm1 - 1) / p.bm1 + (G < rows ? G : rows));
}

// router kind of the persistent kernel: the 512-thread kernel runs the stand-alone path's
// tiled router (same slices, same sums) where that one does
int fused_router_kind(const Shape &s, const FfnPlan &p) {
    if (fused_w8(s, p) && route_tile_slices(s) > 0) return ROUTER_TILE;
    return router_kind(s, route_splitk_slices(s));
}

size_t fused_lds_bytes(const Shape &s, const FfnPlan &p) {
    const int kind = fused_router_kind(s, p);
    size_t b = gemm_lds(s, p);
    const size_t r = kind == ROUTER_TILE ? bf16_tile8_lds() : router_lds(s, kind);
    const size_t m = (size_t)4 * s.E * 8 + (size_t)(s.E + 256) * 4, plan = (2 * 1032 + 256) * 4;
    const size_t cached = p.decode ? (size_t)3 * (s.G() + 1) * 4 : 0;  // the plan, kept in LDS
    for (size_t v : {r, m, plan, cached}) b = v > b ? v : b;
    if (fused_stream_ok(s, p)) {  // the weight streams' plan and staging buffers
        const int rmax = s.T < 32 ? s.T : 32;
        for (size_t v : {fp8_gemv_lds(s.G(), rmax, 1024), fp8_gemv_lds(s.G(), rmax, 2048)}) b = v > b ? v : b;
    }
    return b;
}

hipError_t fused_occupancy(const void *fn, int dev, int threads, size_t lds, int &cus, int &per_cu) {
    struct Entry {
        const void *fn;
        int dev, threads;
        size_t lds;
        int cus, per_cu;
    };
    static std::mutex mu;
    static std::vector<Entry> cache;
    std::lock_guard<std::mutex> lk(mu);
    for (const Entry &c : cache)
        if (c.fn == fn && c.dev == dev && c.threads == threads && c.lds == lds) {
            cus = c.cus;
            per_cu = c.per_cu;
            return hipSuccess;
        }
    if (lds > 65536) {
        // the cap of the kernel's dynamic LDS: the whole 160 KB of a CU, so that every LDS
        // size a later launch asks for is within it
        hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (e != hipSuccess) return e;
    }
    hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, lds);
    if (e != hipSuccess) return e;
    cache.push_back({fn, dev, threads, lds, cus, per_cu});
    return hipSuccess;
}

hipError_t launch_layer_fused(const Shape &s, const FfnPlan &p, FusedArgs &a, int cu_limit, hipStream_t st) {
    a.T = s.T; a.d = s.d; a.E = s.E; a.k = s.k; a.F = s.F; a.S = s.S; a.G = s.G(); a.gating = s.gating;
    a.nks = route_splitk_slices(s);
    a.router = fused_router_kind(s, p);
    a.nblk = dispatch_blocks(s.T);
    a.bm = p.bm1;
    a.ntn1 = p.ntn1;
    a.ntn2 = p.ntn2;
    a.ks = p.ks;
    a.rows = s.rows();
    // row-tile counters: only the decode variant's hand-offs use (and clear) them
    a.nm = p.decode ? fused_row_tiles(s, p) : 0;
    // FP8 activation items: contiguous ranges of at least 64 blocks of 128, at most 256 items
    const long nblocks_q = fp8_act(s.mode) ? (long)s.T * (s.d / 128) : 0;
    long nq = (nblocks_q + 63) / 64;
    if (nq > 256) nq = 256;
    long nr;
    switch (a.router) {
        case ROUTER_SPLITK: nr = (route_splitk_waves(s, a.nks) + 3) / 4; break;
        case ROUTER_TILE: nr = (long)((s.T + 255) / 256) * (s.E / 256) * a.nks; break;
        case ROUTER_MFMA: nr = (s.T + kRouteTok - 1) / kRouteTok; break;
        default: nr = (s.T + 3) / 4; break;
    }
    // selection by waves: tokens per item -- 4 at decode sizes (parallel waves), 32 at large T
    // (each item's hand-off, a few microseconds, is paid once per 32 tokens)
    a.sel4 = router_in_slices(a.router) && route_select_by_wave(s.E, a.nks) ? (s.T >= 2048 ? 32 : 4) : 0;
    const long nsel = !router_in_slices(a.router) ? 0 : a.sel4 ? (s.T + a.sel4 - 1) / a.sel4 : s.T;
    a.b_r = nq;
    a.b_sel = a.b_r + nr;
    a.b_cnt = a.b_sel + nsel;
    // with a single dispatch block the plan item also counts and scatters it
    const long nsplit = a.nblk == 1 ? 0 : a.nblk;
    a.b_plan = a.b_cnt + nsplit;
    a.b_end = (a.b_plan + 1 + nsplit + 7) / 8 * 8;
    a.n1 = (a.rows * s.F + 255) / 256;
    a.n2 = (a.rows * s.d + 255) / 256;
    const int V = s.mode == MODE_F32 ? 4 : 8;
    const long lanes_c = (long)s.T * (s.d / V);
    a.ncb = p.decode ? (lanes_c + kWave - 1) / kWave : (lanes_c + 255) / 256;
    // decode: workgroup weight streams where their shapes apply (column quads per tile as in
    // the stand-alone kernels, 1 where those take 2); the blocks in flight follow from the
    // occupancy at launch
    a.sq1 = a.sq2 = a.sd1 = a.sd2 = 0;
    if (fused_stream_ok(s, p)) {
        a.sq1 = fp8_gemv_qc(s, p.ntn1) == 4 ? 4 : 1;
        a.sq2 = fp8_gemv_qc(s, p.ntn2) == 4 ? 4 : 1;
    }
    const size_t lds = fused_lds_bytes(s, p);
    if (s.mode == MODE_F32) return launch_fused_kernel<MODE_F32, 128, 128>(a, lds, cu_limit, st);
    if (s.mode == MODE_BF16) return launch_fused_bf16(a, p.bm1, p.bn2, lds, cu_limit, st);
    if (s.mode == MODE_FP8X8) return launch_fused_fp8x8(a, p.bn2, lds, cu_limit, st);
    return launch_fused_fp8(a, p.decode, p.bm1, p.bn2, fp8_w8(s), lds, cu_limit, st);
}

}  // namespace moe
