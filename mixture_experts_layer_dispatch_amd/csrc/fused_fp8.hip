// Persistent layer kernel, FP8 x MXFP4 instantiations (tiled and decode) and the FP8 x FP8 one.
#include "fused_dev.hpp"

namespace moe {

// w8: the 8-wave tiles apply (their A operands addressed with 32-bit byte offsets)
hipError_t launch_fused_fp8(FusedArgs &a, bool decode, int bm, int bn2, bool w8, size_t lds, int cu_limit,
                            hipStream_t st) {
    if (decode) {
        if (a.sq1 > 0) {
            // eight weight blocks in flight per wave at one workgroup per CU (the stand-alone
            // kernels' deep ring), four at two
            int dev = 0, cus = 0, per_cu = 0;
            hipError_t e = hipGetDevice(&dev);
            if (e == hipSuccess) e = fused_occupancy((const void *)fused_decode_kernel<0>, dev, 256, lds, cus, per_cu);
            if (e != hipSuccess) return e;
            const bool two = per_cu >= 2;
            a.sd1 = !two && a.sq1 == 4 ? 8 : 4;
            a.sd2 = two ? 4 : 8;
        }
        return launch_fused_fn((const void *)fused_decode_kernel<0>, a, lds, cu_limit, st);
    }
    if (bm == 256 && bn2 == 256 && w8) return launch_fused_kernel8<MODE_FP8>(a, lds, cu_limit, st);
    if (bm == 256 && bn2 == 256) return launch_fused_kernel<MODE_FP8, 256, 256>(a, lds, cu_limit, st);
    if (bm == 256) return launch_fused_kernel<MODE_FP8, 256, 128>(a, lds, cu_limit, st);
    if (bn2 == 256) return launch_fused_kernel<MODE_FP8, 128, 256>(a, lds, cu_limit, st);
    return launch_fused_kernel<MODE_FP8, 128, 128>(a, lds, cu_limit, st);
}

// FP8 x FP8: the 256-thread kernel with the 128-row FP8 x FP8 tiles (linear2 bn2 columns wide)
hipError_t launch_fused_fp8x8(FusedArgs &a, int bn2, size_t lds, int cu_limit, hipStream_t st) {
    if (bn2 == 256) return launch_fused_kernel<MODE_FP8X8, 128, 256>(a, lds, cu_limit, st);
    return launch_fused_kernel<MODE_FP8X8, 128, 128>(a, lds, cu_limit, st);
}

}  // namespace moe
