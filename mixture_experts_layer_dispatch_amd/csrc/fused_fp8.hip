// Persistent layer kernel, FP8 x MXFP4 instantiations (tiled and decode) and the FP8 x FP8 one.
#include "fused_dev.hpp"

namespace moe {

// w8: the 8-wave tiles apply (their A operands addressed with 32-bit byte offsets)
hipError_t launch_fused_fp8(FusedArgs &a, bool decode, int bm, int bn2, bool w8, size_t lds, int cu_limit,
                            hipStream_t st) {
    if (decode) return launch_fused_fn((const void *)fused_decode_kernel<0>, a, lds, cu_limit, st);
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
