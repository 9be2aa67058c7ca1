// Persistent layer kernel, bf16 instantiations.
#include "fused_dev.hpp"

namespace moe {

hipError_t launch_fused_bf16(FusedArgs &a, int bm, int bn2, size_t lds, int cu_limit, hipStream_t st) {
    if (bm == 256 && bn2 == 256) return launch_fused_kernel8<MODE_BF16>(a, lds, cu_limit, st);
    if (bm == 256) return launch_fused_kernel<MODE_BF16, 256, 128>(a, lds, cu_limit, st);
    if (bn2 == 256) return launch_fused_kernel<MODE_BF16, 128, 256>(a, lds, cu_limit, st);
    return launch_fused_kernel<MODE_BF16, 128, 128>(a, lds, cu_limit, st);
}

}  // namespace moe
