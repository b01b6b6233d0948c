// Standalone network kernels, bfloat16 matrix inputs.
#include "mlp_kernel.hpp"

namespace nerf {

void launch_mlp_bf16(int kind, const void* packed, const float* ex, const float* ev, int64_t n, int spr, float* raw,
                    hipStream_t s) {
    switch (kind) {
        case NET_8x256: launch_mlp_t<TBF16, NET_8x256>(packed, ex, ev, n, spr, raw, s); break;
        case NET_4x64: launch_mlp_t<TBF16, NET_4x64>(packed, ex, ev, n, spr, raw, s); break;
        case NET_CELL_2x32: launch_mlp_t<TBF16, NET_CELL_2x32>(packed, ex, ev, n, spr, raw, s); break;
        case NET_HASH_FIELD: launch_mlp_t<TBF16, NET_HASH_FIELD>(packed, ex, ev, n, spr, raw, s); break;
        default: break;
    }
}

}  // namespace nerf
