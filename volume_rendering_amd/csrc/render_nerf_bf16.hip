// Fused NeRF-mode render kernels, bfloat16 networks.
#include "render_common.hpp"

namespace nerf {

template <int KIND>
static void launch_nerf(const RenderArgs& a, hipStream_t s) {
    hipLaunchKernelGGL((k_render_nerf<TBF16, KIND>), dim3((unsigned)((a.n_rays + 3) / 4)), dim3(256), 0, s, a);
}

void launch_render_nerf_bf16(int kind, const RenderArgs& a, hipStream_t s) {
    if (kind == NET_8x256) launch_nerf<NET_8x256>(a, s);
    else if (kind == NET_4x64) launch_nerf<NET_4x64>(a, s);
}

}  // namespace nerf
